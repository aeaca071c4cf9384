// The C interface (include/w4a16.h): argument checks, the work plan and the
// launches.  Nothing here allocates, prints or synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "../../include/w4a16.h"
#include "format.hpp"
#include "internal.hpp"
#include "layout.hpp"

namespace w4a16 {

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];  // 0 = not yet queried

// Compute units of the current device, cached per device.  Returns <= 0 on
// failure.
int current_cus(int* device_out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (device_out) *device_out = dev;
  if (dev >= kMaxDevices) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return -1;
    return cus;
  }
  int cus = g_cus[dev].load(std::memory_order_relaxed);
  if (cus > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return -1;
  g_cus[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Shapes every entry point that reads permuted weights accepts.
int check_kn(int K, int N, bool allow_empty_n) {
  if (K <= 0 || K % kBlockK) return W4A16_ERR_SHAPE;
  if (N < 0 || N % kBlockN || (!allow_empty_n && N == 0)) return W4A16_ERR_SHAPE;
  // the kernels index one column block's K blocks, and divide a K-block
  // index by the group, in 32-bit arithmetic: K < 2^23 keeps both exact
  if (K >= (1 << 23)) return W4A16_ERR_SHAPE;
  // scale offsets (row * N + column) are 32-bit as well
  if ((int64_t)(K / kBlockK) * N >= ((int64_t)1 << 31)) return W4A16_ERR_SHAPE;
  return W4A16_OK;
}

int check_group(int K, int group) {
  if (group <= 0 || group % kBlockK || K % group) return W4A16_ERR_GROUP;
  return W4A16_OK;
}

bool variant_is_compiled(const Plan& q, int fmt) {
  if (q.tile == 4) return fmt <= kFmtBf16Zp && sk_is_compiled(q.mb, q.nb, q.depth, q.wm, q.wk);
  if (fmt == kFmtSp24) {
    if (q.tile == 2) return lds_sp_is_compiled(q.mb, q.nb, q.wm, q.wk, q.depth);
    return q.tile == 0 && q.wm == 1 && sp_is_compiled(q.mb, q.nb, q.wk, q.depth);
  }
  if (q.tile == 2) return lds_is_compiled(q.mb, q.nb, q.wm, q.wk, q.depth);
  if (q.wm != 1 || q.tile != 0) return false;
  return plan_is_compiled(q.mb, q.nb, q.wk, q.depth, fmt);
}

// Test and tuning override of the plan heuristic: a process-wide setting,
// seeded once from the environment variable W4A16_FORCE_PLAN when the
// library first plans a call, and replaced by w4a16_set_forced_plan.  The
// text is "mb,nb,wk,splits[,depth[,tile[,unused[,wm]]]]": a field <= 0 keeps
// the heuristic's value; tile is 0 (the default) for the streaming kernel,
// 2 for the LDS kernel, 4 for the stream-K kernel (wk = its waves along N,
// splits = its grid), and -1 for the plan the heuristic makes when it does
// not pick the stream-K kernel (the other fields are then ignored).  The override feeds the same kernels, and
// w4a16_workspace_bytes sees it as well, so sizes agree as long as it is
// not changed between the two calls.
struct ForcedPlan {
  bool set;
  int mb, nb, wk, splits, depth, tile, wm;
};

std::mutex g_force_mu;
ForcedPlan g_force{};
std::atomic<bool> g_force_any{false};
std::once_flag g_force_env_once;

// Parse an override; false if the text is not one.
bool parse_forced_plan(const char* text, ForcedPlan* out) {
  int mb = 0, nb = 0, wk = 0, splits = 0, depth = 0, tile = 0, unused = 0, wm = 0;
  if (std::sscanf(text, "%d,%d,%d,%d,%d,%d,%d,%d", &mb, &nb, &wk, &splits, &depth, &tile,
                  &unused, &wm) < 4)
    return false;
  if (tile != -1 && tile != 0 && tile != 2 && tile != 4) return false;
  *out = ForcedPlan{true, mb, nb, wk, splits, depth, tile, wm};
  return true;
}

void set_forced(const ForcedPlan& f) {
  std::lock_guard<std::mutex> lock(g_force_mu);
  g_force = f;
  g_force_any.store(f.set, std::memory_order_release);
}

void seed_forced_from_env() {
  std::call_once(g_force_env_once, [] {
    const char* env = std::getenv("W4A16_FORCE_PLAN");
    ForcedPlan f{};
    if (env && *env && parse_forced_plan(env, &f)) set_forced(f);
  });
}

// Returns whether a forced plan replaced the heuristic's.
bool apply_forced_plan(Plan* p, const Plan& base, int KB, int fmt) {
  seed_forced_from_env();
  if (!g_force_any.load(std::memory_order_acquire)) return false;
  ForcedPlan f;
  {
    std::lock_guard<std::mutex> lock(g_force_mu);
    f = g_force;
  }
  if (!f.set) return false;
  if (f.tile == -1) {  // the heuristic's plan without the stream-K kernel
    *p = base;
    return false;
  }
  // fields left open come from the heuristic's plan of the forced family
  Plan q = (f.tile == 4) == (p->tile == 4) ? *p : base;
  q.tile = f.tile;
  if (f.mb > 0) q.mb = f.mb;
  if (f.nb > 0) q.nb = f.nb;
  if (f.wk > 0) q.wk = f.wk;
  if (f.splits > 0) q.splits = (f.tile == 4 || f.splits <= KB) ? f.splits : KB;
  if (q.tile != 4 && q.splits < 1) q.splits = 1;  // the stream-K plan's grid is set later
  if (q.tile == 4 && f.splits <= 0) q.splits = 0;  // stream-K: the heuristic grid
  if (f.depth > 0) q.depth = f.depth;
  q.wm = f.wm > 0 ? f.wm : 1;
  if (!variant_is_compiled(q, fmt)) {
    // keep the forced tile but take the first compiled depth for it
    for (int d : {4, 3, 2, 1}) {
      q.depth = d;
      if (variant_is_compiled(q, fmt)) break;
    }
  }
  if (!variant_is_compiled(q, fmt)) return false;
  *p = q;
  return true;
}

// The plan of one call on a device with `cus` compute units as one line of
// text (w4a16_describe, w4a16_plan_describe).
int describe_plan(int M, int K, int N, int group, int fmt, int cus, char* buf, size_t len) {
  if (!buf || len == 0) return W4A16_ERR_NULL;
  buf[0] = 0;
  if (M <= 0 || N == 0) return W4A16_ERR_SHAPE;
  int rc = check_kn(K, N, false);
  if (rc != W4A16_OK) return rc;
  rc = check_group(K, group);
  if (rc != W4A16_OK) return rc;
  if (cus <= 0) return W4A16_ERR_DEVICE;
  const Plan p = make_plan(M, K, N, group, cus, fmt);
  if (p.tile == 4)
    std::snprintf(buf, len,
                  "gemm_sk_kernel<%d,%d,%d,%d> grid=%dx1x1 block=%d tiles=%dx%d splits=%d "
                  "workspace=%zu",
                  p.mb, p.nb, p.depth, p.wk, p.splits, 64 * p.wk, p.tiles_n,
                  p.tiles_m,
                  p.splits, p.workspace_bytes);
  else if (p.tile == 2) {
    const int tiles = p.tiles_n * p.tiles_m;
    const int head = p.splits > 1 ? p.head : tiles;
    std::snprintf(buf, len,
                  "gemm_lds_kernel<%d,%d,%d,%d,%d> grid=%dx1x1 block=%d tiles=%dx%d whole=%d "
                  "splits=%d workspace=%zu",
                  p.mb, p.nb, p.wm, p.wk, p.depth, head + (tiles - head) * p.splits,
                  64 * p.wm * p.wk, p.tiles_n, p.tiles_m, head, p.splits, p.workspace_bytes);
  }
  else
    std::snprintf(buf, len,
                  "gemm_kernel<%d,%d,%d,%d> grid=%dx%dx%d block=%d splits=%d workspace=%zu%s",
                  p.mb, p.nb, p.wk, p.depth, p.tiles_n, p.tiles_m, p.splits, 64 * p.wk,
                  p.splits, p.workspace_bytes,
                  activations_lds_bytes(p, M, K, fmt) ? " activations=lds" : "");
  return W4A16_OK;
}

int describe_fmt(int M, int K, int N, int group, int fmt, char* buf, size_t len) {
  if (!buf || len == 0) return W4A16_ERR_NULL;
  buf[0] = 0;
  if (M <= 0 || N == 0) return W4A16_ERR_SHAPE;
  int rc = check_kn(K, N, false);
  if (rc != W4A16_OK) return rc;
  rc = check_group(K, group);
  if (rc != W4A16_OK) return rc;
  return describe_plan(M, K, N, group, fmt, current_cus(nullptr), buf, len);
}

size_t workspace_fmt(int M, int K, int N, int group, int fmt) {
  if (M <= 0 || N == 0) return 0;
  if (check_kn(K, N, false) != W4A16_OK || check_group(K, group) != W4A16_OK) return 0;
  const int cus = current_cus(nullptr);
  if (cus <= 0) return 0;
  return make_plan(M, K, N, group, cus, fmt).workspace_bytes;
}

}  // namespace

// The heuristic (measured on MI355X at the Llama-2-7B layer shapes and an
// 8192 x 28672 prefill layer).
// Small batches (M <= 4, or M <= 16 with N < 8192) stream the weights:
// one 16-row block per wave.  Plans were chosen by sweeping every compiled
// variant and split count at the workload shapes (Llama-2-7B layers,
// 18432 x 73728, 28672 x 8192, 13824 x 5120, 8192 x 28672).
// With one activation row the activation fragments cost little, so narrow
// column tiles (16 or 32 columns) give the most workgroups; with 16 rows
// every wave re-reads its activation fragments, so wide tiles (64 columns)
// amortise them when N leaves enough tiles.  K is split across workgroups
// only as far as needed to give every compute unit work, keeping at least
// two K blocks per wave.  Larger batches go to the LDS kernel with 64 or 128
// rows per wave, so each weight is unpacked once for many rows.
//
// 2:4-sparse weights (format 5) take the same plans with three changes,
// measured at the Llama-2-7B layer shapes: the streaming kernel keeps two
// K blocks in flight (a slot is smaller; 11008 x 4096 at M = 16: 14.6 ->
// 12.2 us); 32 < M <= 128 runs 64 x 128 tiles as four waves of 64 x 32 (half
// the matrix instructions per activation fragment of the dense format, so
// wider wave tiles: 4096 x 12288 at M = 128: 26.6 -> 21.1 us); and the K
// split there is twice the dense one below a full wave of workgroups and
// none above it.
// Whether the stream-K kernel takes a call (4-bit dense formats only), and
// its tile: eight waves (two per SIMD, each with its own columns, so no
// weight is unpacked twice), every compute unit an equal share of the
// (tile, K block) iterations.  Measured against the whole-tile plans by
// graph replay over rotating weight copies:
//  * 9 to 64 rows, on a layer with at least 48 K blocks of 256 columns per
//    compute unit: 16*mb x 512 tiles.  18432 x 73728: 144-154 against
//    152-161 us at M = 16, 160 against 176-185 us at M = 32, 211 against
//    232-234 us at M = 64.  On smaller layers the fix-up and pipeline fill
//    cost 10-20 us that a grid of whole tiles does not pay (8192 x 28672,
//    28672 x 8192 and the Llama-2-7B layers: 1.16-2.9x slower).
//  * 65 to 128 rows, where the LDS plan splits K and the layer gives at
//    least 24 iterations of 128 x 256 tiles per compute unit: 128 x 256
//    tiles (waves of 128 x 32, the LDS plan's own), with no partial tiles
//    through the workspace and no last wave of workgroups half empty.
//    18432 x 73728: 329-339 against 354-366 us at M = 65..128; 28672 x 8192
//    at M = 128: 78-80 against 85-86 us.  Below that count (the Llama-2-7B
//    layers: 1.3-2.9x slower) and in prefill, where the LDS plan needs no
//    split (4-14% slower), the LDS kernel stays.
static bool stream_k_plan(int M, int KB, int N, int cus, int fmt, const Plan& base, Plan* p) {
  if (fmt > kFmtBf16Zp || M <= 8 || M > 128) return false;
  Plan q = *p;
  q.tile = 4;
  q.wm = 1;
  q.wk = 8;  // waves along N
  q.splits = 0;  // the stream-K grid is set below
  if (M <= 64) {
    const int64_t blocks = (int64_t)((N + 255) / 256) * KB;  // 256-column K blocks
    if (blocks < (int64_t)48 * cus) return false;
    q.nb = 4;
    q.mb = M <= 16 ? 1 : M <= 32 ? 2 : 4;
    q.depth = q.mb == 1 ? 4 : 3;  // as many stages as fit in LDS
  } else {
    const int64_t iters = (int64_t)((N + 255) / 256) * ((M + 127) / 128) * KB;
    if (base.tile != 2 || base.splits <= 1 || iters < (int64_t)24 * cus) return false;
    q.nb = 2;
    q.mb = 8;
    q.depth = 3;
  }
  *p = q;
  return true;
}

Plan make_plan(int M, int K, int N, int group, int cus, int fmt) {
  (void)group;
  Plan p{};
  p.wm = 1;
  const int n16 = N / kBlockN;
  const int KB = K / kBlockK;
  if (cus <= 0) cus = 256;
  // FP16 formats: the streaming kernel scales its FP32 sums, which makes it
  // the faster one at five to eight rows on every wide layer too
  const bool scaled_sums = fmt == kFmtF16 || fmt == kFmtF16Zp;
  if (M <= 4 || (M <= 16 && N < 8192) || (M <= 8 && (n16 >= 8 * cus || scaled_sums))) {
    // streaming kernel: activations straight from global memory (up to
    // M = 8 on very wide layers too: 18432 x 73728 at M = 8 took 128 us
    // against 145 us in the LDS kernel; at M = 16 the LDS kernel is ahead)
    p.mb = 1;
    if (M <= 4) {
      // 16-column tiles; 32 for wide N or deep K (there split three ways
      // below), 64 for very wide N.  Four waves per workgroup with 16- and
      // 64-column tiles when there are at least two tiles per compute unit,
      // else eight (measured: 18432 x 73728 at M = 1..4 126-131 us against
      // 130-142 us with eight; 4096 x 12288 at M = 1 9.4 against 10.0 us;
      // but 11008 x 4096, 256 tiles, 9.6 against 8.3 us; and 4096 x 22016
      // at M = 1 keeps eight waves of 32 columns, 14.1 against 14.7 us).
      // In the FP16 formats, whose 16-column tiles of eight waves scale the
      // sums (four waves of them scale the weights), 16-column tiles take
      // eight waves throughout: 4096 x 12288 at M = 1 / 2 / 4 7.9 / 8.3 / 9.0
      // against 8.4 / 9.0 / 10.1 us, 4096 x 8192 at M = 1 / 4 6.5 / 7.4
      // against 6.8 / 8.1 us, 5120 x 10240 at M = 1 8.8 against 9.5 us.
      p.nb = n16 >= 8 * cus ? 4 : (n16 >= 4 * cus || KB >= 96) ? 2 : 1;
      p.wk = p.nb != 2 && !(p.nb == 1 && scaled_sums) && n16 / p.nb >= 2 * cus ? 4 : 8;
      p.depth = 2;
    } else if (N >= 8192 && n16 < 8 * cus) {
      // five to eight rows, FP16 formats, wide layers: 64-column tiles of
      // four waves from 1536 column blocks, else 32-column tiles of eight
      // waves, unsplit.  Measured at M = 8 against the LDS kernel's 16-row
      // tiles (graph replay, same box): 8192 x 28672 25.7 against 30.3 us,
      // 4096 x 22016 12.9 against 16.2 us, 4096 x 12288 9.3 against
      // 11.1 us, 28672 x 8192 27.5 against 30.5 us (three K ranges: 30.7).
      p.nb = n16 >= 6 * cus ? 4 : 2;
      p.wk = p.nb == 4 ? 4 : 8;
      p.depth = 2;
    } else {
      p.nb = n16 >= 2 * cus || KB >= 64 ? 4 : 1;
      p.wk = 4;
      p.depth = KB >= 64 && KB < 96 ? 4 : 2;
      if (p.nb == 1 && scaled_sums) {
        // FP16 formats, narrow and shallow layers: 32-column tiles of eight
        // waves (which scale the sums), split in two by the rule below when
        // that still fits one workgroup per compute unit.  Same box:
        // 4096 x 4096 at M = 8 / 12 / 16 6.3 / 6.5 / 6.8 against 6.4 / 6.7 /
        // 7.0 us; 5120 x 5120 at M = 16 9.1 against 12.8 us (320 tiles of
        // 16 columns left a second, mostly empty wave of workgroups).
        p.nb = 2;
        p.wk = 8;
      }
    }
  } else if (M <= 32 && !(fmt != kFmtSp24 && M > 16 && KB >= 32 && KB <= 64 &&
                           (N + 255) / 256 <= cus / 8)) {
    // LDS kernel with 16- or 32-row tiles and 256 columns (eight waves of
    // 16 or 32 x 32): one activation tile in LDS serves every wave, where
    // the streaming kernel would have each wave load its own copy.  (17 to
    // 32 rows on narrow layers, 4096 <= K <= 8192, dense codes, take the
    // 64 x 128 tiles below: 4096 x 4096 at M = 32 10.5 against 11.5 us,
    // 5120 x 5120 11.8 against 13.1 us, 4096 x 8192 11.9 against 12.5 us.
    // 4096 x 12288 and wider keep these, 12.9 against 15.3 us; so does
    // deeper K, where the choice went both ways: 11008 x 4096 15.5 against
    // 16.4 us, but 13824 x 5120 20.3 against 18.1 us.)
    p.tile = 2;
    p.mb = M <= 16 ? 1 : 2;
    p.nb = 2;
    p.wk = 8;
    p.depth = 4;
  } else if (M <= 128) {
    // LDS kernel, 64 x 128 tiles (eight waves of 64 x 16, two per SIMD):
    // small tiles keep enough workgroups; each weight is unpacked once per
    // 64 rows.  Above 64 rows, where N gives at least half a tile per
    // compute unit at 128 columns, 128-row tiles read each weight once:
    // 128 x 128 as a 2 x 4 grid of 64 x 32 wave tiles, or, with two tiles
    // per compute unit, 128 x 256 (eight waves of 128 x 32).  Measured
    // 1.2x at 4096 x 22016 and 18432 x 73728 for M = 128.
    const int n128 = (N + 127) / 128;
    p.tile = 2;
    p.mb = 4;
    p.nb = 1;
    p.wk = 8;
    p.depth = 3;
    if (M > 64 && n128 >= 2 * cus) {
      p.mb = 8;
      p.nb = 2;
    } else if (M > 64 && 2 * n128 >= cus) {
      p.nb = 2;
      p.wm = 2;
      p.wk = 4;
    }
  } else {
    // prefill: 128 x 256 tiles (eight waves of 128 x 32), each weight
    // unpacked once per 128 rows
    p.tile = 2;
    p.mb = 8;
    p.nb = 2;
    p.wk = 8;
    p.depth = 3;
  }
  const bool sparse = fmt == kFmtSp24;
  if (sparse && p.tile == 0) p.depth = 2;
  if (sparse && M > 32 && M <= 128) {
    p.mb = 4;
    p.nb = 2;
    p.wm = 1;
    p.wk = 4;
    p.depth = 3;
  }
  auto shape = [&](Plan& q) {
    q.tm = 16 * q.mb * q.wm;
    q.tn = 16 * q.nb * (q.tile ? q.wk : 1);  // LDS and stream-K kernels split N over waves
    q.tiles_n = (N + q.tn - 1) / q.tn;
    q.tiles_m = (M + q.tm - 1) / q.tm;
  };
  shape(p);
  const int64_t tiles = (int64_t)p.tiles_n * p.tiles_m;
  // Split K only when the tiles leave many compute units idle: the
  // streaming kernel up to one workgroup per compute unit (two for deep K),
  // the tile and LDS kernels up to about one workgroup per compute unit.
  int64_t want;
  int64_t cap;
  if (p.tile && tiles < cus) {
    // fewer tiles than compute units: split K as far as whole splits fill
    // the compute units (a partly filled extra wave of workgroups costs
    // more than idle compute units), a power of two
    want = (sparse && M > 32 && M <= 128 ? 2 : 1) * cus / tiles;
    while (want & (want - 1)) want &= want - 1;
    cap = KB / 4 < 8 ? KB / 4 : 8;
    // from K = 4096 on, at least eight K blocks per split (K = 4096: four
    // splits, not eight).  64 x 128 tiles: 10.5-11.8 us against 11.3-14.4 us
    // with eight splits on 4096 x 4096, 4096 x 6144, 4096 x 8192 and
    // 5120 x 5120 at M = 24..48; 16-row tiles on 4096 x 8192 at M = 8 / 16:
    // 10.6 / 10.8 against 11.2 us.
    if (!sparse && KB >= 32 && KB / 8 < cap) cap = KB / 8;
  } else if (p.tile && sparse && M > 32 && M <= 128) {
    want = 1;
    cap = 1;
  } else if (p.tile) {
    // more tiles than compute units: the last wave of workgroups may run
    // nearly empty (288 tiles on 256 CUs keep 56% of them busy on average).
    // Take the smallest power-of-two split, with at least 16 K blocks per
    // split, that keeps 85% of the compute units busy.
    want = 1;
    for (int64_t sp = 1; sp <= 8 && sp * 16 <= KB; sp *= 2) {
      const int64_t wgs = tiles * sp;
      const int64_t waves_of_wgs = (wgs + cus - 1) / cus;
      if (wgs * 100 >= 85 * waves_of_wgs * cus) {
        want = sp;
        break;
      }
    }
    cap = 8;
  } else if (M <= 4 && KB >= 96 && n16 < 4 * cus) {
    // streaming, one to four rows, deep K (K >= 12288) and moderate N: three
    // K ranges per 32-column tile (measured best for 28672 x 8192 and
    // 13824 x 5120: 1.2-1.25x over unsplit 16-column tiles)
    want = 3;
    cap = KB / (2 * p.wk);
  } else if (M > 4 && KB >= 96 && N < 8192 && tiles < 2 * (int64_t)cus) {
    // streaming, five to sixteen rows, deep K: eight K ranges per 64-column
    // tile (13824 x 5120: 1.3x over the default below)
    want = 8;
    cap = KB / (2 * p.wk);
  } else {
    // one workgroup per compute unit, two for deep K (K >= 8192)
    const int64_t target = (KB >= 64 ? 2 : 1) * (int64_t)cus;
    want = 10 * tiles >= 6 * (int64_t)cus ? 1 : (target + tiles - 1) / tiles;
    cap = KB / (2 * p.wk);
  }
  if (cap < 1) cap = 1;
  if (want > cap) want = cap;
  if (want > 64) want = 64;
  p.splits = (int)(want < 1 ? 1 : want);
  const Plan base = p;  // the plan without the stream-K kernel
  stream_k_plan(M, KB, N, cus, fmt, base, &p);
  const bool forced = apply_forced_plan(&p, base, KB, fmt);
  shape(p);
  const int64_t ftiles = (int64_t)p.tiles_n * p.tiles_m;
  p.head = 0;
  if (p.tile == 4 && !variant_is_compiled(p, fmt)) return Plan{};  // not reached: plans name compiled variants
  if (p.tile == 4) {
    // Stream-K grid: one workgroup per compute unit, each with at least
    // kSkMinIters iterations (fewer workgroups for small problems), never
    // more workgroups than iterations.  With more tiles than the counter
    // header can count (one counter per tile and wave), every workgroup
    // takes whole tiles.
    const int64_t units = ftiles * ((KB + p.depth - 1) / p.depth);  // of depth K blocks
    int64_t g = p.splits > 0 ? p.splits : cus;
    if (p.splits <= 0 && g * kSkMinIters > units * p.depth)
      g = (units * p.depth + kSkMinIters - 1) / kSkMinIters;
    if (g > units) g = units;
    if (g < 1) g = 1;
    if (ftiles * p.wk * p.wm > kMaxSplitTiles) g = ftiles;
    p.splits = (int)g;
    p.workspace_bytes = sk_workspace_bytes(p.splits, p.tm, p.tn, (int)ftiles, KB, p.depth);
    return p;
  }
  if (p.tile == 2 && p.splits == 1 && !forced && ftiles > cus && KB >= 16) {
    // LDS kernel with more tiles than compute units: when the last wave of
    // workgroups would run at most half full, the whole waves' tiles run
    // whole and the rest are split in two along K, so the last wave takes
    // half a tile-time.  8192 x 28672 at M = 1024 (896 tiles on 256 CUs,
    // the fourth wave half full): 417-420 against 436-439 us.  Splitting
    // every tile writes and re-reads partials for all of them (6% slower
    // there), and a four-way split of a three-quarter-full last wave
    // (M = 512) measured 4-5% slower than none.
    const int64_t head = ftiles / cus * cus, tail = ftiles - head;
    if (tail > 0 && 2 * tail <= cus) {
      p.splits = 2;
      p.head = (int)head;
    }
  }
  if (ftiles - p.head > kMaxSplitTiles) {  // the counter header holds one per split tile
    p.splits = 1;
    p.head = 0;
  }
  p.workspace_bytes = 0;
  if (p.splits > 1) {
    p.workspace_bytes = kCounterHeaderBytes + (size_t)(ftiles - p.head) * p.splits * p.tm *
                                                  p.tn * sizeof(float);
  }
  return p;
}

}  // namespace w4a16

using namespace w4a16;

extern "C" {

int w4a16_layout_version(void) { return kLayoutVersion; }

int w4a16_set_forced_plan(const char* spec) {
  seed_forced_from_env();  // a later first plan must not overwrite this
  if (!spec || !*spec) {
    set_forced(ForcedPlan{});
    return W4A16_OK;
  }
  ForcedPlan f{};
  if (!parse_forced_plan(spec, &f)) return W4A16_ERR_SHAPE;
  set_forced(f);
  return W4A16_OK;
}

const char* w4a16_status_string(int status) {
  switch (status) {
    case W4A16_OK: return "W4A16_OK";
    case W4A16_ERR_NULL: return "W4A16_ERR_NULL";
    case W4A16_ERR_SHAPE: return "W4A16_ERR_SHAPE";
    case W4A16_ERR_GROUP: return "W4A16_ERR_GROUP";
    case W4A16_ERR_ALIGN: return "W4A16_ERR_ALIGN";
    case W4A16_ERR_WORKSPACE: return "W4A16_ERR_WORKSPACE";
    case W4A16_ERR_LAUNCH: return "W4A16_ERR_LAUNCH";
    case W4A16_ERR_DEVICE: return "W4A16_ERR_DEVICE";
    case W4A16_ERR_EPILOGUE: return "W4A16_ERR_EPILOGUE";
    case W4A16_ERR_DTYPE: return "W4A16_ERR_DTYPE";
    default: return "W4A16_ERR_UNKNOWN";
  }
}

size_t w4a16_packed_bytes(int K, int N) {
  if (K <= 0 || N <= 0) return 0;
  return (size_t)K * (size_t)N / 2;
}

size_t w4a16_workspace_bytes(int M, int K, int N, int group) {
  return workspace_fmt(M, K, N, group, kFmtF16);
}

int w4a16_describe(int M, int K, int N, int group, char* buf, size_t len) {
  return describe_fmt(M, K, N, group, kFmtF16, buf, len);
}

int w4a16_plan_describe(int M, int K, int N, int group, int format, int cus, char* buf,
                        size_t len) {
  if (!buf || len == 0) return W4A16_ERR_NULL;
  buf[0] = 0;
  if (format < kFmtF16 || format > kFmtSp24) return W4A16_ERR_DTYPE;
  return describe_plan(M, K, N, group, format, cus, buf, len);
}

int w4a16_repack(const uint32_t* Bq, uint32_t* Bpacked, int K, int N, void* stream) {
  if (!Bq || !Bpacked) return W4A16_ERR_NULL;
  int rc = check_kn(K, N, false);
  if (rc != W4A16_OK) return rc;
  if (!aligned16(Bq) || !aligned16(Bpacked)) return W4A16_ERR_ALIGN;
  const size_t bytes = w4a16_packed_bytes(K, N);
  if (overlap(Bq, bytes, Bpacked, bytes)) return W4A16_ERR_SHAPE;
  if (current_cus(nullptr) <= 0) return W4A16_ERR_DEVICE;
  if (launch_repack(Bq, Bpacked, K, N, static_cast<hipStream_t>(stream)) != hipSuccess)
    return W4A16_ERR_LAUNCH;
  return W4A16_OK;
}

int w4a16_dequant_debug(const uint32_t* Bpacked, const uint16_t* scales, uint16_t* W,
                        int K, int N, int group, void* stream) {
  if (!Bpacked || !scales || !W) return W4A16_ERR_NULL;
  int rc = check_kn(K, N, false);
  if (rc != W4A16_OK) return rc;
  rc = check_group(K, group);
  if (rc != W4A16_OK) return rc;
  if (!aligned16(Bpacked) || !aligned16(scales) || !aligned16(W)) return W4A16_ERR_ALIGN;
  if (current_cus(nullptr) <= 0) return W4A16_ERR_DEVICE;
  if (launch_dequant(Bpacked, scales, W, K, N, group, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return W4A16_ERR_LAUNCH;
  return W4A16_OK;
}

int w4a16_dequant_awq_debug(const uint32_t* Bpacked, const uint16_t* scales,
                            const uint8_t* zeros, uint16_t* W, int K, int N, int group,
                            int dtype, void* stream) {
  if (dtype != W4A16_DTYPE_F16 && dtype != W4A16_DTYPE_BF16) return W4A16_ERR_DTYPE;
  if (!Bpacked || !scales || !W) return W4A16_ERR_NULL;
  int rc = check_kn(K, N, false);
  if (rc != W4A16_OK) return rc;
  rc = check_group(K, group);
  if (rc != W4A16_OK) return rc;
  if (!aligned16(Bpacked) || !aligned16(scales) || !aligned16(W) ||
      (zeros && !aligned16(zeros)))
    return W4A16_ERR_ALIGN;
  if (current_cus(nullptr) <= 0) return W4A16_ERR_DEVICE;
  const int fmt = (dtype == W4A16_DTYPE_BF16 ? 2 : 0) + (zeros ? 1 : 0);
  if (launch_dequant_fmt(Bpacked, scales, zeros, W, K, N, group, fmt,
                         static_cast<hipStream_t>(stream)) != hipSuccess)
    return W4A16_ERR_LAUNCH;
  return W4A16_OK;
}

}  // extern "C"

namespace {

// ---- The allocation-free variant (w4a16_gemm_noalloc) -------------------
// Its split-K partials and arrival counters live in this file-scope device
// array instead of a caller's workspace.  Each device the library runs on
// holds its own copy until the process ends.  In host code the name
// `scratch` is only a host-side stand-in: kernels get the device address
// taken with hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = (size_t)W4A16_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes > kCounterHeaderBytes, "the scratch holds the counter header");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// Zero n 32-bit words (the counter header at set-up).  A kernel rather
// than a memset, so that a first call under HIP-graph capture records an
// ordinary kernel node.
__global__ void zero_words_kernel(uint32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The scratch of the current device `dev`; on the first call for a device,
// take its address and clear its counters (on `stream`, ahead of the call's
// own kernels).
int scratch_of(int dev, hipStream_t stream, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return W4A16_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
      return W4A16_ERR_DEVICE;
    hipLaunchKernelGGL(zero_words_kernel, dim3((kMaxSplitTiles + 255) / 256), dim3(256), 0,
                       stream, static_cast<uint32_t*>(p), kMaxSplitTiles);
    if (hipGetLastError() != hipSuccess) return W4A16_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return W4A16_OK;
}

// The GEMM behind every entry point: argument checks, then the plan and the
// launch.  fmt is a weight format of format.hpp (0: FP16, 1: FP16 with zero
// points, 2: BF16, 3: BF16 with zero points, 4: 8-bit codes, 5: 2:4-sparse
// codes).
int gemm_checked(const uint16_t* A, const uint32_t* Bpacked, const uint16_t* scales,
                 const uint8_t* zeros, const uint16_t* bias, int activation, uint16_t* C,
                 int M, int K, int N, int group, int fmt, void* workspace, void* stream,
                 bool use_scratch = false) {
  if (M < 0) return W4A16_ERR_SHAPE;
  int rc = check_kn(K, N, true);
  if (rc != W4A16_OK) return rc;
  rc = check_group(K, group);
  if (rc != W4A16_OK) return rc;
  if (M == 0 || N == 0) return W4A16_OK;  // empty output: nothing to do
  if (!A || !Bpacked || !scales || !C) return W4A16_ERR_NULL;
  if (!aligned16(A) || !aligned16(Bpacked) || !aligned16(scales) || !aligned16(C) ||
      (bias && !aligned16(bias)) || (zeros && !aligned16(zeros)))
    return W4A16_ERR_ALIGN;
  const size_t cbytes = (size_t)M * N * 2;
  const size_t pbytes = fmt == kFmtW8     ? (size_t)K * N
                        : fmt == kFmtSp24 ? w4a16_sparse24_packed_bytes(K, N)
                                          : w4a16_packed_bytes(K, N);
  if (overlap(C, cbytes, A, (size_t)M * K * 2) ||
      overlap(C, cbytes, Bpacked, pbytes) ||
      overlap(C, cbytes, scales, (size_t)(K / group) * N * 2) ||
      (bias && overlap(C, cbytes, bias, (size_t)N * 2)) ||
      (zeros && overlap(C, cbytes, zeros, (size_t)(K / group) * N)))
    return W4A16_ERR_SHAPE;
  int dev = -1;
  const int cus = current_cus(&dev);
  if (cus <= 0) return W4A16_ERR_DEVICE;
  const Plan plan = make_plan(M, K, N, group, cus, fmt);
  if (use_scratch) {
    workspace = nullptr;
    if (plan.workspace_bytes > kScratchBytes) return W4A16_ERR_WORKSPACE;
    if (plan.workspace_bytes > 0) {
      rc = scratch_of(dev, static_cast<hipStream_t>(stream), &workspace);
      if (rc != W4A16_OK) return rc;
    }
  }
  if (plan.workspace_bytes > 0) {
    if (!workspace) return W4A16_ERR_WORKSPACE;
    if (!aligned16(workspace)) return W4A16_ERR_ALIGN;
    // partial tiles are written while other workgroups still read the
    // inputs: the workspace may alias none of the buffers
    const size_t wb = plan.workspace_bytes;
    if (overlap(workspace, wb, C, cbytes) || overlap(workspace, wb, A, (size_t)M * K * 2) ||
        overlap(workspace, wb, Bpacked, pbytes) ||
        overlap(workspace, wb, scales, (size_t)(K / group) * N * 2) ||
        (bias && overlap(workspace, wb, bias, (size_t)N * 2)) ||
        (zeros && overlap(workspace, wb, zeros, (size_t)(K / group) * N)))
      return W4A16_ERR_SHAPE;
  }
  const Epilogue ep{reinterpret_cast<const _Float16*>(bias), activation};
  const WeightFormat wf{fmt, zeros};
  if (launch_gemm(plan, A, Bpacked, scales, C, M, K, N, group, ep, wf, workspace,
                  static_cast<hipStream_t>(stream)) != hipSuccess)
    return W4A16_ERR_LAUNCH;
  return W4A16_OK;
}

}  // namespace

extern "C" {

int w4a16_gemm_fused(const uint16_t* A, const uint32_t* Bpacked, const uint16_t* scales,
                     const uint16_t* bias, int activation, uint16_t* C, int M, int K, int N,
                     int group, void* workspace, void* stream) {
  if (activation != W4A16_ACT_NONE && activation != W4A16_ACT_RELU &&
      activation != W4A16_ACT_SILU)
    return W4A16_ERR_EPILOGUE;
  return gemm_checked(A, Bpacked, scales, nullptr, bias, activation, C, M, K, N, group, 0,
                      workspace, stream);
}

int w4a16_gemm(const uint16_t* A, const uint32_t* Bpacked, const uint16_t* scales,
               uint16_t* C, int M, int K, int N, int group, void* workspace,
               void* stream) {
  return gemm_checked(A, Bpacked, scales, nullptr, nullptr, W4A16_ACT_NONE, C, M, K, N, group,
                      0, workspace, stream);
}

int w4a16_gemm_noalloc(const uint16_t* A, const uint32_t* Bpacked, const uint16_t* scales,
                       uint16_t* C, int M, int K, int N, int group, void* stream) {
  return gemm_checked(A, Bpacked, scales, nullptr, nullptr, W4A16_ACT_NONE, C, M, K, N, group,
                      0, nullptr, stream, /*use_scratch=*/true);
}

size_t w8a16_packed_bytes(int K, int N) {
  if (K <= 0 || N <= 0) return 0;
  return (size_t)K * (size_t)N;
}

int w8a16_repack(const uint32_t* Bq, uint32_t* Bpacked, int K, int N, void* stream) {
  if (!Bq || !Bpacked) return W4A16_ERR_NULL;
  int rc = check_kn(K, N, false);
  if (rc != W4A16_OK) return rc;
  if (!aligned16(Bq) || !aligned16(Bpacked)) return W4A16_ERR_ALIGN;
  const size_t bytes = w8a16_packed_bytes(K, N);
  if (overlap(Bq, bytes, Bpacked, bytes)) return W4A16_ERR_SHAPE;
  if (current_cus(nullptr) <= 0) return W4A16_ERR_DEVICE;
  if (launch_repack8(Bq, Bpacked, K, N, static_cast<hipStream_t>(stream)) != hipSuccess)
    return W4A16_ERR_LAUNCH;
  return W4A16_OK;
}

int w8a16_dequant_debug(const uint32_t* Bpacked, const uint16_t* scales, uint16_t* W, int K,
                        int N, int group, void* stream) {
  if (!Bpacked || !scales || !W) return W4A16_ERR_NULL;
  int rc = check_kn(K, N, false);
  if (rc != W4A16_OK) return rc;
  rc = check_group(K, group);
  if (rc != W4A16_OK) return rc;
  if (!aligned16(Bpacked) || !aligned16(scales) || !aligned16(W)) return W4A16_ERR_ALIGN;
  if (current_cus(nullptr) <= 0) return W4A16_ERR_DEVICE;
  if (launch_dequant_fmt(Bpacked, scales, nullptr, W, K, N, group, kFmtW8,
                         static_cast<hipStream_t>(stream)) != hipSuccess)
    return W4A16_ERR_LAUNCH;
  return W4A16_OK;
}

size_t w8a16_workspace_bytes(int M, int K, int N, int group) {
  return workspace_fmt(M, K, N, group, kFmtW8);
}

int w8a16_describe(int M, int K, int N, int group, char* buf, size_t len) {
  return describe_fmt(M, K, N, group, kFmtW8, buf, len);
}

int w8a16_gemm(const uint16_t* A, const uint32_t* Bpacked, const uint16_t* scales, uint16_t* C,
               int M, int K, int N, int group, void* workspace, void* stream) {
  return gemm_checked(A, Bpacked, scales, nullptr, nullptr, W4A16_ACT_NONE, C, M, K, N, group,
                      kFmtW8, workspace, stream);
}

int w4a16_gemm_awq(const uint16_t* A, const uint32_t* Bpacked, const uint16_t* scales,
                   const uint8_t* zeros, uint16_t* C, int M, int K, int N, int group, int dtype,
                   void* workspace, void* stream) {
  if (dtype != W4A16_DTYPE_F16 && dtype != W4A16_DTYPE_BF16) return W4A16_ERR_DTYPE;
  const int fmt = (dtype == W4A16_DTYPE_BF16 ? 2 : 0) + (zeros ? 1 : 0);
  return gemm_checked(A, Bpacked, scales, zeros, nullptr, W4A16_ACT_NONE, C, M, K, N, group,
                      fmt, workspace, stream);
}

size_t w4a16_sparse24_packed_bytes(int K, int N) {
  if (K <= 0 || N <= 0) return 0;
  return (size_t)K * (size_t)N / 8 * 3;
}

int w4a16_sparse24_repack(const uint32_t* Bq, const uint8_t* mask, uint32_t* Bpacked, int K,
                          int N, void* stream) {
  if (!Bq || !mask || !Bpacked) return W4A16_ERR_NULL;
  int rc = check_kn(K, N, false);
  if (rc != W4A16_OK) return rc;
  if (!aligned16(Bq) || !aligned16(mask) || !aligned16(Bpacked)) return W4A16_ERR_ALIGN;
  const size_t qbytes = w4a16_packed_bytes(K, N);
  const size_t mbytes = (size_t)K * N / 4;
  const size_t pbytes = w4a16_sparse24_packed_bytes(K, N);
  if (overlap(Bq, qbytes, Bpacked, pbytes) || overlap(mask, mbytes, Bpacked, pbytes))
    return W4A16_ERR_SHAPE;
  if (current_cus(nullptr) <= 0) return W4A16_ERR_DEVICE;
  if (launch_repack_sp24(Bq, mask, Bpacked, K, N, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return W4A16_ERR_LAUNCH;
  return W4A16_OK;
}

size_t w4a16_sparse24_workspace_bytes(int M, int K, int N, int group) {
  return workspace_fmt(M, K, N, group, kFmtSp24);
}

int w4a16_sparse24_describe(int M, int K, int N, int group, char* buf, size_t len) {
  return describe_fmt(M, K, N, group, kFmtSp24, buf, len);
}

int w4a16_sparse24_gemm(const uint16_t* A, const uint32_t* Bpacked, const uint16_t* scales,
                        uint16_t* C, int M, int K, int N, int group, void* workspace,
                        void* stream) {
  return gemm_checked(A, Bpacked, scales, nullptr, nullptr, W4A16_ACT_NONE, C, M, K, N, group,
                      kFmtSp24, workspace, stream);
}

int w4a16_sparse24_dequant_debug(const uint32_t* Bpacked, const uint16_t* scales, uint16_t* W,
                                 int K, int N, int group, void* stream) {
  if (!Bpacked || !scales || !W) return W4A16_ERR_NULL;
  int rc = check_kn(K, N, false);
  if (rc != W4A16_OK) return rc;
  rc = check_group(K, group);
  if (rc != W4A16_OK) return rc;
  if (!aligned16(Bpacked) || !aligned16(scales) || !aligned16(W)) return W4A16_ERR_ALIGN;
  if (current_cus(nullptr) <= 0) return W4A16_ERR_DEVICE;
  if (launch_dequant_fmt(Bpacked, scales, nullptr, W, K, N, group, kFmtSp24,
                         static_cast<hipStream_t>(stream)) != hipSuccess)
    return W4A16_ERR_LAUNCH;
  return W4A16_OK;
}

}  // extern "C"
