/*
 * w4a16.h -- C interface of libw4a16, a W4A16 matrix multiply for gfx950.
 *
 *   C[M x N] = A[M x K] . dequant(B)[K x N]
 *
 * A holds FP16 activations (tokens x in-features), B holds 4-bit weight codes
 * q in 0..15 (in-features x out-features) with one FP16 scale s per group of
 * `group` consecutive in-features per output column, the weight is
 * w = (q - 8) * s, products accumulate in FP32 and C is FP16.
 *
 * What the operation is comes from the "Quant Marlin kernel" explainer
 * (aicassindra.com): section "The architecture: every piece explained"
 * (top row: eight 4-bit codes per 32-bit word, one FP16 scale per group,
 * commonly 128; middle row: unpack to FP16, multiply by the group scale,
 * matrix-multiply with FP32 accumulation, split-K with a global reduction;
 * bottom rows: FP16 in, FP16 out, the permuted layout computed once offline)
 * and section "End-to-end flow" (tokens x in-features times in-features x
 * out-features).  The zero point 8, the nibble order and the scale layout
 * are this library's readings where the pages leave them open.
 *
 * Conventions for every entry point:
 *  - FP16 values are passed as uint16_t bit patterns, so callers need no HIP
 *    or half-precision headers.  `stream` is a hipStream_t (NULL = the null
 *    stream of the current device).
 *  - Pointers marked "device" must point to memory of the current HIP device
 *    and be 16-byte aligned.  The caller owns and allocates every buffer;
 *    the library allocates nothing and keeps only a per-device cache of the
 *    compute-unit count.
 *  - Work is enqueued on `stream` and the call returns without waiting for
 *    it.  Nothing is allocated and nothing is synchronised, so calls can be
 *    captured into a HIP graph.
 *  - Arguments are checked before anything is launched; on error nothing is
 *    launched and a negative W4A16_ERR_* code is returned.  W4A16_ERR_LAUNCH
 *    reports a failed kernel launch (hipGetLastError).  The library never
 *    prints, aborts or throws.
 *  - Buffers passed to one call must not overlap, except where stated.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum w4a16_status {
    W4A16_OK = 0,
    W4A16_ERR_NULL = -1,      /* a required pointer is NULL                  */
    W4A16_ERR_SHAPE = -2,     /* M, K or N out of range or not a multiple    */
    W4A16_ERR_GROUP = -3,     /* group not a multiple of 128 dividing K      */
    W4A16_ERR_ALIGN = -4,     /* a pointer is not 16-byte aligned            */
    W4A16_ERR_WORKSPACE = -5, /* workspace NULL although one is needed, or  */
                              /* (noalloc) more than its scratch holds     */
    W4A16_ERR_LAUNCH = -6,    /* the kernel launch failed                    */
    W4A16_ERR_DEVICE = -7,    /* no usable current HIP device                */
    W4A16_ERR_EPILOGUE = -8,  /* unknown activation for w4a16_gemm_fused     */
    W4A16_ERR_DTYPE = -9      /* unknown dtype for the *_awq entry points    */
};

/* 16-bit types of activations, scales and output (the *_awq entry points). */
enum w4a16_dtype {
    W4A16_DTYPE_F16 = 0,      /* IEEE binary16                               */
    W4A16_DTYPE_BF16 = 1      /* bfloat16: 8 exponent bits, 7 mantissa bits  */
};

/* Activations the fused epilogue applies (w4a16_gemm_fused). */
enum w4a16_activation {
    W4A16_ACT_NONE = 0,       /* y = x                                       */
    W4A16_ACT_RELU = 1,       /* y = max(x, 0)                               */
    W4A16_ACT_SILU = 2        /* y = x / (1 + exp(-x))                       */
};

/* Version of the permuted layout written by w4a16_repack.  Callers that
 * store permuted weights should store this number with them: weights
 * permuted for one layout cannot be fed to another without repacking. */
int w4a16_layout_version(void);

/* Static, NUL-terminated name of a status code ("W4A16_OK", ...). */
const char* w4a16_status_string(int status);

/* Bytes of the permuted weights for a K x N matrix: K * N / 2. */
size_t w4a16_packed_bytes(int K, int N);

/* Writes into buf (at most len bytes, NUL-terminated) a one-line
 * description of how w4a16_gemm would run this shape on the current device:
 * the kernel variant, grid, splits and workspace bytes, for example
 *   "gemm_kernel<1,4,4> grid=64x1x4 block=256 splits=4 workspace=1048832".
 * Returns W4A16_OK, W4A16_ERR_NULL (buf NULL or len 0), W4A16_ERR_SHAPE /
 * W4A16_ERR_GROUP (a shape w4a16_gemm rejects, or M or N zero) or
 * W4A16_ERR_DEVICE.  Launches nothing. */
int w4a16_describe(int M, int K, int N, int group, char* buf, size_t len);

/* Weight formats, named by the entry point that takes them. */
enum w4a16_format {
    W4A16_FORMAT_F16 = 0,      /* w4a16_gemm, w4a16_gemm_fused              */
    W4A16_FORMAT_F16_ZP = 1,   /* w4a16_gemm_awq: FP16 with zero points     */
    W4A16_FORMAT_BF16 = 2,     /* w4a16_gemm_awq: BF16                      */
    W4A16_FORMAT_BF16_ZP = 3,  /* w4a16_gemm_awq: BF16 with zero points     */
    W4A16_FORMAT_W8 = 4,       /* w8a16_gemm                                */
    W4A16_FORMAT_SPARSE24 = 5  /* w4a16_sparse24_gemm                       */
};

/* The line w4a16_describe would write for a call of weight format `format`
 * on a device with `cus` compute units, computed without querying any
 * device (for planning tools and tests on a machine without a GPU).
 * Returns as w4a16_describe, with W4A16_ERR_DTYPE for an unknown format and
 * W4A16_ERR_DEVICE for cus <= 0.  Follows the forced plan like
 * w4a16_describe. */
int w4a16_plan_describe(int M, int K, int N, int group, int format, int cus, char* buf,
                        size_t len);

/* Tuning and testing only: replace the plan heuristic of every later call
 * in this process with the text spec
 *   "mb,nb,wk,splits[,depth[,tile[,unused[,wm]]]]"
 * (a field <= 0 keeps the heuristic's value; tile 0 is the streaming
 * kernel, 2 the LDS kernel, 4 the stream-K kernel (wk = its waves along N,
 * splits = its grid), -1 the plan the heuristic makes without the stream-K
 * kernel).  A
 * spec naming a variant that is not compiled leaves the heuristic's plan in
 * place.  NULL or "" restores the heuristic.  The environment variable
 * W4A16_FORCE_PLAN, read once when the library first plans a call, seeds the
 * same setting.  w4a16_workspace_bytes and w4a16_describe follow it, so a
 * caller that changes it between sizing a workspace and a call must size
 * again.  Not to be called while another thread plans a call.
 * Returns W4A16_OK, or W4A16_ERR_SHAPE for text that is not a spec. */
int w4a16_set_forced_plan(const char* spec);

/*
 * w4a16_repack -- offline permutation of canonical codes into the layout
 * the GEMM reads.
 *
 * The pages: weights are pre-permuted once, offline, so that one wide load
 * hands every thread exactly the operand fragment of the matrix instruction
 * ("Quant Marlin kernel" explainer, the paragraph on the permuted weight
 * layout; "Low-Precision Quantization Kernels in Production", section 1,
 * mechanism 1).  The order here is this library's own, for the gfx950
 * 16x16x32 FP16 matrix instruction.
 *
 * Bq      (device, read)  canonical codes, uint32[K/8][N] row-major; code k
 *                         of column n is bits 4*(k%8) .. 4*(k%8)+3 of word
 *                         Bq[k/8][n] (least significant nibble first).
 * Bpacked (device, write) w4a16_packed_bytes(K, N) bytes, layout version 1:
 *                         code (k, n) is in word
 *                           ((n/16 * K/128 + k/128) * 64 + lane) * 4 + (k%128)/32
 *                         with lane = n%16 + 16*((k%32)/8), at nibble
 *                         {0,4,1,5,2,6,3,7}[k%8].  Callers treat it as opaque.
 * K, N    K a positive multiple of 128, N a positive multiple of 16.
 * Errors: NULL pointer, bad shape, misalignment, Bq and Bpacked overlapping
 *         (W4A16_ERR_SHAPE).
 */
int w4a16_repack(const uint32_t* Bq, uint32_t* Bpacked, int K, int N,
                 void* stream);

/*
 * w4a16_workspace_bytes -- bytes of split-K workspace w4a16_gemm needs for
 * this shape (FP32 partial tiles plus one arrival counter per output tile).
 * 0 means the call needs no workspace.  Returns 0 for shapes w4a16_gemm
 * rejects.
 *
 * Layout: a fixed 64 KiB header of 32-bit arrival counters (one per output
 * tile, at the same place for every shape), then the FP32 partial tiles.
 *
 * Contract: the caller allocates at least this many bytes and fills them
 * with zeros once, after allocating.  Every call leaves the counters at zero
 * again, so one workspace serves any number of later calls of any shape
 * whose requirement it covers, as long as those calls are ordered (same
 * stream, or synchronised).  Two calls running at the same time must not
 * share a workspace.  The workspace may not overlap A, Bpacked, scales, C
 * or any other buffer of the call (W4A16_ERR_SHAPE).
 */
size_t w4a16_workspace_bytes(int M, int K, int N, int group);

/*
 * w4a16_gemm -- C = A . dequant(Bpacked, scales).
 *
 * Split-K and its reduction: the pages split the in-feature dimension over
 * several workgroups, each computing a partial sum, combined by a global
 * reduction ("Quant Marlin kernel" explainer, middle row and "End-to-end
 * flow"); the combination here is deterministic ("Low-Precision Quantization
 * Kernels in Production", section 3, mechanism 1): FP32 partials are added
 * in a fixed order, so equal inputs give bit-identical C on every run.
 *
 * A         (device, read)  FP16 [M][K] row-major.
 * Bpacked   (device, read)  output of w4a16_repack for (K, N).
 * scales    (device, read)  FP16 [K/group][N] row-major.
 * C         (device, write) FP16 [M][N] row-major.  Rows are written only
 *                           for m < M; A is read only for m < M.
 * M         >= 0; M == 0 returns W4A16_OK and launches nothing.
 * K         positive multiple of 128.
 * N         multiple of 16, >= 0; N == 0 returns W4A16_OK.
 * group     multiple of 128 that divides K (128 = per-128 groups; K = one
 *           scale per output column).
 * workspace (device, read/write) see w4a16_workspace_bytes; may be NULL
 *           only when that returns 0 for this shape.
 * Numerics: products accumulate in FP32 and C is rounded once to FP16
 *           (round to nearest even; overflow gives +-inf).  Kernel variants
 *           whose tiles have 16 or 32 rows multiply the exact integers q-8
 *           and apply the scale to each 128-deep block's FP32 sum, so no
 *           weight is rounded; those with 64 rows or more round each weight
 *           once to FP16 from the exact (q-8)*s.  Both are the product up to
 *           rounding; w4a16_describe names the variant a shape gets.
 * Errors:   W4A16_ERR_NULL, _SHAPE, _GROUP, _ALIGN, _WORKSPACE, _DEVICE,
 *           _LAUNCH.  C must not overlap A, Bpacked, scales or workspace,
 *           and the workspace none of the inputs.
 */
int w4a16_gemm(const uint16_t* A, const uint32_t* Bpacked,
               const uint16_t* scales, uint16_t* C, int M, int K, int N,
               int group, void* workspace, void* stream);

/*
 * w4a16_gemm_noalloc -- w4a16_gemm for callers that cannot allocate memory
 * (code under HIP-graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same plan and kernels, with the split-K partials and
 * counters in a scratch array the library holds on each device (a static
 * device array of W4A16_NOALLOC_SCRATCH_BYTES, 64 MiB, kept until the
 * process ends) instead of a caller's workspace.
 *
 * A, Bpacked, scales, C, M, K, N, group, stream, numerics and errors: as
 * w4a16_gemm.  No allocation, free, memset or synchronisation happens; the
 * first call on a device takes the scratch's address and clears its
 * counters with a small kernel on `stream`.
 * Limit: a shape whose plan needs more split-K scratch than
 * W4A16_NOALLOC_SCRATCH_BYTES (w4a16_workspace_bytes(M, K, N, group) above
 * it) returns W4A16_ERR_WORKSPACE and launches nothing.
 * Every call on one device shares that device's scratch, which keeps the
 * last call's contents: calls that overlap in time on one device (other
 * streams, other threads) race and must not be issued; calls ordered on one
 * stream, or synchronised, are safe.
 */
#define W4A16_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int w4a16_gemm_noalloc(const uint16_t* A, const uint32_t* Bpacked, const uint16_t* scales,
                       uint16_t* C, int M, int K, int N, int group, void* stream);

/*
 * w4a16_gemm_fused -- C = act(A . dequant(Bpacked, scales) + bias).
 *
 * The pages hand the GEMM's output straight to the next operation -- a bias
 * add, an activation -- with no visible dequantisation step ("Quant Marlin
 * kernel" explainer, section "End-to-end flow").  Here that operation runs
 * in the GEMM's output stage, on the FP32 sum before the one rounding to
 * FP16, so C makes a single trip to memory.
 *
 * bias       (device, read) FP16 [N], or NULL for no bias.
 * activation one of enum w4a16_activation.
 * The other arguments, alignment rules and errors are those of w4a16_gemm,
 * plus W4A16_ERR_EPILOGUE for an unknown activation.  bias must not overlap
 * C.  Numerics: y = act(sum + float(bias[n])) in FP32 (SiLU with the
 * device's single-precision exp), then rounded once to FP16.
 * w4a16_gemm is w4a16_gemm_fused with bias NULL and W4A16_ACT_NONE.
 */
int w4a16_gemm_fused(const uint16_t* A, const uint32_t* Bpacked,
                     const uint16_t* scales, const uint16_t* bias, int activation,
                     uint16_t* C, int M, int K, int N, int group, void* workspace,
                     void* stream);

/*
 * w4a16_gemm_awq -- C = A . W with AWQ-style zero points and/or BF16.
 *
 * The serving stacks the pages describe run AWQ checkpoints through the same
 * kernel ("Low-Precision Quantization Kernels in Production", section 1 on
 * production engines and the comparison table of section 5), and models
 * kept in BF16 (same page, introduction; section 4's activation formats).
 * Here:
 *   w[k][n] = rnd((q[k][n] - z[k/group][n]) * s[k/group][n])
 * with rnd the rounding (to nearest even) to the 16-bit type `dtype`, and
 * z = 8 when `zeros` is NULL.  A, scales and C hold `dtype` values; the sum
 * is FP32 and rounded once to `dtype`.  With FP16 the tiles of 16 or 32
 * rows skip rnd, as in w4a16_gemm: they scale the FP32 sums of the exact
 * (q - z) per 128-deep block.
 *
 * zeros   (device, read) uint8 [K/group][N] row-major, the zero point of
 *         each group and column (AWQ uses 0..15; any byte value gives the
 *         formula above exactly), or NULL.  16-byte aligned.
 * dtype   W4A16_DTYPE_F16 or W4A16_DTYPE_BF16; anything else returns
 *         W4A16_ERR_DTYPE.
 * The other arguments, layouts, alignment, workspace and errors are those
 * of w4a16_gemm (same plan and workspace size).  With dtype F16 and zeros
 * NULL this is w4a16_gemm.  Every format is compiled for the same kernel
 * variants (the ones the library's plans choose).  No fused epilogue here.
 */
int w4a16_gemm_awq(const uint16_t* A, const uint32_t* Bpacked, const uint16_t* scales,
                   const uint8_t* zeros, uint16_t* C, int M, int K, int N, int group,
                   int dtype, void* workspace, void* stream);

/*
 * w4a16_dequant_awq_debug -- the weights of w4a16_gemm_awq, written out:
 * W [K][N] row-major `dtype` values, produced by the GEMM's own unpack
 * routine for that format.  Arguments as in w4a16_dequant_debug plus
 * `zeros` (NULL: z = 8) and `dtype`.
 */
int w4a16_dequant_awq_debug(const uint32_t* Bpacked, const uint16_t* scales,
                            const uint8_t* zeros, uint16_t* W, int K, int N, int group,
                            int dtype, void* stream);

/*
 * 8-bit weights (W8A16).  The same kernel family serves 4-bit and 8-bit
 * checkpoints ("Low-Precision Quantization Kernels in Production", section 1
 * on production engines; the comparison table of section 5: INT4, INT8).
 * Codes q in 0..255 centred on 128:  w = fp16_rne((q - 128) * s), scales as
 * for 4 bits (FP16 [K/group][N]).
 *
 * Canonical input Bq uint32 [K/4][N]: code k = 4j + i of column n is bits
 * 8i..8i+7 of Bq[j][n].  Permuted layout (version 1 for 8 bits): blocks of
 * 16 columns x 64 in-features (1 KiB), block(n16, kb64) = n16 * K/64 + kb64;
 * in a block lane l = (n % 16) + 16 * ((k % 32) / 8) owns words 4l..4l+3,
 * word 2 * ((k % 64) / 32) + (k % 8) / 4 holds codes k0..k0+3 (k0 % 4 == 0),
 * code k0 + i at byte {0,2,1,3}[i].  K*N bytes.
 */

/* Bytes of the permuted 8-bit layout: K*N (0 for non-positive sizes). */
size_t w8a16_packed_bytes(int K, int N);

/* The offline permutation for 8 bits: Bq [K/4][N] -> Bpacked (K*N bytes),
 * device to device on `stream`.  Requirements and errors as w4a16_repack. */
int w8a16_repack(const uint32_t* Bq, uint32_t* Bpacked, int K, int N, void* stream);

/* Workspace bytes of w8a16_gemm for this shape: its plans differ from the
 * 4-bit ones from 16 rows on, so its workspace is sized here (contract as
 * w4a16_workspace_bytes). */
size_t w8a16_workspace_bytes(int M, int K, int N, int group);

/* The plan of w8a16_gemm for this shape, as w4a16_describe. */
int w8a16_describe(int M, int K, int N, int group, char* buf, size_t len);

/* C = A . dequant8(Bpacked, scales): arguments, layouts, alignment and
 * errors as w4a16_gemm; the workspace is sized by w8a16_workspace_bytes. */
int w8a16_gemm(const uint16_t* A, const uint32_t* Bpacked, const uint16_t* scales, uint16_t* C,
               int M, int K, int N, int group, void* workspace, void* stream);

/* The FP16 weights of w8a16_gemm, written out W [K][N] by the GEMM's own
 * unpack routine.  Arguments as w4a16_dequant_debug. */
int w8a16_dequant_debug(const uint32_t* Bpacked, const uint16_t* scales, uint16_t* W, int K,
                        int N, int group, void* stream);

/*
 * 2:4 structured sparsity (Sparse-MARLIN).  The pages report a Sparse-MARLIN
 * variant serving beside MARLIN ("The anthology of the SOTA", the MARLIN
 * note, section "Key results"); they give no format, so this one is the
 * library's own:
 *
 *   in every group of four consecutive in-features k = 4g .. 4g+3 of a
 *   column at most two weights are kept, the others are exactly zero; the
 *   kept ones are fp16_rne((q - 8) * s) as in w4a16_gemm.
 *
 * Input: the dense canonical codes Bq uint32 [K/8][N] (as for w4a16_repack)
 * and a mask uint8 [K/4][N] whose bits 0..3 mark the kept in-features
 * 4g + i.  A group keeps its two lowest set bits; with fewer than two bits
 * set it keeps only those (bits above the lowest two are ignored).
 *
 * Permuted layout (version 1 for 2:4), 768 bytes per block of 16 columns x
 * 128 in-features, block(n16, kb) = n16 * K/128 + kb: words 0..127 of a
 * block hold codes, words 128..191 positions.  Lane l = (n % 16) +
 * 16 * ((k % 64) / 16) owns code words 2l + t (t = (k % 128) / 64) and
 * position word 128 + l.  Code word t holds the two kept codes of each of
 * the lane's four groups (slots 2r, 2r+1 for group r, lower in-feature
 * first) with slot i at nibble {0,4,1,5,2,6,3,7}[i]; bits 16t + 2i .. +1 of
 * the position word hold slot i's position in its group (0..3).  A group
 * with fewer than two kept weights fills its free slot with code 8 at its
 * lowest unused position.  K * N * 3 / 8 bytes: three quarters of the dense
 * 4-bit layout.
 */

/* Bytes of the permuted 2:4 layout: K * N * 3 / 8 (0 for non-positive sizes). */
size_t w4a16_sparse24_packed_bytes(int K, int N);

/* The offline compression and permutation: Bq uint32 [K/8][N] and mask
 * uint8 [K/4][N] (device, read) -> Bpacked (device, write,
 * w4a16_sparse24_packed_bytes(K, N) bytes) on `stream`.  K a positive
 * multiple of 128, N of 16; all three pointers 16-byte aligned; Bpacked
 * must not overlap Bq or mask (W4A16_ERR_SHAPE).  Other errors as
 * w4a16_repack. */
int w4a16_sparse24_repack(const uint32_t* Bq, const uint8_t* mask, uint32_t* Bpacked, int K,
                          int N, void* stream);

/* Workspace bytes of w4a16_sparse24_gemm for this shape (its plans differ
 * from the dense ones); contract as w4a16_workspace_bytes. */
size_t w4a16_sparse24_workspace_bytes(int M, int K, int N, int group);

/* The plan of w4a16_sparse24_gemm for this shape, as w4a16_describe. */
int w4a16_sparse24_describe(int M, int K, int N, int group, char* buf, size_t len);

/* C = A . W with W the 2:4-sparse weights of Bpacked (pruned weights 0),
 * computed by the sparse matrix instruction (half the multiplies of the
 * dense product).  Arguments, layouts, numerics, alignment and errors as
 * w4a16_gemm, with Bpacked from w4a16_sparse24_repack and the workspace
 * sized by w4a16_sparse24_workspace_bytes. */
int w4a16_sparse24_gemm(const uint16_t* A, const uint32_t* Bpacked, const uint16_t* scales,
                        uint16_t* C, int M, int K, int N, int group, void* workspace,
                        void* stream);

/* The weights of w4a16_sparse24_gemm, written out densely: W FP16 [K][N],
 * each kept weight as the GEMM's own unpack routine makes it, +0 at every
 * position no slot names.  (A free slot, code 8 at an unused position,
 * gives (8 - 8) * s: -0 there when s < 0.)  Arguments and errors as
 * w4a16_dequant_debug. */
int w4a16_sparse24_dequant_debug(const uint32_t* Bpacked, const uint16_t* scales, uint16_t* W,
                                 int K, int N, int group, void* stream);

/*
 * w4a16_dequant_debug -- W = dequant(Bpacked, scales), written out.
 *
 * Uses the same device unpack-and-scale routine as w4a16_gemm's tiles of 64
 * rows or more, so it shows bit for bit the FP16 weights they multiply
 * ("Quant Marlin kernel" explainer, middle row: codes to FP16, times the
 * group scale); the smaller tiles take the routine's exact integers q - 8
 * and scale their sums instead.
 *
 * Bpacked (device, read)  output of w4a16_repack for (K, N).
 * scales  (device, read)  FP16 [K/group][N].
 * W       (device, write) FP16 [K][N] row-major,
 *                         W[k][n] = fp16_rne((q[k][n] - 8) * s[k/group][n]).
 * Errors: as w4a16_gemm.
 */
int w4a16_dequant_debug(const uint32_t* Bpacked, const uint16_t* scales,
                        uint16_t* W, int K, int N, int group, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
