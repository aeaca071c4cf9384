// The stream-K kernel (gemm_sk.hpp) for FP16 weights with symmetric codes,
// with and without the fused output stage, and the launcher for every
// format it serves.
#include "gemm_sk.hpp"

namespace w4a16 {

bool sk_is_compiled(int mb, int nb, int ns, int wm, int wn) {
#define W4A16_SKMATCH(MB_, NB_, NS_, WN_) \
  if (mb == MB_ && nb == NB_ && ns == NS_ && wm == 1 && wn == WN_) return true;
  W4A16_SK_VARIANTS(W4A16_SKMATCH)
#undef W4A16_SKMATCH
  return false;
}

size_t sk_workspace_bytes(int wgs, int tm, int tn, int tiles, int KB, int ns) {
  const int64_t upt = (KB + ns - 1) / ns;  // units of ns iterations per tile
  const int64_t U = (int64_t)tiles * upt;
  // no tile is shared between runs when every run is a whole number of tiles
  if (U % wgs == 0 && (U / wgs) % upt == 0) return 0;
  return kCounterHeaderBytes + (size_t)2 * wgs * tm * tn * sizeof(float);
}

hipError_t launch_sk(const Plan& p, const uint16_t* A, const uint32_t* Bp, const uint16_t* S,
                     uint16_t* C, int M, int K, int N, uint64_t gmagic, Epilogue ep,
                     WeightFormat wf, void* workspace, hipStream_t stream) {
  if (wf.fmt == kFmtF16)
    return launch_sk_fmt<kFmtF16>(p, A, Bp, S, C, M, K, N, gmagic, ep, nullptr, workspace, stream);
  if (wf.fmt == kFmtF16Zp || wf.fmt == kFmtBf16 || wf.fmt == kFmtBf16Zp)
    return launch_sk_zp_bf16(p, A, Bp, S, C, M, K, N, gmagic, ep, wf, workspace, stream);
  return hipErrorInvalidValue;
}

}  // namespace w4a16
