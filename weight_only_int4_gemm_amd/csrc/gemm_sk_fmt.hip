// The stream-K kernel (gemm_sk.hpp) for the formats with zero points and
// BF16 (format.hpp, formats 1 to 3), in a translation unit of its own.
#include "gemm_sk.hpp"

namespace w4a16 {

hipError_t launch_sk_zp_bf16(const Plan& p, const uint16_t* A, const uint32_t* Bp,
                             const uint16_t* S, uint16_t* C, int M, int K, int N, uint64_t gmagic,
                             Epilogue ep, WeightFormat wf, void* workspace, hipStream_t stream) {
  if (wf.fmt == kFmtF16Zp)
    return launch_sk_fmt<kFmtF16Zp>(p, A, Bp, S, C, M, K, N, gmagic, ep, wf.zeros, workspace,
                                    stream);
  if (wf.fmt == kFmtBf16)
    return launch_sk_fmt<kFmtBf16>(p, A, Bp, S, C, M, K, N, gmagic, ep, nullptr, workspace,
                                   stream);
  if (wf.fmt == kFmtBf16Zp)
    return launch_sk_fmt<kFmtBf16Zp>(p, A, Bp, S, C, M, K, N, gmagic, ep, wf.zeros, workspace,
                                     stream);
  return hipErrorInvalidValue;
}

}  // namespace w4a16
