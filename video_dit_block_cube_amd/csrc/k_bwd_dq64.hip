// k_bwd_dq64.hip -- block-sparse attention backward, dQ, head_dim 64: the instantiations of the
// one-wave kernel (bsa_bwd_dq.h) for head_dim 64.
//
// Same operation as the head_dim 128 dQ (backward shipped with the forward for training:
// "LongCat-Video 高效長視頻生成探索世界模型的第壹步", meituan.com talk, section 2.2).  A separate
// translation unit so that it can be compiled with every MFMA writing architectural VGPRs
// (build flags): at head_dim 64 the whole kernel fits in 256 VGPRs, and the score accumulators
// then reach the exponentials without AGPR-to-VGPR copies (8% faster at the 720p-class shape;
// at head_dim 128 the same choice was 2% slower, so k_bwd_dq.hip keeps the default).
#include "bsa_bwd_dq.h"

namespace bsa {

hipError_t launch_bwd_dq64(const Geom& g, const bf16_t* q_row, const bf16_t* do_row,
                           const bf16_t* k_row, const bf16_t* v_row, const float2* ld_c,
                           const int32_t* idx, int k_sel, float scale, float c_log2, int cpx,
                           float* dq, hipStream_t s) {
  dim3 grid((unsigned)(g.B * g.Hh * cpx * 8));
#define BSA_DQ64(RG)                                                                            \
  hipLaunchKernelGGL((bwd_dq_mfma_kernel<64, RG>), grid, dim3(64), 0, s, g, q_row, do_row, k_row, \
                     v_row, ld_c, idx, k_sel, scale, c_log2, cpx, dq)
  if (g.ragged) BSA_DQ64(true); else BSA_DQ64(false);
#undef BSA_DQ64
  return hipGetLastError();
}

}  // namespace bsa
