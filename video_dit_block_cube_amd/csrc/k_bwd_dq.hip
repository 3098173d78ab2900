// k_bwd_dq.hip -- block-sparse attention backward, dQ, on bf16 MFMA (gfx950), c == 64: the
// launcher, and the head_dim 128 instantiations of the one-wave kernel (bsa_bwd_dq.h).
//
// The backward ships alongside the forward for training ("LongCat-Video 高效長視頻生成探索世界
// 模型的第壹步", meituan.com talk, section 2.2); the selection is a discrete choice and is held
// constant.  With P = exp(scale*Q_i K_j^T - LSE_i) over every selected pair (i, j):
//   dV_j += P^T dO_i,  dS = P o (dO_i V_j^T - Delta_i),  dQ_i += scale*dS K_j,
//   dK_j += scale*dS^T Q_i.
//
// This file is compiled with LLVM's register-minimising scheduler (build flags): at head_dim 128
// it keeps the score accumulators out of the AGPRs that hold dQ^T, which trims accumulator copies
// in the loop.  At head_dim 128 the launcher runs the software-pipelined variant
// (k_bwd_dq_pipe.hip, k_bwd_dq_pipe_ragged.hip) instead, which gives the same bits, unless the
// pipeline is switched off; head_dim 64 runs the instantiation in k_bwd_dq64.hip.
#include "bsa_bwd_dq.h"

namespace bsa {

hipError_t launch_bwd_dq_mfma(const Geom& g, const bf16_t* q_row, const bf16_t* do_row,
                              const bf16_t* k_row, const bf16_t* v_row, const float2* ld_c,
                              const int32_t* idx, int k_sel, float scale, float* dq,
                              bool pipelined, int walk_ticks, hipStream_t s) {
  if (pipelined && g.D == 128)
    return launch_bwd_dq_pipe(g, q_row, do_row, k_row, v_row, ld_c, idx, k_sel, scale, dq,
                              walk_ticks, s);
  const int cpx = (g.nbq + 7) / 8;
  dim3 grid((unsigned)(g.B * g.Hh * cpx * 8));
  const float c_log2 = scale * kLog2e;
#define BSA_DQ(DD, RG)                                                                          \
  hipLaunchKernelGGL((bwd_dq_mfma_kernel<DD, RG>), grid, dim3(64), 0, s, g, q_row, do_row, k_row, \
                     v_row, ld_c, idx, k_sel, scale, c_log2, cpx, dq)
  if (g.D == 64)
    return launch_bwd_dq64(g, q_row, do_row, k_row, v_row, ld_c, idx, k_sel, scale, c_log2, cpx,
                           dq, s);
  if (g.ragged) BSA_DQ(128, true); else BSA_DQ(128, false);
#undef BSA_DQ
  return hipGetLastError();
}

}  // namespace bsa
