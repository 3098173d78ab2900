// k_bwd_dq_pipe.hip -- block-sparse attention backward, dQ: the software-pipelined kernel
// (bsa_bwd_dq_pipe.h) at head_dim 128 on grids whose sides are cube multiples, and its launcher.
//
// Built with every MFMA writing architectural VGPRs and LLVM's register-minimising scheduler
// (build flags): the accumulators then sit in VGPRs, where the exponentials read the scores
// without a copy per element, and the Q and dO operand fragments, which the products read
// straight from there, fill the AGPRs.  About 8% faster than the plain kernel at the 720p-class
// shape.  The ragged-grid instantiation lives in k_bwd_dq_pipe_ragged.hip: under the VGPR option
// it spills, and spilling under that option gave wrong results, so it is built without it.  At
// head_dim 64 the plain kernel (k_bwd_dq64.hip) is faster.
#include "bsa_bwd_dq_pipe.h"

namespace bsa {

hipError_t launch_bwd_dq_pipe(const Geom& g, const bf16_t* q_row, const bf16_t* do_row,
                              const bf16_t* k_row, const bf16_t* v_row, const float2* ld_c,
                              const int32_t* idx, int k_sel, float scale, float* dq,
                              int walk_ticks, hipStream_t s) {
  if (g.D != 128 || k_sel < 1) return hipErrorInvalidValue;
  const int cpx = (g.nbq + 7) / 8;
  const float c_log2 = scale * kLog2e;
  if (g.ragged)
    return launch_bwd_dq_pipe_ragged(g, q_row, do_row, k_row, v_row, ld_c, idx, k_sel, scale,
                                     c_log2, cpx, walk_ticks, dq, s);
  dim3 grid((unsigned)(g.B * g.Hh * cpx * 8));
  hipLaunchKernelGGL((bwd_dq_pipe_kernel<128, false>), grid, dim3(64), 0, s, g, q_row, do_row,
                     k_row, v_row, ld_c, idx, k_sel, scale, c_log2, cpx, walk_ticks, dq);
  return hipGetLastError();
}

}  // namespace bsa
