// k_bwd_dq_pipe_ragged.hip -- block-sparse attention backward, dQ: the software-pipelined kernel
// (bsa_bwd_dq_pipe.h) at head_dim 128 on ragged grids (H or W not a multiple of the cube side,
// such as the 45-token height of a 720p latent).
//
// Same operation and the same bits as the plain ragged dQ loop (backward shipped with the forward
// for training: "LongCat-Video 高效長視頻生成探索世界模型的第壹步", meituan.com talk, section 2.2).
// Built with LLVM's register-minimising scheduler only: with every MFMA writing architectural
// VGPRs (the option k_bwd_dq_pipe.hip uses) this instantiation spills four registers, and that
// build gave wrong gradients; without the option nothing spills and the result matches the plain
// loop bit for bit, about 2% faster than it on the 24x45x80 grid.
#include "bsa_bwd_dq_pipe.h"

namespace bsa {

hipError_t launch_bwd_dq_pipe_ragged(const Geom& g, const bf16_t* q_row, const bf16_t* do_row,
                                     const bf16_t* k_row, const bf16_t* v_row,
                                     const float2* ld_c, const int32_t* idx, int k_sel,
                                     float scale, float c_log2, int cpx, int walk_ticks,
                                     float* dq, hipStream_t s) {
  dim3 grid((unsigned)(g.B * g.Hh * cpx * 8));
  hipLaunchKernelGGL((bwd_dq_pipe_kernel<128, true>), grid, dim3(64), 0, s, g, q_row, do_row,
                     k_row, v_row, ld_c, idx, k_sel, scale, c_log2, cpx, walk_ticks, dq);
  return hipGetLastError();
}

}  // namespace bsa
