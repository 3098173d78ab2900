// k_gather.hip -- coalesced cube-gather of a [B, N, Hh, D] bf16 token tensor into cube-major
// blocks laid out in MFMA operand order (64-token cubes, D in {64, 128}).
//
// The 3D cube partition ("LongCat-Video : Generate 1 minute long AI videos with this model",
// Data Science in Your Pocket, section "Sparse attention") scatters a cube's 64 tokens over
// 64 token records of Hh*D elements.  The attention kernels instead want each selected cube as
// one contiguous block whose 16-byte pieces land directly in the lanes of a
// v_mfma_f32_32x32x16_bf16 operand, so every operand load of the hot loop is a 1 KB fully
// coalesced wave load.  Two layouts are produced (per (b, h, cube), 64*D elements each):
//
//   ROW   lane = token, 8 consecutive d per lane:
//         elem[((rb*S + s)*64 + lane)*8 + e] = X[token 32rb + lane%32][d = (lane/32)*D/2 + 8s + e]
//         (S = D/16).  This is the A (or B) operand of a product that contracts over d.
//   TRANS lane = d, 8 tokens per lane, tokens in the order of the 32x32 accumulator rows:
//         elem[(((rb*DB + db)*2 + s2)*64 + lane)*8 + e] =
//             X[token 32rb + 16s2 + 8(e/4) + 4(lane/32) + e%4][d = 32db + lane%32]   (DB = D/32)
//         This is the operand of a product that contracts over tokens, matching a P (or dS)
//         tile converted in place from an fp32 32x32 accumulator.
//
// Cube ids run over the condition cubes (read from x_cache) first, then the noise cubes.
// One workgroup per (head, cube, batch) -- heads fastest, so neighbouring workgroups read
// neighbouring 2*D-byte pieces of the same token records -- stages the 64 x D tile in LDS and
// writes the requested layouts as 16-byte vector stores.
#include "bsa_launch.h"

namespace bsa {

template <int D>
__global__ __launch_bounds__(256) void gather_kernel(Geom g, const bf16_t* __restrict__ x,
                                                     const bf16_t* __restrict__ xc, int mode,
                                                     bf16_t* __restrict__ out_row,
                                                     bf16_t* __restrict__ out_trans) {
  constexpr int LD = D + 8;  // padded LDS row (elements)
  constexpr int S = D / 16;
  constexpr int DB = D / 32;
  constexpr int UNITS = 64 * D / 8;  // 16-byte units per cube block
  __shared__ bf16_t tile[64 * LD];
  const int h = blockIdx.x;
  const int j = blockIdx.y;  // global key cube id
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const bool cached = j < g.nbc;
  const bf16_t* src = cached ? xc : x;
  const int N = cached ? g.Nc : g.Nq;
  const int cube = cached ? j : j - g.nbc;
  constexpr int CPR = D / 8;  // 16-byte chunks per token row
  for (int u = tid; u < UNITS; u += 256) {
    const int row = u / CPR, ch = u % CPR;
    const int tok = cube_token(g, cube, row);  // -1: slot outside a ragged grid -> zero row
    *reinterpret_cast<uint4*>(tile + row * LD + ch * 8) =
        tok >= 0 ? *reinterpret_cast<const uint4*>(src + bnhd_offset(g, N, b, tok, h) + ch * 8)
                 : make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  const size_t blk = (((size_t)b * g.Hh + h) * g.nbk + j) * (size_t)(64 * D);
  if (mode & GATHER_ROW) {
    for (int u = tid; u < UNITS; u += 256) {
      const int lane = u % 64;
      const int s = (u / 64) % S;
      const int rb = u / (64 * S);
      const int row = 32 * rb + (lane & 31);
      const int d0 = (lane >> 5) * (D / 2) + 8 * s;
      *reinterpret_cast<uint4*>(out_row + blk + (size_t)u * 8) =
          *reinterpret_cast<const uint4*>(tile + row * LD + d0);
    }
  }
  if (mode & GATHER_TRANS) {
    for (int u = tid; u < UNITS; u += 256) {
      const int lane = u % 64;
      const int s2 = (u / 64) % 2;
      const int db = (u / 128) % DB;
      const int rb = u / (128 * DB);
      const int d = 32 * db + (lane & 31);
      const int rbase = 32 * rb + 16 * s2 + 4 * (lane >> 5);
      uint32_t w[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int e0 = 2 * p, e1 = 2 * p + 1;
        const int r0 = rbase + 8 * (e0 >> 2) + (e0 & 3);
        const int r1 = rbase + 8 * (e1 >> 2) + (e1 & 3);
        w[p] = (uint32_t)tile[r0 * LD + d] | ((uint32_t)tile[r1 * LD + d] << 16);
      }
      *reinterpret_cast<uint4*>(out_trans + blk + (size_t)u * 8) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

size_t gather_bytes(const Geom& g, bool with_cache) {
  const size_t cubes = with_cache ? (size_t)g.nbk : (size_t)g.nbq;
  return (size_t)g.B * g.Hh * cubes * 64 * g.D * sizeof(bf16_t);
}

hipError_t launch_gather(const Geom& g, const void* x, const void* x_cache, int mode,
                         bf16_t* out_row, bf16_t* out_trans, hipStream_t s) {
  dim3 grid(g.Hh, g.nbk, g.B);
  if (g.D == 64)
    hipLaunchKernelGGL(gather_kernel<64>, grid, dim3(256), 0, s, g, (const bf16_t*)x,
                       (const bf16_t*)x_cache, mode, out_row, out_trans);
  else
    hipLaunchKernelGGL(gather_kernel<128>, grid, dim3(256), 0, s, g, (const bf16_t*)x,
                       (const bf16_t*)x_cache, mode, out_row, out_trans);
  return hipGetLastError();
}

}  // namespace bsa
