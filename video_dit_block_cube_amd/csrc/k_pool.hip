// k_pool.hip -- per-cube mean pool of a [B, Nq, Hh, D] token tensor (HBM-bound).
//
// The cube descriptor is the mean of the cube's token vectors, per head (which cubes matter to
// each other is decided by similarity, "LongCat-Video : Generate 1 minute long AI videos with
// this model", Data Science in Your Pocket, section "Sparse attention").
//
// MI355X design: one workgroup per (batch, cube) reads the cube's c token rows; a token row holds
// every head (Hh*D contiguous elements, 8 KB for 32 heads x 128 bf16), so each 16-byte lane load
// is fully coalesced and each lane owns fixed (head, d) columns -- the reduction over the cube's
// tokens runs down the lane's own registers with no cross-lane traffic.  When a row has fewer
// 16-byte chunks than the workgroup has lanes, the tokens are split across lane groups and the
// partial sums meet in LDS.  Accumulation is fp32; the result is sum / c.
#include "bsa_launch.h"

namespace bsa {

template <typename T>
struct Vec16;  // 16 bytes of T
template <>
struct Vec16<float> {
  static constexpr int N = 4;
};
template <>
struct Vec16<bf16_t> {
  static constexpr int N = 8;
};

template <typename T>
__global__ __launch_bounds__(256) void pool_kernel(Geom g, const T* __restrict__ x,
                                                   float* __restrict__ out) {
  constexpr int V = Vec16<T>::N;
  __shared__ float red[256 * V];
  const int cube = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int cols = g.Hh * g.D;
  const int nchunks = cols / V;
  const int G = nchunks < 256 ? nchunks : 256;
  const int tsplit = 256 / G;
  const int tg = tid / G;
  const int cg = tid % G;
  const float cf = (float)cube_count(g, cube);  // fewer than c on a ragged edge

  for (int ch0 = 0; ch0 < nchunks; ch0 += G) {
    const int ch = ch0 + cg;
    const bool active = (tg < tsplit) && (ch < nchunks);
    float acc[V];
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = 0.f;
    if (active) {
#pragma unroll 4
      for (int s = tg; s < g.c; s += tsplit) {
        const int tok = cube_token(g, cube, s);
        if (tok < 0) continue;  // slot outside a ragged grid
        const T* row = x + ((size_t)b * g.Nq + tok) * (size_t)cols + (size_t)ch * V;
        const uint4 raw = *reinterpret_cast<const uint4*>(row);
        const T* vals = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] += load_as_f32<T>(vals + e);
      }
    }
    if (tsplit > 1) {
      if (active) {
#pragma unroll
        for (int e = 0; e < V; ++e) red[(tg * G + cg) * V + e] = acc[e];
      }
      __syncthreads();
      if (tg == 0 && active) {
        for (int t2 = 1; t2 < tsplit; ++t2) {
#pragma unroll
          for (int e = 0; e < V; ++e) acc[e] += red[(t2 * G + cg) * V + e];
        }
      }
      __syncthreads();
    }
    if (tg == 0 && active) {
      const int e0 = ch * V;
      const int h = e0 / g.D;
      const int d = e0 % g.D;
      float* dst = out + (((size_t)b * g.Hh + h) * g.nbq + cube) * (size_t)g.D + d;
#pragma unroll
      for (int e = 0; e < V; e += 4) {
        float4 w = make_float4(acc[e] / cf, acc[e + 1] / cf,
                               acc[e + 2] / cf, acc[e + 3] / cf);
        *reinterpret_cast<float4*>(dst + e) = w;
      }
    }
  }
}

hipError_t launch_pool(const Geom& g, bool bf16, const void* x, float* out, hipStream_t s) {
  dim3 grid(g.nbq, g.B);
  if (bf16)
    hipLaunchKernelGGL(pool_kernel<bf16_t>, grid, dim3(256), 0, s, g,
                       static_cast<const bf16_t*>(x), out);
  else
    hipLaunchKernelGGL(pool_kernel<float>, grid, dim3(256), 0, s, g,
                       static_cast<const float*>(x), out);
  return hipGetLastError();
}

}  // namespace bsa
