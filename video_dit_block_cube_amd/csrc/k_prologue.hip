// k_prologue.hip -- attention prologue fused with the cube pool: QK RMS normalisation, 3D rotary
// position embedding and the per-cube means that feed block selection, in one HBM pass.
//
// Every 3D self-attention layer normalises its queries and keys and encodes position with rotary
// embeddings over the three axes time, height and width ("美团LongCat-Video揭秘：13.6B参数长视频
// 生成模型如何终结画面漂移？", xugj520, section "三、模型架构：Diffusion Transformer 的高维协奏";
// "LongCat-Video deep dive", ai-news-5min-kr, the layer table row for the positional encoding).  The pages give no formula; the kernel
// computes, per (token, head):
//   y = x / sqrt(mean_d x^2 + eps) * gamma,  then channel pairs (2i, 2i+1) of the time, height and
//   width blocks (widths D - 4*floor(D/6), 2*floor(D/6), 2*floor(D/6)) rotated by
//   pos_axis * theta^(-2i / width), pos = the token's coordinate on the full latent grid.
// For the noise segment it also writes the mean of y over each cube (fp32, of the unrounded y).
//
// MI355X design: one workgroup per (batch, cube) of the segment, exactly like the pool: a token row
// holds every head (Hh*D contiguous elements), each lane owns one 16-byte chunk of (head, d)
// columns, so loads and stores are fully coalesced and the cube mean runs down the lane's own
// registers.  The RMS reduction of a (token, head) spans the D/V lanes holding that head's
// columns, all in one wave, and is a butterfly of cross-lane shuffles.  A cube spans only
// ct (ch, cw) positions on the time (height, width) axis, so the workgroup first tabulates
// (cos, sin) for every rotation pair at each of its cube's positions on that pair's axis, in LDS
// (one sincos per thread for 4x4x4 cubes instead of one per pair per token); the angle is formed
// and range-reduced in fp64 and only the reduced angle goes to fp32 sincos, so the rotation is
// accurate at any position.
#include "bsa_launch.h"

namespace bsa {

namespace {

template <typename T>
struct Chunk;  // one 16-byte chunk of T
template <>
struct Chunk<float> {
  static constexpr int N = 4;
};
template <>
struct Chunk<bf16_t> {
  static constexpr int N = 8;
};

__device__ __forceinline__ void store_chunk(float* dst, const float (&y)[4]) {
  *reinterpret_cast<float4*>(dst) = make_float4(y[0], y[1], y[2], y[3]);
}
__device__ __forceinline__ void store_chunk(bf16_t* dst, const float (&y)[8]) {
  uint4 w;
  w.x = (uint32_t)f32_to_bf16_bits(y[0]) | ((uint32_t)f32_to_bf16_bits(y[1]) << 16);
  w.y = (uint32_t)f32_to_bf16_bits(y[2]) | ((uint32_t)f32_to_bf16_bits(y[3]) << 16);
  w.z = (uint32_t)f32_to_bf16_bits(y[4]) | ((uint32_t)f32_to_bf16_bits(y[5]) << 16);
  w.w = (uint32_t)f32_to_bf16_bits(y[6]) | ((uint32_t)f32_to_bf16_bits(y[7]) << 16);
  *reinterpret_cast<uint4*>(dst) = w;
}

}  // namespace

// g: geometry of the segment alone (its frames as T, no condition part); t_offset: grid time of
// the segment's first frame.  out_mean may be null.
template <typename T>
__global__ __launch_bounds__(256) void prologue_kernel(Geom g, int t_offset,
                                                       const T* __restrict__ x,
                                                       const float* __restrict__ gamma,
                                                       float theta, float eps,
                                                       T* __restrict__ y_out,
                                                       float* __restrict__ out_mean) {
  constexpr int V = Chunk<T>::N;
  __shared__ float red[256 * V];
  extern __shared__ float2 rot[];  // (cos, sin): time pairs x ct, height pairs x ch, width x cw
  const int cube = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int cols = g.Hh * g.D;
  const int nchunks = cols / V;
  const int G = nchunks < 256 ? nchunks : 256;  // multiple of D/V (D/V divides 256)
  const int tsplit = 256 / G;
  const int tg = tid / G;
  const int cg = tid % G;
  const int lanes_per_head = g.D / V;  // 8 or 16 (bf16), 16 or 32 (fp32): inside one wave
  const int s6 = 2 * (g.D / 6);
  const int wt = g.D - 2 * s6;  // time block width; height and width blocks are s6 wide
  const float inv_c = 1.0f / (float)cube_count(g, cube);  // fewer than c on a ragged edge
  const double log2_theta = log2((double)theta);
  // cube origin on the grid and the rotation table of this cube
  const int tok0 = cube_token(g, cube, 0);
  const int org[3] = {t_offset + tok0 / (g.H * g.W), (tok0 / g.W) % g.H, tok0 % g.W};
  const int ext[3] = {g.ct, g.ch, g.cw};
  const int npairs[3] = {wt / 2, s6 / 2, s6 / 2};
  const int tbase[3] = {0, npairs[0] * g.ct, npairs[0] * g.ct + npairs[1] * g.ch};
  const int nrot = tbase[2] + npairs[2] * g.cw;
  for (int e = tid; e < nrot; e += 256) {
    const int a = e < tbase[1] ? 0 : (e < tbase[2] ? 1 : 2);
    const int pi = (e - tbase[a]) / ext[a];  // pair index inside the axis block
    const int k = (e - tbase[a]) % ext[a];   // position offset inside the cube
    const int width = a == 0 ? wt : s6;
    const double f = exp2(-(double)(2 * pi) / (double)width * log2_theta);
    const double ang = (double)(org[a] + k) * f;
    const double r = ang - rint(ang * 0.15915494309189535) * 6.283185307179586;
    float sn, cs;
    sincosf((float)r, &sn, &cs);
    rot[e] = make_float2(cs, sn);
  }
  __syncthreads();

  for (int ch0 = 0; ch0 < nchunks; ch0 += G) {
    const int ch = ch0 + cg;
    const bool active = (tg < tsplit) && (ch < nchunks);
    const int e0 = (ch < nchunks ? ch : 0) * V;
    const int d0 = e0 % g.D;
    // this lane's channel gains and, per pair, its axis and row of the rotation table
    float gm[V];
    int axis[V / 2], row[V / 2];
#pragma unroll
    for (int e = 0; e < V; ++e) gm[e] = gamma ? gamma[d0 + e] : 1.0f;
#pragma unroll
    for (int j = 0; j < V / 2; ++j) {
      const int c = d0 + 2 * j;
      const int a = c < wt ? 0 : (c < wt + s6 ? 1 : 2);
      const int start = a == 0 ? 0 : (a == 1 ? wt : wt + s6);
      axis[j] = a;
      row[j] = tbase[a] + ((c - start) / 2) * ext[a];
    }
    float acc[V];
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = 0.f;
    // every lane of a head group runs the same token sequence, so the shuffles line up
    for (int s = tg; s < g.c; s += tsplit) {
      const int tok = cube_token(g, cube, s);
      if (tok < 0) continue;  // slot outside a ragged grid (same for the whole head group)
      const size_t off = ((size_t)b * g.Nq + tok) * (size_t)cols + (size_t)e0;
      float v[V];
      {
        const uint4 raw = active ? *reinterpret_cast<const uint4*>(x + off) : make_uint4(0, 0, 0, 0);
        const T* vals = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int e = 0; e < V; ++e) v[e] = load_as_f32<T>(vals + e);
      }
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < V; ++e) ss = fmaf(v[e], v[e], ss);
      for (int m = 1; m < lanes_per_head; m <<= 1) ss += __shfl_xor(ss, m, 64);
      const float inv = 1.0f / sqrtf(ss / (float)g.D + eps);
      // offsets of slot s inside the cube (raster order within the cube)
      const int off3[3] = {s / (g.ch * g.cw), (s / g.cw) % g.ch, s % g.cw};
      float y[V];
#pragma unroll
      for (int j = 0; j < V / 2; ++j) {
        const float2 cr = rot[row[j] + off3[axis[j]]];
        const float a0 = v[2 * j] * inv * gm[2 * j];
        const float a1 = v[2 * j + 1] * inv * gm[2 * j + 1];
        y[2 * j] = a0 * cr.x - a1 * cr.y;
        y[2 * j + 1] = a0 * cr.y + a1 * cr.x;
      }
      if (active) {
        store_chunk(y_out + off, y);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] += y[e];
      }
    }
    if (out_mean == nullptr) continue;
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
      const int h = e0 / g.D;
      float* dst = out_mean + (((size_t)b * g.Hh + h) * g.nbq + cube) * (size_t)g.D + d0;
#pragma unroll
      for (int e = 0; e < V; e += 4)
        *reinterpret_cast<float4*>(dst + e) = make_float4(acc[e] * inv_c, acc[e + 1] * inv_c,
                                                          acc[e + 2] * inv_c, acc[e + 3] * inv_c);
    }
  }
}

hipError_t launch_prologue(const Geom& seg, int t_offset, bool bf16, const void* x,
                           const float* gamma, float rope_theta, float eps, void* y,
                           float* y_mean, hipStream_t s) {
  if (seg.nbq == 0) return hipSuccess;
  dim3 grid(seg.nbq, seg.B);
  const int s6 = 2 * (seg.D / 6);
  const size_t rot_bytes =
      (size_t)((seg.D - 2 * s6) / 2 * seg.ct + s6 / 2 * seg.ch + s6 / 2 * seg.cw) * sizeof(float2);
  if (bf16)
    hipLaunchKernelGGL(prologue_kernel<bf16_t>, grid, dim3(256), rot_bytes, s, seg, t_offset,
                       static_cast<const bf16_t*>(x), gamma, rope_theta, eps, static_cast<bf16_t*>(y),
                       y_mean);
  else
    hipLaunchKernelGGL(prologue_kernel<float>, grid, dim3(256), rot_bytes, s, seg, t_offset,
                       static_cast<const float*>(x), gamma, rope_theta, eps, static_cast<float*>(y),
                       y_mean);
  return hipGetLastError();
}

}  // namespace bsa
