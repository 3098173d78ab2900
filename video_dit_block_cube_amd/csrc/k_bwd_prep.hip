// k_bwd_prep.hip -- backward preparation: Delta, LSE in cube order, and the CSR transpose of the
// selection (key cube -> ascending list of the query cubes that attend it).
//
// The backward of block-sparse attention (forward and backward both ship, "LongCat-Video
// 高效長視頻生成探索世界模型的第壹步", meituan.com talk, section 2.2) needs Delta_q = <dO_q, O_q>
// per query token, and the key-stationary dK/dV pass needs, for each key cube, the query cubes
// whose selection contains it.
//
// MI355X design: Delta is one wave per (cube, head) with each token row split over 8..32 lanes
// (16-byte loads) and a shuffle reduction; it also re-lays LSE and Delta in cube order so the
// attention kernels read 64 contiguous floats per cube.  The transpose is deterministic and
// atomic-free in global memory: (1) one workgroup per 32 query rows ORs the rows' bits into an
// LDS word per key cube and writes the words column-major, (2) one workgroup per (b, h) popcounts
// each column and scans the counts into the list offsets, (3) one wave per key cube expands its
// column's set bits in ascending row order (a wave prefix sum over the words' bit counts gives
// each lane its first position).
#include "bsa_launch.h"

namespace bsa {

template <typename T>
__global__ __launch_bounds__(64) void delta_kernel(Geom g, const T* __restrict__ o,
                                                   const T* __restrict__ d_o,
                                                   const float* __restrict__ lse,
                                                   float* __restrict__ delta_c,
                                                   float* __restrict__ lse_c,
                                                   float2* __restrict__ ld_c) {
  constexpr int V = 16 / sizeof(T);
  const int i = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / g.Hh, h = bh % g.Hh;
  const int lane = threadIdx.x;
  const int lpr = g.D / V;          // lanes per token row
  const int rpi = 64 / lpr;         // rows per iteration
  const int sub = lane % lpr;
  const int rr = lane / lpr;
  for (int s0 = 0; s0 < g.c; s0 += rpi) {
    const int s = s0 + rr;
    float acc = 0.f;
    const int tok = s < g.c ? cube_token(g, i, s) : -1;
    if (tok >= 0) {
      const size_t off = bnhd_offset(g, g.Nq, b, tok, h) + (size_t)sub * V;
      const uint4 a = *reinterpret_cast<const uint4*>(o + off);
      const uint4 c2 = *reinterpret_cast<const uint4*>(d_o + off);
      const T* av = reinterpret_cast<const T*>(&a);
      const T* cv = reinterpret_cast<const T*>(&c2);
#pragma unroll
      for (int e = 0; e < V; ++e) acc = fmaf(load_as_f32<T>(av + e), load_as_f32<T>(cv + e), acc);
    }
    for (int off = lpr >> 1; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (s < g.c && sub == 0) {
      const size_t dst = ((size_t)bh * g.nbq + i) * g.c + s;
      // a slot outside a ragged grid gets LSE = +inf: P = exp(S - LSE) = 0 for that row
      const float lv = tok >= 0 ? lse[(size_t)bh * g.Nq + tok] : INFINITY;
      delta_c[dst] = acc;
      lse_c[dst] = lv;
      if (ld_c) ld_c[dst] = make_float2(lv * kLog2e, acc);  // base-2 LSE for exp2
    }
  }
}

hipError_t launch_delta(const Geom& g, bool bf16, const void* o, const void* d_o,
                        const float* lse, float* delta_c, float* lse_c, float2* ld_c,
                        hipStream_t s) {
  dim3 grid(g.nbq, g.B * g.Hh);
  if (bf16)
    hipLaunchKernelGGL(delta_kernel<bf16_t>, grid, dim3(64), 0, s, g, (const bf16_t*)o,
                       (const bf16_t*)d_o, lse, delta_c, lse_c, ld_c);
  else
    hipLaunchKernelGGL(delta_kernel<float>, grid, dim3(64), 0, s, g, (const float*)o,
                       (const float*)d_o, lse, delta_c, lse_c, ld_c);
  return hipGetLastError();
}

__host__ __device__ static inline int csr_groups(const Geom& g) { return (g.nbq + 31) / 32; }

size_t csr_bits_words(const Geom& g) {
  return (size_t)g.B * g.Hh * g.nbk * csr_groups(g);
}

__global__ __launch_bounds__(256) void csr_bits_kernel(Geom g, const int32_t* __restrict__ idx,
                                                       int k_sel, uint32_t* __restrict__ bits) {
  extern __shared__ uint32_t words[];  // [nbk]
  const int grp = blockIdx.x;
  const int bh = blockIdx.y;
  const int ngroups = csr_groups(g);
  for (int j = threadIdx.x; j < g.nbk; j += 256) words[j] = 0u;
  __syncthreads();
  const int row0 = grp * 32;
  const int nrows = min(32, g.nbq - row0);
  const int32_t* base = idx + ((size_t)bh * g.nbq + row0) * k_sel;
  for (int e = threadIdx.x; e < nrows * k_sel; e += 256) {
    const int r = e / k_sel;
    const int j = min(max(base[e], 0), g.nbk - 1);
    atomicOr(&words[j], 1u << r);
  }
  __syncthreads();
  for (int j = threadIdx.x; j < g.nbk; j += 256)
    bits[((size_t)bh * g.nbk + j) * ngroups + grp] = words[j];
}

__global__ __launch_bounds__(1024) void csr_fill_kernel(Geom g, int k_sel,
                                                        const uint32_t* __restrict__ bits,
                                                        int32_t* __restrict__ csr_off) {
  extern __shared__ int32_t cnt[];  // [nbk] then [1024] thread totals
  int32_t* tot = cnt + g.nbk;
  const int bh = blockIdx.x;
  const int ngroups = csr_groups(g);
  const int tid = threadIdx.x;
  const uint32_t* colbits = bits + (size_t)bh * g.nbk * ngroups;
  for (int j = tid; j < g.nbk; j += 1024) {
    int c = 0;
    for (int w = 0; w < ngroups; ++w) c += __popc(colbits[(size_t)j * ngroups + w]);
    cnt[j] = c;
  }
  __syncthreads();
  // exclusive scan of cnt[0..nbk): per-thread contiguous segments, then a scan of the totals
  const int seg = (g.nbk + 1023) / 1024;
  const int lo = min(tid * seg, g.nbk), hi = min(lo + seg, g.nbk);
  int run = 0;
  for (int j = lo; j < hi; ++j) run += cnt[j];
  tot[tid] = run;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = (tid >= off) ? tot[tid - off] : 0;
    __syncthreads();
    tot[tid] += v;
    __syncthreads();
  }
  const size_t base = (size_t)bh * g.nbq * k_sel;
  int pre = tot[tid] - run;  // exclusive prefix of this segment
  int32_t* off_bh = csr_off + (size_t)bh * (g.nbk + 1);
  for (int j = lo; j < hi; ++j) {
    off_bh[j] = (int32_t)(base + pre);
    pre += cnt[j];
  }
  if (tid == 1023) off_bh[g.nbk] = (int32_t)(base + tot[1023]);
}

// One wave per key cube j: the query cubes whose bits are set in j's column, ascending, written
// from csr_off[j] on.  Lane l expands word w0 + l of the column after a wave prefix sum of the
// words' bit counts gives its first position.
__global__ __launch_bounds__(1024) void csr_list_kernel(Geom g,
                                                        const uint32_t* __restrict__ bits,
                                                        const int32_t* __restrict__ csr_off,
                                                        int32_t* __restrict__ csr_list) {
  const int bh = blockIdx.y;
  const int j = blockIdx.x * 16 + (threadIdx.x >> 6);
  if (j >= g.nbk) return;
  const int lane = threadIdx.x & 63;
  const int ngroups = csr_groups(g);
  const uint32_t* col = bits + ((size_t)bh * g.nbk + j) * ngroups;
  int pos0 = csr_off[(size_t)bh * (g.nbk + 1) + j];
  for (int w0 = 0; w0 < ngroups; w0 += 64) {
    uint32_t m = (w0 + lane < ngroups) ? col[w0 + lane] : 0u;
    const int c = __popc(m);
    int incl = c;  // inclusive prefix over the lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    int pos = pos0 + incl - c;
    while (m) {
      csr_list[pos++] = (w0 + lane) * 32 + (__ffs(m) - 1);
      m &= m - 1;
    }
    pos0 += __shfl(incl, 63, 64);
  }
}

hipError_t launch_csr(const Geom& g, const int32_t* idx, int k_sel, uint32_t* bits,
                      int32_t* csr_off, int32_t* csr_list, hipStream_t s) {
  const size_t lds1 = (size_t)g.nbk * sizeof(uint32_t);
  const size_t lds2 = ((size_t)g.nbk + 1024) * sizeof(int32_t);
  if (lds1 > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(csr_bits_kernel),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1);
  if (lds2 > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(csr_fill_kernel),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds2);
  hipLaunchKernelGGL(csr_bits_kernel, dim3(csr_groups(g), g.B * g.Hh), dim3(256), lds1, s, g,
                     idx, k_sel, bits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(csr_fill_kernel, dim3(g.B * g.Hh), dim3(1024), lds2, s, g, k_sel, bits,
                     csr_off);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(csr_list_kernel, dim3((unsigned)((g.nbk + 15) / 16), g.B * g.Hh), dim3(1024),
                     0, s, g, bits, csr_off, csr_list);
  return hipGetLastError();
}

}  // namespace bsa

namespace bsa {

// Delta fused with the dO gather (bf16, 64-token cubes): one workgroup per (head, query cube,
// batch) reads the cube's O and dO token rows once, forms Delta = <dO, O> per token, and writes
// the dO cube in the ROW gather layout (see k_gather.hip) plus the interleaved (LSE * log2 e,
// Delta) pairs the MFMA backward kernels read (LSE = +inf, Delta = 0 for a slot outside a ragged
// grid, so such a row's P is 0).  Saves the separate dO gather's second read of dO.
template <int D>
__global__ __launch_bounds__(256) void delta_gather_kernel(Geom g, const bf16_t* __restrict__ o,
                                                           const bf16_t* __restrict__ d_o,
                                                           const float* __restrict__ lse,
                                                           float2* __restrict__ ld_c,
                                                           bf16_t* __restrict__ do_row) {
  constexpr int LD = D + 8;      // padded LDS row (elements)
  constexpr int S = D / 16;
  constexpr int CPR = D / 8;     // 16-byte chunks per token row
  constexpr int UNITS = 64 * CPR;
  __shared__ bf16_t tile[64 * LD];
  __shared__ float dsum[64];
  const int h = blockIdx.x;
  const int i = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int bh = b * g.Hh + h;
  // 256 threads cover 256 / CPR rows per pass; a row's CPR threads are consecutive lanes
  for (int u = tid; u < UNITS; u += 256) {
    const int row = u / CPR, ch = u % CPR;
    const int tok = cube_token(g, i, row);
    uint4 dv = make_uint4(0u, 0u, 0u, 0u);
    float part = 0.f;
    if (tok >= 0) {
      const size_t off = bnhd_offset(g, g.Nq, b, tok, h) + ch * 8;
      dv = *reinterpret_cast<const uint4*>(d_o + off);
      const uint4 ov = *reinterpret_cast<const uint4*>(o + off);
      const uint32_t dw[4] = {dv.x, dv.y, dv.z, dv.w};
      const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        part = fmaf(__uint_as_float(dw[k] << 16), __uint_as_float(ow[k] << 16), part);
        part = fmaf(__uint_as_float(dw[k] & 0xffff0000u), __uint_as_float(ow[k] & 0xffff0000u),
                    part);
      }
    }
    *reinterpret_cast<uint4*>(tile + row * LD + ch * 8) = dv;
#pragma unroll
    for (int off = CPR >> 1; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
    if (ch == 0) dsum[row] = part;
  }
  __syncthreads();
  const size_t blk = ((size_t)bh * g.nbq + i) * (size_t)(64 * D);
  for (int u = tid; u < UNITS; u += 256) {
    const int lane = u % 64;
    const int s = (u / 64) % S;
    const int rb = u / (64 * S);
    const int row = 32 * rb + (lane & 31);
    const int d0 = (lane >> 5) * (D / 2) + 8 * s;
    *reinterpret_cast<uint4*>(do_row + blk + (size_t)u * 8) =
        *reinterpret_cast<const uint4*>(tile + row * LD + d0);
  }
  if (tid < 64) {
    const int tok = cube_token(g, i, tid);
    const float lv = tok >= 0 ? lse[(size_t)bh * g.Nq + tok] : INFINITY;
    ld_c[((size_t)bh * g.nbq + i) * 64 + tid] = make_float2(lv * kLog2e, tok >= 0 ? dsum[tid] : 0.f);
  }
}

hipError_t launch_delta_gather(const Geom& g, const void* o, const void* d_o, const float* lse,
                               float2* ld_c, bf16_t* do_row, hipStream_t s) {
  if (g.c != 64) return hipErrorInvalidValue;
  dim3 grid(g.Hh, g.nbq, g.B);
  if (g.D == 64)
    hipLaunchKernelGGL(delta_gather_kernel<64>, grid, dim3(256), 0, s, g, (const bf16_t*)o,
                       (const bf16_t*)d_o, lse, ld_c, do_row);
  else
    hipLaunchKernelGGL(delta_gather_kernel<128>, grid, dim3(256), 0, s, g, (const bf16_t*)o,
                       (const bf16_t*)d_o, lse, ld_c, do_row);
  return hipGetLastError();
}

}  // namespace bsa
