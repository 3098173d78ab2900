// k_attn_simt.hip -- portable block-sparse attention kernels in fp32 arithmetic.
//
// These serve every shape the bf16 MFMA kernels do not (fp32 inputs, cube sizes other than 64).
// They compute exactly what the MFMA path computes -- attention of each query cube over the
// tokens of its selected key cubes, unselected cube pairs skipped entirely ("LongCat-Video deep
// dive", ai-news-5min-kr, block-sparse attention paragraph), condition cubes read from the K/V
// cache for continuation ("LongCat-Video 高效長視頻生成探索世界模型的第壹步", meituan.com talk,
// section 2.1), and the backward with the selection held constant (same talk, section 2.2) --
// with scalar fp32 FMAs on LDS tiles of 64 queries x 64 keys.
//
// Thread map (256 lanes): lane t owns row t/4 of the 64-row tile; the four lanes of a row split
// the 64 columns of the score tile (column sub + 4m) and the D columns of the output.
#include "bsa_launch.h"

namespace bsa {

namespace {

constexpr int kTile = 64;

template <typename T>
__device__ __forceinline__ void load_row_f32(const T* __restrict__ src, float* __restrict__ dst,
                                             int D, int lane4) {
  // 4 lanes cooperate on one row of D elements
  for (int d = lane4; d < D; d += 4) dst[d] = load_as_f32<T>(src + d);
}

// Token of slot `slot` of a cube, or -1 past the cube or outside a ragged grid.
__device__ __forceinline__ int slot_token(const Geom& g, int cube, int slot) {
  return slot < g.c ? cube_token(g, cube, slot) : -1;
}

__device__ __forceinline__ float group4_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 1, 64));
  v = fmaxf(v, __shfl_xor(v, 2, 64));
  return v;
}
__device__ __forceinline__ float group4_sum(float v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  return v;
}

template <int D>
__device__ __forceinline__ float dot_lds(const float* __restrict__ a, const float* __restrict__ b) {
  float acc = 0.f;
#pragma unroll 8
  for (int d = 0; d < D; d += 4) {
    const float4 x = *reinterpret_cast<const float4*>(a + d);
    const float4 y = *reinterpret_cast<const float4*>(b + d);
    acc = fmaf(x.x, y.x, acc);
    acc = fmaf(x.y, y.y, acc);
    acc = fmaf(x.z, y.z, acc);
    acc = fmaf(x.w, y.w, acc);
  }
  return acc;
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// Forward: grid (nbq * ceil(c/64), B*Hh), 256 lanes.
// ---------------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void fwd_simt_kernel(Geom g, const T* __restrict__ q,
                                                       const T* __restrict__ k,
                                                       const T* __restrict__ v,
                                                       const T* __restrict__ kc,
                                                       const T* __restrict__ vc,
                                                       const int32_t* __restrict__ idx,
                                                       int k_sel, float scale,
                                                       T* __restrict__ o, float* __restrict__ lse) {
  constexpr int LD = D + 4;
  extern __shared__ float sm[];
  float* Qs = sm;
  float* Ks = Qs + kTile * LD;
  float* Vs = Ks + kTile * LD;
  float* Ps = Vs + kTile * LD;  // [64][65]
  float* kok = Ps + kTile * 65;  // 1 where the tile's key slot holds a token
  const int nqc = (g.c + kTile - 1) / kTile;
  const int i = blockIdx.x / nqc;
  const int qc0 = (blockIdx.x % nqc) * kTile;
  const int bh = blockIdx.y;
  const int b = bh / g.Hh, h = bh % g.Hh;
  const int tid = threadIdx.x;
  const int row = tid >> 2, sub = tid & 3;
  const int qrow = qc0 + row;
  const int qtok = slot_token(g, i, qrow);
  const bool row_ok = qtok >= 0;

  {
    float* dst = Qs + row * LD;
    if (row_ok) load_row_f32(q + bnhd_offset(g, g.Nq, b, qtok, h), dst, D, sub);
    else for (int d = sub; d < D; d += 4) dst[d] = 0.f;
  }
  constexpr int DO = D / 4;
  float acc[DO];
#pragma unroll
  for (int e = 0; e < DO; ++e) acc[e] = 0.f;
  float m_run = -INFINITY, l_part = 0.f;
  const int32_t* irow = idx + ((size_t)bh * g.nbq + i) * k_sel;

  for (int t = 0; t < k_sel; ++t) {
    const int j = min(max(irow[t], 0), g.nbk - 1);
    const bool cached = j < g.nbc;
    const T* ksrc = cached ? kc : k;
    const T* vsrc = cached ? vc : v;
    const int N = cached ? g.Nc : g.Nq;
    const int cube = cached ? j : j - g.nbc;
    for (int kc0 = 0; kc0 < g.c; kc0 += kTile) {
      __syncthreads();
      {
        const int ktok = slot_token(g, cube, kc0 + row);
        float* kd = Ks + row * LD;
        float* vd = Vs + row * LD;
        if (ktok >= 0) {
          const size_t off = bnhd_offset(g, N, b, ktok, h);
          load_row_f32(ksrc + off, kd, D, sub);
          load_row_f32(vsrc + off, vd, D, sub);
        } else {
          for (int d = sub; d < D; d += 4) { kd[d] = 0.f; vd[d] = 0.f; }
        }
        if (sub == 0) kok[row] = ktok >= 0 ? 1.f : 0.f;
      }
      __syncthreads();
      float s[16];
      float mt = -INFINITY;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const int key = sub + 4 * m;
        s[m] = kok[key] != 0.f ? dot_lds<D>(Qs + row * LD, Ks + key * LD) * scale : -INFINITY;
        mt = fmaxf(mt, s[m]);
      }
      mt = group4_max(mt);
      const float m_new = fmaxf(m_run, mt);
      // a tile with no key yet seen keeps m at -inf: nothing to rescale (avoids -inf - -inf)
      const float alpha = m_new == -INFINITY ? 1.f : expf(m_run - m_new);
      float psum = 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const float p = s[m] == -INFINITY ? 0.f : expf(s[m] - m_new);
        psum += p;
        Ps[row * 65 + sub + 4 * m] = p;
      }
      l_part = l_part * alpha + psum;
      m_run = m_new;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < DO; ++e) acc[e] *= alpha;
      for (int key = 0; key < kTile; ++key) {
        const float p = Ps[row * 65 + key];
        const float* vr = Vs + key * LD + sub * DO;
#pragma unroll
        for (int e = 0; e < DO; ++e) acc[e] = fmaf(p, vr[e], acc[e]);
      }
    }
  }
  const float l = group4_sum(l_part);
  if (row_ok) {
    const int tok = qtok;
    T* orow = o + bnhd_offset(g, g.Nq, b, tok, h) + sub * DO;
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < DO; ++e) store_from_f32<T>(orow + e, acc[e] * inv);
    if (sub == 0) lse[(size_t)bh * g.Nq + tok] = m_run + logf(l);
  }
}

// ---------------------------------------------------------------------------------------------
// Backward dQ (query-stationary): grid (nbq * ceil(c/64), B*Hh).
// ---------------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dq_simt_kernel(Geom g, const T* __restrict__ q,
                                                          const T* __restrict__ k,
                                                          const T* __restrict__ v,
                                                          const T* __restrict__ d_o,
                                                          const float* __restrict__ lse_c,
                                                          const float* __restrict__ delta_c,
                                                          const int32_t* __restrict__ idx,
                                                          int k_sel, float scale,
                                                          float* __restrict__ dq) {
  constexpr int LD = D + 4;
  extern __shared__ float sm[];
  float* Qs = sm;
  float* dOs = Qs + kTile * LD;
  float* Ks = dOs + kTile * LD;
  float* Vs = Ks + kTile * LD;
  float* Ps = Vs + kTile * LD;  // [64][65]
  float* kok = Ps + kTile * 65;  // 1 where the tile's key slot holds a token
  const int nqc = (g.c + kTile - 1) / kTile;
  const int i = blockIdx.x / nqc;
  const int qc0 = (blockIdx.x % nqc) * kTile;
  const int bh = blockIdx.y;
  const int b = bh / g.Hh, h = bh % g.Hh;
  const int tid = threadIdx.x;
  const int row = tid >> 2, sub = tid & 3;
  const int qrow = qc0 + row;
  const int qtok = slot_token(g, i, qrow);
  const bool row_ok = qtok >= 0;
  float lse_r = 0.f, dl_r = 0.f;
  {
    float* dq_ = Qs + row * LD;
    float* dd = dOs + row * LD;
    if (row_ok) {
      const size_t off = bnhd_offset(g, g.Nq, b, qtok, h);
      load_row_f32(q + off, dq_, D, sub);
      load_row_f32(d_o + off, dd, D, sub);
      lse_r = lse_c[((size_t)bh * g.nbq + i) * g.c + qrow];
      dl_r = delta_c[((size_t)bh * g.nbq + i) * g.c + qrow];
    } else {
      for (int d = sub; d < D; d += 4) { dq_[d] = 0.f; dd[d] = 0.f; }
    }
  }
  constexpr int DO = D / 4;
  float acc[DO];
#pragma unroll
  for (int e = 0; e < DO; ++e) acc[e] = 0.f;
  const int32_t* irow = idx + ((size_t)bh * g.nbq + i) * k_sel;
  for (int t = 0; t < k_sel; ++t) {
    const int cube = min(max(irow[t], 0), g.nbq - 1);  // cond_T == 0 in the backward
    for (int kc0 = 0; kc0 < g.c; kc0 += kTile) {
      __syncthreads();
      {
        const int ktok = slot_token(g, cube, kc0 + row);
        float* kd = Ks + row * LD;
        float* vd = Vs + row * LD;
        if (ktok >= 0) {
          const size_t off = bnhd_offset(g, g.Nq, b, ktok, h);
          load_row_f32(k + off, kd, D, sub);
          load_row_f32(v + off, vd, D, sub);
        } else {
          for (int d = sub; d < D; d += 4) { kd[d] = 0.f; vd[d] = 0.f; }
        }
        if (sub == 0) kok[row] = ktok >= 0 ? 1.f : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const int key = sub + 4 * m;
        float ds = 0.f;
        if (row_ok && kok[key] != 0.f) {
          const float s = dot_lds<D>(Qs + row * LD, Ks + key * LD) * scale;
          const float p = expf(s - lse_r);
          const float dp = dot_lds<D>(dOs + row * LD, Vs + key * LD);
          ds = p * (dp - dl_r);
        }
        Ps[row * 65 + key] = ds;
      }
      __syncthreads();
      for (int key = 0; key < kTile; ++key) {
        const float ds = Ps[row * 65 + key];
        const float* kr = Ks + key * LD + sub * DO;
#pragma unroll
        for (int e = 0; e < DO; ++e) acc[e] = fmaf(ds, kr[e], acc[e]);
      }
    }
  }
  if (row_ok) {
    float* out = dq + bnhd_offset(g, g.Nq, b, qtok, h) + sub * DO;
#pragma unroll
    for (int e = 0; e < DO; ++e) out[e] = acc[e] * scale;
  }
}

// ---------------------------------------------------------------------------------------------
// Backward dK, dV (key-stationary over the CSR transpose): grid (nbq * ceil(c/64), B*Hh).
// ---------------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dkdv_simt_kernel(
    Geom g, const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ d_o, const float* __restrict__ lse_c,
    const float* __restrict__ delta_c, const int32_t* __restrict__ csr_off,
    const int32_t* __restrict__ csr_list, float scale, float* __restrict__ dk,
    float* __restrict__ dv) {
  constexpr int LD = D + 4;
  extern __shared__ float sm[];
  float* Ks = sm;
  float* Vs = Ks + kTile * LD;
  float* Qs = Vs + kTile * LD;
  float* dOs = Qs + kTile * LD;
  float* Ps = dOs + kTile * LD;  // [64][65], P^T then dS^T
  float* lse_s = Ps + kTile * 65;
  float* dl_s = lse_s + kTile;
  const int nkc = (g.c + kTile - 1) / kTile;
  const int j = blockIdx.x / nkc;
  const int kc0 = (blockIdx.x % nkc) * kTile;
  const int bh = blockIdx.y;
  const int b = bh / g.Hh, h = bh % g.Hh;
  const int tid = threadIdx.x;
  const int row = tid >> 2, sub = tid & 3;  // row = key within the tile
  const int key = kc0 + row;
  const int ktok = slot_token(g, j, key);
  const bool key_ok = ktok >= 0;
  {
    float* kd = Ks + row * LD;
    float* vd = Vs + row * LD;
    if (key_ok) {
      const size_t off = bnhd_offset(g, g.Nq, b, ktok, h);
      load_row_f32(k + off, kd, D, sub);
      load_row_f32(v + off, vd, D, sub);
    } else {
      for (int d = sub; d < D; d += 4) { kd[d] = 0.f; vd[d] = 0.f; }
    }
  }
  constexpr int DO = D / 4;
  float acc_k[DO], acc_v[DO];
#pragma unroll
  for (int e = 0; e < DO; ++e) { acc_k[e] = 0.f; acc_v[e] = 0.f; }
  // csr_off holds absolute positions into csr_list ([B*Hh][nbk + 1])
  const int32_t* off_bh = csr_off + (size_t)bh * (g.nbk + 1);
  const int beg = off_bh[j], end = off_bh[j + 1];
  for (int n = beg; n < end; ++n) {
    const int i = csr_list[n];
    for (int qc0 = 0; qc0 < g.c; qc0 += kTile) {
      __syncthreads();
      {
        const int qrow = qc0 + row;
        const int qtok = slot_token(g, i, qrow);
        float* qd = Qs + row * LD;
        float* dd = dOs + row * LD;
        // a slot without a token has LSE = +inf (from the delta pass): its P row is 0
        if (qtok >= 0) {
          const size_t off = bnhd_offset(g, g.Nq, b, qtok, h);
          load_row_f32(q + off, qd, D, sub);
          load_row_f32(d_o + off, dd, D, sub);
          if (sub == 0) {
            lse_s[row] = lse_c[((size_t)bh * g.nbq + i) * g.c + qrow];
            dl_s[row] = delta_c[((size_t)bh * g.nbq + i) * g.c + qrow];
          }
        } else {
          for (int d = sub; d < D; d += 4) { qd[d] = 0.f; dd[d] = 0.f; }
          if (sub == 0) { lse_s[row] = INFINITY; dl_s[row] = 0.f; }
        }
      }
      __syncthreads();
      float p[16], ds[16];
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const int qq = sub + 4 * m;
        p[m] = 0.f;
        ds[m] = 0.f;
        if (key_ok && qc0 + qq < g.c) {
          const float s = dot_lds<D>(Ks + row * LD, Qs + qq * LD) * scale;
          p[m] = expf(s - lse_s[qq]);
          const float dp = dot_lds<D>(Vs + row * LD, dOs + qq * LD);
          ds[m] = p[m] * (dp - dl_s[qq]);
        }
        Ps[row * 65 + qq] = p[m];
      }
      __syncthreads();
      for (int qq = 0; qq < kTile; ++qq) {
        const float pv = Ps[row * 65 + qq];
        const float* dr = dOs + qq * LD + sub * DO;
#pragma unroll
        for (int e = 0; e < DO; ++e) acc_v[e] = fmaf(pv, dr[e], acc_v[e]);
      }
      __syncthreads();
#pragma unroll
      for (int m = 0; m < 16; ++m) Ps[row * 65 + sub + 4 * m] = ds[m];
      __syncthreads();
      for (int qq = 0; qq < kTile; ++qq) {
        const float dsv = Ps[row * 65 + qq];
        const float* qr = Qs + qq * LD + sub * DO;
#pragma unroll
        for (int e = 0; e < DO; ++e) acc_k[e] = fmaf(dsv, qr[e], acc_k[e]);
      }
    }
  }
  if (key_ok) {
    const size_t off = bnhd_offset(g, g.Nq, b, ktok, h) + sub * DO;
#pragma unroll
    for (int e = 0; e < DO; ++e) {
      dk[off + e] = acc_k[e] * scale;
      dv[off + e] = acc_v[e];
    }
  }
}

// ---------------------------------------------------------------------------------------------
static size_t simt_lds(int D, int tiles, bool stats) {
  return ((size_t)tiles * kTile * (D + 4) + kTile * 65 + (stats ? 2 * kTile : 0)) * sizeof(float);
}

#define BSA_SET_LDS(kern, bytes)                                                     \
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),                          \
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)(bytes))

hipError_t launch_fwd_simt(const Geom& g, bool bf16, const void* q, const void* k, const void* v,
                           const void* kc, const void* vc, const int32_t* idx, int k_sel,
                           float scale, void* o, float* lse, hipStream_t s) {
  const int nqc = (g.c + kTile - 1) / kTile;
  dim3 grid(g.nbq * nqc, g.B * g.Hh);
  const size_t lds = simt_lds(g.D, 3, true);  // stats region holds the key flags
#define BSA_FWD(T, DD)                                                                        \
  do {                                                                                         \
    auto kern = fwd_simt_kernel<T, DD>;                                                        \
    BSA_SET_LDS(kern, lds);                                                                    \
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, s, g, (const T*)q, (const T*)k,             \
                       (const T*)v, (const T*)kc, (const T*)vc, idx, k_sel, scale, (T*)o, lse); \
  } while (0)
  if (bf16) {
    if (g.D == 64) BSA_FWD(bf16_t, 64); else BSA_FWD(bf16_t, 128);
  } else {
    if (g.D == 64) BSA_FWD(float, 64); else BSA_FWD(float, 128);
  }
#undef BSA_FWD
  return hipGetLastError();
}

hipError_t launch_bwd_dq_simt(const Geom& g, bool bf16, const void* q, const void* k,
                              const void* v, const void* d_o, const float* lse_c,
                              const float* delta_c, const int32_t* idx, int k_sel, float scale,
                              float* dq, hipStream_t s) {
  const int nqc = (g.c + kTile - 1) / kTile;
  dim3 grid(g.nbq * nqc, g.B * g.Hh);
  const size_t lds = simt_lds(g.D, 4, true);  // stats region holds the key flags
#define BSA_DQ(T, DD)                                                                          \
  do {                                                                                          \
    auto kern = bwd_dq_simt_kernel<T, DD>;                                                      \
    BSA_SET_LDS(kern, lds);                                                                     \
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, s, g, (const T*)q, (const T*)k, (const T*)v, \
                       (const T*)d_o, lse_c, delta_c, idx, k_sel, scale, dq);                   \
  } while (0)
  if (bf16) {
    if (g.D == 64) BSA_DQ(bf16_t, 64); else BSA_DQ(bf16_t, 128);
  } else {
    if (g.D == 64) BSA_DQ(float, 64); else BSA_DQ(float, 128);
  }
#undef BSA_DQ
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_simt(const Geom& g, bool bf16, const void* q, const void* k,
                                const void* v, const void* d_o, const float* lse_c,
                                const float* delta_c, const int32_t* csr_off,
                                const int32_t* csr_list, float scale, float* dk, float* dv,
                                hipStream_t s) {
  const int nkc = (g.c + kTile - 1) / kTile;
  dim3 grid(g.nbq * nkc, g.B * g.Hh);
  const size_t lds = simt_lds(g.D, 4, true);
#define BSA_DKDV(T, DD)                                                                        \
  do {                                                                                          \
    auto kern = bwd_dkdv_simt_kernel<T, DD>;                                                    \
    BSA_SET_LDS(kern, lds);                                                                     \
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, s, g, (const T*)q, (const T*)k, (const T*)v, \
                       (const T*)d_o, lse_c, delta_c, csr_off, csr_list, scale, dk, dv);        \
  } while (0)
  if (bf16) {
    if (g.D == 64) BSA_DKDV(bf16_t, 64); else BSA_DKDV(bf16_t, 128);
  } else {
    if (g.D == 64) BSA_DKDV(float, 64); else BSA_DKDV(float, 128);
  }
#undef BSA_DKDV
  return hipGetLastError();
}

}  // namespace bsa
