// k_bwd_mfma.hip -- block-sparse attention backward on bf16 MFMA (gfx950), c == 64.
//
// The backward ships alongside the forward for training ("LongCat-Video 高效長視頻生成探索世界
// 模型的第壹步", meituan.com talk, section 2.2); the selection is a discrete choice and is held
// constant.  With P = exp(scale*Q_i K_j^T - LSE_i) over every selected pair (i, j):
//   dV_j += P^T dO_i,  dS = P o (dO_i V_j^T - Delta_i),  dQ_i += scale*dS K_j,
//   dK_j += scale*dS^T Q_i.
//
// MI355X design: two kernels, each owning its output in registers so no fp32 atomics are needed.
//  * dQ (query-stationary, one wave = one 64-token query cube): Q^T and dO^T operand fragments in
//    LDS; per 32-key half cube, S^T = K Q^T and dP^T = V dO^T on MFMA (K, V from the ROW gather
//    layout), then dS^T in place in the accumulator registers, converted to bf16, is the B
//    operand of dQ^T += K^T dS^T (K^T from the TRANS gather layout).
//  * dK/dV (key-stationary over the CSR transpose, one wave = one 64-token key cube): K and V in
//    LDS as B operands; per 32-query half of each query cube that selected this key cube,
//    S = Q K^T and dP = dO V^T (Q, dO from ROW layouts), then P and dS converted in place are
//    the B operands of dV^T += dO^T P and dK^T += Q^T dS (dO^T, Q^T from TRANS layouts).
//  Operands of the next step are requested as soon as the current ones are consumed; per-lane
//  byte offsets stay constant and the wave-uniform tile offset rides in an SGPR (buffer loads).
#include "bsa_launch.h"

namespace bsa {

namespace {

__device__ __forceinline__ bf16x8 ld16g(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ bf16x8 bld16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void zero16(f32x16& a) {
#pragma unroll
  for (int e = 0; e < 16; ++e) a[e] = 0.f;
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// dQ: grid = B*Hh*cpx*8 (head-major, XCD-aware like the forward), one wave per query cube.
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void bwd_dq_mfma_kernel(
    Geom g, const bf16_t* __restrict__ q, const bf16_t* __restrict__ d_o,
    const bf16_t* __restrict__ k_row, const bf16_t* __restrict__ k_trans,
    const bf16_t* __restrict__ v_row, const float* __restrict__ lse_c,
    const float* __restrict__ delta_c, const int32_t* __restrict__ idx, int k_sel, float scale,
    float c_log2, int cpx, float* __restrict__ dq) {
  constexpr int S = D / 16;
  constexpr int DB = D / 32;
  constexpr int cube_bytes = 64 * D * 2;
  __shared__ bf16x8 qs[S * 2 * 64];
  __shared__ bf16x8 dos[S * 2 * 64];

  const int L = blockIdx.x;
  const int xcd = L & 7;
  const int k8 = L >> 3;
  const int bh = k8 / cpx;
  const int i = xcd * cpx + (k8 % cpx);
  if (i >= g.nbq) return;
  const int b = bh / g.Hh, h = bh % g.Hh;
  const int lane = threadIdx.x;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  float lse2[2], dl[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int tq = cube_token(g, i, 32 * qb + l32);
    const size_t off = bnhd_offset(g, g.Nq, b, tq, h) + hh * (D / 2);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      qs[(s * 2 + qb) * 64 + lane] = ld16g(q + off + 8 * s);
      dos[(s * 2 + qb) * 64 + lane] = ld16g(d_o + off + 8 * s);
    }
    const size_t ci = ((size_t)bh * g.nbq + i) * 64 + 32 * qb + l32;
    lse2[qb] = lse_c[ci] * kLog2e;
    dl[qb] = delta_c[ci];
  }

  f32x16 acc[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db) { zero16(acc[db][0]); zero16(acc[db][1]); }

  const int32_t* irow = idx + ((size_t)bh * g.nbq + i) * k_sel;
  const size_t bh_bytes = (size_t)g.nbk * cube_bytes;
  const size_t bh_elems = (size_t)g.nbk * 64 * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k_row + bh * bh_elems, bh_bytes);
  const __amdgpu_buffer_rsrc_t rkt = make_rsrc(k_trans + bh * bh_elems, bh_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v_row + bh * bh_elems, bh_bytes);
  const int vlane = lane * 16;
  const int ntiles = 2 * k_sel;

  bf16x8 kr[S], vr[S], kt[DB * 2];
  {
    const int off0 = irow[0] * cube_bytes;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      kr[s] = bld16(rk, vlane, off0 + s * 1024);
      vr[s] = bld16(rv, vlane, off0 + s * 1024);
    }
#pragma unroll
    for (int u = 0; u < DB * 2; ++u) kt[u] = bld16(rkt, vlane, off0 + u * 1024);
  }

  for (int t = 0; t < ntiles; ++t) {
    asm volatile("" ::: "memory");
    f32x16 st[2], dpt[2];
    zero16(st[0]); zero16(st[1]); zero16(dpt[0]); zero16(dpt[1]);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const bf16x8 q0 = qs[(s * 2 + 0) * 64 + lane];
      const bf16x8 q1 = qs[(s * 2 + 1) * 64 + lane];
      st[0] = mfma32(kr[s], q0, st[0]);
      st[1] = mfma32(kr[s], q1, st[1]);
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const bf16x8 d0 = dos[(s * 2 + 0) * 64 + lane];
      const bf16x8 d1 = dos[(s * 2 + 1) * 64 + lane];
      dpt[0] = mfma32(vr[s], d0, dpt[0]);
      dpt[1] = mfma32(vr[s], d1, dpt[1]);
    }
    const int tn = t + 1 < ntiles ? t + 1 : t;
    const int noff = irow[tn >> 1] * cube_bytes + (tn & 1) * (32 * D * 2);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      kr[s] = bld16(rk, vlane, noff + s * 1024);
      vr[s] = bld16(rv, vlane, noff + s * 1024);
    }
    bf16x8 dsb[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * s2 + e;
          const float p = fast_exp2(fmaf(st[qb][r], c_log2, -lse2[qb]));
          dsb[s2][qb][e] = (__bf16)(p * (dpt[qb][r] - dl[qb]));
        }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) acc[db][qb] = mfma32(kt[db * 2 + s2], dsb[s2][qb], acc[db][qb]);
#pragma unroll
    for (int u = 0; u < DB * 2; ++u) kt[u] = bld16(rkt, vlane, noff + u * 1024);
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int tq = cube_token(g, i, 32 * qb + l32);
    float* out = dq + bnhd_offset(g, g.Nq, b, tq, h);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * db + 8 * r4 + 4 * hh;
        *reinterpret_cast<float4*>(out + d) =
            make_float4(acc[db][qb][4 * r4] * scale, acc[db][qb][4 * r4 + 1] * scale,
                        acc[db][qb][4 * r4 + 2] * scale, acc[db][qb][4 * r4 + 3] * scale);
      }
  }
}

// ---------------------------------------------------------------------------------------------
// dK, dV: grid = B*Hh*cpx*8, one wave per key cube (cond_T == 0, so key cube j = noise cube j).
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void bwd_dkdv_mfma_kernel(
    Geom g, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ q_row, const bf16_t* __restrict__ q_trans,
    const bf16_t* __restrict__ do_row, const bf16_t* __restrict__ do_trans,
    const float* __restrict__ lse_c, const float* __restrict__ delta_c,
    const int32_t* __restrict__ csr_off, const int32_t* __restrict__ csr_list, float scale,
    float c_log2, int cpx, float* __restrict__ dk, float* __restrict__ dv) {
  constexpr int S = D / 16;
  constexpr int DB = D / 32;
  constexpr int cube_bytes = 64 * D * 2;
  __shared__ bf16x8 ks[2 * S * 64];
  __shared__ bf16x8 vs[2 * S * 64];

  const int L = blockIdx.x;
  const int xcd = L & 7;
  const int k8 = L >> 3;
  const int bh = k8 / cpx;
  const int j = xcd * cpx + (k8 % cpx);
  if (j >= g.nbq) return;
  const int b = bh / g.Hh, h = bh % g.Hh;
  const int lane = threadIdx.x;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // K, V as B operands: lane = key, 8 consecutive d (same d split as the ROW layout).
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int tk = cube_token(g, j, 32 * kb + l32);
    const size_t off = bnhd_offset(g, g.Nq, b, tk, h) + hh * (D / 2);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      ks[(kb * S + s) * 64 + lane] = ld16g(k + off + 8 * s);
      vs[(kb * S + s) * 64 + lane] = ld16g(v + off + 8 * s);
    }
  }

  f32x16 acck[DB][2], accv[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) { zero16(acck[db][kb]); zero16(accv[db][kb]); }

  const int32_t* offs = csr_off + (size_t)bh * (g.nbk + 1);
  const int beg = offs[j], end = offs[j + 1];
  const size_t bh_bytes = (size_t)g.nbq * cube_bytes;
  const size_t bh_elems = (size_t)g.nbq * 64 * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q_row + bh * bh_elems, bh_bytes);
  const __amdgpu_buffer_rsrc_t rqt = make_rsrc(q_trans + bh * bh_elems, bh_bytes);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(do_row + bh * bh_elems, bh_bytes);
  const __amdgpu_buffer_rsrc_t rdt = make_rsrc(do_trans + bh * bh_elems, bh_bytes);
  const int vlane = lane * 16;
  const float* lse_bh = lse_c + (size_t)bh * g.nbq * 64;
  const float* dl_bh = delta_c + (size_t)bh * g.nbq * 64;
  const int nsteps = 2 * (end - beg);

  bf16x8 qr[S], dr[S];
  if (nsteps > 0) {
    const int off0 = csr_list[beg] * cube_bytes;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      qr[s] = bld16(rq, vlane, off0 + s * 1024);
      dr[s] = bld16(rd, vlane, off0 + s * 1024);
    }
  }

  for (int t = 0; t < nsteps; ++t) {
    asm volatile("" ::: "memory");
    const int i = csr_list[beg + (t >> 1)];
    const int qb = t & 1;
    const int coff = i * cube_bytes + qb * (32 * D * 2);
    f32x16 st[2], dp[2];
    zero16(st[0]); zero16(st[1]); zero16(dp[0]); zero16(dp[1]);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      st[0] = mfma32(qr[s], ks[(0 * S + s) * 64 + lane], st[0]);
      st[1] = mfma32(qr[s], ks[(1 * S + s) * 64 + lane], st[1]);
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
      dp[0] = mfma32(dr[s], vs[(0 * S + s) * 64 + lane], dp[0]);
      dp[1] = mfma32(dr[s], vs[(1 * S + s) * 64 + lane], dp[1]);
    }
    // transposed operands of this step, into registers the row operands no longer need
    bf16x8 qt[DB * 2], dt[DB * 2];
#pragma unroll
    for (int u = 0; u < DB * 2; ++u) {
      qt[u] = bld16(rqt, vlane, coff + u * 1024);
      dt[u] = bld16(rdt, vlane, coff + u * 1024);
    }
    // P and dS for the 16 query rows this lane holds (rows 8*r4 + 4*hh + e4 of the 32-row half)
    bf16x8 pb[2][2], dsb[2][2];
    const float* lp = lse_bh + (size_t)i * 64 + 32 * qb + 4 * hh;
    const float* dlp = dl_bh + (size_t)i * 64 + 32 * qb + 4 * hh;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const float4 a4 = *reinterpret_cast<const float4*>(lp + 8 * r4);
      const float4 c4 = *reinterpret_cast<const float4*>(dlp + 8 * r4);
      const float la[4] = {a4.x * kLog2e, a4.y * kLog2e, a4.z * kLog2e, a4.w * kLog2e};
      const float da[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int r = 4 * r4 + e4;
          const float p = fast_exp2(fmaf(st[kb][r], c_log2, -la[e4]));
          pb[kb][r >> 3][r & 7] = (__bf16)p;
          dsb[kb][r >> 3][r & 7] = (__bf16)(p * (dp[kb][r] - da[e4]));
        }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          accv[db][kb] = mfma32(dt[db * 2 + s2], pb[kb][s2], accv[db][kb]);
          acck[db][kb] = mfma32(qt[db * 2 + s2], dsb[kb][s2], acck[db][kb]);
        }
    // row operands of the next step
    const int tn = t + 1 < nsteps ? t + 1 : t;
    const int noff = csr_list[beg + (tn >> 1)] * cube_bytes + (tn & 1) * (32 * D * 2);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      qr[s] = bld16(rq, vlane, noff + s * 1024);
      dr[s] = bld16(rd, vlane, noff + s * 1024);
    }
  }

#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int tk = cube_token(g, j, 32 * kb + l32);
    const size_t off = bnhd_offset(g, g.Nq, b, tk, h);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * db + 8 * r4 + 4 * hh;
        const f32x16& ak = acck[db][kb];
        const f32x16& av = accv[db][kb];
        *reinterpret_cast<float4*>(dk + off + d) =
            make_float4(ak[4 * r4] * scale, ak[4 * r4 + 1] * scale, ak[4 * r4 + 2] * scale,
                        ak[4 * r4 + 3] * scale);
        *reinterpret_cast<float4*>(dv + off + d) =
            make_float4(av[4 * r4], av[4 * r4 + 1], av[4 * r4 + 2], av[4 * r4 + 3]);
      }
  }
}

hipError_t launch_bwd_dq_mfma(const Geom& g, const void* q, const void* d_o,
                              const bf16_t* k_row, const bf16_t* k_trans, const bf16_t* v_row,
                              const float* lse_c, const float* delta_c, const int32_t* idx,
                              int k_sel, float scale, float* dq, hipStream_t s) {
  const int cpx = (g.nbq + 7) / 8;
  dim3 grid((unsigned)(g.B * g.Hh * cpx * 8));
  const float c_log2 = scale * kLog2e;
  if (g.D == 64)
    hipLaunchKernelGGL(bwd_dq_mfma_kernel<64>, grid, dim3(64), 0, s, g, (const bf16_t*)q,
                       (const bf16_t*)d_o, k_row, k_trans, v_row, lse_c, delta_c, idx, k_sel,
                       scale, c_log2, cpx, dq);
  else
    hipLaunchKernelGGL(bwd_dq_mfma_kernel<128>, grid, dim3(64), 0, s, g, (const bf16_t*)q,
                       (const bf16_t*)d_o, k_row, k_trans, v_row, lse_c, delta_c, idx, k_sel,
                       scale, c_log2, cpx, dq);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_mfma(const Geom& g, const void* k, const void* v,
                                const bf16_t* q_row, const bf16_t* q_trans,
                                const bf16_t* do_row, const bf16_t* do_trans,
                                const float* lse_c, const float* delta_c,
                                const int32_t* csr_off, const int32_t* csr_list, float scale,
                                float* dk, float* dv, hipStream_t s) {
  const int cpx = (g.nbq + 7) / 8;
  dim3 grid((unsigned)(g.B * g.Hh * cpx * 8));
  const float c_log2 = scale * kLog2e;
  if (g.D == 64)
    hipLaunchKernelGGL(bwd_dkdv_mfma_kernel<64>, grid, dim3(64), 0, s, g, (const bf16_t*)k,
                       (const bf16_t*)v, q_row, q_trans, do_row, do_trans, lse_c, delta_c,
                       csr_off, csr_list, scale, c_log2, cpx, dk, dv);
  else
    hipLaunchKernelGGL(bwd_dkdv_mfma_kernel<128>, grid, dim3(64), 0, s, g, (const bf16_t*)k,
                       (const bf16_t*)v, q_row, q_trans, do_row, do_trans, lse_c, delta_c,
                       csr_off, csr_list, scale, c_log2, cpx, dk, dv);
  return hipGetLastError();
}

}  // namespace bsa
