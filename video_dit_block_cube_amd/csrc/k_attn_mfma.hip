// k_attn_mfma.hip -- gathered block-sparse flash attention forward on bf16 MFMA (gfx950).
//
// For each query cube, softmax attention over the tokens of its selected key cubes only, every
// unselected cube pair skipped ("LongCat-Video deep dive", ai-news-5min-kr, block-sparse
// attention paragraph); condition cubes come from the cached K/V of the condition frames
// ("LongCat-Video 高效長視頻生成探索世界模型的第壹步", meituan.com talk, section 2.1).  Both
// products are dense contractions, so they run on v_mfma_f32_32x32x16_bf16 with fp32
// accumulation; the softmax is online, in fp32, in the base-2 domain (hardware v_exp_f32).
//
// MI355X design (one wave64 = one 64-token query cube):
//  * S^T = K Q^T per 32-key half cube: A = K rows (ROW gather layout, 1 KB coalesced loads
//    straight into the operand registers), B = Q^T (kept in LDS in operand order, 16 KB).
//  * The S^T accumulator holds, per lane, one query column and 16 keys, so P^T converted to bf16
//    in place IS the B operand of O^T = V^T P^T; V^T comes pre-transposed (TRANS gather layout)
//    in the matching key order.  No LDS round trip and no shuffles for P.
//  * Row max needs one xor-32 shuffle per query block; the row sum stays per lane until the end.
//  * Lazy rescale: the running max only moves when a tile's max exceeds it by more than 8 (base 2),
//    so P <= 256 and the O accumulators are rescaled rarely; the result is exact either way
//    because O and l are always scaled by the same exp2(m_used).
//  * Next tile's K is requested right after this tile's S MFMAs, next V right after the PV
//    MFMAs; about 230 live VGPRs, so two waves share each SIMD and hide each other's latency.
//  * Work order is head-major (all XCDs work on the same (b, h) at a time, keeping that head's
//    K/V hot in the shared Infinity Cache) and XCD-aware: workgroup L runs on XCD L%8, which gets
//    a contiguous run of query cubes of the head (spatial neighbours select similar key cubes).
#include "bsa_launch.h"

namespace bsa {

namespace {

__device__ __forceinline__ bf16x8 ld16(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// 16-byte buffer load: wave-uniform byte offset `soff` (SGPR) + per-lane `voff` (VGPR).
__device__ __forceinline__ bf16x8 bld16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& a, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)a[base + e];
  return r;
}

}  // namespace

template <int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_mfma_kernel(Geom g, const bf16_t* __restrict__ q,
                                                      const bf16_t* __restrict__ krow,
                                                      const bf16_t* __restrict__ vtr,
                                                      const int32_t* __restrict__ idx, int k_sel,
                                                      float c_log2, int cpx,
                                                      bf16_t* __restrict__ o,
                                                      float* __restrict__ lse) {
  constexpr int S = D / 16;   // k-steps of the QK^T contraction
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  __shared__ bf16x8 qs[S * 2 * 64];

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

  // Q^T operand fragments -> LDS (each lane stores exactly what it will read back).
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int tq = cube_token(g, i, 32 * qb + l32);
    const bf16_t* src = q + bnhd_offset(g, g.Nq, b, tq, h) + hh * (D / 2);
#pragma unroll
    for (int s = 0; s < S; ++s) qs[(s * 2 + qb) * 64 + lane] = ld16(src + 8 * s);
  }

  f32x16 acc[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[db][qb][e] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_part[2] = {0.f, 0.f};

  const int32_t* irow = idx + ((size_t)bh * g.nbq + i) * k_sel;
  constexpr int cube_bytes = 64 * D * 2;
  const size_t bh_bytes = (size_t)g.nbk * cube_bytes;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(krow + (size_t)bh * g.nbk * (64 * D), bh_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vtr + (size_t)bh * g.nbk * (64 * D), bh_bytes);
  const int vlane = lane * 16;
  const int ntiles = 2 * k_sel;

  bf16x8 kr[S], vr[DB * 2];
  {
    const int off0 = irow[0] * cube_bytes;
#pragma unroll
    for (int s = 0; s < S; ++s) kr[s] = bld16(rk, vlane, off0 + s * 1024);
#pragma unroll
    for (int u = 0; u < DB * 2; ++u) vr[u] = bld16(rv, vlane, off0 + u * 1024);
  }

  for (int t = 0; t < ntiles; ++t) {
    // Q^T lives in LDS, not registers: keep the compiler from hoisting its loop-invariant reads.
    asm volatile("" ::: "memory");
    // ---- S^T = K Q^T for this 32-key half cube ----
    f32x16 st[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int e = 0; e < 16; ++e) st[qb][e] = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const bf16x8 q0 = qs[(s * 2 + 0) * 64 + lane];
      const bf16x8 q1 = qs[(s * 2 + 1) * 64 + lane];
      st[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[s], q0, st[0], 0, 0, 0);
      st[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[s], q1, st[1], 0, 0, 0);
    }
    // ---- request next tile's K ----
    const int tn = t + 1 < ntiles ? t + 1 : t;
    const int noff = irow[tn >> 1] * cube_bytes + (tn & 1) * (32 * D * 2);
#pragma unroll
    for (int s = 0; s < S; ++s) kr[s] = bld16(rk, vlane, noff + s * 1024);

    // ---- online softmax (base 2) ----
    float tgt[2];
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = st[qb][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, st[qb][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      tgt[qb] = mx * c_log2;
      need |= tgt[qb] > m_run[qb] + 8.0f;
    }
    if (__ballot(need)) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float m_new = (tgt[qb] > m_run[qb] + 8.0f) ? tgt[qb] : m_run[qb];
        const float alpha = fast_exp2(m_run[qb] - m_new);
        m_run[qb] = m_new;
        l_part[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[db][qb][e] *= alpha;
      }
    }
    bf16x8 pb[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float ls = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = fast_exp2(fmaf(st[qb][8 * s2 + e], c_log2, -m_run[qb]));
          ls += p;
          pb[s2][qb][e] = (__bf16)p;
        }
      }
      l_part[qb] += ls;
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          acc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[db * 2 + s2], pb[s2][qb],
                                                                acc[db][qb], 0, 0, 0);
    // ---- request next tile's V ----
#pragma unroll
    for (int u = 0; u < DB * 2; ++u) vr[u] = bld16(rv, vlane, noff + u * 1024);
  }

  // ---- epilogue: normalise, write O (bf16) and LSE ----
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = l_part[qb] + __shfl_xor(l_part[qb], 32, 64);
    const float inv = 1.0f / l;
    const int tq = cube_token(g, i, 32 * qb + l32);
    bf16_t* orow = o + bnhd_offset(g, g.Nq, b, tq, h);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * db + 8 * r4 + 4 * hh;
        uint32_t w0 = (uint32_t)f32_to_bf16_bits(acc[db][qb][4 * r4 + 0] * inv) |
                      ((uint32_t)f32_to_bf16_bits(acc[db][qb][4 * r4 + 1] * inv) << 16);
        uint32_t w1 = (uint32_t)f32_to_bf16_bits(acc[db][qb][4 * r4 + 2] * inv) |
                      ((uint32_t)f32_to_bf16_bits(acc[db][qb][4 * r4 + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + d) = make_uint2(w0, w1);
      }
    }
    if (hh == 0) lse[(size_t)bh * g.Nq + tq] = (m_run[qb] + fast_log2(l)) * kLn2;
  }
}

hipError_t launch_fwd_mfma(const Geom& g, const void* q, const bf16_t* k_row,
                           const bf16_t* v_trans, const int32_t* idx, int k_sel, float scale,
                           void* o, float* lse, hipStream_t s) {
  const int cpx = (g.nbq + 7) / 8;
  dim3 grid((unsigned)(g.B * g.Hh * cpx * 8));
  const float c_log2 = scale * kLog2e;
  if (g.D == 64)
    hipLaunchKernelGGL(fwd_mfma_kernel<64>, grid, dim3(64), 0, s, g, (const bf16_t*)q, k_row,
                       v_trans, idx, k_sel, c_log2, cpx, (bf16_t*)o, lse);
  else
    hipLaunchKernelGGL(fwd_mfma_kernel<128>, grid, dim3(64), 0, s, g, (const bf16_t*)q, k_row,
                       v_trans, idx, k_sel, c_log2, cpx, (bf16_t*)o, lse);
  return hipGetLastError();
}

}  // namespace bsa
