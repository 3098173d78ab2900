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
//  * Next tile's V (and K) is requested right after this tile's PV MFMAs -- at D = 64 the next K
//    already after the S MFMAs, a longer lead that D = 128 has no registers for; about 245 live
//    VGPRs at D = 128, so two waves share each SIMD and hide each other's latency.
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

// Q^T operand fragments straight from the ROW-gathered Q cube into LDS, no VGPRs in between:
// instruction (s, qb) moves the 1 KB block of lanes' 16-byte fragments to qs[(s*2 + qb)*64 ...].
template <int D>
__device__ __forceinline__ void load_q_lds(__amdgpu_buffer_rsrc_t rq, int qoff, bf16x8* qs,
                                           int lane) {
  constexpr int S = D / 16;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int s = 0; s < S; ++s)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rq, (__attribute__((address_space(3))) void*)(qs + (s * 2 + qb) * 64), 16, lane * 16,
          qoff + (qb * S + s) * 1024, 0, 0);
}

__device__ __forceinline__ void wait_vmem_all() {
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): every vector memory load of this wave is done
}

// [lo, hi) = positions of the ascending selection row whose cube ids lie in [key_lo, key_hi),
// counted with one coalesced pass over the row.
__device__ __forceinline__ void row_span(const int32_t* __restrict__ irow, int k_sel, int key_lo,
                                         int key_hi, int lane, int& lo, int& hi) {
  int below_lo = 0, below_hi = 0;
  for (int c0 = 0; c0 < k_sel; c0 += 64) {
    const int e = c0 + lane;
    const int v = e < k_sel ? irow[e] : 0x7fffffff;
    below_lo += __popcll(__ballot(v < key_lo));
    below_hi += __popcll(__ballot(v < key_hi));
  }
  lo = below_lo;
  hi = below_hi;
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& a, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)a[base + e];
  return r;
}

}  // namespace

// Slot mask of key cube j's 32-key half `half` from the per-launch table (ragged grids).
__device__ __forceinline__ uint32_t key_half_mask(const uint2* __restrict__ kmask, int j,
                                                  int half) {
  const uint2 m = kmask[j];
  return half ? m.y : m.x;
}

// Online-softmax attention of one 64-token query cube over the 32-key half cubes
// [t_begin, t_end) of its (ascending) selection row, where row position p stands for entry
// p + (p >= p_split ? p_skip : 0) (two disjoint spans walked as one; p_skip = 0 for one span).
// Accumulates O^T (unnormalised), the running base-2 max and this lane's partial row sums.  On a
// ragged grid (RAGGED, a separate instantiation so divisible grids carry none of its registers),
// key slots of a partial edge cube that hold no token get S = -inf.
template <int D, bool EARLY_K, bool RAGGED>
__device__ __forceinline__ void attend_span(const Geom& g, const bf16x8* __restrict__ qs,
                                            __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                            const int32_t* __restrict__ irow, int t_begin,
                                            int t_end, int p_split, int p_skip, float c_log2,
                                            const uint2* __restrict__ kmask, int lane,
                                            f32x16 (&acc)[D / 32][2], float (&m_run)[2],
                                            float (&l_part)[2]) {
  constexpr int S = D / 16;
  constexpr int DB = D / 32;
  constexpr int cube_bytes = 64 * D * 2;
  const int vlane = lane * 16;
  int cur_j;                   // key cube id of tile t
  uint32_t km_cur = ~0u;       // its slot mask (RAGGED): bit k set iff key slot k holds a token
  bf16x8 kr[S], vr[DB * 2];
  {
    const int p0 = t_begin >> 1;
    cur_j = irow[p0 + (p0 >= p_split ? p_skip : 0)];
    if constexpr (RAGGED) km_cur = key_half_mask(kmask, cur_j, t_begin & 1);
    const int off0 = cur_j * cube_bytes + (t_begin & 1) * (32 * D * 2);
#pragma unroll
    for (int s = 0; s < S; ++s) kr[s] = bld16(rk, vlane, off0 + s * 1024);
#pragma unroll
    for (int u = 0; u < DB * 2; ++u) vr[u] = bld16(rv, vlane, off0 + u * 1024);
  }
  wait_vmem_all();  // Q^T fragments were written to LDS by buffer loads issued before these
  for (int t = t_begin; t < t_end; ++t) {
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
    if constexpr (RAGGED) {
      // accumulator row 8*(e/4) + 4*(lane/32) + e%4 of S^T is key slot 32*(t&1) + that row
      if (km_cur != 0xffffffffu) {
        // this lane's rows, shifted so each row's bit sits at a compile-time position
        const uint32_t kml = km_cur >> (4 * (lane >> 5));
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if (!((kml >> (8 * (e >> 2) + (e & 3))) & 1u)) {
            st[0][e] = -INFINITY;
            st[1][e] = -INFINITY;
          }
        }
      }
    }
    const int tn = t + 1 < t_end ? t + 1 : t;
    const int pn = tn >> 1;
    const int nxt_j = irow[pn + (pn >= p_split ? p_skip : 0)];
    const int noff = nxt_j * cube_bytes + (tn & 1) * (32 * D * 2);
    // the next tile's slot mask is requested a whole tile ahead of its use
    uint32_t km_nxt = ~0u;
    if constexpr (RAGGED) km_nxt = key_half_mask(kmask, nxt_j, tn & 1);
    if constexpr (EARLY_K) {
      // ---- request next tile's K now (longer lead, more live registers) ----
#pragma unroll
      for (int s = 0; s < S; ++s) kr[s] = bld16(rk, vlane, noff + s * 1024);
    }

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
    // ---- P^T (bf16, in place of S^T) and O^T += V^T P^T, one 16-key half at a time ----
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8 pb[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float ls = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = fast_exp2(fmaf(st[qb][8 * s2 + e], c_log2, -m_run[qb]));
          ls += p;
          pb[qb][e] = (__bf16)p;
        }
        l_part[qb] += ls;
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          acc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[db * 2 + s2], pb[qb],
                                                                acc[db][qb], 0, 0, 0);
    }
    // ---- request next tile's V (and K when not requested earlier) ----
    if constexpr (!EARLY_K) {
#pragma unroll
      for (int s = 0; s < S; ++s) kr[s] = bld16(rk, vlane, noff + s * 1024);
    }
#pragma unroll
    for (int u = 0; u < DB * 2; ++u) vr[u] = bld16(rv, vlane, noff + u * 1024);
    cur_j = nxt_j;
    km_cur = km_nxt;
  }
}

template <int D>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[D / 32][2]) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[db][qb][e] = 0.f;
}

// Single pass: one wave per query cube over its whole selection; writes O (bf16) and LSE.
template <int D, bool EARLY_K, bool RAGGED>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_mfma_kernel(
    Geom g, const bf16_t* __restrict__ q_row, const bf16_t* __restrict__ krow,
    const bf16_t* __restrict__ vtr, const int32_t* __restrict__ idx, int k_sel, float c_log2,
    int cpx, const uint2* __restrict__ kmask, bf16_t* __restrict__ o, float* __restrict__ lse) {
  constexpr int DB = D / 32;
  constexpr int cube_bytes = 64 * D * 2;
  __shared__ bf16x8 qs[(D / 16) * 2 * 64];
  const int L = blockIdx.x;
  const int xcd = L & 7;
  const int k8 = L >> 3;
  const int bh = k8 / cpx;
  const int i = xcd * cpx + (k8 % cpx);
  if (i >= g.nbq) return;
  const int b = bh / g.Hh, h = bh % g.Hh;
  const int lane = threadIdx.x;
  const int l32 = lane & 31, hh = lane >> 5;
  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc(q_row + (size_t)bh * g.nbq * (64 * D), (size_t)g.nbq * cube_bytes);
  load_q_lds<D>(rq, i * cube_bytes, qs, lane);
  const size_t bh_bytes = (size_t)g.nbk * cube_bytes;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(krow + (size_t)bh * g.nbk * (64 * D), bh_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vtr + (size_t)bh * g.nbk * (64 * D), bh_bytes);
  const int32_t* irow = idx + ((size_t)bh * g.nbq + i) * k_sel;
  f32x16 acc[DB][2];
  zero_acc<D>(acc);
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_part[2] = {0.f, 0.f};
  attend_span<D, EARLY_K, RAGGED>(g, qs, rk, rv, irow, 0, 2 * k_sel, k_sel, 0, c_log2, kmask,
                                  lane, acc, m_run, l_part);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = l_part[qb] + __shfl_xor(l_part[qb], 32, 64);
    const float inv = 1.0f / l;
    const int tq = cube_token(g, i, 32 * qb + l32);
    if (tq < 0) continue;  // slot outside a ragged grid
    bf16_t* orow = o + bnhd_offset(g, g.Nq, b, tq, h);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * db + 8 * r4 + 4 * hh;
        uint32_t w0 = (uint32_t)f32_to_bf16_bits(acc[db][qb][4 * r4 + 0] * inv) |
                      ((uint32_t)f32_to_bf16_bits(acc[db][qb][4 * r4 + 1] * inv) << 16);
        uint32_t w1 = (uint32_t)f32_to_bf16_bits(acc[db][qb][4 * r4 + 2] * inv) |
                      ((uint32_t)f32_to_bf16_bits(acc[db][qb][4 * r4 + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + d) = make_uint2(w0, w1);
      }
    if (hh == 0) lse[(size_t)bh * g.Nq + tq] = (m_run[qb] + fast_log2(l)) * kLn2;
  }
}

// Split over key ranges: range s holds the s-th of NS contiguous runs of the condition cube ids
// (`rcc` cubes each) and the s-th of NS runs of the noise cube ids (`rcn` each), so every range
// carries the same share of the always-selected condition cubes.  Work item (range s, b, h, query
// cube i) attends only the selected cubes of range s and writes a normalised partial O plus, per
// query row, (base-2 max, row sum, scale exponent e).  Range s runs on XCD s%8, whose L2 then
// only ever holds that range of the head's K/V; the XCD takes its ranges one after the other
// (s = xcd, xcd + 8, ...), heads in order within each.  A pass with r < 8 ranges deals range
// x % r to XCD x, so every XCD works and the XCDs holding one range split its query cubes.
//
// The partial O is stored as fp16 (11 significant bits, against bf16's 8), scaled by 2^-e with
// the smallest e >= 0 that keeps the row's largest magnitude at or below 2^15: a convex
// combination of V rows never exceeds max|V|, so e = 0 unless |V| reaches fp16's range, and the
// power-of-two scale is exact.  The merge then rounds O once more, to the output's bf16; with
// bf16 partials the two roundings together could reach 2 * 2^-9 * |O|.
template <int D, bool EARLY_K, bool RAGGED>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_split_kernel(
    Geom g, const bf16_t* __restrict__ q_row, const bf16_t* __restrict__ krow,
    const bf16_t* __restrict__ vtr, const int32_t* __restrict__ idx, int k_sel, float c_log2,
    int ns, int rcc, int rcn, const uint2* __restrict__ kmask, uint16_t* __restrict__ o_part,
    float4* __restrict__ ml_part) {
  constexpr int DB = D / 32;
  constexpr int cube_bytes = 64 * D * 2;
  __shared__ bf16x8 qs[(D / 16) * 2 * 64];
  const int L = blockIdx.x;
  const int xcd = L & 7;
  const int k8 = L >> 3;
  const int per_pass = g.B * g.Hh * g.nbq;
  const int pass = k8 / per_pass;
  const int rem = k8 % per_pass;
  const int bh = rem / g.nbq;
  const int i = rem % g.nbq;
  int sr = xcd + 8 * pass;
  const int r_left = ns - 8 * pass;  // ranges in this pass
  if (r_left < 8) {
    // fewer ranges than XCDs: XCD x takes range x % r_left, and the c XCDs that share a range
    // split its query cubes (cube i goes to the one with x / r_left == i % c)
    const int s_in = xcd % r_left;
    const int c = (8 - s_in + r_left - 1) / r_left;
    if (i % c != xcd / r_left) return;
    sr = 8 * pass + s_in;
  }
  const int b = bh / g.Hh, h = bh % g.Hh;
  const int lane = threadIdx.x;
  const int l32 = lane & 31, hh = lane >> 5;
  const int32_t* irow = idx + ((size_t)bh * g.nbq + i) * k_sel;
  int lo1, hi1, lo2, hi2;  // selected condition cubes of the range, then its noise cubes
  row_span(irow, k_sel, sr * rcc, min((sr + 1) * rcc, g.nbc), lane, lo1, hi1);
  row_span(irow, k_sel, g.nbc + sr * rcn, g.nbc + (sr + 1) * rcn, lane, lo2, hi2);
  if (hi1 < lo1) hi1 = lo1;  // empty condition run (sr * rcc >= nbc)
  const int n_sel = (hi1 - lo1) + (hi2 - lo2);
  const size_t item = ((size_t)sr * g.B * g.Hh + bh) * g.nbq + i;
  float4* ml = ml_part + item * 64;
  if (n_sel == 0) {
    if (hh == 0) {
      ml[l32] = make_float4(-INFINITY, 0.f, 0.f, 0.f);
      ml[32 + l32] = make_float4(-INFINITY, 0.f, 0.f, 0.f);
    }
    return;
  }
  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc(q_row + (size_t)bh * g.nbq * (64 * D), (size_t)g.nbq * cube_bytes);
  load_q_lds<D>(rq, i * cube_bytes, qs, lane);
  const size_t bh_bytes = (size_t)g.nbk * cube_bytes;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(krow + (size_t)bh * g.nbk * (64 * D), bh_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vtr + (size_t)bh * g.nbk * (64 * D), bh_bytes);
  f32x16 acc[DB][2];
  zero_acc<D>(acc);
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_part[2] = {0.f, 0.f};
  attend_span<D, EARLY_K, RAGGED>(g, qs, rk, rv, irow, 2 * lo1, 2 * (lo1 + n_sel), hi1,
                                  lo2 - hi1, c_log2, kmask, lane, acc, m_run, l_part);
  uint16_t* op = o_part + item * (64 * D);
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = l_part[qb] + __shfl_xor(l_part[qb], 32, 64);
    const float inv = 1.0f / l;
    const int row = 32 * qb + l32;
    // the row's largest |O| (its 128 values sit in this lane and the one 32 lanes away)
    float amax = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(acc[db][qb][e]));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64)) * inv;
    int ex;
    (void)__builtin_frexpf(amax, &ex);  // amax < 2^ex
    const int sc = ex > 15 ? ex - 15 : 0;
    const float mul = __builtin_ldexpf(inv, -sc);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * db + 8 * r4 + 4 * hh;
        const f16x2 h0 = {(_Float16)(acc[db][qb][4 * r4 + 0] * mul),
                          (_Float16)(acc[db][qb][4 * r4 + 1] * mul)};
        const f16x2 h1 = {(_Float16)(acc[db][qb][4 * r4 + 2] * mul),
                          (_Float16)(acc[db][qb][4 * r4 + 3] * mul)};
        *reinterpret_cast<uint2*>(op + row * D + d) =
            make_uint2(__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1));
      }
    if (hh == 0) ml[row] = make_float4(m_run[qb], l, (float)sc, 0.f);
  }
}

// Merge of the range partials of one query cube: O = sum_s w_s 2^e_s O'_s / sum_s w_s with
// w_s = l_s * 2^(m_s - M), M = max_s m_s, O'_s the stored fp16 partial; LSE = (M + log2 sum_s
// w_s) * ln 2.  The ranges are summed in their fixed order, so the result does not depend on
// which range finished first.
template <int D>
__global__ __launch_bounds__(256) void fwd_merge_kernel(Geom g, int ns,
                                                        const uint16_t* __restrict__ o_part,
                                                        const float4* __restrict__ ml_part,
                                                        bf16_t* __restrict__ o,
                                                        float* __restrict__ lse) {
  constexpr int DQ = D / 4;  // columns per thread
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const int i = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / g.Hh, h = bh % g.Hh;
  const int t = threadIdx.x;
  const int row = t >> 2, part = t & 3;
  const size_t per_s = (size_t)g.B * g.Hh * g.nbq;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) {
    const float4 v = ml_part[(s * per_s + (size_t)bh * g.nbq + i) * 64 + row];
    if (v.y > 0.f) M = fmaxf(M, v.x);
  }
  float acc[DQ];
#pragma unroll
  for (int e = 0; e < DQ; ++e) acc[e] = 0.f;
  float Lsum = 0.f;
  for (int s = 0; s < ns; ++s) {
    const size_t item = s * per_s + (size_t)bh * g.nbq + i;
    const float4 v = ml_part[item * 64 + row];
    if (!(v.y > 0.f)) continue;
    const float w = v.y * fast_exp2(v.x - M);
    Lsum += w;
    const float wo = __builtin_ldexpf(w, (int)v.z);
    const uint4* src =
        reinterpret_cast<const uint4*>(o_part + item * (64 * D) + row * D + part * DQ);
#pragma unroll
    for (int c8 = 0; c8 < DQ / 8; ++c8) {
      const uint4 u = src[c8];
      const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f16x2 hv = __builtin_bit_cast(f16x2, wd[k]);
        acc[c8 * 8 + 2 * k] = fmaf(wo, (float)hv[0], acc[c8 * 8 + 2 * k]);
        acc[c8 * 8 + 2 * k + 1] = fmaf(wo, (float)hv[1], acc[c8 * 8 + 2 * k + 1]);
      }
    }
  }
  const float inv = 1.0f / Lsum;
  const int tok = cube_token(g, i, row);
  if (tok < 0) return;  // slot outside a ragged grid
  bf16_t* orow = o + bnhd_offset(g, g.Nq, b, tok, h) + part * DQ;
#pragma unroll
  for (int c8 = 0; c8 < DQ / 8; ++c8) {
    uint32_t wd[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      wd[k] = (uint32_t)f32_to_bf16_bits(acc[c8 * 8 + 2 * k] * inv) |
              ((uint32_t)f32_to_bf16_bits(acc[c8 * 8 + 2 * k + 1] * inv) << 16);
    reinterpret_cast<uint4*>(orow)[c8] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  }
  if (part == 0) lse[(size_t)bh * g.Nq + tok] = (M + fast_log2(Lsum)) * kLn2;
}

size_t fwd_split_bytes(const Geom& g, int ns) {
  if (ns <= 1) return 0;
  const size_t items = (size_t)ns * g.B * g.Hh * g.nbq;
  return items * 64 * g.D * sizeof(uint16_t) + items * 64 * sizeof(float4) + 256;
}

size_t fwd_kmask_bytes(const Geom& g) { return g.ragged ? (size_t)g.nbk * sizeof(uint2) : 0; }

int fwd_split_ranges(const Geom& g, int k_sel, int requested) {
  if (requested >= 0) return requested <= 1 ? 1 : requested;
  // Split when the noise cubes a query cube selects out of a head's noise K/V (32 KB per cube)
  // are most of its row and that K/V is far larger than one XCD's 4 MB L2.  When the forced
  // condition cubes dominate, every query cube streams them in the same ascending order and
  // the L2 already reuses them; the partials and their merge would only add work.
  const double head_kv = (double)g.nbq * 64 * g.D * 2 * 2;
  const bool mostly_noise = 2 * (k_sel - g.nbc) >= k_sel;
  return (head_kv > 8.0 * (1 << 20) && mostly_noise) ? 8 : 1;
}

// Slot masks of every key cube of a ragged grid, condition cubes first: word h of cube j has
// bit k set iff slot 32*h + k of the 64-token cube holds a token.
__global__ __launch_bounds__(256) void key_mask_kernel(Geom g, uint2* __restrict__ kmask) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= g.nbk) return;
  const int jc = j < g.nbc ? j : j - g.nbc;  // cube index inside its segment
  kmask[j] = make_uint2(cube_half_mask(g, jc, 0), cube_half_mask(g, jc, 1));
}

template <int D, bool EK, bool RG>
static hipError_t launch_fwd_t(const Geom& g, const bf16_t* q_row, const bf16_t* k_row,
                               const bf16_t* v_trans, const int32_t* idx, int k_sel,
                               float c_log2, void* o, float* lse, int ns, void* split_ws,
                               uint2* kmask, hipStream_t s) {
  if constexpr (RG) {
    // slot masks of every key cube, once per call (the tile loop only loads them)
    hipLaunchKernelGGL(key_mask_kernel, dim3((unsigned)((g.nbk + 255) / 256)), dim3(256), 0, s, g,
                       kmask);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (ns <= 1) {
    const int cpx = (g.nbq + 7) / 8;
    dim3 grid((unsigned)(g.B * g.Hh * cpx * 8));
    hipLaunchKernelGGL((fwd_mfma_kernel<D, EK, RG>), grid, dim3(64), 0, s, g, q_row,
                       k_row, v_trans, idx, k_sel, c_log2, cpx, kmask, (bf16_t*)o, lse);
    return hipGetLastError();
  }
  const int rcc = (g.nbc + ns - 1) / ns;
  const int rcn = (g.nbq + ns - 1) / ns;
  const size_t items = (size_t)ns * g.B * g.Hh * g.nbq;
  uint16_t* o_part = static_cast<uint16_t*>(split_ws);
  float4* ml_part = reinterpret_cast<float4*>(o_part + items * 64 * g.D);
  const int passes = (ns + 7) / 8;
  dim3 grid((unsigned)(8 * passes * g.B * g.Hh * g.nbq));
  hipLaunchKernelGGL((fwd_split_kernel<D, EK, RG>), grid, dim3(64), 0, s, g, q_row,
                     k_row, v_trans, idx, k_sel, c_log2, ns, rcc, rcn, kmask, o_part, ml_part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 mgrid(g.nbq, g.B * g.Hh);
  hipLaunchKernelGGL(fwd_merge_kernel<D>, mgrid, dim3(256), 0, s, g, ns, o_part, ml_part,
                     (bf16_t*)o, lse);
  return hipGetLastError();
}

hipError_t launch_fwd_mfma(const Geom& g, const bf16_t* q_row, const bf16_t* k_row,
                           const bf16_t* v_trans, const int32_t* idx, int k_sel, float scale,
                           void* o, float* lse, int ns, void* split_ws, uint2* kmask,
                           hipStream_t s) {
  const float c_log2 = scale * kLog2e;
  // The next K tile is requested right after the S MFMAs at D = 64.  D = 128 requests it with
  // V after the PV MFMAs: the earlier request needs registers it does not have at two waves per
  // SIMD (the compiler spills, or, with another scheduler, fits it at no measured gain).
#define BSA_FWD_CALL(DD, EK)                                                                   \
  (g.ragged ? launch_fwd_t<DD, EK, true>(g, q_row, k_row, v_trans, idx, k_sel, c_log2, o, lse, \
                                         ns, split_ws, kmask, s)                                 \
            : launch_fwd_t<DD, EK, false>(g, q_row, k_row, v_trans, idx, k_sel, c_log2, o, lse, \
                                          ns, split_ws, kmask, s))
  const hipError_t e = g.D == 64 ? BSA_FWD_CALL(64, true) : BSA_FWD_CALL(128, false);
#undef BSA_FWD_CALL
  return e;
}

}  // namespace bsa
