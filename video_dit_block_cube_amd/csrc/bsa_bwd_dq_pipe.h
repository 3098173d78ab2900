// bsa_bwd_dq_pipe.h -- the software-pipelined dQ kernel of the block-sparse attention backward
// (head_dim 128, bf16 MFMA, gfx950) as a template shared by the translation units that
// instantiate it: k_bwd_dq_pipe.hip (grids whose sides are cube multiples) and
// k_bwd_dq_pipe_ragged.hip (ragged grids), which need different compiler options (see there).
//
// Same operation as the one-wave dQ kernel (backward shipped with the forward for training:
// "LongCat-Video 高效長視頻生成探索世界模型的第壹步", meituan.com talk, section 2.2): with
// P = exp(scale*Q_i K_j^T - LSE_i) and dS = P o (dO_i V_j^T - Delta_i) over every selected pair,
// dQ_i = scale * sum_j dS K_j.
//
// MI355X design: one wave per query cube, as in the plain dQ kernel, but the tile loop is
// software-pipelined by one tile.  S^T and dP^T of tile t+1 go to the MFMA unit while the VALU
// forms P and dS of tile t, then dQ^T takes tile t's product.  At head_dim 128 the dQ^T
// accumulators, the score accumulators of two tiles and the Q/dO operands need about 490
// registers, so one wave runs per SIMD and no other wave can fill the MFMA unit during the
// exponentials.  Each tile's arithmetic and the order of the dQ^T updates are those of the plain
// loop, so the result is the same bit for bit.
#pragma once

#include "bsa_bwd_tiles.h"

namespace bsa {

template <int D, bool RAGGED>
__global__ __launch_bounds__(64) void bwd_dq_pipe_kernel(
    Geom g, const bf16_t* __restrict__ q_row, const bf16_t* __restrict__ do_row,
    const bf16_t* __restrict__ k_row, const bf16_t* __restrict__ v_row,
    const float2* __restrict__ ld_c, const int32_t* __restrict__ idx, int k_sel, float scale,
    float c_log2, int cpx, int walk_ticks, float* __restrict__ dq) {
  constexpr int S = D / 16;
  constexpr int DB = D / 32;
  constexpr int cube_bytes = 64 * D * 2;
  constexpr int half_bytes = 32 * D * 2;            // a 32-row half block in memory
  constexpr int lds_half = staged_half_bytes<D>();  // the same block staged in LDS
  __shared__ __attribute__((aligned(16))) char stage0[2 * lds_half];  // K rows | V rows
  __shared__ __attribute__((aligned(16))) char stage1[2 * lds_half];

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

  const size_t bh_bytes = (size_t)g.nbk * cube_bytes;
  const size_t bh_elems = (size_t)g.nbk * 64 * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k_row + bh * bh_elems, bh_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v_row + bh * bh_elems, bh_bytes);
  const int32_t* irow = idx + ((size_t)bh * g.nbq + i) * k_sel;
  const int ntiles = 2 * k_sel;  // even and >= 2
  // first entry of the walk: 0, or (walk phase) the first selected cube at or past the clock's
  // phase within the period, the walk wrapping around the row
  int s0 = 0;
  if (walk_ticks > 0) {
    const int phase = (int)((wall_clock64() % (uint64_t)walk_ticks) * (uint64_t)g.nbk /
                            (uint64_t)walk_ticks);
    for (int e0 = 0; e0 < k_sel; e0 += 64) {
      const int e = e0 + lane;
      s0 += __popcll(__ballot(e < k_sel && irow[e] < phase));
    }
    if (s0 >= k_sel) s0 = 0;
  }
  auto entry = [&](int e) { return irow[e + s0 < k_sel ? e + s0 : e + s0 - k_sel]; };
  lds_char* st0 = (lds_char*)stage0;
  lds_char* st1 = (lds_char*)stage1;
  auto stage = [&](int t, lds_char* dst) {  // K and V rows of tile t -> dst
    const int off = entry(t >> 1) * cube_bytes + (t & 1) * half_bytes;
    stage_half<D>(rk, off, dst, lane);
    stage_half<D>(rv, off, dst + lds_half, lane);
  };
  stage(0, st0);

  // Q and dO rows of this query cube as B operands (lane = query, 8 consecutive d).
  const size_t q_bh = (size_t)bh * g.nbq * (64 * D);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q_row + q_bh, (size_t)g.nbq * cube_bytes);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(do_row + q_bh, (size_t)g.nbq * cube_bytes);
  bf16x8 qreg[2][S], dreg[2][S];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int s = 0; s < S; ++s) {
      qreg[qb][s] = bld16(rq, lane * 16, i * cube_bytes + (qb * S + s) * 1024);
      dreg[qb][s] = bld16(rd, lane * 16, i * cube_bytes + (qb * S + s) * 1024);
    }
  float lse2[2], dl[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float2 ld = ld_c[((size_t)bh * g.nbq + i) * 64 + 32 * qb + l32];
    lse2[qb] = ld.x;  // LSE in base 2
    dl[qb] = ld.y;
  }
  stage(1, st1);
  // vmcnt(2S): every vector load but the last tile request (2S buffer loads) has completed
  constexpr int kWaitTile = 0x0f70 | ((2 * S) & 0xf) | (((2 * S) >> 4) << 14);

  f32x16 acc[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db) { zero16(acc[db][0]); zero16(acc[db][1]); }
  const int trb = tr_lane_base(lane);

  // S^T = K Q^T and dP^T = V dO^T of the tile staged at src
  auto scores = [&](const lds_char* src, f32x16 (&st)[2], f32x16 (&dpt)[2]) {
    zero16(st[0]); zero16(st[1]); zero16(dpt[0]); zero16(dpt[1]);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const bf16x8 ka = lds_row_frag(src, lane, s);
      st[0] = mfma32(ka, qreg[0][s], st[0]);
      st[1] = mfma32(ka, qreg[1][s], st[1]);
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const bf16x8 va = lds_row_frag(src + lds_half, lane, s);
      dpt[0] = mfma32(va, dreg[0][s], dpt[0]);
      dpt[1] = mfma32(va, dreg[1][s], dpt[1]);
    }
  };
  auto make_ds = [&](const f32x16 (&st)[2], const f32x16 (&dpt)[2], bf16x8 (&dsb)[2][2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * s2 + e;
          float p = fast_exp2(fmaf(st[qb][r], c_log2, -lse2[qb]));
          // ragged grids: the plain kernel's clamp (a key slot without a token has a zero K row;
          // P <= 1 keeps its dS finite), so both loops give the same bits
          if constexpr (RAGGED) p = fminf(p, 1.0f);
          dsb[s2][qb][e] = (__bf16)(p * (dpt[qb][r] - dl[qb]));
        }
  };
  auto k_trans = [&](const lds_char* src, bf16x8 (&kt)[DB * 2]) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) kt[db * 2 + s2] = lds_trans_frag<D>(src, trb, db, s2);
  };
  auto add_dq = [&](const bf16x8 (&kt)[DB * 2], const bf16x8 (&dsb)[2][2]) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        acc[db][0] = mfma32(kt[db * 2 + s2], dsb[s2][0], acc[db][0]);
        acc[db][1] = mfma32(kt[db * 2 + s2], dsb[s2][1], acc[db][1]);
      }
  };

  f32x16 stc[2], dpc[2];  // scores of the tile whose dQ^T term comes next
  __builtin_amdgcn_s_waitcnt(kWaitTile);  // tile 0 and the Q, dO rows have landed
  scores(st0, stc, dpc);
  // Iteration t: K^T of tile t (staged at cur) is read, cur is refilled with tile t+2 (the last
  // tile re-stages itself so every wait stays the same), the scores of tile t+1 (staged at nxt)
  // are issued, P and dS of tile t are formed from the scores of the previous iteration, and
  // dQ^T takes tile t's term.
  auto body = [&](int t, lds_char* cur, lds_char* nxt) {
    bf16x8 kt[DB * 2];
    k_trans(cur, kt);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): tile t's rows have all been read
    stage(t + 2 < ntiles ? t + 2 : ntiles - 1, cur);
    __builtin_amdgcn_s_waitcnt(kWaitTile);  // tile t+1 has landed
    f32x16 stn[2], dpn[2];
    bf16x8 dsb[2][2];
    scores(nxt, stn, dpn);
    make_ds(stc, dpc, dsb);
    add_dq(kt, dsb);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) { stc[qb] = stn[qb]; dpc[qb] = dpn[qb]; }
  };
  int t = 0;
  for (; t + 2 < ntiles; t += 2) {
    body(t, st0, st1);
    body(t + 1, st1, st0);
  }
  body(t, st0, st1);  // t = ntiles - 2
  {
    bf16x8 kt[DB * 2], dsb[2][2];  // the last tile, staged at st1
    k_trans(st1, kt);
    make_ds(stc, dpc, dsb);
    add_dq(kt, dsb);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the last re-staging has landed

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int tq = cube_token(g, i, 32 * qb + l32);
    if (RAGGED && tq < 0) continue;  // slot outside a ragged grid
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

}  // namespace bsa
