// bsa_bwd_dq.h -- the one-wave dQ kernel of the block-sparse attention backward on bf16 MFMA
// (gfx950), c == 64, as a template shared by the translation units that instantiate it.
//
// The backward ships alongside the forward for training ("LongCat-Video 高效長視頻生成探索世界
// 模型的第壹步", meituan.com talk, section 2.2); the selection is a discrete choice and is held
// constant.  With P = exp(scale*Q_i K_j^T - LSE_i) over every selected pair (i, j):
//   dS = P o (dO_i V_j^T - Delta_i),  dQ_i += scale*dS K_j.
//
// MI355X design: one wave per query cube owns its dQ^T in registers, so no fp32 atomics are
// needed.  Every operand comes from the ROW gather layout; the streamed operand's rows are staged
// straight into LDS with buffer_load ... lds and its transposed uses are read back with
// ds_read_b64_tr_b16, so each tile crosses the fabric once.  The next tile is requested as soon
// as the current one is staged; per-lane byte offsets stay constant and the wave-uniform tile
// offset rides in an SGPR (buffer loads).
//
// Head dim 128 (k_bwd_dq.hip) and head dim 64 (k_bwd_dq64.hip) are instantiated in separate
// files because they want different register allocations from the compiler (see those files).
#pragma once

#include "bsa_bwd_tiles.h"

namespace bsa {

// ---------------------------------------------------------------------------------------------
// dQ (query-stationary): grid = B*Hh*cpx*8, one wave per query cube.  Per 32-key half cube:
// K and V rows are staged straight into LDS (double buffered, the next tile in flight while this
// one computes), S^T = K Q^T and dP^T = V dO^T take the K/V rows as A operands and Q, dO rows
// (held in registers) as B operands; dS^T stays in the accumulator registers and, as bf16, is
// the B operand of dQ^T += K^T dS^T, whose A operand is read transposed from the staged K rows.
// ---------------------------------------------------------------------------------------------
template <int D, bool RAGGED>
__global__ __launch_bounds__(64) void bwd_dq_mfma_kernel(
    Geom g, const bf16_t* __restrict__ q_row, const bf16_t* __restrict__ do_row,
    const bf16_t* __restrict__ k_row, const bf16_t* __restrict__ v_row,
    const float2* __restrict__ ld_c, const int32_t* __restrict__ idx, int k_sel, float scale,
    float c_log2, int cpx, float* __restrict__ dq) {
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
  const int ntiles = 2 * k_sel;
  lds_char* st0 = (lds_char*)stage0;
  lds_char* st1 = (lds_char*)stage1;
  {
    const int off0 = irow[0] * cube_bytes;
    stage_half<D>(rk, off0, st0, lane);
    stage_half<D>(rv, off0, st0 + lds_half, lane);
  }

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

  f32x16 acc[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db) { zero16(acc[db][0]); zero16(acc[db][1]); }
  const int trb = tr_lane_base(lane);

  auto tile = [&](int t, lds_char* cur, lds_char* nxt) {
    // next tile's K and V rows -> the other stage (its previous reads were consumed last tile);
    // the last tile re-stages itself so every tile waits the same way
    const int tn = t + 1 < ntiles ? t + 1 : t;
    const int noff = irow[tn >> 1] * cube_bytes + (tn & 1) * half_bytes;
    stage_half<D>(rk, noff, nxt, lane);
    stage_half<D>(rv, noff, nxt + lds_half, lane);
    __builtin_amdgcn_s_waitcnt(0x0f70 | ((2 * S) & 0xf) | (((2 * S) >> 4) << 14));  // vmcnt(2S)
    f32x16 st[2], dpt[2];
    zero16(st[0]); zero16(st[1]); zero16(dpt[0]); zero16(dpt[1]);
    bf16x8 ka[S];
#pragma unroll
    for (int s = 0; s < S; ++s) ka[s] = lds_row_frag(cur, lane, s);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      st[0] = mfma32(ka[s], qreg[0][s], st[0]);
      st[1] = mfma32(ka[s], qreg[1][s], st[1]);
    }
#pragma unroll
    for (int s = 0; s < S; ++s) ka[s] = lds_row_frag(cur + lds_half, lane, s);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      dpt[0] = mfma32(ka[s], dreg[0][s], dpt[0]);
      dpt[1] = mfma32(ka[s], dreg[1][s], dpt[1]);
    }
    // Ragged grids need no key mask here: a key slot without a token has a zero K row in the
    // gather, so its dS adds nothing to dQ = dS K as long as it is finite.  Its P = exp(-LSE)
    // could overflow for a very negative LSE, so the ragged instantiation clamps P at 1 (a valid
    // P is <= 1; the clamp only trims rounding).  A query slot without a token has LSE = +inf,
    // so its P row is 0.
    bf16x8 kt[DB * 2];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) kt[db * 2 + s2] = lds_trans_frag<D>(cur, trb, db, s2);
    bf16x8 dsb[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * s2 + e;
          float p = fast_exp2(fmaf(st[qb][r], c_log2, -lse2[qb]));
          if constexpr (RAGGED) p = fminf(p, 1.0f);
          dsb[s2][qb][e] = (__bf16)(p * (dpt[qb][r] - dl[qb]));
        }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        acc[db][0] = mfma32(kt[db * 2 + s2], dsb[s2][0], acc[db][0]);
        acc[db][1] = mfma32(kt[db * 2 + s2], dsb[s2][1], acc[db][1]);
      }
  };
  for (int t = 0; t < ntiles; t += 2) {
    tile(t, st0, st1);
    if (t + 1 < ntiles) tile(t + 1, st1, st0);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the last re-staging has landed

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int tq = cube_token(g, i, 32 * qb + l32);
    if (tq < 0) continue;  // slot outside a ragged grid
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
