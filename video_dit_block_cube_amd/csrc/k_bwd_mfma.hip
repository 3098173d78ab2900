// k_bwd_mfma.hip -- block-sparse attention backward, dK and dV, on bf16 MFMA (gfx950), c == 64.
//
// The backward ships alongside the forward for training ("LongCat-Video 高效長視頻生成探索世界
// 模型的第壹步", meituan.com talk, section 2.2); the selection is a discrete choice and is held
// constant.  With P = exp(scale*Q_i K_j^T - LSE_i) over every selected pair (i, j):
//   dV_j += P^T dO_i,  dS = P o (dO_i V_j^T - Delta_i),  dQ_i += scale*dS K_j,
//   dK_j += scale*dS^T Q_i.
//
// MI355X design: the backward is two passes (dK/dV here, dQ in k_bwd_dq.hip), each owning its
// output in registers so no fp32 atomics are needed.  Every operand comes from the ROW gather
// layout; the streamed operand's rows are staged straight into LDS with buffer_load ... lds and
// their transposed uses are read back with ds_read_b64_tr_b16, so each tile crosses the fabric
// once.  Per-lane byte offsets stay constant and the wave-uniform tile offset rides in an SGPR
// (buffer loads).
#include <type_traits>

#include "bsa_bwd_tiles.h"

namespace bsa {

// ---------------------------------------------------------------------------------------------
// dK, dV (key-stationary over the CSR transpose): grid = B*Hh*(ccx+ncx)*8 work items, one per key
// cube (condition cubes, read from the cache and written to the cache gradients, and noise
// cubes), longest lists first within each (b, h).  For every query cube that selected the key
// cube, the Q and dO rows of each 32-query half are staged straight into LDS (double buffered);
// S = Q K^T and dP = dO V^T take them as A operands against the key cube's K and V rows held in
// registers, and P, dS are the B operands of dV^T += dO^T P and dK^T += Q^T dS, whose A operands
// are read transposed from the same staged rows.  Two kernels:
//   bwd_dkdv_mfma_kernel (D = 64): one wave per key cube, 16-query sub-steps (254 VGPRs, every
//     MFMA writing VGPRs by the build flags, so no AGPR copies; two waves per SIMD);
//   bwd_dkdv_pair_kernel (D = 128): two waves per key cube split by output (below).
// ---------------------------------------------------------------------------------------------
// XCD x takes the x-th run of ccx condition cube ids and the x-th run of ncx noise cube ids of
// every (b, h), condition cubes (whose lists hold every query cube) first, so the XCDs carry
// equal work.  Slot k8 of XCD x -> (bh, key cube j: condition cubes first, then noise cubes);
// false for a slot past the last cube.
__device__ __forceinline__ bool dkdv_identity_item(const Geom& g, int x, int k8, int ccx, int ncx,
                                                   int& bh, int& j) {
  const int per = ccx + ncx;
  bh = k8 / per;
  const int m = k8 % per;
  if (m < ccx) {
    j = x * ccx + m;
    return j < g.nbc;
  }
  j = x * ncx + (m - ccx);
  if (j >= g.nbq) return false;
  j += g.nbc;
  return true;
}

constexpr int kOrderBuckets = 256;

// Longest-first dispatch order of the dK/dV items inside each (b, h): a key cube's item takes
// time in proportion to its list length (the query cubes that selected it), which varies about
// +-16% around k_sel on these workloads and up to 1.5x.  The (b, h) groups keep their sequence,
// so the items running together on an XCD still share one head's Q/dO rows in the Infinity
// Cache (sorting across heads made dK/dV 9% slower).  Workgroup (x, bh) sorts XCD x's slots of
// bh into buckets of list length (width 2^shift), longest first, and writes them to
// order[8*(bh*per + pos) + x]; its slots past the item count get -1.  Items of one bucket land
// in atomic (run-dependent) order, which changes nothing in any item's arithmetic.
__global__ __launch_bounds__(256) void dkdv_order_kernel(Geom g,
                                                         const int32_t* __restrict__ csr_off,
                                                         int ccx, int ncx, int shift,
                                                         int32_t* __restrict__ order) {
  __shared__ int cnt[kOrderBuckets];
  __shared__ int total;
  const int x = blockIdx.x, bh = blockIdx.y;
  const int per = ccx + ncx;
  for (int i = threadIdx.x; i < kOrderBuckets; i += 256) cnt[i] = 0;
  __syncthreads();
  const int32_t* o = csr_off + (size_t)bh * (g.nbk + 1);
  auto bucket = [&](int j) {
    const int b = (o[j + 1] - o[j]) >> shift;
    return kOrderBuckets - 1 - (b < kOrderBuckets - 1 ? b : kOrderBuckets - 1);
  };
  for (int m = threadIdx.x; m < per; m += 256) {
    int bh2, j;
    if (dkdv_identity_item(g, x, bh * per + m, ccx, ncx, bh2, j)) atomicAdd(&cnt[bucket(j)], 1);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int sum = 0;
    for (int i = 0; i < kOrderBuckets; ++i) {
      const int c = cnt[i];
      cnt[i] = sum;
      sum += c;
    }
    total = sum;
  }
  __syncthreads();
  const size_t base = (size_t)bh * per;
  for (int m = threadIdx.x; m < per; m += 256) {
    int bh2, j;
    if (dkdv_identity_item(g, x, bh * per + m, ccx, ncx, bh2, j)) {
      const int pos = atomicAdd(&cnt[bucket(j)], 1);
      order[8 * (base + pos) + x] = bh * g.nbk + j;
    }
  }
  for (int k = total + threadIdx.x; k < per; k += 256) order[8 * (base + k) + x] = -1;
}

template <int D>
__global__ __launch_bounds__(64) void bwd_dkdv_mfma_kernel(
    Geom g, const bf16_t* __restrict__ k_row, const bf16_t* __restrict__ v_row,
    const bf16_t* __restrict__ q_row, const bf16_t* __restrict__ do_row,
    const float2* __restrict__ ld_c, const int32_t* __restrict__ csr_off,
    const int32_t* __restrict__ csr_list, const int32_t* __restrict__ order, float scale,
    float c_log2, int ccx, int ncx, float* __restrict__ dk, float* __restrict__ dv,
    float* __restrict__ dk_cache, float* __restrict__ dv_cache) {
  static_assert(D == 64, "D = 128 runs bwd_dkdv_pair_kernel");
  constexpr int S = D / 16;
  constexpr int DB = D / 32;
  constexpr int cube_bytes = 64 * D * 2;
  constexpr int half_bytes = 32 * D * 2;              // a 32-row half block in memory
  constexpr int lds_half = staged_half_bytes<D>();    // the same block staged in LDS
  constexpr int stage_bytes = 2 * lds_half + 256;     // Q rows | dO rows | 32 (LSE2, Delta) pairs
  __shared__ __attribute__((aligned(16))) char stage0[stage_bytes];
  __shared__ __attribute__((aligned(16))) char stage1[stage_bytes];

  // Work item (b*Hh + h, key cube j) of workgroup L, which runs on XCD L % 8.
  int bh, j;
  if (order) {
    // longest lists first inside each XCD's share (dkdv_order_kernel); -1: idle slot
    const int it = order[blockIdx.x];
    if (it < 0) return;
    bh = it / g.nbk;
    j = it % g.nbk;
  } else if (!dkdv_identity_item(g, blockIdx.x & 7, blockIdx.x >> 3, ccx, ncx, bh, j)) {
    return;
  }
  const int b = bh / g.Hh, h = bh % g.Hh;
  const int lane = threadIdx.x;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int32_t* offs = csr_off + (size_t)bh * (g.nbk + 1);
  const int beg = offs[j], end = offs[j + 1];
  const int nsteps = 2 * (end - beg);
  const size_t bh_bytes = (size_t)g.nbq * cube_bytes;
  const size_t bh_elems = (size_t)g.nbq * 64 * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q_row + bh * bh_elems, bh_bytes);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(do_row + bh * bh_elems, bh_bytes);
  const __amdgpu_buffer_rsrc_t rl =
      make_rsrc(ld_c + (size_t)bh * g.nbq * 64, (size_t)g.nbq * 64 * sizeof(float2));
  lds_char* st0 = (lds_char*)stage0;
  lds_char* st1 = (lds_char*)stage1;
  // one 32-query half of query cube i: Q rows, dO rows and the (base-2 LSE, Delta) pairs -> a
  // stage
  auto stage_step = [&](int i, int qb, lds_char* dst) {
    stage_half<D>(rq, i * cube_bytes + qb * half_bytes, dst, lane);
    stage_half<D>(rd, i * cube_bytes + qb * half_bytes, dst + lds_half, lane);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rl, (__attribute__((address_space(3))) void*)(dst + 2 * lds_half), 4, lane * 4,
        (i * 64 + 32 * qb) * (int)sizeof(float2), 0, 0);
  };
  if (nsteps > 0) stage_step(csr_list[beg], 0, st0);

  // K and V rows of this key cube as B operands of the 16x16x32 products; the K/V gathers hold
  // every key cube (condition cubes from the cache first).
  // kreg[nb*S4 + s] = (lane%16 = key of 16-block nb, d = 32s + 8*(lane/16) + 0..7).
  constexpr int S4 = D / 32;
  const size_t kv_elems = (size_t)g.nbk * 64 * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k_row + bh * kv_elems, (size_t)g.nbk * cube_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v_row + bh * kv_elems, (size_t)g.nbk * cube_bytes);
  const int r16 = row16_lane(lane);
  const int r16m = row16_lane_mem(lane);
  bf16x8 kreg[4 * S4], vreg[4 * S4];
#pragma unroll
  for (int f = 0; f < 4 * S4; ++f) {
    const int nb = f / S4, s = f % S4;
    const int soff =
        j * cube_bytes + (nb >> 1) * half_bytes + row16_const_mem<D>(s, 16 * (nb & 1));
    kreg[f] = bld16(rk, r16m, soff);
    vreg[f] = bld16(rv, r16m, soff);
  }

  f32x16 acck[DB][2], accv[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) { zero16(acck[db][kb]); zero16(accv[db][kb]); }
  const int trb = tr16_lane(lane);

  auto step = [&](int t, lds_char* cur, lds_char* nxt) {
    const int tn = t + 1 < nsteps ? t + 1 : t;
    stage_step(csr_list[beg + (tn >> 1)], tn & 1, nxt);
    __builtin_amdgcn_s_waitcnt(0x0f70 | ((2 * S + 1) & 0xf) | (((2 * S + 1) >> 4) << 14));
    const __attribute__((address_space(3))) f32x4* ldp =
        (const __attribute__((address_space(3))) f32x4*)(cur + 2 * lds_half);
    // two 16-query sub-steps per staged half
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      // (base-2 LSE, Delta) of this lane's queries 16*sub + 4*(lane/16) + 0..3
      const f32x4 p01 = ldp[8 * sub + 2 * (lane >> 4)];
      const f32x4 p23 = ldp[8 * sub + 2 * (lane >> 4) + 1];
      const float lv[4] = {p01[0], p01[2], p23[0], p23[2]};
      // dP's accumulators start at -Delta of the lane's queries, so the products leave the
      // factor dP - Delta of dS with no subtraction per element
      const f32x4v ndl = f32x4v{-p01[1], -p01[3], -p23[1], -p23[3]};
      f32x4v sc[4], dp[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        sc[nb] = f32x4v{0.f, 0.f, 0.f, 0.f};
        dp[nb] = ndl;
      }
#pragma unroll
      for (int s = 0; s < S4; ++s) {
        const bf16x8 a = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            cur + r16 + row16_const<D>(s, 16 * sub));
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          sc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, kreg[nb * S4 + s], sc[nb], 0, 0, 0);
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[nb][i] = fast_exp2(fmaf(sc[nb][i], c_log2, -lv[i]));
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) pb[kb] = acc16_to_b32(sc[2 * kb], sc[2 * kb + 1]);
#pragma unroll
      for (int s = 0; s < S4; ++s) {
        const bf16x8 a = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            cur + lds_half + r16 + row16_const<D>(s, 16 * sub));
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          dp[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, vreg[nb * S4 + s], dp[nb], 0, 0, 0);
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) dp[nb][i] = sc[nb][i] * dp[nb][i];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) dsb[kb] = acc16_to_b32(dp[2 * kb], dp[2 * kb + 1]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 dt = lds_tr16<D>(cur + lds_half, trb, db, sub);
        const bf16x8 qt = lds_tr16<D>(cur, trb, db, sub);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          accv[db][kb] = mfma32(dt, pb[kb], accv[db][kb]);
          acck[db][kb] = mfma32(qt, dsb[kb], acck[db][kb]);
        }
      }
    }
  };
  // nsteps is even (two 32-query halves per listed query cube); fixed stage roles per half let
  // the compiler see that this step's LDS reads never alias the next step's LDS-bound loads,
  // so it does not drain those loads before the transposed reads
  for (int t = 0; t < nsteps; t += 2) {
    step(t, st0, st1);
    step(t + 1, st1, st0);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the last re-staging has landed

  const bool cond = j < g.nbc;  // condition key cube: its gradients go to the cache tensors
  float* dk_out = cond ? dk_cache : dk;
  float* dv_out = cond ? dv_cache : dv;
  const int jc = cond ? j : j - g.nbc;  // cube index inside its segment
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int tk = cube_token(g, jc, 32 * kb + l32);
    if (tk < 0) continue;  // slot outside a ragged grid
    const size_t off = bnhd_offset(g, cond ? g.Nc : g.Nq, b, tk, h);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * db + 8 * r4 + 4 * hh;
        const f32x16& ak = acck[db][kb];
        const f32x16& av = accv[db][kb];
        *reinterpret_cast<float4*>(dk_out + off + d) =
            make_float4(ak[4 * r4] * scale, ak[4 * r4 + 1] * scale, ak[4 * r4 + 2] * scale,
                        ak[4 * r4 + 3] * scale);
        *reinterpret_cast<float4*>(dv_out + off + d) =
            make_float4(av[4 * r4], av[4 * r4 + 1], av[4 * r4 + 2], av[4 * r4 + 3]);
      }
  }
}


// ---------------------------------------------------------------------------------------------
// dK, dV at D = 128 with two waves per key cube.  The accumulators of one 64-key cube (dV^T and
// dK^T, 128 registers each) hold a single wave at one wave per SIMD, where its softmax VALU,
// LDS reads and MFMAs serialise.  Split by output instead: wave 0 holds K and accumulates dV,
// wave 1 holds V and accumulates dK, each within 256 registers, so two waves share every SIMD
// and overlap each other's VALU and MFMA work.  Per 16-query sub-step (16x16x32 products, as
// in the D = 64 path of the one-wave kernel):
//   wave 0: S = Q K^T, P = exp2(S*scale*log2e - LSE2) -> bf16 P to LDS; barrier; dV^T += dO^T P
//   wave 1: dP = dO V^T; barrier; dS = P o (dP - Delta) with the bf16 P; dK^T += Q^T dS
// Wave 0 stages the Q rows and wave 1 the dO rows of every 32-query half (each with its own
// copy of the (LSE2, Delta) pairs), so each reads its own rows before the barrier; the next
// half is requested right after the first barrier of a step, when both waves are past the
// previous step.  The roles run separate copies of the loop with the same barrier sequence.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void pair_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done (no vmcnt
                                       // wait: the next half's LDS-bound loads stay in flight)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2))) void
bwd_dkdv_pair_kernel(Geom g, const bf16_t* __restrict__ k_row, const bf16_t* __restrict__ v_row,
                     const bf16_t* __restrict__ q_row, const bf16_t* __restrict__ do_row,
                     const float2* __restrict__ ld_c, const int32_t* __restrict__ csr_off,
                     const int32_t* __restrict__ csr_list, const int32_t* __restrict__ order,
                     float scale, float c_log2, int ccx, int ncx, int walk_ticks,
                     float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dk_cache,
                     float* __restrict__ dv_cache) {
  constexpr int S4 = D / 32;
  constexpr int DB = D / 32;
  constexpr int cube_bytes = 64 * D * 2;
  constexpr int half_bytes = 32 * D * 2;              // a 32-row half block in memory
  constexpr int lds_half = staged_half_bytes<D>();    // the same block staged in LDS
  constexpr int stage_bytes = 2 * lds_half + 512;     // Q | dO | pairs (wave 0) | pairs (wave 1)
  __shared__ __attribute__((aligned(16))) char stage0[stage_bytes];
  __shared__ __attribute__((aligned(16))) char stage1[stage_bytes];
  // bf16 P of a sub-step: 8 words per lane as two 16-byte blocks, [block][lane] (lane stride 16
  // bytes: conflict-free 16-byte accesses)
  __shared__ __attribute__((aligned(16))) char xch[2][16 * 64 * 2];

  int bh, j;
  if (order) {
    const int it = order[blockIdx.x];
    if (it < 0) return;
    bh = it / g.nbk;
    j = it % g.nbk;
  } else if (!dkdv_identity_item(g, blockIdx.x & 7, blockIdx.x >> 3, ccx, ncx, bh, j)) {
    return;
  }
  const int b = bh / g.Hh, h = bh % g.Hh;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // 0: K, dV   1: V, dK
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hh = lane >> 5;

  const int32_t* offs = csr_off + (size_t)bh * (g.nbk + 1);
  const int beg = offs[j], end = offs[j + 1];
  const int nsteps = 2 * (end - beg);
  // first entry of the walk: 0, or (walk phase) the first query cube at or past the clock's
  // phase within the period, read once for both waves, the walk wrapping around the list
  const int nlist = end - beg;
  int s0 = 0;
  if (walk_ticks > 0) {
    __shared__ int walk_phase;
    if (threadIdx.x == 0)
      walk_phase = (int)((wall_clock64() % (uint64_t)walk_ticks) * (uint64_t)g.nbq /
                         (uint64_t)walk_ticks);
    __syncthreads();
    const int phase = walk_phase;
    for (int e0 = 0; e0 < nlist; e0 += 64) {
      const int e = e0 + lane;
      s0 += __popcll(__ballot(e < nlist && csr_list[beg + e] < phase));
    }
    if (s0 >= nlist) s0 = 0;
  }
  auto entry = [&](int e) { return csr_list[beg + (e + s0 < nlist ? e + s0 : e + s0 - nlist)]; };
  const size_t bh_bytes = (size_t)g.nbq * cube_bytes;
  const size_t bh_elems = (size_t)g.nbq * 64 * D;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc((wave ? do_row : q_row) + bh * bh_elems, bh_bytes);
  const __amdgpu_buffer_rsrc_t rl =
      make_rsrc(ld_c + (size_t)bh * g.nbq * 64, (size_t)g.nbq * 64 * sizeof(float2));
  lds_char* st0 = (lds_char*)stage0;
  lds_char* st1 = (lds_char*)stage1;
  const int own_rows = wave * lds_half;             // this wave's rows inside a stage
  const int own_pairs = 2 * lds_half + 256 * wave;  // this wave's (LSE2, Delta) pairs
  auto stage_step = [&](int i, int qb, lds_char* dst) {
    stage_half<D>(rs, i * cube_bytes + qb * half_bytes, dst + own_rows, lane);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rl, (__attribute__((address_space(3))) void*)(dst + own_pairs), 4, lane * 4,
        (i * 64 + 32 * qb) * (int)sizeof(float2), 0, 0);
  };
  if (nsteps > 0) stage_step(entry(0), 0, st0);

  // K (wave 0) or V (wave 1) rows of the key cube: B operands of the 16x16x32 products,
  // kv[nb*S4 + s] = (lane%16 = key of 16-block nb, d = 32s + 8*(lane/16) + 0..7)
  const size_t kv_elems = (size_t)g.nbk * 64 * D;
  const __amdgpu_buffer_rsrc_t rkv =
      make_rsrc((wave ? v_row : k_row) + bh * kv_elems, (size_t)g.nbk * cube_bytes);
  const int r16 = row16_lane(lane);
  const int r16m = row16_lane_mem(lane);
  bf16x8 kv[4 * S4];
#pragma unroll
  for (int f = 0; f < 4 * S4; ++f) {
    const int nb = f / S4, s = f % S4;
    kv[f] = bld16(rkv, r16m,
                  j * cube_bytes + (nb >> 1) * half_bytes + row16_const_mem<D>(s, 16 * (nb & 1)));
  }
  f32x16 acc[DB][2];  // dV^T (wave 0) or dK^T (wave 1)
#pragma unroll
  for (int db = 0; db < DB; ++db) { zero16(acc[db][0]); zero16(acc[db][1]); }
  const int trb = tr16_lane(lane);

  auto step = [&](int t, lds_char* cur, lds_char* nxt, auto role_c) {
    constexpr int R = decltype(role_c)::value;
    const int tn = t + 1 < nsteps ? t + 1 : t;  // the last step re-stages itself
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's rows of the half have landed
    const __attribute__((address_space(3))) float2* ldp =
        (const __attribute__((address_space(3))) float2*)(cur + own_pairs);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int q0 = 16 * sub + 4 * (lane >> 4);  // this lane's first query of the sub-step
      // Score accumulators start at 0 for S (wave 0) and at -Delta of the lane's four queries
      // for dP (wave 1), so the products leave dP - Delta, the factor dS needs, with no
      // subtraction per element (the four values serve all four key blocks).
      f32x4v sc[4];
      f32x4v c0 = f32x4v{0.f, 0.f, 0.f, 0.f};
      if constexpr (R == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) c0[i] = -ldp[q0 + i].y;
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) sc[nb] = c0;
      // Operand reads are issued ahead of their products, so the LDS latency overlaps other
      // work: the wave's own row fragments of the sub-step first, and the transposed fragments
      // of the other wave's rows (dO^T for wave 0, Q^T for wave 1) as soon as they are visible:
      // at the start of sub-step 1, and right after the barrier in sub-step 0 (the barrier that
      // follows both waves' waits for this step's rows).
      bf16x8 ar[S4];
#pragma unroll
      for (int s = 0; s < S4; ++s)
        ar[s] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            cur + own_rows + r16 + row16_const<D>(s, 16 * sub));
      bf16x8 tf[DB];
      const lds_char* tsrc = R == 0 ? cur + lds_half : cur;
      if (sub == 1) {
#pragma unroll
        for (int db = 0; db < DB; ++db) tf[db] = lds_tr16<D>(tsrc, trb, db, sub);
      }
      __builtin_amdgcn_sched_barrier(0);
      // S = Q K^T (wave 0) or dP = dO V^T (wave 1), from the wave's own staged rows
#pragma unroll
      for (int s = 0; s < S4; ++s)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          sc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar[s], kv[nb * S4 + s], sc[nb], 0, 0, 0);
      // this lane's 8 words of the exchanged P: words 0-3 at lane*16, words 4-7 at 1024 + lane*16
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      __attribute__((address_space(3))) u32x4* x =
          (__attribute__((address_space(3))) u32x4*)(xch[sub]) + lane;
      if constexpr (R == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lv = ldp[q0 + i].x;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) sc[nb][i] = fast_exp2(fmaf(sc[nb][i], c_log2, -lv));
        }
        x[0] = u32x4{pack_bf16x2(sc[0][0], sc[0][1]), pack_bf16x2(sc[0][2], sc[0][3]),
                     pack_bf16x2(sc[1][0], sc[1][1]), pack_bf16x2(sc[1][2], sc[1][3])};
        x[64] = u32x4{pack_bf16x2(sc[2][0], sc[2][1]), pack_bf16x2(sc[2][2], sc[2][3]),
                      pack_bf16x2(sc[3][0], sc[3][1]), pack_bf16x2(sc[3][2], sc[3][3])};
        bf16x8 pb[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) pb[kb] = acc16_to_b32(sc[2 * kb], sc[2 * kb + 1]);
        pair_barrier();  // P is in LDS; both waves have finished the previous step
        if (sub == 0) {
#pragma unroll
          for (int db = 0; db < DB; ++db) tf[db] = lds_tr16<D>(tsrc, trb, db, sub);
          __builtin_amdgcn_sched_barrier(0);
          stage_step(entry(tn >> 1), tn & 1, nxt);
        }
        // dV^T += dO^T P
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) acc[db][kb] = mfma32(tf[db], pb[kb], acc[db][kb]);
      } else {
        pair_barrier();
        if (sub == 0) {
#pragma unroll
          for (int db = 0; db < DB; ++db) tf[db] = lds_tr16<D>(tsrc, trb, db, sub);
        }
        const u32x4 xa = x[0], xb = x[64];
        __builtin_amdgcn_sched_barrier(0);
        if (sub == 0) stage_step(entry(tn >> 1), tn & 1, nxt);
        // dS = P o (dP - Delta) from wave 0's bf16 P (same lane layout as this accumulator,
        // which already holds dP - Delta)
        const uint32_t xw[8] = {xa[0], xa[1], xa[2], xa[3], xb[0], xb[1], xb[2], xb[3]};
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const uint32_t w0 = xw[2 * nb], w1 = xw[2 * nb + 1];
          const float pv[4] = {__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xffff0000u),
                               __uint_as_float(w1 << 16), __uint_as_float(w1 & 0xffff0000u)};
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[nb][i] = pv[i] * sc[nb][i];
        }
        bf16x8 dsb[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) dsb[kb] = acc16_to_b32(sc[2 * kb], sc[2 * kb + 1]);
        // dK^T += Q^T dS
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) acc[db][kb] = mfma32(tf[db], dsb[kb], acc[db][kb]);
      }
    }
  };
  // nsteps is even; fixed stage roles per pair of steps (see the one-wave kernel)
  if (wave == 0) {
    for (int t = 0; t < nsteps; t += 2) {
      step(t, st0, st1, std::integral_constant<int, 0>{});
      step(t + 1, st1, st0, std::integral_constant<int, 0>{});
    }
  } else {
    for (int t = 0; t < nsteps; t += 2) {
      step(t, st0, st1, std::integral_constant<int, 1>{});
      step(t + 1, st1, st0, std::integral_constant<int, 1>{});
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the last re-staging has landed

  const bool cond = j < g.nbc;  // condition key cube: its gradients go to the cache tensors
  float* out = wave ? (cond ? dk_cache : dk) : (cond ? dv_cache : dv);
  const float mul = wave ? scale : 1.0f;
  const int jc = cond ? j : j - g.nbc;  // cube index inside its segment
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int tk = cube_token(g, jc, 32 * kb + l32);
    if (tk < 0) continue;  // slot outside a ragged grid
    const size_t off = bnhd_offset(g, cond ? g.Nc : g.Nq, b, tk, h);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * db + 8 * r4 + 4 * hh;
        const f32x16& a = acc[db][kb];
        *reinterpret_cast<float4*>(out + off + d) = make_float4(
            a[4 * r4] * mul, a[4 * r4 + 1] * mul, a[4 * r4 + 2] * mul, a[4 * r4 + 3] * mul);
      }
  }
}

// ---------------------------------------------------------------------------------------------
// dK, dV at D = 128 with two waves per key cube split by KEYS (the more accurate alternative,
// BSA_TUNE_DKDV_SPLIT = 1): wave w holds K and V of keys 32w..32w+31 and accumulates both dK^T
// and dV^T of those keys.  Per 16-query sub-step each wave forms S and dP of its keys (16x16x32),
// P and dS = P o (dP - Delta) from the fp32 P (the same dS the dQ pass forms), then dV^T += dO^T P
// and dK^T += Q^T dS (32x32x16).  No hand-off between the waves: both run the same loop and meet
// at one barrier per 32-query step, where the step's staged rows are complete and the other
// stage is free to be refilled (wave 0 stages the Q rows and the pairs, wave 1 the dO rows).
// Each wave reads Q, dO, Q^T and dO^T from LDS, twice the LDS reads of the split by output,
// which keeps this variant a few percent slower.
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2))) void
bwd_dkdv_keys_kernel(Geom g, const bf16_t* __restrict__ k_row, const bf16_t* __restrict__ v_row,
                     const bf16_t* __restrict__ q_row, const bf16_t* __restrict__ do_row,
                     const float2* __restrict__ ld_c, const int32_t* __restrict__ csr_off,
                     const int32_t* __restrict__ csr_list, const int32_t* __restrict__ order,
                     float scale, float c_log2, int ccx, int ncx, int walk_ticks,
                     float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dk_cache,
                     float* __restrict__ dv_cache) {
  constexpr int S4 = D / 32;
  constexpr int DB = D / 32;
  constexpr int cube_bytes = 64 * D * 2;
  constexpr int half_bytes = 32 * D * 2;              // a 32-row half block in memory
  constexpr int lds_half = staged_half_bytes<D>();    // the same block staged in LDS
  constexpr int stage_bytes = 2 * lds_half + 256;     // Q rows | dO rows | 32 (LSE2, Delta) pairs
  __shared__ __attribute__((aligned(16))) char stage0[stage_bytes];
  __shared__ __attribute__((aligned(16))) char stage1[stage_bytes];

  int bh, j;
  if (order) {
    const int it = order[blockIdx.x];
    if (it < 0) return;
    bh = it / g.nbk;
    j = it % g.nbk;
  } else if (!dkdv_identity_item(g, blockIdx.x & 7, blockIdx.x >> 3, ccx, ncx, bh, j)) {
    return;
  }
  const int b = bh / g.Hh, h = bh % g.Hh;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // keys 32*wave .. +31
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hh = lane >> 5;

  const int32_t* offs = csr_off + (size_t)bh * (g.nbk + 1);
  const int beg = offs[j], end = offs[j + 1];
  const int nsteps = 2 * (end - beg);
  // first entry of the walk, as in the split by output
  const int nlist = end - beg;
  int s0 = 0;
  if (walk_ticks > 0) {
    __shared__ int walk_phase;
    if (threadIdx.x == 0)
      walk_phase = (int)((wall_clock64() % (uint64_t)walk_ticks) * (uint64_t)g.nbq /
                         (uint64_t)walk_ticks);
    __syncthreads();
    const int phase = walk_phase;
    for (int e0 = 0; e0 < nlist; e0 += 64) {
      const int e = e0 + lane;
      s0 += __popcll(__ballot(e < nlist && csr_list[beg + e] < phase));
    }
    if (s0 >= nlist) s0 = 0;
  }
  auto entry = [&](int e) { return csr_list[beg + (e + s0 < nlist ? e + s0 : e + s0 - nlist)]; };
  const size_t bh_bytes = (size_t)g.nbq * cube_bytes;
  const size_t bh_elems = (size_t)g.nbq * 64 * D;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc((wave ? do_row : q_row) + bh * bh_elems, bh_bytes);
  const __amdgpu_buffer_rsrc_t rl =
      make_rsrc(ld_c + (size_t)bh * g.nbq * 64, (size_t)g.nbq * 64 * sizeof(float2));
  lds_char* st0 = (lds_char*)stage0;
  lds_char* st1 = (lds_char*)stage1;
  auto stage_step = [&](int i, int qb, lds_char* dst) {
    stage_half<D>(rs, i * cube_bytes + qb * half_bytes, dst + wave * lds_half, lane);
    if (wave == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rl, (__attribute__((address_space(3))) void*)(dst + 2 * lds_half), 4, lane * 4,
          (i * 64 + 32 * qb) * (int)sizeof(float2), 0, 0);
  };
  if (nsteps > 0) stage_step(entry(0), 0, st0);

  // K and V rows of this wave's 32 keys as B operands of the 16x16x32 products,
  // f = nb*S4 + s: lane%16 = key 32*wave + 16*nb + lane%16, d = 32s + 8*(lane/16) + 0..7
  const size_t kv_elems = (size_t)g.nbk * 64 * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k_row + bh * kv_elems, (size_t)g.nbk * cube_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v_row + bh * kv_elems, (size_t)g.nbk * cube_bytes);
  const int r16 = row16_lane(lane);
  const int r16m = row16_lane_mem(lane);
  bf16x8 kf[2 * S4], vf[2 * S4];
#pragma unroll
  for (int f = 0; f < 2 * S4; ++f) {
    const int nb = f / S4, s = f % S4;
    const int off = j * cube_bytes + wave * half_bytes + row16_const_mem<D>(s, 16 * nb);
    kf[f] = bld16(rk, r16m, off);
    vf[f] = bld16(rv, r16m, off);
  }
  f32x16 accv[DB], acck[DB];  // dV^T, dK^T of this wave's keys (lane%32 = key)
#pragma unroll
  for (int db = 0; db < DB; ++db) { zero16(accv[db]); zero16(acck[db]); }
  const int trb = tr16_lane(lane);

  auto step = [&](int t, lds_char* cur, lds_char* nxt) {
    const int tn = t + 1 < nsteps ? t + 1 : t;  // the last step re-stages itself
    __builtin_amdgcn_s_waitcnt(0x0f70);          // vmcnt(0): this wave's rows of the step landed
    pair_barrier();  // both waves' rows have landed, and both are done with the other stage
    stage_step(entry(tn >> 1), tn & 1, nxt);
    const __attribute__((address_space(3))) float2* ldp =
        (const __attribute__((address_space(3))) float2*)(cur + 2 * lds_half);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int q0 = 16 * sub + 4 * (lane >> 4);  // this lane's first query of the sub-step
      // dP's accumulators start at -Delta of the lane's four queries (dP - Delta comes out of
      // the products)
      f32x4v ndl;
#pragma unroll
      for (int i = 0; i < 4; ++i) ndl[i] = -ldp[q0 + i].y;
      f32x4v sc[2], dp[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        sc[nb] = f32x4v{0.f, 0.f, 0.f, 0.f};
        dp[nb] = ndl;
      }
#pragma unroll
      for (int s = 0; s < S4; ++s) {
        const bf16x8 a = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            cur + r16 + row16_const<D>(s, 16 * sub));
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          sc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, kf[nb * S4 + s], sc[nb], 0, 0, 0);
      }
#pragma unroll
      for (int s = 0; s < S4; ++s) {
        const bf16x8 a = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            cur + lds_half + r16 + row16_const<D>(s, 16 * sub));
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          dp[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, vf[nb * S4 + s], dp[nb], 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lx = ldp[q0 + i].x;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const float p = fast_exp2(fmaf(sc[nb][i], c_log2, -lx));
          sc[nb][i] = p;
          dp[nb][i] = p * dp[nb][i];
        }
      }
      const bf16x8 pb = acc16_to_b32(sc[0], sc[1]);
      const bf16x8 dsb = acc16_to_b32(dp[0], dp[1]);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        accv[db] = mfma32(lds_tr16<D>(cur + lds_half, trb, db, sub), pb, accv[db]);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        acck[db] = mfma32(lds_tr16<D>(cur, trb, db, sub), dsb, acck[db]);
    }
  };
  for (int t = 0; t < nsteps; t += 2) {
    step(t, st0, st1);
    step(t + 1, st1, st0);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the last re-staging has landed

  const bool cond = j < g.nbc;  // condition key cube: its gradients go to the cache tensors
  const int jc = cond ? j : j - g.nbc;
  const int tk = cube_token(g, jc, 32 * wave + l32);
  if (tk < 0) return;  // slot outside a ragged grid
  const size_t off = bnhd_offset(g, cond ? g.Nc : g.Nq, b, tk, h);
  float* outk = (cond ? dk_cache : dk) + off;
  float* outv = (cond ? dv_cache : dv) + off;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * db + 8 * r4 + 4 * hh;
      const f32x16& a = acck[db];
      const f32x16& c = accv[db];
      *reinterpret_cast<float4*>(outk + d) = make_float4(
          a[4 * r4] * scale, a[4 * r4 + 1] * scale, a[4 * r4 + 2] * scale, a[4 * r4 + 3] * scale);
      *reinterpret_cast<float4*>(outv + d) =
          make_float4(c[4 * r4], c[4 * r4 + 1], c[4 * r4 + 2], c[4 * r4 + 3]);
    }
}

size_t dkdv_order_bytes(const Geom& g) {
  const int ccx = (g.nbc + 7) / 8, ncx = (g.nbq + 7) / 8;
  return (size_t)g.B * g.Hh * (ccx + ncx) * 8 * sizeof(int32_t);
}

hipError_t launch_bwd_dkdv_mfma(const Geom& g, const bf16_t* k_row, const bf16_t* v_row,
                                const bf16_t* q_row, const bf16_t* do_row, const float2* ld_c,
                                const int32_t* csr_off, const int32_t* csr_list, int32_t* order,
                                float scale, int walk_ticks, bool by_keys, float* dk, float* dv,
                                float* dk_cache, float* dv_cache, hipStream_t s) {
  const int ccx = (g.nbc + 7) / 8, ncx = (g.nbq + 7) / 8;
  dim3 grid((unsigned)(g.B * g.Hh * (ccx + ncx) * 8));
  const float c_log2 = scale * kLog2e;
  if (order) {
    int shift = 0;  // list lengths are at most nbq: fit them into the buckets
    while ((g.nbq >> shift) >= kOrderBuckets - 1) ++shift;
    hipLaunchKernelGGL(dkdv_order_kernel, dim3(8, (unsigned)(g.B * g.Hh)), dim3(256), 0, s, g,
                       csr_off, ccx, ncx, shift, order);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (g.D == 64)
    hipLaunchKernelGGL(bwd_dkdv_mfma_kernel<64>, grid, dim3(64), 0, s, g, k_row, v_row, q_row,
                       do_row, ld_c, csr_off, csr_list, order, scale, c_log2, ccx, ncx, dk, dv,
                       dk_cache, dv_cache);
  else if (by_keys)
    hipLaunchKernelGGL(bwd_dkdv_keys_kernel<128>, grid, dim3(128), 0, s, g, k_row, v_row, q_row,
                       do_row, ld_c, csr_off, csr_list, order, scale, c_log2, ccx, ncx, walk_ticks,
                       dk, dv, dk_cache, dv_cache);
  else
    hipLaunchKernelGGL(bwd_dkdv_pair_kernel<128>, grid, dim3(128), 0, s, g, k_row, v_row, q_row,
                       do_row, ld_c, csr_off, csr_list, order, scale, c_log2, ccx, ncx, walk_ticks,
                       dk, dv, dk_cache, dv_cache);
  return hipGetLastError();
}

}  // namespace bsa
