// k_select.hip -- block scores and top-r key cube selection.
//
// Each query cube keeps its own cube, every condition cube, and the r noise cubes most similar
// to it (top-r key blocks: "LongCat-Video视频生成模型发布 迈出世界模型探索第一步", youleyou,
// section "块稀疏注意力（BSA）"; chosen by similarity: Data Science in Your Pocket page, section
// "Sparse attention"; own cube always kept: "LongCat-Video deep dive", ai-news-5min-kr, the
// same-table analogy).  Score S[i,j] = D^-1/2 <q_mean_i, k_mean_j> in fp32; order is score
// descending, then cube id ascending; -0.0 counts as +0.0.
//
// MI355X design: a workgroup of NW waves owns R query rows of one (b, h): R = 16 rows and 16 waves
// when the score rows fit in LDS (every row of the 16-row MFMA operand in use, each key descriptor
// read once per 16 rows), else R <= 8 rows and 4 waves.  Phase 1 computes the R x nbq
// scores on fp32 MFMA (v_mfma_f32_16x16x4f32, 16 key cubes per wave step) and writes them into LDS
// as order-preserving uint32 keys (every score is summed over d in the same order, so equal
// descriptors give bitwise-equal scores and exact ties stay exact).  Phase 2:
// one wave per row runs a 4-pass MSB-first radix select (8-bit digits, LDS histogram, wave suffix
// scan with shuffles) to find the r-th largest key T and how many keys equal to T to take; the
// lower-id rule among equal keys falls out of walking the ids in ascending order.  Phase 3 walks
// key cube ids in 64-lane chunks and compacts the selected ids with ballot + mbcnt, which emits
// every row already ascending, and writes the optional mask row as coalesced bytes.
#include "bsa_launch.h"

namespace bsa {

__device__ __forceinline__ uint32_t order_key(float s) {
  s = s + 0.0f;  // -0.0 -> +0.0
  uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ void lds_fence_wave() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS operations have completed
  __builtin_amdgcn_wave_barrier();
}

template <int R, int NW>
__global__ __launch_bounds__(64 * NW) void select_kernel(Geom g, const float* __restrict__ qm,
                                                     const float* __restrict__ km, int r_eff,
                                                     int k_sel, int32_t* __restrict__ idx,
                                                     uint8_t* __restrict__ mask) {
  extern __shared__ uint32_t smem[];
  const int D = g.D;
  const int nbq = g.nbq;
  float* qs = reinterpret_cast<float*>(smem);          // [R][D]
  uint32_t* keys = smem + R * D;                       // [R][nbq]
  uint32_t* hist = keys + (size_t)R * nbq;             // [NW][256]
  const int bh = blockIdx.y;
  const int row0 = blockIdx.x * R;
  const int tid = threadIdx.x;
  const float* qbase = qm + (size_t)bh * nbq * D;
  const float* kbase = km + (size_t)bh * nbq * D;

  // Phase 1: scores -> order keys in LDS, on v_mfma_f32_16x16x4f32.  A = the R query
  // descriptors (rows R..15 zero), B = 16 key descriptors per step of a wave.  The contraction
  // index is permuted the same way on both sides: at step (c, e) lane group grp = lane/16 holds
  // d = 16c + 4grp + e, so each lane's operands are float4 reads (a key row's four lane groups read
  // 64 contiguous bytes) and every score is summed over d in one fixed order.
  for (int e = tid; e < R * D; e += 64 * NW) {
    const int r = e / D;
    qs[e] = (row0 + r < nbq) ? qbase[(size_t)(row0 + r) * D + (e % D)] : 0.f;
  }
  __syncthreads();
  const float scale = 1.0f / sqrtf((float)D);
  {
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int m = lane & 15, grp = lane >> 4;
    const int nc = D / 16;  // 4 or 8
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 qa[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
      qa[c] = (c < nc && m < R)
                  ? *reinterpret_cast<const f32x4*>(qs + m * D + 16 * c + 4 * grp)
                  : zero4;
    for (int jb = wave * 16; jb < nbq; jb += 16 * NW) {
      const int n = jb + m;  // this lane's key cube (B column)
      f32x4 kb[8];
#pragma unroll
      for (int c = 0; c < 8; ++c)
        kb[c] = (c < nc && n < nbq)
                    ? *reinterpret_cast<const f32x4*>(kbase + (size_t)n * D + 16 * c + 4 * grp)
                    : zero4;
      f32x4 acc = zero4;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if (c < nc) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[c][e], kb[c][e], acc, 0, 0, 0);
        }
      }
      // lane holds rows 4*grp + i of the 16 x 16 block, column m
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * grp + i;
        if (r < R && n < nbq)
          keys[(size_t)r * nbq + n] = (row0 + r == n) ? 0u : order_key(acc[i] * scale);
      }
    }
  }
  __syncthreads();

  // Phase 2 + 3: one wave per row.
  const int wave = tid >> 6;
  const int lane = tid & 63;
  uint32_t* wh = hist + wave * 256;
  for (int r = wave; r < R; r += NW) {
    const int i = row0 + r;
    if (i >= nbq) break;
    const uint32_t* kr = keys + (size_t)r * nbq;
    uint32_t T;
    int take_eq;
    if (r_eff == 0) {
      T = 0xFFFFFFFFu;
      take_eq = 0;
    } else if (r_eff >= nbq - 1) {
      T = 0u;  // every finite candidate key is > 0; the own cube (key 0) is handled separately
      take_eq = 0;
    } else {
      uint32_t prefix = 0, pmask = 0;
      int kk = r_eff;
      for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
#pragma unroll
        for (int q = 0; q < 4; ++q) wh[lane * 4 + q] = 0u;
        lds_fence_wave();
        for (int j = lane; j < nbq; j += 64) {
          const uint32_t u = kr[j];
          if ((u & pmask) == prefix) atomicAdd(&wh[(u >> shift) & 255u], 1u);
        }
        lds_fence_wave();
        const uint32_t h0 = wh[lane * 4 + 0], h1 = wh[lane * 4 + 1];
        const uint32_t h2 = wh[lane * 4 + 2], h3 = wh[lane * 4 + 3];
        const int local = (int)(h0 + h1 + h2 + h3);
        int incl = local;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int t = __shfl_down(incl, off, 64);
          if (lane + off < 64) incl += t;
        }
        const int after = incl - local;  // keys in bins above this lane's four bins
        int digit = -1, above_d = 0;
        int above = after;
        const uint32_t hb[4] = {h0, h1, h2, h3};
#pragma unroll
        for (int bb = 3; bb >= 0; --bb) {
          if (digit < 0 && above < kk && above + (int)hb[bb] >= kk) {
            digit = lane * 4 + bb;
            above_d = above;
          }
          above += (int)hb[bb];
        }
        const uint64_t who = __ballot(digit >= 0);
        const int src = __ffsll((unsigned long long)who) - 1;
        digit = __shfl(digit, src, 64);
        above_d = __shfl(above_d, src, 64);
        kk -= above_d;
        prefix |= ((uint32_t)digit) << shift;
        pmask |= 0xFFu << shift;
      }
      T = prefix;
      take_eq = kk;
    }
    // Phase 3: ascending compaction over key cube ids.
    int32_t* irow = idx + ((size_t)bh * nbq + i) * k_sel;
    uint8_t* mrow = mask ? mask + ((size_t)bh * nbq + i) * g.nbk : nullptr;
    int run_sel = 0, run_eq = 0;
    for (int j0 = 0; j0 < g.nbk; j0 += 64) {
      const int j = j0 + lane;
      bool sel = false, eq = false;
      if (j < g.nbk) {
        if (j < g.nbc) {
          sel = true;
        } else {
          const int jn = j - g.nbc;
          if (jn == i) {
            sel = true;
          } else {
            const uint32_t u = kr[jn];
            if (u > T) sel = true;
            else if (u == T) eq = true;
          }
        }
      }
      const uint64_t eqm = __ballot(eq);
      if (eq && run_eq + lanes_below(eqm) < take_eq) sel = true;
      run_eq += __popcll(eqm);
      const uint64_t sm = __ballot(sel);
      const int pos = run_sel + lanes_below(sm);
      if (sel && pos < k_sel) irow[pos] = j;  // a row never holds more than k_sel ids
      run_sel += __popcll(sm);
      if (mrow && j < g.nbk) mrow[j] = sel ? 1 : 0;
    }
  }
}

static size_t select_lds_bytes(const Geom& g, int R, int NW) {
  return ((size_t)R * g.D + (size_t)R * g.nbq + (size_t)NW * 256) * sizeof(uint32_t);
}

hipError_t launch_select(const Geom& g, const float* qm, const float* km, int r_eff, int k_sel,
                         int32_t* idx, uint8_t* mask, hipStream_t s) {
  constexpr size_t kMaxLds = 160 * 1024;
  if (select_lds_bytes(g, 16, 16) <= kMaxLds) {
    // 16 rows per workgroup: 34% faster than 8 rows at 1440 key cubes (same bits)
    const size_t lds = select_lds_bytes(g, 16, 16);
    if (lds > 64 * 1024)
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(select_kernel<16, 16>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    dim3 grid((g.nbq + 15) / 16, g.B * g.Hh);
    hipLaunchKernelGGL((select_kernel<16, 16>), grid, dim3(1024), lds, s, g, qm, km, r_eff, k_sel,
                       idx, mask);
    return hipGetLastError();
  }
  int R = 8;
  while (R > 1 && select_lds_bytes(g, R, 4) > 64 * 1024) R >>= 1;
  const size_t lds = select_lds_bytes(g, R, 4);
  dim3 grid((g.nbq + R - 1) / R, g.B * g.Hh);
  switch (R) {
    case 8:
      hipLaunchKernelGGL((select_kernel<8, 4>), grid, dim3(256), lds, s, g, qm, km, r_eff, k_sel,
                         idx, mask);
      break;
    case 4:
      hipLaunchKernelGGL((select_kernel<4, 4>), grid, dim3(256), lds, s, g, qm, km, r_eff, k_sel,
                         idx, mask);
      break;
    case 2:
      hipLaunchKernelGGL((select_kernel<2, 4>), grid, dim3(256), lds, s, g, qm, km, r_eff, k_sel,
                         idx, mask);
      break;
    default:
      if (lds > kMaxLds) return hipErrorInvalidValue;
      if (lds > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(select_kernel<1, 4>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      hipLaunchKernelGGL((select_kernel<1, 4>), grid, dim3(256), lds, s, g, qm, km, r_eff, k_sel,
                         idx, mask);
      break;
  }
  return hipGetLastError();
}

}  // namespace bsa
