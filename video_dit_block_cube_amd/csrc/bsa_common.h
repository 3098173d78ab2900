// bsa_common.h -- kernel-side geometry and small device helpers shared by the gfx950 BSA kernels.
//
// Cube partition of the latent grid (tokens grouped into small 3D cubes: "LongCat-Video :
// Generate 1 minute long AI videos with this model", Data Science in Your Pocket, section
// "Sparse attention"): cubes are numbered in raster order over cube coordinates (t slowest, then
// h, then w) inside each segment (condition frames, noise frames); the c slots of a cube are
// visited in raster order over (dt, dh, dw).  On a ragged grid (H or W not a multiple of the cube
// side) the last cube row / column is partial: its slots outside the grid hold no token.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

struct Geom {
  int B, Hh, D;
  int T, H, W;
  int ct, ch, cw;
  int condT;
  // derived
  int c;         // tokens per cube
  int nT;        // noise frames
  int Nq, Nc;    // tokens in the noise / condition segment
  int gh, gw;    // cubes along h, w
  int gtq, gtc;  // cubes along t in the noise / condition segment
  int nbq, nbc, nbk;
  int ragged;    // H % ch or W % cw non-zero: partial edge cubes exist
};

inline Geom make_geom(int B, int Hh, int D, int T, int H, int W, int ct, int ch, int cw,
                      int condT) {
  Geom g;
  g.B = B; g.Hh = Hh; g.D = D; g.T = T; g.H = H; g.W = W;
  g.ct = ct; g.ch = ch; g.cw = cw; g.condT = condT;
  g.c = ct * ch * cw;
  g.nT = T - condT;
  g.Nq = g.nT * H * W;
  g.Nc = condT * H * W;
  g.gh = (H + ch - 1) / ch;
  g.gw = (W + cw - 1) / cw;
  g.ragged = (H % ch) != 0 || (W % cw) != 0;
  g.gtq = g.nT / ct;
  g.gtc = condT / ct;
  g.nbq = g.gtq * g.gh * g.gw;
  g.nbc = g.gtc * g.gh * g.gw;
  g.nbk = g.nbq + g.nbc;
  return g;
}

// Token index (raster order inside its segment) of slot `slot` of cube `cube` of a segment.
__host__ __device__ inline int cube_token(const Geom& g, int cube, int slot) {
  const int e = cube % g.gw;
  const int r = cube / g.gw;
  const int bb = r % g.gh;
  const int a = r / g.gh;
  const int dw = slot % g.cw;
  const int r2 = slot / g.cw;
  const int dh = r2 % g.ch;
  const int dt = r2 / g.ch;
  const int hh = bb * g.ch + dh, ww = e * g.cw + dw;
  if (hh >= g.H || ww >= g.W) return -1;  // slot of a partial edge cube outside the grid
  return ((a * g.ct + dt) * g.H + hh) * g.W + ww;
}

// Extent of cube `cube` of a segment along h and w (ch, cw except on a ragged edge).
__host__ __device__ inline void cube_extent(const Geom& g, int cube, int& he, int& we) {
  const int e = cube % g.gw, bb = (cube / g.gw) % g.gh;
  he = g.H - bb * g.ch < g.ch ? g.H - bb * g.ch : g.ch;
  we = g.W - e * g.cw < g.cw ? g.W - e * g.cw : g.cw;
}

// Number of tokens of cube `cube` of a segment.
__host__ __device__ inline int cube_count(const Geom& g, int cube) {
  int he, we;
  cube_extent(g, cube, he, we);
  return g.ct * he * we;
}

// Bit k set iff slot 32*half + k of the cube holds a token (all bits off the ragged edge).
__device__ inline uint32_t cube_half_mask(const Geom& g, int cube, int half) {
  int he, we;
  cube_extent(g, cube, he, we);
  if (he == g.ch && we == g.cw) return 0xffffffffu;
  uint32_t m = 0u;
  for (int k = 0; k < 32; ++k) {
    const int s = 32 * half + k;
    const int dw = s % g.cw, dh = (s / g.cw) % g.ch;
    if (s < g.c && dh < he && dw < we) m |= 1u << k;
  }
  return m;
}

// Element offset of (b, token, head, 0) in a [B, N, Hh, D] tensor.
__host__ __device__ inline size_t bnhd_offset(const Geom& g, int N, int b, int tok, int h) {
  return ((size_t)((size_t)b * N + tok) * g.Hh + h) * (size_t)g.D;
}

typedef uint16_t bf16_t;  // raw bfloat16 bits in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(bf16_t x) {
  return __uint_as_float(((uint32_t)x) << 16);
}

// fp32 -> bf16 with round-to-nearest-even (gfx950 v_cvt_pk_bf16_f32); finite inputs.
__device__ __forceinline__ bf16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(bf16_t, h);
}

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_as_f32<bf16_t>(const bf16_t* p) {
  return bf16_bits_to_f32(*p);
}

template <typename T>
__device__ __forceinline__ void store_from_f32(T* p, float v);
template <>
__device__ __forceinline__ void store_from_f32<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_from_f32<bf16_t>(bf16_t* p, float v) {
  *p = f32_to_bf16_bits(v);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Number of lanes below this one whose bit is set in `m` (wave64).
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

}  // namespace bsa
