// bsa_bwd_tiles.h -- tile helpers shared by the gfx950 backward kernels (dQ and dK/dV): buffer
// loads, the bf16 MFMA step, and the LDS staging of ROW-layout half cubes with their plain and
// transposed (ds_read_b64_tr_b16) operand reads.
//
// ROW gather layout (lane = token, 8 consecutive d per 16 bytes): a 32-row half block is D/16
// steps of 1 KB, step s holding lane l's 16 bytes at (s*64 + l)*16.
#pragma once

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
// Shared LDS helpers.
//
// A staged ROW half block keeps the D/16 steps of the global layout (1 KB each: lane l's 16 bytes
// at l*16) but places step s' at s' * kStageStep in LDS, 64 bytes further apart than in memory.
// The transposed reads take 8-byte runs from four different steps at once; with the steps exactly
// 1 KB apart those runs fall on the same LDS banks (2- to 4-way conflicts), with the 64-byte skew
// they cover every bank once.  A byte of the staged block: s' * kStageStep + lane' * 16 + e' * 2
// for ROW element (step s', lane' = (d / (D/2)) * 32 + row, e' = d % 8).
// ---------------------------------------------------------------------------------------------
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kStageStep = 1024 + 64;
// LDS bytes of one staged 32-row half block.
template <int D>
__host__ __device__ constexpr int staged_half_bytes() {
  return (D / 16) * kStageStep;
}
__device__ __forceinline__ constexpr int stage_off(int step, int lane_row, int elem) {
  return step * kStageStep + lane_row * 16 + elem * 2;
}

// Operand fragment of a ROW-layout 32-row half block staged in LDS: lane's 16 bytes of step s.
__device__ __forceinline__ bf16x8 lds_row_frag(const lds_char* stage, int lane, int s) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
      stage + stage_off(s, lane, 0));
}

// Byte offset (inside a staged ROW half block) of lane's transposed read for operand (db, s2),
// half eh: ds_read_b64_tr_b16 gives lane m of each 16-lane group g element k of
// v[4k + m/4][m%4], where v[n] is the 4-element run at lane n's address.  Pointing lane n at
// row 16*s2 + 8*eh + 4*(g/2) + n/4, columns d = 32*db + 16*(g%2) + 4*(n%4) .. +3 turns the run
// into the TRANS operand (lane = d, 8 rows in accumulator-row order).  In ROW terms the lane
// part is step 2*(g%2) + (n%4)/2, lane' 4*(g/2) + n/4, element 4*(n%2).
__device__ __forceinline__ int tr_lane_base(int lane) {
  const int g = lane >> 4, n = lane & 15;
  return stage_off(2 * (g & 1) + ((n & 3) >> 1), 4 * (g >> 1) + (n >> 2), 4 * (n & 1));
}
// The row-split point of the ROW layout is d = D/2: column d lives at lane' = (d/(D/2))*32 + r,
// step s' = (d%(D/2))/8.  With d = 32*db + (lane part), that gives per-(db, s2, eh) constants:
template <int D>
__device__ __forceinline__ int tr_const(int db, int s2, int eh) {
  if constexpr (D == 128) return stage_off(4 * (db & 1), 32 * (db >> 1) + 16 * s2 + 8 * eh, 0);
  else return stage_off(0, 32 * db + 16 * s2 + 8 * eh, 0);  // D == 64
}
template <int D>
__device__ __forceinline__ bf16x8 lds_trans_frag(const lds_char* stage, int lane_base, int db,
                                                 int s2) {
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(stage + lane_base + tr_const<D>(db, s2, 0)));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(stage + lane_base + tr_const<D>(db, s2, 1)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

// ---------------------------------------------------------------------------------------------
// 16-row steps on v_mfma_f32_16x16x32_bf16 (A: lane = row 16-block position, 8 consecutive k at
// 8*(lane/16); D: lane holds rows 4*(lane/16) + i of column lane%16).
// ---------------------------------------------------------------------------------------------
typedef float f32x4v __attribute__((ext_vector_type(4)));

// Byte offset inside a staged ROW half block of the 16-byte fragment holding row r0 + lane%16,
// columns 32*s + 8*(lane/16) .. +7: lane part (step lane/16, lane' lane%16) and (s, r0) part.
__device__ __forceinline__ int row16_lane(int lane) { return stage_off(lane >> 4, lane & 15, 0); }
template <int D>
__device__ __forceinline__ int row16_const(int s, int r0) {
  return stage_off(((32 * s) % (D / 2)) / 8, ((32 * s) / (D / 2)) * 32 + r0, 0);
}

// The same fragment in the gathered ROW layout in memory (steps 1 KB apart), for loads straight
// into registers.
__device__ __forceinline__ int row16_lane_mem(int lane) {
  return ((lane >> 4) * 64 + (lane & 15)) * 16;
}
template <int D>
__device__ __forceinline__ int row16_const_mem(int s, int r0) {
  return ((((32 * s) % (D / 2)) / 8) * 64 + ((32 * s) / (D / 2)) * 32 + r0) * 16;
}

// Transposed read (ds_read_b64_tr_b16) of the 16-row block `sub` of a staged half: lane gets
// rows 16*sub + 8*(lane/32) + 0..7, in natural order, of column 32*db + lane%32 (the same
// pointing rule as lds_trans_frag with the row index 8*(g/2) + 4*eh + n/4).
__device__ __forceinline__ int tr16_lane(int lane) {
  const int g = lane >> 4, n = lane & 15;
  return stage_off(2 * (g & 1) + ((n & 3) >> 1), 8 * (g >> 1) + (n >> 2), 4 * (n & 1));
}
template <int D>
__device__ __forceinline__ int tr16_const(int db, int sub, int eh) {
  if constexpr (D == 128) return stage_off(4 * (db & 1), 32 * (db >> 1) + 16 * sub + 4 * eh, 0);
  else return stage_off(0, 32 * db + 16 * sub + 4 * eh, 0);  // D == 64
}
template <int D>
__device__ __forceinline__ bf16x8 lds_tr16(const lds_char* stage, int lane_base, int db, int sub) {
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(stage + lane_base + tr16_const<D>(db, sub, 0)));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(stage + lane_base + tr16_const<D>(db, sub, 1)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Two 16x16 accumulators x, y of key blocks 2kb, 2kb+1 (lane: query 4*(lane/16) + i, key
// lane%16 of its block) -> the bf16 B operand of a 32x32x16 product over those 16 queries (lane:
// key 32kb + lane%32, queries 8*(lane/32) + 0..7).  v_permlane16_swap exchanges the odd 16-lane
// rows of the first register with the even rows of the second, which moves every lane's missing
// four queries of its key in from the neighbouring row.
__device__ __forceinline__ bf16x8 acc16_to_b32(const f32x4v& x, const f32x4v& y) {
  const auto s0 = __builtin_amdgcn_permlane16_swap(pack_bf16x2(x[0], x[1]), pack_bf16x2(y[0], y[1]),
                                                   false, false);
  const auto s1 = __builtin_amdgcn_permlane16_swap(pack_bf16x2(x[2], x[3]), pack_bf16x2(y[2], y[3]),
                                                   false, false);
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
  return __builtin_bit_cast(bf16x8, v);
}

// One 32-row half block (D/16 steps of 1 KB) of a ROW-gathered tensor -> LDS at the staged
// layout (steps kStageStep apart), no VGPRs in between.
template <int D>
__device__ __forceinline__ void stage_half(__amdgpu_buffer_rsrc_t r, int soff, lds_char* dst,
                                           int lane) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(dst + s * kStageStep), 16, lane * 16,
        soff + s * 1024, 0, 0);
}

}  // namespace bsa
