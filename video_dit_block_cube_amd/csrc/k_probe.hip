// k_probe.hip -- two microbenchmarks that bound the attention kernels on MI355X (diagnostics; no
// part of block sparse attention runs here):
//
//  * mfma_probe_kernel: back-to-back v_mfma_f32_32x32x16_bf16 (or 16x16x32) on every SIMD, with
//    1, 2, 4 or 8 independent accumulator chains per wave, operands taken from a caller buffer.  With N(0,1) bf16 operands
//    (the data the attention products see) the chip lowers its clock under load, so this is the
//    rate bf16 MFMA work can reach on such data; constant operands show the clock effect.
//  * coexec_probe_kernel: bf16 MFMA and VALU work on one SIMD, either interleaved in each wave
//    or split between the two waves that share the SIMD, against each kind alone: how much
//    VALU work (softmax arithmetic) can run beside the products, and in which arrangement.
//  * tile_read_kernel: every wave reads whole tiles (tile_bytes, a multiple of 1 KB) at the tile
//    ids of its row of a caller table, as 1 KB wave-wide 16-byte-per-lane buffer loads -- the
//    access pattern of the attention kernels' K/V and Q/dO tiles.  The caller picks the ids, and
//    with them the working set each XCD (workgroup w runs on XCD w % 8) touches.
#include "bsa_launch.h"

namespace bsa {

namespace {
__device__ __forceinline__ __amdgpu_buffer_rsrc_t probe_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes < 0x7fffffffu ? bytes : 0x7fffffffu),
                                           0x00020000);
}
}  // namespace

// SHAPE 0: v_mfma_f32_32x32x16_bf16, 8 products per iteration; SHAPE 1: v_mfma_f32_16x16x32_bf16,
// 16 products per iteration (262144 FLOP per iteration either way).  CH independent accumulator
// chains per wave, product u adding into chain u % CH: one chain makes every product depend on
// the one before it.
template <int SHAPE, int CH>
__global__ __launch_bounds__(64) void mfma_probe_kernel(const bf16_t* __restrict__ operands,
                                                        int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x;
  bf16x8 a[8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
    a[u] = __builtin_bit_cast(bf16x8,
                              *reinterpret_cast<const uint4*>(operands + (u * 64 + lane) * 8));
  float s = 0.f;
  if constexpr (SHAPE == 0) {
    f32x16 acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        acc[u % CH] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], a[(u + 3) & 7], acc[u % CH],
                                                              0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[c][e];
  } else {
    typedef float f32x4p __attribute__((ext_vector_type(4)));
    f32x4p acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[c][e] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < 16; ++u)
        acc[u % CH] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u & 7], a[(u + 3) & 7],
                                                              acc[u % CH], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) s += acc[c][e];
  }
  sink[blockIdx.x * 64 + lane] = s;
}

// Eight-wave workgroups, one per CU at a time, two waves on every SIMD.  Each iteration is four products
// (v_mfma_f32_32x32x16_bf16, four independent accumulators) and/or, after each product, V VALU
// instructions on eight independent fp32 chains (OP 0: v_fma_f32; OP 1: v_exp_f32 of the negated
// value, whose fixed point keeps the chain finite).  mode 0: every wave does both, the VALU
// instructions scheduled right after each product; mode 1: on each SIMD one wave does the
// products and the other the VALU instructions (the wave's SIMD read from the HW_ID register,
// the first of the two in wave order taking the products); mode 2: products only; mode 3: VALU
// only.
// The loop of one wave: iters x 4 slots, each slot a product (DO_M) and/or V VALU instructions
// (DO_V); with both, the VALU instructions are scheduled right after their slot's product.
template <int V, int OP, bool DO_M, bool DO_V>
__device__ __forceinline__ float coexec_loop(const bf16x8 a, const bf16x8 b, int lane, int iters) {
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  float x[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = 0.001f * (float)(lane + k);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if constexpr (DO_M) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
      if constexpr (DO_V) {
#pragma unroll
        for (int k = 0; k < V; ++k) {
          if constexpr (OP == 0) x[k & 7] = fmaf(x[k & 7], 0.999f, 0.001f);
          else x[k & 7] = __builtin_amdgcn_exp2f(-x[k & 7]);
        }
      }
      if constexpr (DO_M && DO_V) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, V, 0);  // then V VALU instructions
      }
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += acc[c][e];
#pragma unroll
  for (int k = 0; k < 8; ++k) sum += x[k];
  return sum;
}

// Eight-wave workgroups, one per CU at a time, two waves on every SIMD.  Each iteration is four
// products (v_mfma_f32_32x32x16_bf16, four independent accumulators) and/or, after each product,
// V VALU instructions on eight independent fp32 chains (OP 0: v_fma_f32; OP 1: v_exp_f32 of the
// negated value, whose fixed point keeps the chain finite).  mode 0: every wave does both;
// mode 1: on each SIMD one wave does the products and the other the VALU instructions (the
// wave's SIMD read from the HW_ID register, the first of the two in wave order taking the
// products); mode 2: products only; mode 3: VALU only.
template <int V, int OP, int ACC>
__global__ __launch_bounds__(512) void coexec_probe_kernel(const bf16_t* __restrict__ operands,
                                                           int mode, int iters,
                                                           float* __restrict__ sink) {
  // ACC 1: an (empty) use of an AGPR tells the compiler the kernel may use AGPRs, which makes it
  // give every product an AGPR accumulator; ACC 0 leaves them in VGPRs (the kernel fits in 256)
  if constexpr (ACC == 1) asm volatile("; agpr in use %0" ::"a"(0));
  __shared__ int simd_of[8];
  // 84 KB of LDS, so that one workgroup holds a CU and every SIMD runs exactly its two waves
  __shared__ int hold[21504];
  if (iters < 0) hold[threadIdx.x] = 0;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // SIMD_ID is bits 5:4 of HW_ID (s_getreg_b32 hwreg(HW_REG_HW_ID, 4, 2))
  const int simd = (int)(__builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4) & 3);
  if (lane == 0) simd_of[wv] = simd;
  __syncthreads();
  int before = 0;  // earlier waves of this workgroup on the same SIMD
  for (int w = 0; w < wv; ++w) before += simd_of[w] == simd ? 1 : 0;
  const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(operands + lane * 8));
  const bf16x8 b =
      __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(operands + (64 + lane) * 8));
  float sum;
  if (mode == 0) sum = coexec_loop<V, OP, true, true>(a, b, lane, iters);
  else if (mode == 2 || (mode == 1 && before == 0)) sum = coexec_loop<V, OP, true, false>(a, b, lane, iters);
  else sum = coexec_loop<V, OP, false, true>(a, b, lane, iters);
  sink[blockIdx.x * 512 + threadIdx.x] = sum;
}

__global__ __launch_bounds__(64) void tile_read_kernel(const bf16_t* __restrict__ buf,
                                                       size_t buf_bytes, int tile_bytes,
                                                       const int32_t* __restrict__ ids,
                                                       int tiles_per_wave,
                                                       uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x;
  const __amdgpu_buffer_rsrc_t r = probe_rsrc(buf, buf_bytes);
  const int32_t* row = ids + (size_t)blockIdx.x * tiles_per_wave;
  const int loads = tile_bytes / 1024;
  uint32_t x = 0u;
  const long long n_tiles = (long long)(buf_bytes / (size_t)tile_bytes);
  for (int t = 0; t < tiles_per_wave; ++t) {
    const int id = row[t];
    if (id < 0 || id >= n_tiles) continue;  // not a tile of buf
    const int base = id * tile_bytes;
    for (int l0 = 0; l0 < loads; l0 += 8) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                             r, lane * 16, base + (l0 + u) * 1024, 0));
#pragma unroll
      for (int u = 0; u < 8; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  sink[blockIdx.x * 64 + lane] = x;
}

hipError_t launch_mfma_probe(const bf16_t* operands, int shape, int chains, int waves, int iters,
                             float* sink, hipStream_t s) {
  const dim3 grid((unsigned)waves), block(64);
#define BSA_PROBE(SH, CH) \
  hipLaunchKernelGGL((mfma_probe_kernel<SH, CH>), grid, block, 0, s, operands, iters, sink)
  switch (shape * 16 + chains) {
    case 1: BSA_PROBE(0, 1); break;
    case 2: BSA_PROBE(0, 2); break;
    case 4: BSA_PROBE(0, 4); break;
    case 8: BSA_PROBE(0, 8); break;
    case 17: BSA_PROBE(1, 1); break;
    case 18: BSA_PROBE(1, 2); break;
    case 20: BSA_PROBE(1, 4); break;
    case 24: BSA_PROBE(1, 8); break;
    default: return hipErrorInvalidValue;
  }
#undef BSA_PROBE
  return hipGetLastError();
}

hipError_t launch_coexec_probe(const bf16_t* operands, int mode, int valu, int op, int acc,
                               int workgroups, int iters, float* sink, hipStream_t s) {
  const dim3 grid((unsigned)workgroups), block(512);
#define BSA_COEXEC(VV, OO, AA)                                                                   \
  hipLaunchKernelGGL((coexec_probe_kernel<VV, OO, AA>), grid, block, 0, s, operands, mode, iters, \
                     sink)
#define BSA_COEXEC2(VV, OO) \
  if (acc) BSA_COEXEC(VV, OO, 1); else BSA_COEXEC(VV, OO, 0);
  switch (op * 32 + valu) {
    case 0: BSA_COEXEC2(0, 0); break;
    case 2: BSA_COEXEC2(2, 0); break;
    case 4: BSA_COEXEC2(4, 0); break;
    case 8: BSA_COEXEC2(8, 0); break;
    case 16: BSA_COEXEC2(16, 0); break;
    case 33: BSA_COEXEC2(1, 1); break;
    case 34: BSA_COEXEC2(2, 1); break;
    case 36: BSA_COEXEC2(4, 1); break;
    default: return hipErrorInvalidValue;
  }
#undef BSA_COEXEC2
#undef BSA_COEXEC
  return hipGetLastError();
}

hipError_t launch_tile_read(const bf16_t* buf, size_t buf_bytes, int tile_bytes,
                            const int32_t* ids, int waves, int tiles_per_wave, uint32_t* sink,
                            hipStream_t s) {
  hipLaunchKernelGGL(tile_read_kernel, dim3((unsigned)waves), dim3(64), 0, s, buf, buf_bytes,
                     tile_bytes, ids, tiles_per_wave, sink);
  return hipGetLastError();
}

}  // namespace bsa
