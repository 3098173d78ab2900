// k_probe.hip -- two microbenchmarks that bound the attention kernels on MI355X (diagnostics; no
// part of block sparse attention runs here):
//
//  * mfma_probe_kernel: back-to-back v_mfma_f32_32x32x16_bf16 on every SIMD, four independent
//    accumulator chains per wave, operands taken from a caller buffer.  With N(0,1) bf16 operands
//    (the data the attention products see) the chip lowers its clock under load, so this is the
//    rate bf16 MFMA work can reach on such data; constant operands show the clock effect.
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

__global__ __launch_bounds__(64) void mfma_probe_kernel(const bf16_t* __restrict__ operands,
                                                        int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x;
  bf16x8 a[8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
    a[u] = __builtin_bit_cast(bf16x8,
                              *reinterpret_cast<const uint4*>(operands + (u * 64 + lane) * 8));
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      acc[u & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], a[(u + 3) & 7], acc[u & 3], 0,
                                                           0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  sink[blockIdx.x * 64 + lane] = s;
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

hipError_t launch_mfma_probe(const bf16_t* operands, int waves, int iters, float* sink,
                             hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)waves), dim3(64), 0, s, operands, iters,
                     sink);
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
