// k_validate.hip -- checks a selection against the contract of the attention calls: every entry a
// key cube id in [0, nbk) and every row strictly ascending (the top-r key cubes of each query
// cube, "LongCat-Video视频生成模型发布 迈出世界模型探索第一步", youleyou, section
// "块稀疏注意力（BSA）", written as ascending ids).  The attention kernels assume both: the split
// forward counts a row's ids per key range with one pass, and the backward's CSR transpose maps
// each id to one key cube.  A malformed row would give dQ that disagrees with dK/dV.
//
// One wave per row: lane l checks entry l (and l + 64, ...) against its range and against the
// entry before it; the row's result is one ballot, and the first lane of a bad row adds one to
// the counter.
#include "bsa_launch.h"

namespace bsa {

__global__ __launch_bounds__(64) void zero_counter_kernel(int32_t* __restrict__ bad_rows) {
  if (threadIdx.x == 0) *bad_rows = 0;
}

__global__ __launch_bounds__(256) void validate_idx_kernel(Geom g, const int32_t* __restrict__ idx,
                                                           int k_sel, long long rows,
                                                           int32_t* __restrict__ bad_rows) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int32_t* r = idx + row * k_sel;
  bool bad = false;
  for (int e = lane; e < k_sel; e += 64) {
    const int32_t v = r[e];
    bad |= v < 0 || v >= g.nbk;
    if (e > 0) bad |= v <= r[e - 1];
  }
  if (__ballot(bad) && lane == 0) atomicAdd(bad_rows, 1);
}

hipError_t launch_validate_idx(const Geom& g, const int32_t* idx, int k_sel, int32_t* bad_rows,
                               hipStream_t s) {
  hipLaunchKernelGGL(zero_counter_kernel, dim3(1), dim3(64), 0, s, bad_rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long rows = (long long)g.B * g.Hh * g.nbq;
  hipLaunchKernelGGL(validate_idx_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, g,
                     idx, k_sel, rows, bad_rows);
  return hipGetLastError();
}

}  // namespace bsa
