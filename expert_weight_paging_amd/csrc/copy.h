// Record copy shared by the kernels that page experts in from the host store's
// device mapping: a workgroup's share of one record.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace moepage {

// Workgroup b of nb copies its chunks of a record of `bytes` (a multiple of
// 16) from src to dst: 16-byte chunks, NT threads with U loads in flight each,
// the workgroups taking consecutive runs of NT * U chunks in turn.
template <int NT, int U>
__device__ inline void copy_record_share(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                         size_t bytes, int b, int nb) {
  const size_t n16 = bytes / 16;
  const size_t step = (size_t)nb * NT * U;
  const uint4* s = (const uint4*)src;
  uint4* d = (uint4*)dst;
  for (size_t i = (size_t)b * NT * U + threadIdx.x; i < n16; i += step) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t j = i + (size_t)u * NT;
      if (j < n16) v[u] = s[j];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t j = i + (size_t)u * NT;
      if (j < n16) d[j] = v[u];
    }
  }
}

}  // namespace moepage
