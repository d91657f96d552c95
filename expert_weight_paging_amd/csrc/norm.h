// Unit-gain RMSNorm of a bf16 hidden-state row staged in LDS, shared by the
// standalone norm kernel and the decode up kernels (which normalise the row
// they have just staged), so both give the same bits: the same thread-to-chunk
// map, the same fixed-order reduction, the same rounding.
//
// A stack of MoE layers reads the residual stream through this norm, as the
// MoE block of the model the pages run (Qwen3-30B-A3B) does; the pages train
// nothing here, so the gain is one.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "moepage.h"
#include "wave.h"

namespace moepage {

constexpr int kNormThreads = 256;

__device__ inline uint32_t norm_bf16_rne(float v) {
  uint32_t b = __float_as_uint(v);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return b >> 16;
}

// row: nx16 16-byte chunks (8 bf16 each) of one row of H values in LDS; red:
// 4 floats of LDS. Called by all kNormThreads threads of the workgroup (a
// barrier must separate the row's staging from the call); thread i sums the
// squares of chunks i, i + 256, ... in order, the wavefront sums combine in
// wavefront order, and every value becomes bf16_rne(v / sqrt(mean(v^2) + eps)).
// Ends with a barrier.
__device__ inline void rmsnorm_row_lds(uint4* row, int nx16, int H, float* red) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  float ss = 0.f;
  for (int c = tid; c < nx16; c += kNormThreads) {
    const uint4 q = row[c];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xFFFF0000u);
      ss = fmaf(lo, lo, ss);
      ss = fmaf(hi, hi, ss);
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wid] = ss;
  __syncthreads();
  const float tot = ((red[0] + red[1]) + red[2]) + red[3];
  const float inv = 1.0f / sqrtf(tot / (float)H + MOE_RMS_EPS);
  for (int c = tid; c < nx16; c += kNormThreads) {
    const uint4 q = row[c];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(w[i] << 16) * inv, hi = __uint_as_float(w[i] & 0xFFFF0000u) * inv;
      o[i] = norm_bf16_rne(lo) | (norm_bf16_rne(hi) << 16);
    }
    row[c] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  __syncthreads();
}

}  // namespace moepage
