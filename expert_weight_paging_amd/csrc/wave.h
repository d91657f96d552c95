// Wavefront (64-lane) reductions on gfx950 with DPP lane moves, which stay in
// the VALU instead of going through the LDS crossbar.
#pragma once

#include <hip/hip_runtime.h>

namespace moepage {

// DPP controls (GFX9 encoding).
constexpr int kDppQuad1032 = 0xB1;   // quad_perm:[1,0,3,2]
constexpr int kDppQuad2301 = 0x4E;   // quad_perm:[2,3,0,1]
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xF>
__device__ inline float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over the 64 lanes, returned to every lane.
__device__ inline float wave_sum(float v) {
  v += dpp_f<kDppQuad1032>(v);      // pairs
  v += dpp_f<kDppQuad2301>(v);      // quads
  v += dpp_f<kDppRowHalfMirror>(v); // 8 lanes
  v += dpp_f<kDppRowMirror>(v);     // rows of 16
  v += dpp_f<kDppRowBcast15, 0xA>(v);  // rows 1, 3 add the row before
  v += dpp_f<kDppRowBcast31, 0xC>(v);  // rows 2, 3 add lanes 0..31's total
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

}  // namespace moepage
