// Decode up projection (gate/up GEMV + SiLU) and the format helpers it shares
// with the down kernel, included by ffn_gemv.hip and by plan.hip (whose
// route-and-page-in launch for the next layer of a stack also runs this
// layer's up projection).
#pragma once

#include "internal.h"
#include "norm.h"
#include "wave.h"

namespace moepage {
namespace gemv {

constexpr int kWave = 64;


__device__ inline uint16_t f32_to_bf16_rne(float v) {
  uint32_t b = __float_as_uint(v);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__device__ inline float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
// 16 bytes of weights read once per step: a streaming load, so the L2 keeps
// the small tables the next launch reads (slot map, h)
__device__ inline uint4 nt_load16(const uint8_t* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));

// e4m3fn pair -> two floats (gfx950 converts OCP e4m3 in hardware); HI selects
// bytes 2..3 of the word instead of bytes 0..1.
template <bool HI>
__device__ inline f32x2 fp8x2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// acc + lo(w)*lo(x) + hi(w)*hi(x) over two packed bf16 pairs (products exact
// in fp32; one fp32 accumulation per pair).
__device__ inline float dot2_bf16(uint32_t w, uint32_t x, float acc) {
  bf16x2_t a, b;
  __builtin_memcpy(&a, &w, 4);
  __builtin_memcpy(&b, &x, 4);
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, acc, false);
}

__device__ inline float half_to_float(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, 2);
  return (float)v;
}

// ------------------------------------------------------------------ formats
// Per format: values per 16-byte chunk of a W13 row (CV1), bytes and values
// per chunk of a W_d row (CB2, CV2).
template <int F> struct Fmt;
template <> struct Fmt<MOE_FMT_F32> { static constexpr int CV1 = 4, CB2 = 16, CV2 = 4; };
template <> struct Fmt<MOE_FMT_BF16> { static constexpr int CV1 = 8, CB2 = 8, CV2 = 4; };
template <> struct Fmt<MOE_FMT_FP8_E4M3_B128> { static constexpr int CV1 = 16, CB2 = 4, CV2 = 4; };
template <> struct Fmt<MOE_FMT_INT4_ASYM_G128> { static constexpr int CV1 = 32, CB2 = 4, CV2 = 8; };
template <> struct Fmt<MOE_FMT_MXFP4_B32> { static constexpr int CV1 = 32, CB2 = 4, CV2 = 8; };

// MXFP4: one word of 8 E2M1 codes (byte b = codes 2b, 2b+1) -> the same values
// as e4m3 bytes, converted in hardware. Every E2M1 value is exact in e4m3: a
// byte permute maps the 3 magnitude bits through the table {0, 0.5, 1, 1.5,
// 2, 3, 4, 6} (as e4m3: 00 30 38 3C 40 44 48 4C) and the sign bit moves from
// bit 3 to bit 7 of each byte. Returns the codes 0,2,4,6 (ev) and 1,3,5,7 (od).
__device__ inline void e2m1x8_to_e4m3(uint32_t w, uint32_t* ev, uint32_t* od) {
  const uint32_t lo = 0x3C383000u, hi = 0x4C484440u;
  const uint32_t e = w & 0x0F0F0F0Fu, o = (w >> 4) & 0x0F0F0F0Fu;
  *ev = __builtin_amdgcn_perm(hi, lo, e & 0x07070707u) | ((e & 0x08080808u) << 4);
  *od = __builtin_amdgcn_perm(hi, lo, o & 0x07070707u) | ((o & 0x08080808u) << 4);
}

__device__ inline float e8m0_to_float(uint8_t b) {  // 2^(b - 127); 255 is NaN
  return b == 255 ? __uint_as_float(0x7FC00000u)
                  : (b == 0 ? 5.877471754111438e-39f : __uint_as_float((uint32_t)b << 23));
}

// Raw sum of e2m1(q) * x over 8 codes (one word) and the matching activations.
__device__ inline float dot_e2m1x8(uint32_t w, const float* x, float acc) {
  uint32_t ev, od;
  e2m1x8_to_e4m3(w, &ev, &od);
  const f32x2 a = fp8x2<false>(ev), b = fp8x2<true>(ev), c = fp8x2<false>(od), d = fp8x2<true>(od);
  acc = fmaf(a.x, x[0], acc);
  acc = fmaf(c.x, x[1], acc);
  acc = fmaf(a.y, x[2], acc);
  acc = fmaf(c.y, x[3], acc);
  acc = fmaf(b.x, x[4], acc);
  acc = fmaf(d.x, x[5], acc);
  acc = fmaf(b.y, x[6], acc);
  acc = fmaf(d.y, x[7], acc);
  return acc;
}

// The same sum with the block's E8M0 scale s = 2^(e - 127) applied by the
// conversion (gfx950 v_cvt_scalef32_pk_f32_fp4: selector b converts byte b,
// low nibble first, and multiplies by 2 to the exponent of its f32 scale
// operand, exactly): codes times s, in index order. In the normal range each
// step is the unscaled step times s, so the result is the raw sum times s,
// bit for bit.
__device__ inline float dot_e2m1x8_scaled(uint32_t w, const float* x, float s, float acc) {
  const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 0);
  const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 1);
  const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 2);
  const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 3);
  acc = fmaf(a.x, x[0], acc);
  acc = fmaf(a.y, x[1], acc);
  acc = fmaf(b.x, x[2], acc);
  acc = fmaf(b.y, x[3], acc);
  acc = fmaf(c.x, x[4], acc);
  acc = fmaf(c.y, x[5], acc);
  acc = fmaf(d.x, x[6], acc);
  acc = fmaf(d.y, x[7], acc);
  return acc;
}

// Load CV1 activations starting at column col, as float.
template <int F, typename XT>
__device__ inline void load_x(const XT* x, int col, float* v) {
  constexpr int CV1 = Fmt<F>::CV1;
  if constexpr (sizeof(XT) == 4) {
#pragma unroll
    for (int i = 0; i < CV1; i += 4) {
      const float4 q = *(const float4*)((const float*)x + col + i);
      v[i] = q.x; v[i + 1] = q.y; v[i + 2] = q.z; v[i + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < CV1; i += 8) {
      const uint4 q = *(const uint4*)((const uint16_t*)x + col + i);
      v[i] = bf16lo(q.x); v[i + 1] = bf16hi(q.x);
      v[i + 2] = bf16lo(q.y); v[i + 3] = bf16hi(q.y);
      v[i + 4] = bf16lo(q.z); v[i + 5] = bf16hi(q.z);
      v[i + 6] = bf16lo(q.w); v[i + 7] = bf16hi(q.w);
    }
  }
}

// Raw dot of one 16-byte W13 chunk with CV1 activations (no scale/zero).
// For int4 also returns the activation sum (for the zero point).
template <int F>
__device__ inline float dot1(const uint4 w, const float* x, float* xsum) {
  const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
  float acc = 0.f;
  if constexpr (F == MOE_FMT_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(__uint_as_float(wv[i]), x[i], acc);
  } else if constexpr (F == MOE_FMT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(bf16lo(wv[i]), x[2 * i], acc);
      acc = fmaf(bf16hi(wv[i]), x[2 * i + 1], acc);
    }
  } else if constexpr (F == MOE_FMT_FP8_E4M3_B128) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 a = fp8x2<false>(wv[i]), b = fp8x2<true>(wv[i]);
      acc = fmaf(a.x, x[4 * i], acc);
      acc = fmaf(a.y, x[4 * i + 1], acc);
      acc = fmaf(b.x, x[4 * i + 2], acc);
      acc = fmaf(b.y, x[4 * i + 3], acc);
    }
  } else if constexpr (F == MOE_FMT_MXFP4_B32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = dot_e2m1x8(wv[i], x + 8 * i, acc);
  } else {
    // int4: handled by dot1_int4 (fp16 pair path)
  }
  return acc;
}

// int4 codes against bf16 activations with the two-element bf16 dot: a code
// pair (q_a, q_b) becomes the bf16 pair (128 + q_a, 128 + q_b) exactly by
// setting the exponent of 128 (0x4300) under the nibbles (the ulp of bf16 at
// 128 is 1), so dot2 sums (128 + q) * x, and the 128 is folded into the zero
// point: sum (q - z) x = sum (128 + q) x - (128 + z) * sum x. Activations stay
// bf16 (any finite bf16 value); products are exact in fp32.
//
// Activations of one int4 chunk (32 values, 4 words of 8 codes) as bf16 pairs
// in the order the code pairs come out of a word: word i, step n pairs values
// 8i + n and 8i + n + 4. Built once per token from the packed bf16 row.
struct XPairs {
  uint32_t p[16];
  float sum;  // sum of the 32 activations (for the zero point)
};

// xw: the chunk's 32 bf16 activations as 16 packed words (2 per word, in order)
__device__ inline void make_xpairs(const uint32_t* xw, XPairs& xp) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a0 = xw[4 * i], a1 = xw[4 * i + 1], a2 = xw[4 * i + 2], a3 = xw[4 * i + 3];
    xp.p[4 * i + 0] = __builtin_amdgcn_perm(a2, a0, 0x05040100u);  // (x0, x4)
    xp.p[4 * i + 1] = __builtin_amdgcn_perm(a2, a0, 0x07060302u);  // (x1, x5)
    xp.p[4 * i + 2] = __builtin_amdgcn_perm(a3, a1, 0x05040100u);  // (x2, x6)
    xp.p[4 * i + 3] = __builtin_amdgcn_perm(a3, a1, 0x07060302u);  // (x3, x7)
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) s += bf16lo(xw[v]) + bf16hi(xw[v]);
  xp.sum = s;
}

// Raw sum of (128 + q) * x over one 16-byte int4 chunk (32 codes).
__device__ inline float dot1_int4(const uint4 w, const XPairs& xp) {
  const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const uint32_t q = ((wv[i] >> (4 * n)) & 0x000F000Fu) | 0x43004300u;
      acc = dot2_bf16(q, xp.p[4 * i + n], acc);
    }
  }
  return acc;
}

// ------------------------------------------------------------------ up
// The up kernel's work for block (bx, by) of its grid (I / (4 * RPW) x
// experts); 256 threads. Also run by the launch that routes and pages in the
// next layer (plan.hip), hence a function of the block coordinates.
template <int F, int NJ, int RPW, typename XT>
__device__ __forceinline__ void ffn_up_body(const FfnArgs& a, int bx, int by) {
  constexpr int CV1 = Fmt<F>::CV1;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int H = a.H, I = a.I;
  const int i0 = (bx * 4 + wid) * RPW;
  // Every wavefront takes part in the workgroup barriers below (one past the
  // last row loads row I - 1 again and stores nothing): each pair's
  // activation row is read from memory once per workgroup into LDS and
  // shared by its four wavefronts.
  __shared__ uint4 xs[kWave * NJ * CV1 * sizeof(XT) / 16];
  __shared__ float red[4];
  const int nx16 = H * (int)sizeof(XT) / 16;  // 16-byte chunks of one activation row
  const int o = a.o_lo + by;
  // The expert's slot and the device-resolved expert count are both read
  // before either is used, so they share one round trip ahead of the weight
  // loads (the empty asm keeps the compiler from moving the slot's read below
  // the count's test). The slot's position is clamped into the array and its
  // value used only when the expert exists; without a device count the read
  // goes to the slot map and is ignored.
  // Several tokens: the expert's CSR pair range is read in the same round
  // trip (one token: its one pair is at position o).
  int slot = a.order_slot[min(o, a.E - 1)];
  int nd = *(a.n_dev ? a.n_dev : a.order_slot);
  int p0 = o, p1 = o + 1;
  if (a.T > 1) {
    p0 = a.pair_off[min(o, a.E - 1)];
    p1 = a.pair_off[min(o, a.E - 1) + 1];
  }
  asm volatile("" : "+s"(slot), "+s"(nd));
  if (a.n_dev && by >= nd - a.o_lo) return;  // device-resolved count: uniform per block
  const uint8_t* rec = a.slots + (size_t)slot * a.stride;
  const RecLayout L = rec_layout(F, H, I);
  const int nch = H / CV1;
  const size_t row_bytes = (size_t)H * fmt_elem_bits(F) / 8;
  const uint8_t* w13 = rec + L.w13;

  uint4 wg[RPW][NJ], wu[RPW][NJ];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int i = min(i0 + r, I - 1);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = lane + kWave * j;
      if (c < nch) {
        wg[r][j] = nt_load16(w13 + (size_t)i * row_bytes + (size_t)c * 16);
        wu[r][j] = nt_load16(w13 + (size_t)(I + i) * row_bytes + (size_t)c * 16);
      } else {
        wg[r][j] = make_uint4(0, 0, 0, 0);
        wu[r][j] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  // per-chunk scale (fp8: 128x128 tiles; int4: per row and group of 128)
  float sg[RPW][NJ], su[RPW][NJ], zg[RPW][NJ], zu[RPW][NJ];
  if constexpr (F == MOE_FMT_FP8_E4M3_B128) {
    const float* s13 = (const float*)(rec + L.s13);
    const int nb = H / 128;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int i = min(i0 + r, I - 1);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = min(lane + kWave * j, nch - 1);
        sg[r][j] = s13[(i / 128) * nb + (c * CV1) / 128];
        su[r][j] = s13[((I + i) / 128) * nb + (c * CV1) / 128];
      }
    }
  } else if constexpr (F == MOE_FMT_INT4_ASYM_G128) {
    const uint16_t* s13 = (const uint16_t*)(rec + L.s13);
    const uint16_t* z13 = (const uint16_t*)(rec + L.z13);
    const int ng = H / 128;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int i = min(i0 + r, I - 1);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int g = min(lane + kWave * j, nch - 1) * CV1 / 128;
        sg[r][j] = half_to_float(s13[(size_t)i * ng + g]);
        zg[r][j] = half_to_float(z13[(size_t)i * ng + g]);
        su[r][j] = half_to_float(s13[(size_t)(I + i) * ng + g]);
        zu[r][j] = half_to_float(z13[(size_t)(I + i) * ng + g]);
      }
    }
  } else if constexpr (F == MOE_FMT_MXFP4_B32) {
    const uint8_t* s13 = rec + L.s13;  // one scale byte per chunk of 32
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int i = min(i0 + r, I - 1);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = min(lane + kWave * j, nch - 1);
        sg[r][j] = e8m0_to_float(s13[(size_t)i * nch + c]);
        su[r][j] = e8m0_to_float(s13[(size_t)(I + i) * nch + c]);
      }
    }
  }

  // the token of each of the expert's pairs (at most one per token, so at
  // most 64), pair p0 + i in lane i, read beside the weights; one token: 0
  int tq = 0;
  if (a.T > 1 && lane < p1 - p0) tq = a.pair_list[p0 + lane] / a.k;
  auto token_of = [&](int q) { return a.T == 1 ? 0 : __builtin_amdgcn_readlane(tq, q - p0); };
  const XT* xbase = (const XT*)a.x;
  if constexpr (F == MOE_FMT_BF16 && sizeof(XT) == 2) {
    // bf16 weights and activations: dot the packed pairs directly (8 values
    // per 16-byte chunk in 4 words), activations never widened to fp32
    for (int q = p0; q < p1; ++q) {
      const int t = token_of(q);
      if (q > p0) __syncthreads();  // the previous pair's reads of xs are done
      for (int c = threadIdx.x; c < nx16; c += 4 * kWave)
        xs[c] = ((const uint4*)(xbase + (size_t)t * H))[c];
      __syncthreads();
      if (a.norm) rmsnorm_row_lds(xs, nx16, H, red);
      uint4 xw[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = lane + kWave * j;
        xw[j] = c < nch ? xs[c] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          g = dot2_bf16(wg[r][j].x, xw[j].x, g);
          g = dot2_bf16(wg[r][j].y, xw[j].y, g);
          g = dot2_bf16(wg[r][j].z, xw[j].z, g);
          g = dot2_bf16(wg[r][j].w, xw[j].w, g);
          u = dot2_bf16(wu[r][j].x, xw[j].x, u);
          u = dot2_bf16(wu[r][j].y, xw[j].y, u);
          u = dot2_bf16(wu[r][j].z, xw[j].z, u);
          u = dot2_bf16(wu[r][j].w, xw[j].w, u);
        }
        g = wave_sum(g);
        u = wave_sum(u);
        if (lane == 0 && i0 + r < I) a.h[(size_t)q * I + i0 + r] = g / (1.f + __expf(-g)) * u;
      }
    }
    return;
  }
  for (int q = p0; q < p1; ++q) {
    const int t = token_of(q);
    if (q > p0) __syncthreads();  // the previous pair's reads of xs are done
    for (int c = threadIdx.x; c < nx16; c += 4 * kWave) xs[c] = ((const uint4*)(xbase + (size_t)t * H))[c];
    __syncthreads();
    if constexpr (sizeof(XT) == 2) {
      if (a.norm) rmsnorm_row_lds(xs, nx16, H, red);
    }
    const XT* xrow = (const XT*)xs;
    float xv[NJ][CV1];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = lane + kWave * j;
      if (c < nch) load_x<F, XT>(xrow, c * CV1, xv[j]);
      else {
#pragma unroll
        for (int v = 0; v < CV1; ++v) xv[j][v] = 0.f;
      }
    }
    XPairs xp[F == MOE_FMT_INT4_ASYM_G128 ? NJ : 1];
    if constexpr (F == MOE_FMT_INT4_ASYM_G128 && sizeof(XT) == 2) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = lane + kWave * j;
        uint32_t xw[16];
        if (c < nch) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint4 q = xs[c * 4 + u];
            xw[4 * u] = q.x; xw[4 * u + 1] = q.y; xw[4 * u + 2] = q.z; xw[4 * u + 3] = q.w;
          }
        } else {
#pragma unroll
          for (int u = 0; u < 16; ++u) xw[u] = 0u;
        }
        make_xpairs(xw, xp[j]);
      }
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      float g = 0.f, u = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        // FP8 and MXFP4: opaque to the compiler at each use, which stops the
        // weight-to-float conversions from being hoisted out of the pair loop
        // (that would keep every converted value of the wavefront's rows live
        // at once: spills, one wavefront per SIMD); at one pair per expert
        // nothing is recomputed, and each use waits only for its own load.
        // (int4 measured faster without it.)
        if constexpr (F == MOE_FMT_FP8_E4M3_B128 || F == MOE_FMT_MXFP4_B32) {
          asm volatile("" : "+v"(wg[r][j].x), "+v"(wg[r][j].y), "+v"(wg[r][j].z), "+v"(wg[r][j].w));
          asm volatile("" : "+v"(wu[r][j].x), "+v"(wu[r][j].y), "+v"(wu[r][j].z), "+v"(wu[r][j].w));
        }
        if constexpr (F == MOE_FMT_INT4_ASYM_G128) {
          const float dg = dot1_int4(wg[r][j], xp[j]);
          const float du = dot1_int4(wu[r][j], xp[j]);
          g = fmaf(sg[r][j], dg - (zg[r][j] + 128.f) * xp[j].sum, g);
          u = fmaf(su[r][j], du - (zu[r][j] + 128.f) * xp[j].sum, u);
        } else {
          if constexpr (F == MOE_FMT_MXFP4_B32) {  // scales applied by the conversions
            const uint32_t gv[4] = {wg[r][j].x, wg[r][j].y, wg[r][j].z, wg[r][j].w};
            const uint32_t uv[4] = {wu[r][j].x, wu[r][j].y, wu[r][j].z, wu[r][j].w};
            float dg = 0.f, du = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              dg = dot_e2m1x8_scaled(gv[i], xv[j] + 8 * i, sg[r][j], dg);
              du = dot_e2m1x8_scaled(uv[i], xv[j] + 8 * i, su[r][j], du);
            }
            g += dg;
            u += du;
            continue;
          }
          float xs = 0.f;
          const float dg = dot1<F>(wg[r][j], xv[j], &xs);
          const float du = dot1<F>(wu[r][j], xv[j], &xs);
          if constexpr (F == MOE_FMT_FP8_E4M3_B128) {
            g = fmaf(dg, sg[r][j], g);
            u = fmaf(du, su[r][j], u);
          } else {
            g += dg;
            u += du;
          }
        }
      }
      g = wave_sum(g);
      u = wave_sum(u);
      if (lane == 0 && i0 + r < I) {
        const float h = g / (1.f + __expf(-g)) * u;
        a.h[(size_t)q * I + i0 + r] = h;
      }
    }
  }
}

// h rows per wavefront (up), chosen by measurement on the cache-cold batch-1
// layer (8 experts per launch): two for int4 (6.4 against 6.8 us with one),
// one for the other formats (MXFP4 7.0 against 7.2 us with two, FP8 7.24
// against 7.30).
template <int F> constexpr int rpw() {
  return F == MOE_FMT_INT4_ASYM_G128 ? 2 : 1;
}

}  // namespace gemv
}  // namespace moepage
