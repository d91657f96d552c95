// Decode-path expert FFN (few tokens per expert): weight streaming GEMVs.
//
// [PE] "What does Paged Experts actually do?": once a wave's experts are in
// their slots, the expert math runs on the GPU over the slots. [SRV]
// ("Mastering the LLM Inference Serving Engine SGLang", the prefill/decode
// discussion): batch-1 decode does about one flop per weight byte, so it is
// bound by reading the weights, and smaller weight formats read less.
//
// Two launches per wave:
//   up   : one workgroup per (expert of the wave, block of h rows). Every
//          wavefront streams RPW gate rows and RPW up rows of its expert once
//          (16-byte loads, all issued before any arithmetic), dots them with
//          the tokens routed to that expert, reduces across the wavefront and
//          writes h = SiLU(g) * u (fp32) for each (token, expert) pair.
//   down : one workgroup of 8 wavefronts per RW output rows; the wave's
//          experts are split over the wavefronts, each streaming the RW rows
//          of its experts' W_d, dotting them with h and adding w_tj * y into
//          the accumulator of token t held by lane t; the partial sums are
//          combined in LDS in a fixed order.
// Every weight byte of the wave is read from HBM exactly once; the summation
// order is fixed, so results are bitwise reproducible.
#include "copy.h"
#include "gemv_up.h"

namespace moepage {

namespace {

using namespace gemv;

template <int F, int NJ, int RPW, typename XT>
__global__ __launch_bounds__(256) void ffn_up_kernel(FfnArgs a) {
  ffn_up_body<F, NJ, RPW, XT>(a, blockIdx.x, blockIdx.y);
}

// ------------------------------------------------------------------ down
template <int F>
__device__ inline void load_w2(const uint8_t* p, uint32_t* w) {
  if constexpr (Fmt<F>::CB2 == 16) {
    const uint4 v = nt_load16(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (Fmt<F>::CB2 == 8) {
    const u32x2 v = __builtin_nontemporal_load((const u32x2*)p);
    w[0] = v.x; w[1] = v.y;
  } else {
    w[0] = __builtin_nontemporal_load((const uint32_t*)p);
  }
}

// BYTES (int4): convert the codes from even and odd nibble bytes (one
// instruction per code, two more registers) instead of one bit-field
// extract and conversion per code; the same products in the same order.
template <int F, bool BYTES>
__device__ inline float dot2(const uint32_t* w, const float* h, float* hsum) {
  float acc = 0.f;
  if constexpr (F == MOE_FMT_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(__uint_as_float(w[i]), h[i], acc);
  } else if constexpr (F == MOE_FMT_BF16) {
    acc = fmaf(bf16lo(w[0]), h[0], acc);
    acc = fmaf(bf16hi(w[0]), h[1], acc);
    acc = fmaf(bf16lo(w[1]), h[2], acc);
    acc = fmaf(bf16hi(w[1]), h[3], acc);
  } else if constexpr (F == MOE_FMT_FP8_E4M3_B128) {
    const f32x2 a = fp8x2<false>(w[0]), b = fp8x2<true>(w[0]);
    acc = fmaf(a.x, h[0], acc);
    acc = fmaf(a.y, h[1], acc);
    acc = fmaf(b.x, h[2], acc);
    acc = fmaf(b.y, h[3], acc);
  } else if constexpr (F == MOE_FMT_MXFP4_B32) {
    acc = dot_e2m1x8(w[0], h, acc);
  } else if constexpr (BYTES) {
    // int4 codes in index order (the low nibble of byte b is code 2b)
    uint32_t ev = w[0] & 0x0F0F0F0Fu, od = (w[0] >> 4) & 0x0F0F0F0Fu;
    asm("" : "+v"(ev), "+v"(od));  // keeps the byte conversions (not a bit-field extract per code)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      acc = fmaf((float)((ev >> (8 * b)) & 0xFFu), h[2 * b], acc);
      acc = fmaf((float)((od >> (8 * b)) & 0xFFu), h[2 * b + 1], acc);
    }
  } else {
#pragma unroll
    for (int n = 0; n < 8; ++n) acc = fmaf((float)((w[0] >> (4 * n)) & 0xFu), h[n], acc);
  }
  return acc;
}

// Down projection: a workgroup of 8 wavefronts owns RW output rows;
// wavefront w takes experts w, w+8, ... of the wave, keeps the per-token sums
// in lane t, and the eight partial sums are added in LDS in wavefront order
// (fixed, so the result is bitwise reproducible).
// Loads are arranged so that an expert costs no dependent round trip of its
// own: each wavefront first reads the slot and the CSR pair range of all of
// its experts (one per lane) in one round trip, and (MULTI: launches of more
// than 8 experts, several per wavefront) while it computes one expert it has
// the next one's rows, scales, first pair's h, token and router weight in
// flight. An expert's second and later pairs are read when they are reached
// (decode batches rarely have them).
template <int F, int NJ, int RW>
struct DownStage {
  uint32_t w[RW][NJ][Fmt<F>::CB2 / 4];  // the expert's RW rows of W_d, chunk lane + 64 j
  // scales of chunk lane + 64 j, kept as stored: FP8, the fp32 block scale
  // (row 0's entry: the RW rows share a 128-row block); int4, the fp16 scale
  // (low half) and zero point (high half) of row r's group; MXFP4, row r's
  // E8M0 byte
  uint32_t sc[RW][NJ];
  float hv[NJ][Fmt<F>::CV2];            // h of the pair being computed (first: the expert's first)
  int t;                                // that pair's token
  float wq;                             // and its router weight
};

template <int F, int NJ, int RW, bool MULTI>
__device__ __forceinline__ void ffn_down_body(const FfnArgs& a, int bx) {
  constexpr int CB2 = Fmt<F>::CB2, CV2 = Fmt<F>::CV2, NW = CB2 / 4;
  static_assert(128 % RW == 0, "a workgroup's rows lie in one 128-row block");
  using Stage = DownStage<F, NJ, RW>;
  __shared__ float part[8][kWave][RW];
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int H = a.H, I = a.I;
  const int r0 = bx * RW;
  const RecLayout L = rec_layout(F, H, I);
  const int nch = I / CV2;
  const size_t row_bytes = (size_t)I * fmt_elem_bits(F) / 8;
  float acc[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) acc[r] = 0.f;
  const int T = a.T;

  // h, token and router weight of CSR position q
  auto load_pair = [&](int q, float (&hv)[NJ][CV2], int& t, float& wq) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = lane + kWave * j;
      if (c < nch) {
#pragma unroll
        for (int v = 0; v < CV2; v += 4) {
          const float4 f = *(const float4*)(a.h + (size_t)q * I + c * CV2 + v);
          hv[j][v] = f.x; hv[j][v + 1] = f.y; hv[j][v + 2] = f.z; hv[j][v + 3] = f.w;
        }
      } else {
#pragma unroll
        for (int v = 0; v < CV2; ++v) hv[j][v] = 0.f;
      }
    }
    t = T == 1 ? 0 : a.pair_list[q] / a.k;  // one token: every pair is token 0's
    wq = a.pair_w[q];
  };
  // everything an expert's first pair needs, from its slot and CSR position
  auto load_stage = [&](int slot, int p0, Stage& s) {
    const uint8_t* rec = a.slots + (size_t)slot * a.stride;
    const uint8_t* wd = rec + L.wd;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int row = min(r0 + r, H - 1);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = lane + kWave * j;
        if (c < nch) load_w2<F>(wd + (size_t)row * row_bytes + (size_t)c * CB2, s.w[r][j]);
        else {
#pragma unroll
          for (int n = 0; n < NW; ++n) s.w[r][j][n] = 0u;
        }
      }
    }
    if constexpr (F == MOE_FMT_FP8_E4M3_B128) {
      const uint32_t* sd = (const uint32_t*)(rec + L.sd);
      const int nb = I / 128;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = min(lane + kWave * j, nch - 1);
        s.sc[0][j] = sd[(min(r0, H - 1) / 128) * nb + (c * CV2) / 128];
      }
    } else if constexpr (F == MOE_FMT_INT4_ASYM_G128) {
      const uint16_t* sd = (const uint16_t*)(rec + L.sd);
      const uint16_t* zd = (const uint16_t*)(rec + L.zd);
      const int ng = I / 128;
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int g = min(lane + kWave * j, nch - 1) * CV2 / 128;
          const size_t row = (size_t)min(r0 + r, H - 1);
          s.sc[r][j] = (uint32_t)sd[row * ng + g] | ((uint32_t)zd[row * ng + g] << 16);
        }
    } else if constexpr (F == MOE_FMT_MXFP4_B32) {
      const uint8_t* sd = rec + L.sd;  // one scale byte per 32 weights = 4 chunks
      const int nb = I / 32;
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int c = min(lane + kWave * j, nch - 1);
          s.sc[r][j] = sd[(size_t)min(r0 + r, H - 1) * nb + (c * CV2) / 32];
        }
    }
    load_pair(p0, s.hv, s.t, s.wq);
  };
  // one pair: the RW rows dotted with its h, reduced over the wavefront and
  // added, times the router weight, into token t's lane
  auto do_pair = [&](Stage& s) {
    float hsum[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      hsum[j] = 0.f;
      if constexpr (F == MOE_FMT_INT4_ASYM_G128) {
#pragma unroll
        for (int v = 0; v < CV2; ++v) hsum[j] += s.hv[j][v];
      }
    }
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      float y = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const float hs = hsum[j];
        float unused = 0.f;
#pragma unroll
        for (int n = 0; n < NW; ++n)  // no hoisting of conversions (as in the up kernel)
          asm volatile("" : "+v"(s.w[r][j][n]));
        if constexpr (F == MOE_FMT_MXFP4_B32) {  // the scale applied by the conversions
          y += dot_e2m1x8_scaled(s.w[r][j][0], s.hv[j], e8m0_to_float((uint8_t)s.sc[r][j]), 0.f);
          continue;
        }
        const float d = dot2<F, !MULTI>(s.w[r][j], s.hv[j], &unused);  // the prefetching variant keeps its registers
        if constexpr (F == MOE_FMT_FP8_E4M3_B128) {
          y = fmaf(d, __uint_as_float(s.sc[0][j]), y);
        } else if constexpr (F == MOE_FMT_INT4_ASYM_G128) {
          const float sv = half_to_float((uint16_t)s.sc[r][j]), zv = half_to_float((uint16_t)(s.sc[r][j] >> 16));
          y = fmaf(sv, d - zv * hs, y);
        } else {
          y += d;
        }
      }
      y = wave_sum(y);
      if (lane == s.t) acc[r] = fmaf(s.wq, y, acc[r]);
    }
  };

  // Expert i of this wavefront (wave-order position o_lo + wid + 8 i): its
  // slot and CSR pair range [p0, p1) in lane i % 64 of register i / 64 (a
  // wave holds at most MOE_MAX_EXPERTS = 1024 experts, 128 per wavefront).
  // Positions are clamped into the launch's range, whose entries the arrays
  // hold; the values of positions past the step's last expert are never
  // used. One token: expert o's one pair is at o.
  const int pos_max = max(min(a.o_lo + a.n_exp, a.E) - 1, 0);
  int m_slot[2] = {0, 0}, m_p0[2] = {0, 0}, m_p1[2] = {0, 0};
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (c == 1 && a.n_exp <= 8 * kWave) break;  // uniform
    const int pos = min(a.o_lo + wid + 8 * (c * kWave + lane), pos_max);
    m_slot[c] = a.order_slot[pos];
    if (T == 1) {
      m_p0[c] = pos;
      m_p1[c] = pos + 1;
    } else {
      m_p0[c] = a.pair_off[pos];
      m_p1[c] = a.pair_off[pos + 1];
    }
  }
  auto meta = [&](const int (&m)[2], int i) {
    return __builtin_amdgcn_readlane((i >> 6) ? m[1] : m[0], i & (kWave - 1));
  };
  // The final value of each (token, row) this thread stores (at most one: T *
  // RW <= 256 < 512 threads): its previous out and x_res values are loaded now,
  // so their latency overlaps the weight stream instead of ending the kernel.
  const int my_t = threadIdx.x / RW, my_r = threadIdx.x % RW;
  const bool mine = (int)threadIdx.x < T * RW && r0 + my_r < H;
  // device-resolved steps: the step's distinct experts D, read on the device
  // (in the same round trip as the metadata above)
  const int D = a.n_dev ? *a.n_dev : a.o_lo + a.n_exp;
  const bool res = a.x_res && (!a.res_last || (a.o_lo < D && D <= a.o_lo + a.n_exp));
  float o_prev = 0.f;
  uint32_t x_prev = 0;
  if (mine) {
    if (a.accumulate) o_prev = a.out[(size_t)my_t * H + r0 + my_r];
    if (res) x_prev = a.x_res[(size_t)my_t * H + r0 + my_r];
  }
  const int n_exp = min(a.n_exp, D - a.o_lo);  // none past the step's last expert
  Stage cur, nxt;
  if (wid < n_exp) load_stage(meta(m_slot, 0), meta(m_p0, 0), cur);
  int i = 0;
  for (int e = wid; e < n_exp; e += 8, ++i) {
    const int p0 = meta(m_p0, i), p1 = meta(m_p1, i);
    if (MULTI && e + 8 < n_exp) load_stage(meta(m_slot, i + 1), meta(m_p0, i + 1), nxt);
    if (p1 > p0) do_pair(cur);
    for (int q = p0 + 1; q < p1; ++q) {  // later pairs, into the first's registers
      load_pair(q, cur.hv, cur.t, cur.wq);
      do_pair(cur);
    }
    if (!MULTI) break;  // the launch holds at most 8 experts: one per wavefront
    if (e + 8 < n_exp) cur = nxt;
  }
#pragma unroll
  for (int r = 0; r < RW; ++r) part[wid][lane][r] = acc[r];
  __syncthreads();
  if (mine) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) v += part[w][my_t][my_r];
    const float ov = o_prev + v;
    a.out[(size_t)my_t * H + r0 + my_r] = ov;
    if (res) {  // stack residual on the final value of out
      // x_prev passes through an empty asm here, at its use, so that the
      // compiler cannot widen it next to its load, which would make this
      // wavefront wait for that load before it issues its weight loads
      uint32_t xp = x_prev;
      asm volatile("" : "+v"(xp));
      a.x_res[(size_t)my_t * H + r0 + my_r] = f32_to_bf16_rne(__uint_as_float(xp << 16) + ov);
    }
  }
}

template <int F, int NJ, int RW, bool MULTI>
__global__ __launch_bounds__(512) void ffn_down_kernel(FfnArgs a) {
  ffn_down_body<F, NJ, RW, MULTI>(a, blockIdx.x);
}

// The down launch of a stack step with lookahead: workgroups 0 .. kCopyBlocks-1
// copy bytes [n.cp_len, n.stride) of every record the next layer's plan (its
// wave order and counts, stored by the up launch before) pages in, the others
// run this layer's down projection exactly as ffn_down_kernel does.
constexpr int kCopyBlocks = 64;

template <int F, int NJ, int RW, bool MULTI>
__global__ __launch_bounds__(512) void down_copy_next_kernel(FfnArgs a, NextStep n) {
  const int b = blockIdx.x;
  if (b < kCopyBlocks) {
    const int D = n.dev.counts[0], nH = n.dev.counts[1];
    for (int m = nH; m < D; ++m) {
      const int e = n.dev.order_expert[m], sl = n.dev.order_slot[m];
      if (e < 0 || e >= n.E || sl < 0 || sl >= n.K) continue;  // never produced by the plan
      copy_record_share<512, 4>(n.host + (size_t)e * n.stride + n.cp_len, n.slots + (size_t)sl * n.stride + n.cp_len,
                                n.stride - n.cp_len, b, kCopyBlocks);
    }
    return;
  }
  ffn_down_body<F, NJ, RW, MULTI>(a, b - kCopyBlocks);
}

// output rows per down workgroup, chosen by measurement
template <int F> constexpr int rw() { return 4; }  // measured: 4 rows beat 8 and 16 for every format, and 2 for bf16

template <int F, typename XT>
hipError_t up_dispatch(const FfnArgs& a, hipStream_t s) {
  constexpr int kRPW = rpw<F>();
  const int nj = (a.H / Fmt<F>::CV1 + kWave - 1) / kWave;
  const dim3 grid((a.I + 4 * kRPW - 1) / (4 * kRPW), a.n_exp), block(256);
  switch (nj) {
    case 1: launch_k(ffn_up_kernel<F, 1, kRPW, XT>, grid, block, s, a.ev0, a.ev1, a); break;
    case 2: launch_k(ffn_up_kernel<F, 2, kRPW, XT>, grid, block, s, a.ev0, a.ev1, a); break;
    case 3: launch_k(ffn_up_kernel<F, 3, kRPW, XT>, grid, block, s, a.ev0, a.ev1, a); break;
    case 4: launch_k(ffn_up_kernel<F, 4, kRPW, XT>, grid, block, s, a.ev0, a.ev1, a); break;
    case 6: launch_k(ffn_up_kernel<F, 6, kRPW, XT>, grid, block, s, a.ev0, a.ev1, a); break;
    case 8: launch_k(ffn_up_kernel<F, 8, kRPW, XT>, grid, block, s, a.ev0, a.ev1, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The down kernels come in two variants: launches of at most 8 experts (one
// per wavefront: no prefetch of a next expert, fewer registers) and larger ones.
template <int F, bool MULTI>
hipError_t down_copy_dispatch_m(const FfnArgs& a, const NextStep& n, hipStream_t s) {
  constexpr int kRW = rw<F>();
  const int nj = (a.I / Fmt<F>::CV2 + kWave - 1) / kWave;
  const dim3 grid(kCopyBlocks + (a.H + kRW - 1) / kRW), block(512);
  switch (nj) {
    case 1: launch_k(down_copy_next_kernel<F, 1, kRW, MULTI>, grid, block, s, a.ev0, a.ev1, a, n); break;
    case 2: launch_k(down_copy_next_kernel<F, 2, kRW, MULTI>, grid, block, s, a.ev0, a.ev1, a, n); break;
    case 3: launch_k(down_copy_next_kernel<F, 3, kRW, MULTI>, grid, block, s, a.ev0, a.ev1, a, n); break;
    case 4: launch_k(down_copy_next_kernel<F, 4, kRW, MULTI>, grid, block, s, a.ev0, a.ev1, a, n); break;
    case 6: launch_k(down_copy_next_kernel<F, 6, kRW, MULTI>, grid, block, s, a.ev0, a.ev1, a, n); break;
    case 8: launch_k(down_copy_next_kernel<F, 8, kRW, MULTI>, grid, block, s, a.ev0, a.ev1, a, n); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
template <int F>
hipError_t down_copy_dispatch(const FfnArgs& a, const NextStep& n, hipStream_t s) {
  return a.n_exp > 8 ? down_copy_dispatch_m<F, true>(a, n, s) : down_copy_dispatch_m<F, false>(a, n, s);
}

template <int F, bool MULTI>
hipError_t down_dispatch_m(const FfnArgs& a, hipStream_t s) {
  constexpr int kRW = rw<F>();
  const int nj = (a.I / Fmt<F>::CV2 + kWave - 1) / kWave;
  const dim3 grid((a.H + kRW - 1) / kRW), block(512);
  switch (nj) {
    case 1: launch_k(ffn_down_kernel<F, 1, kRW, MULTI>, grid, block, s, a.ev0, a.ev1, a); break;
    case 2: launch_k(ffn_down_kernel<F, 2, kRW, MULTI>, grid, block, s, a.ev0, a.ev1, a); break;
    case 3: launch_k(ffn_down_kernel<F, 3, kRW, MULTI>, grid, block, s, a.ev0, a.ev1, a); break;
    case 4: launch_k(ffn_down_kernel<F, 4, kRW, MULTI>, grid, block, s, a.ev0, a.ev1, a); break;
    case 6: launch_k(ffn_down_kernel<F, 6, kRW, MULTI>, grid, block, s, a.ev0, a.ev1, a); break;
    case 8: launch_k(ffn_down_kernel<F, 8, kRW, MULTI>, grid, block, s, a.ev0, a.ev1, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
template <int F>
hipError_t down_dispatch(const FfnArgs& a, hipStream_t s) {
  return a.n_exp > 8 ? down_dispatch_m<F, true>(a, s) : down_dispatch_m<F, false>(a, s);
}

// ------------------------------------------------------------------ dequant
// Prefill with quantised experts: the wave's records are expanded once into
// bf16 records (the bf16 format's layout) that the grouped MFMA GEMMs read.
// Each thread writes 8 consecutive bf16 values of one row (16 bytes), the
// dequantised weight rounded to nearest even; the formats' decodings are
// those of the GEMV kernels above.
template <int F>
__device__ inline void decode8(const uint8_t* rec, const RecLayout& L, bool up, int r, int c, int H, int I,
                               float* v) {
  const int cols = up ? H : I;
  if constexpr (F == MOE_FMT_FP8_E4M3_B128) {
    const uint2 q = *(const uint2*)(rec + (up ? L.w13 : L.wd) + (size_t)r * cols + (size_t)c * 8);
    const float s = ((const float*)(rec + (up ? L.s13 : L.sd)))[(r / 128) * (cols / 128) + (c * 8) / 128];
    const f32x2 a = fp8x2<false>(q.x), b = fp8x2<true>(q.x), d = fp8x2<false>(q.y), e = fp8x2<true>(q.y);
    v[0] = a.x * s; v[1] = a.y * s; v[2] = b.x * s; v[3] = b.y * s;
    v[4] = d.x * s; v[5] = d.y * s; v[6] = e.x * s; v[7] = e.y * s;
  } else {
    const uint32_t w = *(const uint32_t*)(rec + (up ? L.w13 : L.wd) + (size_t)r * (cols / 2) + (size_t)c * 4);
    if constexpr (F == MOE_FMT_INT4_ASYM_G128) {
      const size_t g = (size_t)r * (cols / 128) + (c * 8) / 128;
      const float s = half_to_float(((const uint16_t*)(rec + (up ? L.s13 : L.sd)))[g]);
      const float z = half_to_float(((const uint16_t*)(rec + (up ? L.z13 : L.zd)))[g]);
#pragma unroll
      for (int n = 0; n < 8; ++n) v[n] = ((float)((w >> (4 * n)) & 0xFu) - z) * s;
    } else {  // MXFP4
      const float s = e8m0_to_float((rec + (up ? L.s13 : L.sd))[(size_t)r * (cols / 32) + (c * 8) / 32]);
      uint32_t ev, od;
      e2m1x8_to_e4m3(w, &ev, &od);
      const f32x2 a = fp8x2<false>(ev), b = fp8x2<true>(ev), d = fp8x2<false>(od), e = fp8x2<true>(od);
      v[0] = a.x * s; v[1] = d.x * s; v[2] = a.y * s; v[3] = d.y * s;
      v[4] = b.x * s; v[5] = e.x * s; v[6] = b.y * s; v[7] = e.y * s;
    }
  }
}

constexpr int kDqBlocks = 64;  // workgroups per expert (grid-stride over its rows)

template <int F>
__global__ __launch_bounds__(256) void dequant_bf16_kernel(FfnArgs a, uint8_t* dst, size_t dst_stride) {
  const int o = a.o_lo + blockIdx.y;
  const int H = a.H, I = a.I;
  const uint8_t* rec = a.slots + (size_t)a.order_slot[o] * a.stride;
  uint16_t* out = (uint16_t*)(dst + (size_t)blockIdx.y * dst_stride);
  const RecLayout L = rec_layout(F, H, I);
  const size_t n13 = (size_t)2 * I * (H / 8), n = n13 + (size_t)H * (I / 8);
  for (size_t w = (size_t)blockIdx.x * 256 + threadIdx.x; w < n; w += (size_t)gridDim.x * 256) {
    const bool up = w < n13;
    const size_t ww = up ? w : w - n13;
    const int cpr = (up ? H : I) / 8;  // 8-value chunks per row
    const int r = (int)(ww / cpr), c = (int)(ww % cpr);
    float v[8];
    decode8<F>(rec, L, up, r, c, H, I, v);
    uint4 q;
    q.x = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
    q.y = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
    q.z = (uint32_t)f32_to_bf16_rne(v[4]) | ((uint32_t)f32_to_bf16_rne(v[5]) << 16);
    q.w = (uint32_t)f32_to_bf16_rne(v[6]) | ((uint32_t)f32_to_bf16_rne(v[7]) << 16);
    *(uint4*)(out + (up ? (size_t)0 : (size_t)2 * I * H) + (size_t)r * (up ? H : I) + (size_t)c * 8) = q;
  }
}

int nj_of(int n) {
  const int nj = (n + kWave - 1) / kWave;
  return (nj == 1 || nj == 2 || nj == 3 || nj == 4 || nj == 6 || nj == 8) ? nj : 0;
}

}  // namespace

bool ffn_shape_supported(int fmt, int H, int I) {
  if (H <= 0 || I <= 0) return false;
  int cv1 = 0, cv2 = 0;
  switch (fmt) {
    case MOE_FMT_F32: cv1 = 4; cv2 = 4; break;
    case MOE_FMT_BF16: cv1 = 8; cv2 = 4; break;
    case MOE_FMT_FP8_E4M3_B128: cv1 = 16; cv2 = 4; break;
    case MOE_FMT_INT4_ASYM_G128: cv1 = 32; cv2 = 8; break;
    case MOE_FMT_MXFP4_B32: cv1 = 32; cv2 = 8; break;
    default: return false;
  }
  if (fmt == MOE_FMT_FP8_E4M3_B128 || fmt == MOE_FMT_INT4_ASYM_G128) {
    if (H % 128 || I % 128) return false;
  }
  if (fmt == MOE_FMT_MXFP4_B32 && (H % 32 || I % 32)) return false;  // whole scale blocks
  if (H % cv1 || I % cv2) return false;
  return nj_of(H / cv1) && nj_of(I / cv2);
}

hipError_t launch_ffn_up(const FfnArgs& a, hipStream_t s) {
  if (a.n_exp <= 0) return hipSuccess;
  switch (a.fmt) {
    case MOE_FMT_F32: return up_dispatch<MOE_FMT_F32, float>(a, s);
    case MOE_FMT_BF16: return up_dispatch<MOE_FMT_BF16, uint16_t>(a, s);
    case MOE_FMT_FP8_E4M3_B128: return up_dispatch<MOE_FMT_FP8_E4M3_B128, uint16_t>(a, s);
    case MOE_FMT_INT4_ASYM_G128: return up_dispatch<MOE_FMT_INT4_ASYM_G128, uint16_t>(a, s);
    case MOE_FMT_MXFP4_B32: return up_dispatch<MOE_FMT_MXFP4_B32, uint16_t>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dequant_bf16(const FfnArgs& a, uint8_t* dst, size_t dst_stride, hipStream_t s) {
  if (a.n_exp <= 0) return hipSuccess;
  const dim3 grid(kDqBlocks, a.n_exp), block(256);
  switch (a.fmt) {
    case MOE_FMT_FP8_E4M3_B128: launch_k(dequant_bf16_kernel<MOE_FMT_FP8_E4M3_B128>, grid, block, s, a.ev0, a.ev1, a, dst, dst_stride); break;
    case MOE_FMT_INT4_ASYM_G128: launch_k(dequant_bf16_kernel<MOE_FMT_INT4_ASYM_G128>, grid, block, s, a.ev0, a.ev1, a, dst, dst_stride); break;
    case MOE_FMT_MXFP4_B32: launch_k(dequant_bf16_kernel<MOE_FMT_MXFP4_B32>, grid, block, s, a.ev0, a.ev1, a, dst, dst_stride); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_ffn_down_copy_next(const FfnArgs& a, const NextStep& n, hipStream_t s) {
  if (n.cp_len > n.stride || (n.cp_len & 15)) return hipErrorInvalidValue;
  switch (a.fmt) {
    case MOE_FMT_BF16: return down_copy_dispatch<MOE_FMT_BF16>(a, n, s);
    case MOE_FMT_FP8_E4M3_B128: return down_copy_dispatch<MOE_FMT_FP8_E4M3_B128>(a, n, s);
    case MOE_FMT_INT4_ASYM_G128: return down_copy_dispatch<MOE_FMT_INT4_ASYM_G128>(a, n, s);
    case MOE_FMT_MXFP4_B32: return down_copy_dispatch<MOE_FMT_MXFP4_B32>(a, n, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_ffn_down(const FfnArgs& a, hipStream_t s) {
  switch (a.fmt) {
    case MOE_FMT_F32: return down_dispatch<MOE_FMT_F32>(a, s);
    case MOE_FMT_BF16: return down_dispatch<MOE_FMT_BF16>(a, s);
    case MOE_FMT_FP8_E4M3_B128: return down_dispatch<MOE_FMT_FP8_E4M3_B128>(a, s);
    case MOE_FMT_INT4_ASYM_G128: return down_dispatch<MOE_FMT_INT4_ASYM_G128>(a, s);
    case MOE_FMT_MXFP4_B32: return down_dispatch<MOE_FMT_MXFP4_B32>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moepage
