// Prefill-path expert FFN (many tokens per expert): token-grouped bf16 GEMMs
// on the gfx950 matrix cores, then a deterministic weighted combine.
//
// [PE] ("Running an MoE Model Larger Than Your VRAM: SGLang Paged Experts, the
// PCIe Math, and the 4-Request Cliff"), "Why do short prompts get slower first
// tokens?": a prefill touches nearly every expert; its expert math runs over
// the slots like decode, but with many tokens per expert, so it is a grouped
// matrix product rather than a matrix-vector product. [SRV] ("Mastering the LLM
// Inference Serving Engine SGLang", prefill vs decode): prefill multiplies a
// large activation matrix by the weights.
//
// Per wave of the plan, for every expert e of the wave with M_e routed pairs
// (rows grouped by the plan's CSR lists):
//   up   : C = X_e (M_e x H, gathered token rows) * W13^T; h = SiLU(C[:, :I]) *
//          C[:, I:] in fp32, stored as a pair of bf16 arrays h_hi = bf16(h),
//          h_lo = bf16(h - h_hi), so that h keeps about 16 significant bits
//   down : Y = h_hi * W_d^T + h_lo * W_d^T (M_e x I times I x H, both on the
//          matrix cores against the same weight fragments);
//          y[pair] = w_pair * Y (fp32 [pair][H])
//   combine: out[t] (+)= sum over j in 0..k-1 of y[pair (t, j)] for the pairs
//          of this wave, j ascending (fixed order -> bitwise reproducible)
//
// Tiling (v_mfma_f32_16x16x32_bf16, 64-wide wavefronts). A workgroup of eight
// wavefronts, one per CU, owns one expert and 256 weight rows (up: 128 gate
// rows and the 128 matching up rows of W13; down: 256 rows of W_d) and covers
// up to 256 of the expert's rows per pass, so each weight byte leaves HBM
// once per expert for all but the hottest experts, and each activation row is
// copied once per 256 weight rows. The k loop runs in steps of 64 (up) or 32
// (down). Each step's weight tile (256 x 64 or 256 x 32) and activation
// tile(s) are filled by direct global-to-LDS copies (no register staging) into
// two LDS rings: the weight ring, fed from HBM, runs 2 to 6 steps ahead of the
// matrix cores; the activation ring, mostly fed from L2, 1 or 2 steps ahead.
// A wait on the vector-memory counter plus a barrier hands a step over. Only
// the 64-row groups that hold routed rows are copied (template RG; the down
// GEMM rounds up to an even count). The
// 16-byte chunks of a tile row are XOR-swizzled by row (see lds_chunk), which
// makes the fragment reads free of LDS bank conflicts; the swizzle is applied
// by choosing each copy lane's source chunk, since one copy instruction
// writes its 64 lanes contiguously.
// The eight wavefronts form a 2 x 4 grid: wavefront (wm, wn) takes the 16-row
// sub-tiles with index = wm (mod 2) and 64 of the output columns (up: h
// columns wn*32 .. wn*32+31 from their gate and up rows; down: wn*64 ..).
// Workgroups are numbered so that each XCD (which schedules every eighth
// workgroup and has its own L2) works through a contiguous run of experts,
// keeping an expert's activation rows in one L2.
#include "gemv_up.h"
#include "internal.h"

namespace moepage {

namespace {

constexpr int kWave = 64;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kThreads = 512;              // eight wavefronts per workgroup
constexpr int BN = 256;                    // weight rows per workgroup
constexpr int UP_HCOLS = BN / 2;           // h columns per workgroup (up)
constexpr int DN_COLS = BN;                // output columns per workgroup (down)
constexpr int kXcd = 8;                    // XCDs; consecutive workgroups go round-robin over them

__device__ inline bf16x8 as_bf16x8(const uint4& v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Eight e4m3 weights (one B fragment's k-run) to bf16 operands: each exact in
// fp32, times its block scale in fp32, rounded to nearest even.
__device__ inline bf16x8 fp8x8_to_bf16(uint2 q, float s) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.x, false), b = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.x, true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.y, false), d = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.y, true);
  bf16x8 r;
  r[0] = (__bf16)(a.x * s); r[1] = (__bf16)(a.y * s); r[2] = (__bf16)(b.x * s); r[3] = (__bf16)(b.y * s);
  r[4] = (__bf16)(c.x * s); r[5] = (__bf16)(c.y * s); r[6] = (__bf16)(d.x * s); r[7] = (__bf16)(d.y * s);
  return r;
}

// Eight E2M1 codes (one word, code 2b in the low nibble of byte b) to bf16
// operands: each code times the block's E8M0 scale s = 2^(e - 127), by
// gfx950's scaled conversion (selector b converts byte b, low nibble first,
// times 2 to the exponent of s). A code has at most two significant bits, so
// the product is exact in bf16: the same values as the expansion of MXFP4
// records (exact product in fp32, rounded to nearest even).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ inline bf16x8 fp4x8_to_bf16(uint32_t q, float s) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 0);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 1);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 2);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 3);
  bf16x8 r;
  r[0] = a.x; r[1] = a.y; r[2] = b.x; r[3] = b.y;
  r[4] = c.x; r[5] = c.y; r[6] = d.x; r[7] = d.y;
  return r;
}

// Eight int4 codes (one word, code 2b in the low nibble of byte b) of one
// 128-group to bf16 operands: (q - z) * s in fp32 with the group's fp16 scale
// and zero point (exact in fp32), rounded to nearest even; the same arithmetic
// as the decode kernels' expansion of int4 records.
__device__ inline bf16x8 int4x8_to_bf16(uint32_t q, float s, float z) {
  const uint32_t ev = q & 0x0F0F0F0Fu, od = (q >> 4) & 0x0F0F0F0Fu;
  bf16x8 r;
  r[0] = (__bf16)(((float)(ev & 0xFFu) - z) * s);
  r[1] = (__bf16)(((float)(od & 0xFFu) - z) * s);
  r[2] = (__bf16)(((float)((ev >> 8) & 0xFFu) - z) * s);
  r[3] = (__bf16)(((float)((od >> 8) & 0xFFu) - z) * s);
  r[4] = (__bf16)(((float)((ev >> 16) & 0xFFu) - z) * s);
  r[5] = (__bf16)(((float)((od >> 16) & 0xFFu) - z) * s);
  r[6] = (__bf16)(((float)((ev >> 24) & 0xFFu) - z) * s);
  r[7] = (__bf16)(((float)((od >> 24) & 0xFFu) - z) * s);
  return r;
}

__device__ inline uint16_t f32_to_bf16_rne(float v) {
  uint32_t b = __float_as_uint(v);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// Tile rows of CPR 16-byte chunks (CPR = 4: 32 bf16 per row, CPR = 8: 64;
// CPR = 2: 32 FP8 or 64 FP4 weights per row).
// LDS chunk of logical chunk c of tile row r; and, for LDS chunk p, the
// logical chunk it holds (its row is p / CPR): the two are inverse of each
// other. The XOR spreads the rows that one fragment read touches over the
// banks (CPR = 2: rows 8..15 of a sub-tile hold their two chunks swapped).
template <int CPR>
__device__ inline int lds_chunk(int r, int c) {
  if constexpr (CPR == 2) return r * 2 + (c ^ ((r >> 3) & 1));
  else if constexpr (CPR == 4) return r * 4 + (c ^ ((r >> 1) & 3));
  else return r * 8 + (c ^ (r & 7));
}
template <int CPR>
__device__ inline int src_chunk(int p) {
  if constexpr (CPR == 2) return (p & 1) ^ ((p >> 4) & 1);
  else if constexpr (CPR == 4) return (p & 3) ^ ((p >> 3) & 3);
  else return (p & 7) ^ ((p >> 3) & 7);
}

// Global-to-LDS copy of 16 bytes per lane: lane l's bytes land at LDS byte
// address lds + 16 * l (lds wave-uniform, passed in M0). Issued from inline
// assembly so that the compiler neither waits for it before every LDS read nor
// counts it: the pipeline below does its own waiting on the vector-memory
// counter. M0 is saved and restored around the copy (the compiler reserves it).
// NT: a streaming (non-temporal) read, for weights that are read once.
template <bool NT = false>
__device__ inline void dma16(const void* src, uint32_t lds) {
  uint32_t save;
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off nt\n\ts_mov_b32 m0, %0"
        : "=&s"(save)
        : "v"(src), "s"(lds)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
        : "=&s"(save)
        : "v"(src), "s"(lds)
        : "memory");
}

__device__ inline uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(const lds_void_t*)p);
}

// Stage hand-over: this wavefront's copies, except the newest N, have landed
// in LDS (copies complete in issue order), its LDS reads are done, and every
// wavefront of the workgroup has got this far.
template <int N>
__device__ inline void stage_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

// Two LDS rings per pass with RG 64-row groups (RG = 2 or 4). The weight tile
// of a k-step comes from HBM and the activation tile(s) mostly from L2, so the
// weight ring runs deeper (SW stages) than the activation ring (SA stages) to
// keep enough HBM bytes in flight. One workgroup per CU owns the 160 KB LDS.
// The up GEMM (k = H) runs k-steps of 64, so that every copy instruction moves
// whole 128-byte lines (8 rows); the down GEMM (k = I, two activation tiles)
// keeps k-steps of 32 to fit its rings.
// WF: the weight tile's format in LDS. bf16 weights (MOE_FMT_BF16) are read
// as MFMA operands directly; FP8 e4m3 weights (MOE_FMT_FP8_E4M3_B128) reach LDS
// at one byte each and become bf16 operands in registers, each weight times
// its 128 x 128 block scale in fp32, rounded to nearest even (the same bf16
// values as an expanded bf16 record).
// MXFP4 weights (MOE_FMT_MXFP4_B32) and int4 weights (MOE_FMT_INT4_ASYM_G128)
// reach LDS at half a byte each, and the tile's scale rows are copied to an
// LDS region once per workgroup: MXFP4, one E8M0 byte per 32 reduction
// elements of a row (each weight becomes its value times 2^(scale - 127) in
// fp32); int4, the row's fp16 scales then its fp16 zero points, one each per
// 128-group (each weight becomes (q - z) * s in fp32); either way rounded to
// nearest even. Both take KD / 32 bytes per row; the scale region holds up to
// 64 bytes per row for the up GEMM and 32 for the down GEMM (H <= 2048, I <=
// 1024); larger shapes read expanded bf16 copies.
template <int WF> struct WBits { static constexpr int B = 16; };
template <> struct WBits<MOE_FMT_FP8_E4M3_B128> { static constexpr int B = 8; };
template <> struct WBits<MOE_FMT_MXFP4_B32> { static constexpr int B = 4; };
template <> struct WBits<MOE_FMT_INT4_ASYM_G128> { static constexpr int B = 4; };
constexpr int kQ4ScRowUp = 64, kQ4ScRowDn = 32;  // scale-region bytes per tile row

template <bool UP, int WF = MOE_FMT_BF16>
struct Tiles {
  static constexpr bool Q4 = WF == MOE_FMT_MXFP4_B32 || WF == MOE_FMT_INT4_ASYM_G128;  // 4-bit weights
  static constexpr int NA = UP ? 1 : 2;  // activation tiles: x, or (h_hi, h_lo)
  // the down GEMM's k-steps are 32 wide (two activation tiles per stage),
  // except with 4-bit weights, whose 32-wide tile rows would be 16 bytes
  static constexpr int BK = (UP || Q4) ? 64 : 32;  // reduction elements per k-step
  static constexpr int CPR = BK / 8;       // 16-byte chunks per activation tile row
  static constexpr int WBITS = WBits<WF>::B;  // bits per weight
  static constexpr int CPRW = BK * WBITS / 128;  // 16-byte chunks per weight tile row
  static constexpr int W_CH = BN * CPRW;   // chunks of the weight tile
  static constexpr int NW = W_CH / kThreads;  // weight copies per thread per stage
  static_assert(NW >= 1 && W_CH % kThreads == 0, "whole weight copies per thread");
  static constexpr int SC_ROW = Q4 ? (UP ? kQ4ScRowUp : kQ4ScRowDn) : 0;
  static constexpr int SC_CH = BN * SC_ROW / 16;  // the 4-bit formats' scale region, after the rings
  static constexpr int BUDGET_CH = 160 * 1024 / 16 - SC_CH;  // for the two rings
};
template <bool UP, int RG, int WF = MOE_FMT_BF16>
struct Ring {
  static constexpr int W_CH = Tiles<UP, WF>::W_CH;
  static constexpr int A_CH = Tiles<UP, WF>::NA * RG * 64 * Tiles<UP, WF>::CPR;  // activation chunks per stage
  static constexpr int SW3 = (Tiles<UP, WF>::BUDGET_CH - 3 * A_CH) / W_CH;
  static constexpr int SA = SW3 > 3 ? 3 : 2;
  static constexpr int SW_FIT = (Tiles<UP, WF>::BUDGET_CH - SA * A_CH) / W_CH;
  static constexpr int SW = SW_FIT > 8 ? 8 : SW_FIT;
  static_assert(SW > SA && SA >= 2, "LDS budget too small for the two rings");
};

// Weight-tile row of B fragment n for this lane. up: h columns wn*32 +
// (n%2)*16 .. (gate rows for n < 2, the matching up rows 128 further down the
// tile for n >= 2); down: columns wn*64 + n*16 ..
template <bool UP>
__device__ inline int frag_row(int n, int wn, int lane) {
  return UP ? ((n < 2 ? 0 : UP_HCOLS) + wn * 32 + (n & 1) * 16 + (lane & 15)) : (wn * 64 + n * 16 + (lane & 15));
}

// Weight copies as streaming reads: measured on the all-resident 2048-token
// layer, they shorten the bf16 up GEMM (180 -> 170 us) but lengthen the down
// GEMM (173 -> 197 us) and every quantised format's GEMMs, so only the bf16
// up GEMM takes them.
template <bool UP, int WF>
constexpr bool kNtWeights = UP && WF == MOE_FMT_BF16;

// One pass over rows [mb, mb + mcnt) of expert position o, mcnt <= 64 * RG.
// Copies are issued per k-step as [activation stage it + SA - 1][weight stage
// it + SW - 1]; since SW > SA, the activation copy of a stage is issued after
// its weight copy, so "stage it has landed" is "all copies up to the
// activation copy of stage it have completed" (copies complete in order).
// wsrc: byte addresses of this thread's weight copies of k-step 0. FP8
// weights: sc0 (up: the gate rows' block row of scales; down: this
// wavefront's) and sc1 (up: the up rows') point at the block-scale rows of
// this tile, one float per 128 reduction elements. 4-bit weights: the scales
// (and int4 zero points) are in the LDS scale region, row r of the weight
// tile at byte r * SC_ROW.
template <bool UP, int RG, int WF>
__device__ void gemm_pass(const FfnArgs& a, uint4* smem, const uint8_t* const (&wsrc)[Tiles<UP, WF>::NW],
                          const float* sc0, const float* sc1, int col0, int q0, int mb, int mcnt) {
  static_assert(RG >= 1 && RG <= 4 && (RG * 64 * Tiles<UP, WF>::CPR) % kThreads == 0,
                "a pass covers 64 * RG rows, copied by whole 512-chunk instructions");
  using R = Ring<UP, RG, WF>;
  using Tl = Tiles<UP, WF>;
  constexpr int NA = Tl::NA, SA = R::SA, SW = R::SW, BK = Tl::BK, CPR = Tl::CPR, CPRW = Tl::CPRW;
  constexpr int WBITS = Tl::WBITS;
  constexpr int GI = RG * 64 * CPR / kThreads;  // activation copies per tile per thread
  constexpr int nA = NA * GI, nW = Tl::NW;      // copy instructions per thread per stage
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform, kept in an SGPR
  const int wm = wid >> 2, wn = wid & 3;
  const int H = a.H, I = a.I;
  const int KD = UP ? H : I;
  const int nit = KD / BK;

  // Activation sources: chunk p = g * 512 + tid of tile u is row p / CPR; rows
  // past the expert's end reload the pass's first row (their results are
  // discarded: a row of the product depends only on that row of A).
  const uint16_t* asrc[NA][GI];
#pragma unroll
  for (int g = 0; g < GI; ++g) {
    const int p = g * kThreads + tid;
    const int r = p / CPR, c = src_chunk<CPR>(p);
    const int q = q0 + mb + (r < mcnt ? r : 0);
    if (UP) {
      asrc[0][g] = (const uint16_t*)a.x + (size_t)(a.pair_list[q] / a.k) * H + c * 8;
    } else {
      asrc[0][g] = a.hb + (size_t)q * I + c * 8;
      asrc[NA - 1][g] = a.hb_lo + (size_t)q * I + c * 8;
    }
  }
  // LDS: activation ring [SA][A_CH], then weight ring [SW][W_CH]
  const uint32_t lds0 = lds_addr(smem) + wid * kWave * 16;
  const uint32_t ldsw = lds0 + SA * R::A_CH * 16;
  auto issue_a = [&](int s) {
    if (s < 0 || s >= nit) return;
    const uint32_t st = lds0 + (s % SA) * R::A_CH * 16;
#pragma unroll
    for (int u = 0; u < NA; ++u)
#pragma unroll
      for (int g = 0; g < GI; ++g) dma16(asrc[u][g] + s * BK, st + (u * GI + g) * kThreads * 16);
  };
  auto issue_w = [&](int s) {
    if (s < 0 || s >= nit) return;
    const uint32_t st = ldsw + (s % SW) * R::W_CH * 16;
#pragma unroll
    for (int i = 0; i < nW; ++i) dma16<kNtWeights<UP, WF>>(wsrc[i] + (size_t)s * BK * WBITS / 8, st + (i * kThreads) * 16);
  };

  constexpr int MT = RG * 2;  // 16-row sub-tiles per wavefront
  f32x4 acc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  // prologue: the k-steps before 0 of the same issue schedule
  for (int j = 1 - SW; j < 0; ++j) {
    issue_a(j + SA - 1);
    issue_w(j + SW - 1);
  }
  for (int it = 0; it < nit; ++it) {
    // Copies issued after the activation copy of stage it: the weight copy of
    // its own k-step (stage it - SA + SW) and, for SA = 3, both copies of
    // k-step it - 1 (stages it + 1 and it + SW - 2); only those below nit exist.
    {
      const bool w0 = it - SA + SW < nit;
      if (SA == 3) {
        const bool a1 = it + 1 < nit, w1 = it + SW - 2 < nit;  // w1 implies w0 implies a1
        if (w1) stage_barrier<2 * nW + nA>();
        else if (w0) stage_barrier<nW + nA>();
        else if (a1) stage_barrier<nA>();
        else stage_barrier<0>();
      } else {
        if (w0) stage_barrier<nW>();
        else stage_barrier<0>();
      }
    }
    issue_a(it + SA - 1);
    issue_w(it + SW - 1);
    const uint4* st = smem + (it % SA) * R::A_CH;
    const uint4* wt = smem + SA * R::A_CH + (it % SW) * R::W_CH;
    // FP8: the block scales of this k-step (wave-uniform, one per 128 elements)
    float s_lo = 1.f, s_hi = 1.f;
    if constexpr (WF == MOE_FMT_FP8_E4M3_B128) {
      const int kb = it * BK / 128;
      s_lo = sc0[kb];
      s_hi = UP ? sc1[kb] : s_lo;
    }
    // MXFP4: the two E8M0 scales of this k-step for each of the lane's rows;
    // int4: the fp16 scale (low half) and zero point (high half) of the
    // 128-group holding this k-step
    uint32_t sc2[4] = {0u, 0u, 0u, 0u};
    if constexpr (Tl::Q4) {
      const uint8_t* scl = (const uint8_t*)(smem + Tl::BUDGET_CH);
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const uint8_t* rr = scl + frag_row<UP>(n, wn, lane) * Tl::SC_ROW;
        if constexpr (WF == MOE_FMT_MXFP4_B32) sc2[n] = *(const uint16_t*)(rr + it * 2);
        else sc2[n] = *(const uint32_t*)(rr + (it >> 1) * 4);
      }
    }
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {  // 32-element sub-steps of one MFMA each
      // B fragments: lane holds weight-tile row (lane % 16) of the sub-tile,
      // chunk 4 * ks + lane / 16
      bf16x8 bf[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int trow = frag_row<UP>(n, wn, lane);
        if constexpr (Tl::Q4) {
          // elements 32 ks + 8 (lane / 16) .. + 7 of the row: word lane / 16 of chunk ks
          const uint32_t q = ((const uint32_t*)&wt[lds_chunk<CPRW>(trow, ks)])[lane >> 4];
          if constexpr (WF == MOE_FMT_MXFP4_B32)
            bf[n] = fp4x8_to_bf16(q, gemv::e8m0_to_float((uint8_t)(sc2[n] >> (8 * ks))));
          else
            bf[n] = int4x8_to_bf16(q, gemv::half_to_float((uint16_t)sc2[n]),
                                   gemv::half_to_float((uint16_t)(sc2[n] >> 16)));
        } else if constexpr (WF == MOE_FMT_FP8_E4M3_B128) {
          // elements 32 ks + 8 (lane / 16) .. + 7 of the row: half (lane / 16) % 2
          // of chunk 2 ks + lane / 32
          const uint2* w2 = (const uint2*)&wt[lds_chunk<CPRW>(trow, 2 * ks + (lane >> 5))];
          bf[n] = fp8x8_to_bf16(w2[(lane >> 4) & 1], n < 2 ? s_lo : s_hi);
        } else {
          bf[n] = as_bf16x8(wt[lds_chunk<CPRW>(trow, 4 * ks + (lane >> 4))]);
        }
      }
#pragma unroll
      for (int u = 0; u < NA; ++u) {
        // all of this wavefront's A fragments are read up front (sub-tiles past the
        // expert's end read stale LDS rows, in bounds and unused); the empty asm
        // keeps the reads from being sunk into the per-sub-tile branches below,
        // which would serialise read, wait and MFMA
        bf16x8 af[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m)
          af[m] = as_bf16x8(st[u * GI * kThreads +
                               lds_chunk<CPR>((2 * m + wm) * 16 + (lane & 15), 4 * ks + (lane >> 4))]);
#pragma unroll
        for (int m = 0; m < MT; ++m) asm volatile("" : "+v"(af[m]));
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if ((2 * m + wm) * 16 >= mcnt) break;  // uniform per wavefront
#pragma unroll
          for (int n = 0; n < 4; ++n)
            acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m], bf[n], acc[m][n], 0, 0, 0);
        }
      }
    }
  }
  __syncthreads();  // all wavefronts are done with the stages before they are refilled

  // epilogue: D[row = 4*(lane/16) + j][col = lane % 16] of each 16 x 16 tile
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int sub = 2 * m + wm;
    if (sub * 16 >= mcnt) break;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = sub * 16 + 4 * (lane >> 4) + j;
      if (row >= mcnt) continue;
      const int q = q0 + mb + row;
      if (UP) {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const float g = acc[m][n][j], v = acc[m][n + 2][j];
          const float h = g / (1.f + __expf(-g)) * v;
          const uint16_t hi = f32_to_bf16_rne(h);
          const size_t at = (size_t)q * I + col0 + wn * 32 + n * 16 + (lane & 15);
          a.hb[at] = hi;
          a.hb_lo[at] = f32_to_bf16_rne(h - __uint_as_float((uint32_t)hi << 16));
        }
      } else if (col0 + wn * 64 < H) {  // the last tile may hold only 128 columns
        const float w = a.pair_w[q];
#pragma unroll
        for (int n = 0; n < 4; ++n)
          a.y[(size_t)q * H + col0 + wn * 64 + n * 16 + (lane & 15)] = w * acc[m][n][j];
      }
    }
  }
}

template <bool UP, int WF>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(FfnArgs a, int tiles_per_expert) {
  using Tl = Tiles<UP, WF>;
  __shared__ __attribute__((aligned(16))) uint4 smem[Tl::BUDGET_CH + Tl::SC_CH];
  constexpr int BMP = 256;  // rows per pass
  // XCD-contiguous numbering: hardware block b runs on XCD b % 8; give the
  // blocks of one XCD consecutive virtual ids.
  const int nb = gridDim.x, b = blockIdx.x;
  const int xcd = b % kXcd, per = nb / kXcd, rem = nb % kXcd;
  const int v = xcd * per + min(xcd, rem) + b / kXcd;
  const int o = a.o_lo + v / tiles_per_expert;
  const int tile = v % tiles_per_expert;
  const int q0 = a.pair_off[o];
  const int M = a.pair_off[o + 1] - q0;
  if (M <= 0) return;  // uniform over the workgroup
  const int H = a.H, I = a.I;
  const int KD = UP ? H : I;
  // bf16 weights: the slot itself or (quantised formats expanded first) the
  // dequantised copy; FP8 and 4-bit weights: the slot
  const uint8_t* rec = a.wbase ? a.wbase + (size_t)(o - a.o_lo) * a.wstride
                               : a.slots + (size_t)a.order_slot[o] * a.stride;
  constexpr int WBITS = Tl::WBITS;
  const uint8_t* W = rec + (UP ? (size_t)0 : (size_t)2 * I * H * WBITS / 8);
  const int col0 = tile * (UP ? UP_HCOLS : DN_COLS);
  // weight copy sources: chunk p = i * 512 + tid of the weight tile is tile row
  // p / CPRW (down: rows past H, in a last half-width tile, reread row H - 1)
  constexpr int CPRW = Tl::CPRW, NW = Tl::NW;
  const uint8_t* wsrc[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int p = i * kThreads + threadIdx.x;
    const int r = p / CPRW, c = src_chunk<CPRW>(p);
    const int wrow = UP ? (r < UP_HCOLS ? col0 + r : I + col0 + (r - UP_HCOLS)) : min(col0 + r, H - 1);
    wsrc[i] = W + (size_t)wrow * KD * WBITS / 8 + c * 16;
  }
  // FP8 block-scale rows of this tile: up, the gate rows' and the up rows' (a
  // tile's 128 gate rows are one block row, and so are its 128 up rows);
  // down, the block row of this wavefront's 64 columns (clamped for a last
  // half-width tile, whose extra columns are discarded)
  const float* sc0 = nullptr;
  const float* sc1 = nullptr;
  if constexpr (WF == MOE_FMT_FP8_E4M3_B128) {
    const RecLayout L = rec_layout(MOE_FMT_FP8_E4M3_B128, H, I);
    const int wn = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave)) & 3;
    if (UP) {
      const float* s13 = (const float*)(rec + L.s13);
      sc0 = s13 + (size_t)(col0 / 128) * (H / 128);
      sc1 = s13 + (size_t)((I + col0) / 128) * (H / 128);
    } else {
      const float* sd = (const float*)(rec + L.sd);
      sc0 = sd + (size_t)min((col0 + wn * 64) / 128, H / 128 - 1) * (I / 128);
    }
  }
  // 4-bit formats: the tile's scale rows (in the row order of the weight
  // tile) into the LDS scale region, once for all passes. MXFP4: KD / 32
  // E8M0 bytes per row; int4: per 128-group its fp16 scale then its fp16
  // zero point (KD / 32 bytes per row)
  if constexpr (Tl::Q4) {
    uint8_t* scl = (uint8_t*)(smem + Tl::BUDGET_CH);
    auto tile_row = [&](int r) {
      return UP ? (r < UP_HCOLS ? col0 + r : I + col0 + (r - UP_HCOLS)) : min(col0 + r, H - 1);
    };
    if constexpr (WF == MOE_FMT_MXFP4_B32) {
      const RecLayout L = rec_layout(MOE_FMT_MXFP4_B32, H, I);
      const uint8_t* sb = rec + (UP ? L.s13 : L.sd);
      const int words = KD / 128;  // 4-byte words of scales per row
      for (int i = threadIdx.x; i < BN * words; i += kThreads) {
        const int r = i / words, w = i - r * words;
        *(uint32_t*)(scl + r * Tl::SC_ROW + 4 * w) =
            *(const uint32_t*)(sb + (size_t)tile_row(r) * (KD / 32) + 4 * w);
      }
    } else {
      const RecLayout L = rec_layout(MOE_FMT_INT4_ASYM_G128, H, I);
      const uint16_t* sb = (const uint16_t*)(rec + (UP ? L.s13 : L.sd));
      const uint16_t* zb = (const uint16_t*)(rec + (UP ? L.z13 : L.zd));
      const int G = KD / 128;  // groups per row
      for (int i = threadIdx.x; i < BN * 2 * G; i += kThreads) {
        const int r = i / (2 * G), c = i - r * 2 * G;
        const size_t at = (size_t)tile_row(r) * G + (c >> 1);
        ((uint16_t*)(scl + r * Tl::SC_ROW))[c] = (c & 1) ? zb[at] : sb[at];
      }
    }
    __syncthreads();
  }
  for (int mb = 0; mb < M; mb += BMP) {
    const int mcnt = min(BMP, M - mb);
    // uniform branches: the smallest pass shape that holds mcnt rows (up: any
    // number of 64-row groups; down, with 32-wide rows: an even number)
    const int rg = (mcnt + 63) >> 6;
    if (UP && rg == 1) gemm_pass<UP, (UP ? 1 : 2), WF>(a, smem, wsrc, sc0, sc1, col0, q0, mb, mcnt);
    else if (rg <= 2) gemm_pass<UP, 2, WF>(a, smem, wsrc, sc0, sc1, col0, q0, mb, mcnt);
    else if (UP && rg == 3) gemm_pass<UP, (UP ? 3 : 4), WF>(a, smem, wsrc, sc0, sc1, col0, q0, mb, mcnt);
    else gemm_pass<UP, 4, WF>(a, smem, wsrc, sc0, sc1, col0, q0, mb, mcnt);
  }
}

// out[t][n] (+)= sum_j y[pos(t, j)][n] over the pairs of this wave, j ascending.
// With x_res, the residual of a layer stack is applied to the final out:
// x_res = bf16_rne(x_res + out).
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const int32_t* __restrict__ wave_of, int wave,
                                                      int T, int k, int H, float* out, int accumulate,
                                                      uint16_t* x_res) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= (int64_t)T * H) return;
  const int t = (int)(i / H), n = (int)(i % H);
  float4 acc = accumulate ? *(const float4*)(out + i) : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int p = t * k + j;
    if (wave_of[p] != wave) continue;
    const float4 v = *(const float4*)(y + (size_t)pair_pos[p] * H + n);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  *(float4*)(out + i) = acc;
  if (x_res) {
    const uint2 xv = *(const uint2*)(x_res + i);
    uint2 r;
    r.x = (uint32_t)f32_to_bf16_rne(__uint_as_float(xv.x << 16) + acc.x) |
          ((uint32_t)f32_to_bf16_rne(__uint_as_float(xv.x & 0xFFFF0000u) + acc.y) << 16);
    r.y = (uint32_t)f32_to_bf16_rne(__uint_as_float(xv.y << 16) + acc.z) |
          ((uint32_t)f32_to_bf16_rne(__uint_as_float(xv.y & 0xFFFF0000u) + acc.w) << 16);
    *(uint2*)(x_res + i) = r;
  }
}

}  // namespace

bool gemm_shape_supported(int H, int I) {
  return H > 0 && I > 0 && H % 128 == 0 && I % 128 == 0;
}

// The GEMMs read bf16 and FP8 records in place, and MXFP4 and int4 records
// whose scale rows fit the LDS scale region; larger 4-bit shapes are expanded
// to bf16 copies first (a.wbase).
bool gemm_reads_record(int fmt, int H, int I) {
  if (fmt == MOE_FMT_BF16 || fmt == MOE_FMT_FP8_E4M3_B128) return true;
  // scale-region bytes per row: MXFP4 KD / 32 E8M0 bytes; int4 KD / 128 fp16
  // scales and as many zero points, KD / 32 bytes too
  if (fmt == MOE_FMT_MXFP4_B32 || fmt == MOE_FMT_INT4_ASYM_G128)
    return H / 32 <= kQ4ScRowUp && I / 32 <= kQ4ScRowDn;
  return false;
}

template <bool UP>
static hipError_t launch_gemm(const FfnArgs& a, hipStream_t s) {
  if (a.n_exp <= 0) return hipSuccess;
  const int tpe = UP ? a.I / UP_HCOLS : (a.H + DN_COLS - 1) / DN_COLS;
  const int wf = a.wbase ? MOE_FMT_BF16 : a.fmt;
  if (!a.wbase && !gemm_reads_record(wf, a.H, a.I)) return hipErrorInvalidValue;
  const dim3 grid(tpe * a.n_exp), block(kThreads);
  switch (wf) {
    case MOE_FMT_BF16: launch_k(grouped_gemm_kernel<UP, MOE_FMT_BF16>, grid, block, s, a.ev0, a.ev1, a, tpe); break;
    case MOE_FMT_FP8_E4M3_B128:
      launch_k(grouped_gemm_kernel<UP, MOE_FMT_FP8_E4M3_B128>, grid, block, s, a.ev0, a.ev1, a, tpe);
      break;
    case MOE_FMT_MXFP4_B32:
      launch_k(grouped_gemm_kernel<UP, MOE_FMT_MXFP4_B32>, grid, block, s, a.ev0, a.ev1, a, tpe);
      break;
    case MOE_FMT_INT4_ASYM_G128:
      launch_k(grouped_gemm_kernel<UP, MOE_FMT_INT4_ASYM_G128>, grid, block, s, a.ev0, a.ev1, a, tpe);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_up(const FfnArgs& a, hipStream_t s) { return launch_gemm<true>(a, s); }
hipError_t launch_gemm_down(const FfnArgs& a, hipStream_t s) { return launch_gemm<false>(a, s); }

hipError_t launch_combine(const FfnArgs& a, const int32_t* pair_pos, const int32_t* wave_of,
                          int wave, hipStream_t s) {
  const int64_t n4 = ((int64_t)a.T * a.H) / 4;
  if (n4 <= 0) return hipSuccess;
  launch_k(combine_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), s, a.ev0, a.ev1, a.y, pair_pos,
           wave_of, wave, a.T, a.k, a.H, a.out, a.accumulate, a.x_res);
  return hipGetLastError();
}

}  // namespace moepage
