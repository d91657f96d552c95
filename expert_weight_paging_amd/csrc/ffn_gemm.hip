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
// Tiling (v_mfma_f32_16x16x32_bf16, 64-wide wavefronts). A workgroup of four
// wavefronts owns one expert and 128 output columns (up: 64 gate rows and the
// 64 matching up rows of W13; down: 128 rows of W_d) and covers up to 256 of
// the expert's rows per pass, so each weight byte leaves HBM once per expert
// for all but the hottest experts. The k loop runs in steps of 32; each step
// is one pipeline stage in LDS holding the weight tile (128 x 32) and the
// activation tile(s) (rows x 32). Stages are filled by direct global-to-LDS
// loads (no register staging), NSTAGE - 1 steps ahead of the matrix cores,
// so HBM latency hides behind the MFMAs; a wait on the vector-memory counter
// plus a barrier hands a stage over. Only the 64-row groups that hold routed
// rows are loaded (template RG). The 16-byte chunks of a tile row are
// XOR-swizzled by (row / 2) mod 4, which makes the fragment reads free of
// LDS bank conflicts; the swizzle is applied by choosing each DMA lane's
// source chunk, since a DMA instruction writes its 64 lanes contiguously.
// The four wavefronts form a 2 x 2 grid: wavefront (wm, wn) takes the 16-row
// sub-tiles with index = wm (mod 2) and output columns wn*64 .. wn*64+63.
// Workgroups are numbered so that each XCD (which schedules every eighth
// workgroup and has its own L2) works through a contiguous run of experts,
// keeping an expert's activation rows in one L2.
#include "internal.h"

namespace moepage {

namespace {

constexpr int kWave = 64;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int BM = 256;                    // expert rows per pass
constexpr int BN = 128;                    // weight rows per workgroup
constexpr int BK = 32;                     // reduction elements per stage
constexpr int A_CH = BM * BK * 2 / 16;     // 16-byte chunks of an activation tile (1024)
constexpr int W_CH = BN * BK * 2 / 16;     // 16-byte chunks of the weight tile (512)
constexpr int UP_HCOLS = BN / 2;           // h columns per workgroup (up)
constexpr int DN_COLS = BN;                // output columns per workgroup (down)
constexpr int kXcd = 8;                    // XCDs; consecutive workgroups go round-robin over them

__device__ inline bf16x8 as_bf16x8(const uint4& v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

__device__ inline uint16_t f32_to_bf16_rne(float v) {
  uint32_t b = __float_as_uint(v);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// LDS chunk of logical chunk c (0..3) of tile row r; and, for LDS chunk p, the
// logical chunk it holds (row p / 4): the two are inverse of each other.
__device__ inline int lds_chunk(int r, int c) { return r * 4 + (c ^ ((r >> 1) & 3)); }
__device__ inline int src_chunk(int p) { return (p & 3) ^ ((p >> 3) & 3); }

// Global-to-LDS copy of 16 bytes per lane: lane l's bytes land at LDS byte
// address lds + 16 * l (lds wave-uniform, in M0). Issued from inline assembly
// so that the compiler neither waits for it before every LDS read nor counts
// it: the pipeline below does its own waiting on the vector-memory counter.
__device__ inline void dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds)
               : "memory", "m0");
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

template <bool UP>
struct Tiles {
  static constexpr int NA = UP ? 1 : 2;                 // activation tiles: x, or (h_hi, h_lo)
  static constexpr int NSTAGE = UP ? 3 : 2;             // pipeline depth (LDS: 72 KB / 80 KB)
  static constexpr int STAGE_CH = NA * A_CH + W_CH;
};

// One pass over rows [mb, mb + mcnt) of expert position o, mcnt <= 64 * RG.
template <bool UP, int RG>
__device__ void gemm_pass(const FfnArgs& a, uint4* smem, const uint16_t* const (&wsrc)[2], int col0,
                          int q0, int mb, int mcnt) {
  using Tl = Tiles<UP>;
  constexpr int NA = Tl::NA, NSTAGE = Tl::NSTAGE, STAGE_CH = Tl::STAGE_CH;
  constexpr int NIS = NA * RG + 2;  // DMA instructions per thread per stage
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform, kept in an SGPR
  const int wm = wid >> 1, wn = wid & 1;
  const int H = a.H, I = a.I;
  const int KD = UP ? H : I;
  const int nit = KD / BK;

  // Activation sources: chunk p = g * 256 + tid of tile u is row p / 4; rows
  // past the expert's end reload the pass's first row (their results are
  // discarded: a row of the product depends only on that row of A).
  const uint16_t* asrc[NA][RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    const int p = g * 256 + tid;
    const int r = p >> 2, c = src_chunk(p);
    const int q = q0 + mb + (r < mcnt ? r : 0);
    if (UP) {
      asrc[0][g] = (const uint16_t*)a.x + (size_t)(a.pair_list[q] / a.k) * H + c * 8;
    } else {
      asrc[0][g] = a.hb + (size_t)q * I + c * 8;
      asrc[NA - 1][g] = a.hb_lo + (size_t)q * I + c * 8;
    }
  }
  const uint32_t lds0 = lds_addr(smem) + wid * kWave * 16;
  auto issue = [&](int it) {
    const uint32_t st = lds0 + (it % NSTAGE) * STAGE_CH * 16;
    const int ko = it * BK;
#pragma unroll
    for (int u = 0; u < NA; ++u)
#pragma unroll
      for (int g = 0; g < RG; ++g) dma16(asrc[u][g] + ko, st + (u * A_CH + g * 256) * 16);
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(wsrc[i] + ko, st + (NA * A_CH + i * 256) * 16);
  };

  constexpr int MT = RG * 2;  // 16-row sub-tiles per wavefront
  f32x4 acc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < nit) issue(s);
  for (int it = 0; it < nit; ++it) {
    // stage `it` has landed once at most the NSTAGE - 2 later stages are in flight
    if (it + NSTAGE - 2 < nit) stage_barrier<NIS * (NSTAGE - 2)>();
    else stage_barrier<0>();
    if (it + NSTAGE - 1 < nit) issue(it + NSTAGE - 1);
    const uint4* st = smem + (it % NSTAGE) * STAGE_CH;
    const uint4* wt = st + NA * A_CH;
    // B fragments: lane holds weight-tile row (lane % 16) of the sub-tile, chunk lane / 16
    bf16x8 bf[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      // up: h columns wn*32 + (n%2)*16 .. (gate rows for n < 2, the matching up
      // rows 64 further down the tile for n >= 2); down: columns wn*64 + n*16 ..
      const int trow = UP ? ((n < 2 ? 0 : UP_HCOLS) + wn * 32 + (n & 1) * 16 + (lane & 15))
                          : (wn * 64 + n * 16 + (lane & 15));
      bf[n] = as_bf16x8(wt[lds_chunk(trow, lane >> 4)]);
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
        af[m] = as_bf16x8(st[u * A_CH + lds_chunk((2 * m + wm) * 16 + (lane & 15), lane >> 4)]);
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
      } else {
        const float w = a.weights[a.pair_list[q]];
#pragma unroll
        for (int n = 0; n < 4; ++n)
          a.y[(size_t)q * H + col0 + wn * 64 + n * 16 + (lane & 15)] = w * acc[m][n][j];
      }
    }
  }
}

template <bool UP>
__global__ __launch_bounds__(256, 2) void grouped_gemm_kernel(FfnArgs a, int tiles_per_expert) {
  using Tl = Tiles<UP>;
  __shared__ __attribute__((aligned(16))) uint4 smem[Tl::NSTAGE * Tl::STAGE_CH];
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
  const uint8_t* rec = a.slots + (size_t)a.order_slot[o] * a.stride;
  const uint16_t* W = (const uint16_t*)(rec + (UP ? (size_t)0 : (size_t)2 * I * H * 2));
  const int col0 = tile * (UP ? UP_HCOLS : DN_COLS);
  // weight DMA sources: chunk p = i * 256 + tid of the weight tile is tile row p / 4
  const uint16_t* wsrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = i * 256 + threadIdx.x;
    const int r = p >> 2, c = src_chunk(p);
    const int wrow = UP ? (r < UP_HCOLS ? col0 + r : I + col0 + (r - UP_HCOLS)) : col0 + r;
    wsrc[i] = W + (size_t)wrow * KD + c * 8;
  }
  for (int mb = 0; mb < M; mb += BM) {
    const int mcnt = min(BM, M - mb);
    switch ((mcnt + 63) >> 6) {  // uniform over the workgroup
      case 1: gemm_pass<UP, 1>(a, smem, wsrc, col0, q0, mb, mcnt); break;
      case 2: gemm_pass<UP, 2>(a, smem, wsrc, col0, q0, mb, mcnt); break;
      case 3: gemm_pass<UP, 3>(a, smem, wsrc, col0, q0, mb, mcnt); break;
      default: gemm_pass<UP, 4>(a, smem, wsrc, col0, q0, mb, mcnt); break;
    }
  }
}

// out[t][n] (+)= sum_j y[pos(t, j)][n] over the pairs of this wave, j ascending.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const int32_t* __restrict__ wave_of, int wave,
                                                      int T, int k, int H, float* out, int accumulate) {
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
}

}  // namespace

bool gemm_shape_supported(int H, int I) {
  return H > 0 && I > 0 && H % 128 == 0 && I % 128 == 0;
}

hipError_t launch_gemm_up(const FfnArgs& a, hipStream_t s) {
  if (a.n_exp <= 0) return hipSuccess;
  const int tpe = a.I / UP_HCOLS;
  launch_k(grouped_gemm_kernel<true>, dim3(tpe * a.n_exp), dim3(256), s, a.ev0, a.ev1, a, tpe);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const FfnArgs& a, hipStream_t s) {
  if (a.n_exp <= 0) return hipSuccess;
  const int tpe = a.H / DN_COLS;
  launch_k(grouped_gemm_kernel<false>, dim3(tpe * a.n_exp), dim3(256), s, a.ev0, a.ev1, a, tpe);
  return hipGetLastError();
}

hipError_t launch_combine(const FfnArgs& a, const int32_t* pair_pos, const int32_t* wave_of,
                          int wave, hipStream_t s) {
  const int64_t n4 = ((int64_t)a.T * a.H) / 4;
  if (n4 <= 0) return hipSuccess;
  launch_k(combine_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), s, a.ev0, a.ev1, a.y, pair_pos,
           wave_of, wave, a.T, a.k, a.H, a.out, a.accumulate);
  return hipGetLastError();
}

}  // namespace moepage
