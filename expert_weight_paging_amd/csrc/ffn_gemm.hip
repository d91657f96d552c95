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
// Tiling (v_mfma_f32_16x16x32_bf16, 64-wide wavefronts): a workgroup of 4
// wavefronts owns one expert and a block of output columns and walks all of
// the expert's rows in passes of 128, so each weight byte is streamed from HBM
// once per pass. Weights go straight from global memory into each
// wavefront's B fragments (prefetched one k-step ahead); the 128 x 64 tile of
// activations is staged once per k-step in LDS (double buffered, 16-byte
// chunks XOR-swizzled by row) and shared by the four wavefronts.
#include "internal.h"

namespace moepage {

namespace {

constexpr int kWave = 64;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;       // rows per pass
constexpr int BK = 64;        // reduction elements per main-loop step
constexpr int MS = BM / 16;   // 16-row sub-tiles per pass
constexpr int NS = 4;         // 16-column sub-tiles per wavefront
constexpr int UP_COLS = 128;  // h columns per workgroup (up)
constexpr int DN_COLS = 256;  // output columns per workgroup (down)

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

// element offset of 16-byte chunk c of row r in an LDS A tile
__device__ inline int a_off(int r, int c) { return r * BK + ((c ^ (r & 7)) << 3); }

template <bool UP>
__global__ __launch_bounds__(256, 2) void grouped_gemm_kernel(FfnArgs a) {
  constexpr int NA = UP ? 1 : 2;  // A tiles per k-step: x, or (h_hi, h_lo)
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][NA][BM * BK];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int o = a.o_lo + blockIdx.y;
  const int q0 = a.pair_off[o];
  const int M = a.pair_off[o + 1] - q0;
  if (M <= 0) return;  // uniform over the workgroup
  const int H = a.H, I = a.I;
  const int KD = UP ? H : I;
  const uint8_t* rec = a.slots + (size_t)a.order_slot[o] * a.stride;
  const uint16_t* W = (const uint16_t*)(rec + (UP ? (size_t)0 : (size_t)2 * I * H * 2));
  int brow[NS];
  int col0;
  if (UP) {
    col0 = blockIdx.x * UP_COLS + wid * 32;  // h columns col0 .. col0+31
    brow[0] = col0;
    brow[1] = col0 + 16;
    brow[2] = I + col0;
    brow[3] = I + col0 + 16;
  } else {
    col0 = blockIdx.x * DN_COLS + wid * 64;
#pragma unroll
    for (int s = 0; s < NS; ++s) brow[s] = col0 + 16 * s;
  }
  const int nit = KD / BK;
  const uint16_t* bptr[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
    bptr[s] = W + (size_t)(brow[s] + (lane & 15)) * KD + 8 * (lane >> 4);

  for (int mb = 0; mb < M; mb += BM) {
    const int mcnt = min(BM, M - mb);
    const uint16_t* asrc[NA][4];
    int aoff[4];
    bool aval[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 3, c = idx & 7;
      aval[i] = r < mcnt;
      aoff[i] = a_off(r, c);
      const int q = q0 + mb + (aval[i] ? r : 0);
      if (UP) {
        const int t = a.pair_list[q] / a.k;
        asrc[0][i] = (const uint16_t*)a.x + (size_t)t * H + c * 8;
      } else {
        asrc[0][i] = a.hb + (size_t)q * I + c * 8;
        asrc[NA - 1][i] = a.hb_lo + (size_t)q * I + c * 8;
      }
    }
    f32x4 acc[MS][NS];
#pragma unroll
    for (int m = 0; m < MS; ++m)
#pragma unroll
      for (int s = 0; s < NS; ++s) acc[m][s] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 areg[NA][4], bcur[NS][2], bnxt[NS][2];
    auto load_a = [&](int k0) {
#pragma unroll
      for (int u = 0; u < NA; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          areg[u][i] = aval[i] ? *(const uint4*)(asrc[u][i] + k0) : make_uint4(0, 0, 0, 0);
    };
    auto load_b = [&](int k0, uint4 (&dst)[NS][2]) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) dst[s][ks] = *(const uint4*)(bptr[s] + k0 + 32 * ks);
    };
    auto store_a = [&](int buf) {
#pragma unroll
      for (int u = 0; u < NA; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) *(uint4*)&sA[buf][u][aoff[i]] = areg[u][i];
    };

    load_a(0);
    load_b(0, bcur);
    store_a(0);
    __syncthreads();
    for (int it = 0; it < nit; ++it) {
      const int buf = it & 1;
      const bool more = it + 1 < nit;
      if (more) {
        load_a((it + 1) * BK);
        load_b((it + 1) * BK, bnxt);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 bf[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) bf[s] = as_bf16x8(bcur[s][ks]);
#pragma unroll
        for (int m = 0; m < MS; ++m) {
          if (m * 16 < mcnt) {
            const int off = a_off(m * 16 + (lane & 15), ks * 4 + (lane >> 4));
#pragma unroll
            for (int u = 0; u < NA; ++u) {
              const bf16x8 af = as_bf16x8(*(const uint4*)&sA[buf][u][off]);
#pragma unroll
              for (int s = 0; s < NS; ++s)
                acc[m][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[s], acc[m][s], 0, 0, 0);
            }
          }
        }
      }
      if (more) {
        store_a(buf ^ 1);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          bcur[s][0] = bnxt[s][0];
          bcur[s][1] = bnxt[s][1];
        }
      }
      __syncthreads();
    }

    // epilogue: D[row = 4*(lane/16) + j][col = lane % 16] of each 16x16 tile
#pragma unroll
    for (int m = 0; m < MS; ++m) {
      if (m * 16 >= mcnt) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = m * 16 + 4 * (lane >> 4) + j;
        if (row >= mcnt) continue;
        const int q = q0 + mb + row;
        if (UP) {
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const float g = acc[m][s][j], u = acc[m][s + 2][j];
            const float h = g / (1.f + __expf(-g)) * u;
            const uint16_t hi = f32_to_bf16_rne(h);
            const size_t at = (size_t)q * I + col0 + 16 * s + (lane & 15);
            a.hb[at] = hi;
            a.hb_lo[at] = f32_to_bf16_rne(h - __uint_as_float((uint32_t)hi << 16));
          }
        } else {
          const float w = a.weights[a.pair_list[q]];
#pragma unroll
          for (int s = 0; s < NS; ++s)
            a.y[(size_t)q * H + col0 + 16 * s + (lane & 15)] = w * acc[m][s][j];
        }
      }
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
  return H > 0 && I > 0 && H % DN_COLS == 0 && I % UP_COLS == 0 && H % BK == 0 && I % BK == 0;
}

hipError_t launch_gemm_up(const FfnArgs& a, hipStream_t s) {
  if (a.n_exp <= 0) return hipSuccess;
  launch_k(grouped_gemm_kernel<true>, dim3(a.I / UP_COLS, a.n_exp), dim3(256), s, a.ev0, a.ev1, a);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const FfnArgs& a, hipStream_t s) {
  if (a.n_exp <= 0) return hipSuccess;
  launch_k(grouped_gemm_kernel<false>, dim3(a.H / DN_COLS, a.n_exp), dim3(256), s, a.ev0, a.ev1, a);
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
