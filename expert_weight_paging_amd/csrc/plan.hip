// Router, slot-plan, grouping and residual kernels for gfx950.
//
// [PE] = "Running an MoE Model Larger Than Your VRAM: SGLang Paged Experts, the
// PCIe Math, and the 4-Request Cliff". [LRU] = "Locality of reference helped
// 94GB Qwen3.8-Flash-Next runs at 68 tok/s on one RTX 5090".
#include "internal.h"

namespace moepage {

namespace {

constexpr int kWave = 64;

// Order-preserving integer key of a float32: equal floats (including +0/-0)
// map to equal keys, larger floats to larger keys.
__device__ inline uint32_t float_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// ------------------------------------------------------------------ router
// One wavefront per token ([PE] "What does Paged Experts actually do?": each
// token goes to top_k of E experts). k rounds of a wavefront arg-max over
// packed (key << 32 | ~id): the largest logit wins, equal logits go to the
// smaller id, so the result is unique and listed by descending logit. The
// weights are the softmax of the selected logits, which equals the softmax
// over all E renormalised over the selected k.
template <int NJ>
__global__ __launch_bounds__(256) void router_kernel(const float* __restrict__ logits, int T, int E,
                                                     int k, int32_t* __restrict__ ids,
                                                     float* __restrict__ weights) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  if (t >= T) return;  // uniform per wavefront
  const float* z = logits + (size_t)t * E;
  uint32_t key[NJ];
  uint32_t valid = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + kWave * j;
    key[j] = 0;
    if (e < E) {
      key[j] = float_key(z[e]);
      valid |= 1u << j;
    }
  }
  int my_id = 0;
  float my_z = 0.f;
  for (int r = 0; r < k; ++r) {
    unsigned long long best = 0ull;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (valid & (1u << j)) {
        const unsigned long long p =
            ((unsigned long long)key[j] << 32) | (uint32_t)(~(uint32_t)(lane + kWave * j));
        best = p > best ? p : best;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const unsigned long long o = __shfl_xor(best, off, kWave);
      best = o > best ? o : best;
    }
    const int e = (int)(~(uint32_t)best);
    if ((e & (kWave - 1)) == lane) valid &= ~(1u << (e / kWave));
    if (lane == r) {
      my_id = e;
      my_z = z[e];
    }
  }
  const float zmax = __shfl(my_z, 0, kWave);
  const float ex = lane < k ? __expf(my_z - zmax) : 0.f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    weights[(size_t)t * k + lane] = ex / sum;
  }
}

// ------------------------------------------------------------------ block scan
constexpr int kPlanThreads = 1024;

// Exclusive prefix sum over the block (1024 threads); *total gets the sum.
__device__ inline int block_exscan(int v, int* s_warp, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  int inc = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += o;
  }
  if (lane == kWave - 1) s_warp[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    int w = lane < kPlanThreads / kWave ? s_warp[lane] : 0;
    int winc = w;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(winc, off, kWave);
      if (lane >= off) winc += o;
    }
    if (lane < kPlanThreads / kWave) s_warp[lane] = winc - w;
    if (lane == kPlanThreads / kWave - 1) s_warp[kPlanThreads / kWave] = winc;
  }
  __syncthreads();
  const int res = s_warp[wid] + inc - v;
  *total = s_warp[kPlanThreads / kWave];
  __syncthreads();
  return res;
}

// ------------------------------------------------------------------ slot plan
// One workgroup of 1024 threads; thread e owns expert e, thread s owns slot s.
// [PE] "TL;DR" / "What does Paged Experts actually do?": only routed experts
// that are not resident are copied in, the least recently used slot goes out.
// [PE] "What happens with more than one request?": a step that routes more
// distinct experts than fit runs as several waves, each with its own page-in.
// Readings (the oracle follows the same ones): residents first then missing
// experts, each ascending; waves are chunks of K; the clock ticks per wave;
// victims are slots not used by the wave, ordered by (stamp, slot); the i-th
// missing expert goes to the i-th victim.
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ ids, int P,
                                                            int T, int E, int K, uint8_t* state,
                                                            StateLayout sl, PlanDev dev,
                                                            PlanHdr* hdr, int32_t seq) {
  __shared__ int s_cnt[MOE_MAX_EXPERTS];
  __shared__ int s_pos[MOE_MAX_EXPERTS];
  __shared__ int s_order_e[MOE_MAX_EXPERTS];
  __shared__ int s_order_s[MOE_MAX_EXPERTS];
  __shared__ int s_slot_expert[MOE_MAX_EXPERTS];
  __shared__ int s_expert_slot[MOE_MAX_EXPERTS];
  __shared__ long long s_stamp[MOE_MAX_EXPERTS];
  __shared__ int s_prot[MOE_MAX_EXPERTS];
  __shared__ int s_warp[kPlanThreads / kWave + 1];

  int32_t* g_slot_expert = (int32_t*)(state + sl.slot_expert);
  int32_t* g_expert_slot = (int32_t*)(state + sl.expert_slot);
  long long* g_stamp = (long long*)(state + sl.stamp);
  long long* g_clock = (long long*)(state + sl.clock);

  const int tid = threadIdx.x;
  if (tid < E) {
    s_cnt[tid] = 0;
    s_expert_slot[tid] = g_expert_slot[tid];
  }
  if (tid < K) {
    s_slot_expert[tid] = g_slot_expert[tid];
    s_stamp[tid] = g_stamp[tid];
  }
  long long clock = *g_clock;
  __syncthreads();
  for (int p = tid; p < P; p += kPlanThreads) atomicAdd(&s_cnt[ids[p]], 1);
  __syncthreads();

  const bool ref = tid < E && s_cnt[tid] > 0;
  const bool hit = ref && s_expert_slot[tid] >= 0;
  const bool miss = ref && !hit;
  int nH, nM;
  const int hit_rank = block_exscan(hit ? 1 : 0, s_warp, &nH);
  const int miss_rank = block_exscan(miss ? 1 : 0, s_warp, &nM);
  const int D = nH + nM;
  if (tid < E) {
    const int pos = hit ? hit_rank : (miss ? nH + miss_rank : -1);
    s_pos[tid] = pos;
    if (pos >= 0) s_order_e[pos] = tid;
  }
  const int n_waves = (D + K - 1) / K;
  __syncthreads();

  for (int w = 0; w < n_waves; ++w) {
    clock += 1;
    const int lo = w * K;
    const int hi = min(lo + K, D);
    const int m_lo = max(lo, nH);
    const int nm = hi - m_lo;
    int prot = 1;
    long long my_stamp = 0;
    if (tid < K) {
      const int e = s_slot_expert[tid];
      prot = (e >= 0 && s_pos[e] >= lo && s_pos[e] < hi) ? 1 : 0;
      s_prot[tid] = prot;
      my_stamp = s_stamp[tid];
    }
    __syncthreads();
    if (tid < K && !prot && nm > 0) {
      int rank = 0;
      for (int s = 0; s < K; ++s) {
        if (s_prot[s]) continue;
        const long long st = s_stamp[s];
        rank += (st < my_stamp || (st == my_stamp && s < tid)) ? 1 : 0;
      }
      if (rank < nm) {
        const int e_new = s_order_e[m_lo + rank];
        const int old = s_slot_expert[tid];
        if (old >= 0) s_expert_slot[old] = -1;
        s_slot_expert[tid] = e_new;
        s_expert_slot[e_new] = tid;
        s_order_s[m_lo + rank] = tid;
      }
    }
    __syncthreads();
    if (tid >= lo && tid < min(hi, nH)) s_order_s[tid] = s_expert_slot[s_order_e[tid]];
    __syncthreads();
    if (tid >= lo && tid < hi) s_stamp[s_order_s[tid]] = clock;
    __syncthreads();
  }

  // table state back to HBM
  if (tid < E) g_expert_slot[tid] = s_expert_slot[tid];
  if (tid < K) {
    g_slot_expert[tid] = s_slot_expert[tid];
    g_stamp[tid] = s_stamp[tid];
  }
  if (tid == 0) *g_clock = clock;

  // per-pair slot and wave
  for (int p = tid; p < P; p += kPlanThreads) {
    const int pos = s_pos[ids[p]];
    dev.slot_ids[p] = s_order_s[pos];
    dev.wave_of[p] = pos / K;
  }
  // CSR offsets of the pairs of each expert, in wave order
  int total;
  const int c = tid < D ? s_cnt[s_order_e[tid]] : 0;
  const int off = block_exscan(c, s_warp, &total);
  if (tid < E) dev.pair_off[tid] = tid < D ? off : P;
  if (tid == 0) dev.pair_off[E] = P;

  // wave order, device and host-visible copies
  int32_t* h_order_e = (int32_t*)(hdr + 1);
  int32_t* h_order_s = h_order_e + E;
  if (tid < D) {
    dev.order_expert[tid] = s_order_e[tid];
    dev.order_slot[tid] = s_order_s[tid];
    h_order_e[tid] = s_order_e[tid];
    h_order_s[tid] = s_order_s[tid];
  }
  if (tid == 0) {
    dev.counts[0] = D;
    dev.counts[1] = nH;
    dev.counts[2] = n_waves;
    dev.counts[3] = T;
    hdr->num_tokens = T;
    hdr->num_distinct = D;
    hdr->num_hits = nH;
    hdr->num_waves = n_waves;
  }
  __threadfence_system();
  __syncthreads();
  if (tid == 0) __hip_atomic_store(&hdr->seq, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ------------------------------------------------------------------ grouping
// One wavefront per position of the wave order: collects the pair indices of
// its expert in ascending order (ballot + prefix popcount), so that the list
// and therefore every later summation order is deterministic.
__global__ __launch_bounds__(256) void group_kernel(const int32_t* __restrict__ ids, int P,
                                                    PlanDev dev) {
  const int lane = threadIdx.x & (kWave - 1);
  const int i = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int D = dev.counts[0];
  if (i >= D) return;
  const int e = dev.order_expert[i];
  const int base = dev.pair_off[i];
  int running = 0;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int c = 0; c < P; c += kWave) {
    const int p = c + lane;
    const bool m = p < P && ids[p] == e;
    const unsigned long long mask = __ballot(m);
    if (m) {
      const int q = base + running + __popcll(mask & below);
      dev.pair_list[q] = p;
      dev.pair_pos[p] = q;
    }
    running += __popcll(mask);
  }
}

// ------------------------------------------------------------------ residual
__device__ inline uint16_t f32_to_bf16_rne(float v) {
  uint32_t b = __float_as_uint(v);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__global__ __launch_bounds__(256) void residual_kernel(const uint16_t* x_in, const float* out,
                                                       uint16_t* x_out, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i + 4 <= n) {
    const uint2 xv = *(const uint2*)(x_in + i);
    const float4 ov = *(const float4*)(out + i);
    const float a0 = __uint_as_float(xv.x << 16) + ov.x;
    const float a1 = __uint_as_float(xv.x & 0xFFFF0000u) + ov.y;
    const float a2 = __uint_as_float(xv.y << 16) + ov.z;
    const float a3 = __uint_as_float(xv.y & 0xFFFF0000u) + ov.w;
    uint2 r;
    r.x = (uint32_t)f32_to_bf16_rne(a0) | ((uint32_t)f32_to_bf16_rne(a1) << 16);
    r.y = (uint32_t)f32_to_bf16_rne(a2) | ((uint32_t)f32_to_bf16_rne(a3) << 16);
    *(uint2*)(x_out + i) = r;
  } else {
    for (int64_t j = i; j < n; ++j)
      x_out[j] = f32_to_bf16_rne(__uint_as_float((uint32_t)x_in[j] << 16) + out[j]);
  }
}

}  // namespace

hipError_t launch_router(const float* logits, int T, int E, int k, int32_t* ids, float* weights,
                         hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int nj = (E + kWave - 1) / kWave;
  const dim3 grid((T + 3) / 4), block(256);
  if (nj <= 1) router_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, ids, weights);
  else if (nj <= 2) router_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, ids, weights);
  else if (nj <= 4) router_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, ids, weights);
  else if (nj <= 8) router_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, ids, weights);
  else router_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k, ids, weights);
  return hipGetLastError();
}

hipError_t launch_plan(const int32_t* ids, int T, int k, int E, int K, void* state, PlanDev dev,
                       PlanHdr* host_hdr_dev, int32_t seq, hipStream_t s) {
  plan_kernel<<<1, kPlanThreads, 0, s>>>(ids, T * k, T, E, K, (uint8_t*)state, state_layout(E, K),
                                         dev, host_hdr_dev, seq);
  return hipGetLastError();
}

hipError_t launch_group(const int32_t* ids, int T, int k, int E, PlanDev dev, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  group_kernel<<<(E + 3) / 4, 256, 0, s>>>(ids, T * k, dev);
  return hipGetLastError();
}

hipError_t launch_residual(const uint16_t* x_in, const float* out, uint16_t* x_out, int64_t n,
                           hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t threads = (n + 3) / 4;
  residual_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(x_in, out, x_out, n);
  return hipGetLastError();
}

}  // namespace moepage
