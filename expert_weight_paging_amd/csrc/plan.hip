// Router, slot-plan, grouping and residual kernels for gfx950.
//
// [PE] = "Running an MoE Model Larger Than Your VRAM: SGLang Paged Experts, the
// PCIe Math, and the 4-Request Cliff". [LRU] = "Locality of reference helped
// 94GB Qwen3.8-Flash-Next runs at 68 tok/s on one RTX 5090".
#include "copy.h"
#include "gemv_up.h"
#include "internal.h"
#include "norm.h"
#include "wave.h"

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

// (key, id) packed so that a larger packed value means a larger logit, or an
// equal logit and a smaller id: all packed values of a token are distinct.
__device__ inline unsigned long long pack_logit(float v, int e) {
  return ((unsigned long long)float_key(v) << 32) | (uint32_t)(~(uint32_t)e);
}


// Orders LDS accesses of one wavefront (its lanes exchange data through LDS).
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier that orders LDS only: this wavefront's LDS accesses are
// complete, then every wavefront has arrived. Unlike __syncthreads it does not
// wait for outstanding global stores, which no wavefront of the workgroup
// reads back.
__device__ inline void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// ------------------------------------------------------------------ router
// One wavefront per token ([PE] "What does Paged Experts actually do?": each
// token goes to top_k of E experts). Every logit's rank is the number of
// packed (logit, id) values above it, counted over the token's E values in
// LDS; ranks 0..k-1 are the selection, listed by descending logit with equal
// logits in ascending id. The weights are the softmax of the selected logits,
// which equals the softmax over all E renormalised over the selected k.
// pk: wavefront-private LDS of E (rounded up to even) entries, 16-byte
// aligned; zs: of k entries. Lane l owns experts l, l+64, ... (NJ of them).
template <int NJ>
__device__ inline void route_token(const float* __restrict__ z, int E, int k, int lane,
                                   unsigned long long* pk, float* zs, int32_t* ids_out,
                                   float* w_out) {
  unsigned long long mine[NJ];
  float zv[NJ];
  // every load issued before any is used (indices clamped in range, the
  // lanes past E discard theirs)
#pragma unroll
  for (int j = 0; j < NJ; ++j) zv[j] = z[min(lane + kWave * j, E - 1)];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + kWave * j;
    mine[j] = ~0ull;
    if (e < E) {
      mine[j] = pack_logit(zv[j], e);
      pk[e] = mine[j];
    } else {
      zv[j] = 0.f;
    }
  }
  // a zero entry is below every packed logit, so it pads E to even harmlessly
  if ((E & 1) && lane == 0) pk[E] = 0ull;
  wave_lds_sync();
  int rank[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) rank[j] = 0;
  const ulonglong2* pk2 = (const ulonglong2*)pk;
  const int n2 = (E + 1) >> 1;
#pragma unroll 8
  for (int u = 0; u < n2; ++u) {
    const ulonglong2 v = pk2[u];  // same address in every lane: a broadcast read
#pragma unroll
    for (int j = 0; j < NJ; ++j) rank[j] += (v.x > mine[j] ? 1 : 0) + (v.y > mine[j] ? 1 : 0);
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + kWave * j;
    if (e < E && rank[j] < k) {
      ids_out[rank[j]] = e;
      zs[rank[j]] = zv[j];
    }
  }
  wave_lds_sync();
  const float zr = lane < k ? zs[lane] : 0.f;
  const float zmax = zs[0];
  const float ex = lane < k ? __expf(zr - zmax) : 0.f;
  const float sum = wave_sum(ex);
  if (lane < k) w_out[lane] = ex / sum;
  wave_lds_sync();
}

// Large steps: 4 wavefronts per workgroup, one token each.
template <int NJ>
__global__ __launch_bounds__(256) void router_kernel(const float* __restrict__ logits, int T, int E,
                                                     int k, int32_t* __restrict__ ids,
                                                     float* __restrict__ weights) {
  __shared__ __attribute__((aligned(16))) unsigned long long s_pk[4][MOE_MAX_EXPERTS];
  __shared__ float s_z[4][MOE_MAX_TOP_K];
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int t = blockIdx.x * 4 + wid;
  if (t >= T) return;  // uniform per wavefront; no workgroup barrier below
  route_token<NJ>(logits + (size_t)t * E, E, k, lane, s_pk[wid], s_z[wid], ids + (size_t)t * k,
                  weights + (size_t)t * k);
}

// ------------------------------------------------------------------ block scan
// Exclusive prefix sum over a block of NT threads; *total gets the sum.
template <int NT>
__device__ inline int block_exscan(int v, int* s_warp, int* total) {
  constexpr int NWV = NT / kWave;
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
    const int w = lane < NWV ? s_warp[lane] : 0;
    int winc = w;
#pragma unroll
    for (int off = 1; off < NWV; off <<= 1) {
      const int o = __shfl_up(winc, off, kWave);
      if (lane >= off) winc += o;
    }
    if (lane < NWV) s_warp[lane] = winc - w;
    if (lane == NWV - 1) s_warp[NWV] = winc;
  }
  __syncthreads();
  const int res = s_warp[wid] + inc - v;
  *total = s_warp[NWV];
  __syncthreads();
  return res;
}

// ------------------------------------------------------------------ slot plan
// One workgroup of NT >= E threads; thread e owns expert e, thread s owns slot s.
// [PE] "TL;DR" / "What does Paged Experts actually do?": only routed experts
// that are not resident are copied in, the least recently used slot goes out.
// [PE] "What happens with more than one request?": a step that routes more
// distinct experts than fit runs as several waves, each with its own page-in.
// Readings (the oracle follows the same ones): residents first then missing
// experts, each ascending; waves are chunks of K; the clock ticks per wave;
// victims are slots not used by the wave, ordered by (stamp, slot); the i-th
// missing expert goes to the i-th victim.
struct PlanSmem {
  int cnt[MOE_MAX_EXPERTS];
  int pos[MOE_MAX_EXPERTS];
  int order_e[MOE_MAX_EXPERTS];
  int order_s[MOE_MAX_EXPERTS];
  int slot_expert[MOE_MAX_EXPERTS];
  int expert_slot[MOE_MAX_EXPERTS];
  long long stamp[MOE_MAX_EXPERTS];
  __attribute__((aligned(16))) unsigned long long vkey[MOE_MAX_EXPERTS];
  int cpos[MOE_MAX_EXPERTS];  // routed pairs of each wave-order position (one-wavefront plan)
  int warp[MOE_MAX_EXPERTS / kWave + 1];
};

// Victim order key of a slot: empty slots (stamp -1) first, then by stamp,
// then by slot index; slots of the current wave never become victims.
__device__ inline unsigned long long victim_key(long long stamp, int slot, bool prot) {
  return prot ? ~0ull : (((unsigned long long)(stamp + 1)) << 11) | (unsigned)slot;
}

// This thread's part of the table state, loaded from HBM (issued early so
// that its latency overlaps other work).
struct StateRegs {
  int expert_slot, slot_expert;
  long long stamp, clock;
};

__device__ inline StateRegs load_state(const uint8_t* state, const StateLayout& sl, int E, int K) {
  const int tid = threadIdx.x;
  StateRegs r;
  r.expert_slot = tid < E ? ((const int32_t*)(state + sl.expert_slot))[tid] : -1;
  r.slot_expert = tid < K ? ((const int32_t*)(state + sl.slot_expert))[tid] : -1;
  r.stamp = tid < K ? ((const long long*)(state + sl.stamp))[tid] : 0;
  r.clock = *(const long long*)(state + sl.clock);
  return r;
}

// ids: the step's routed ids (LDS or global), P = T * k of them.
template <int NT>
__device__ void plan_body(const int32_t* ids, int P, int T, int E, int K, uint8_t* state,
                          const StateLayout& sl, const StateRegs& pre, const PlanDev& dev,
                          PlanSmem& sm, int* D_out, int* nH_out, int* nw_out) {
  int32_t* g_slot_expert = (int32_t*)(state + sl.slot_expert);
  int32_t* g_expert_slot = (int32_t*)(state + sl.expert_slot);
  long long* g_stamp = (long long*)(state + sl.stamp);
  long long* g_clock = (long long*)(state + sl.clock);

  const int tid = threadIdx.x;
  if (tid < E) {
    sm.cnt[tid] = 0;
    sm.expert_slot[tid] = pre.expert_slot;
  }
  if (tid < K) {
    sm.slot_expert[tid] = pre.slot_expert;
    sm.stamp[tid] = pre.stamp;
  }
  long long clock = pre.clock;
  __syncthreads();
#pragma unroll 4
  for (int p = tid; p < P; p += NT) atomicAdd(&sm.cnt[ids[p]], 1);
  __syncthreads();

  const bool ref = tid < E && sm.cnt[tid] > 0;
  const bool hit = ref && sm.expert_slot[tid] >= 0;
  const bool miss = ref && !hit;
  int nH, nM;
  const int hit_rank = block_exscan<NT>(hit ? 1 : 0, sm.warp, &nH);
  const int miss_rank = block_exscan<NT>(miss ? 1 : 0, sm.warp, &nM);
  const int D = nH + nM;
  if (tid < E) {
    const int pos = hit ? hit_rank : (miss ? nH + miss_rank : -1);
    sm.pos[tid] = pos;
    if (pos >= 0) sm.order_e[pos] = tid;
  }
  const int n_waves = (D + K - 1) / K;
  __syncthreads();

  for (int w = 0; w < n_waves; ++w) {
    clock += 1;
    const int lo = w * K;
    const int hi = min(lo + K, D);
    const int m_lo = max(lo, nH);
    const int nm = hi - m_lo;
    unsigned long long my_key = ~0ull;
    if (tid < K) {
      const int e = sm.slot_expert[tid];
      const bool prot = e >= 0 && sm.pos[e] >= lo && sm.pos[e] < hi;
      my_key = victim_key(sm.stamp[tid], tid, prot);
      sm.vkey[tid] = my_key;
    }
    __syncthreads();
    if (tid < K && my_key != ~0ull && nm > 0) {
      int rank = 0;
      for (int s = 0; s < K; ++s) rank += sm.vkey[s] < my_key ? 1 : 0;
      if (rank < nm) {
        const int e_new = sm.order_e[m_lo + rank];
        const int old = sm.slot_expert[tid];
        if (old >= 0) sm.expert_slot[old] = -1;
        sm.slot_expert[tid] = e_new;
        sm.expert_slot[e_new] = tid;
        sm.order_s[m_lo + rank] = tid;
      }
    }
    __syncthreads();
    if (tid >= lo && tid < min(hi, nH)) sm.order_s[tid] = sm.expert_slot[sm.order_e[tid]];
    __syncthreads();
    if (tid >= lo && tid < hi) sm.stamp[sm.order_s[tid]] = clock;
    __syncthreads();
  }

  // table state back to HBM
  if (tid < E) g_expert_slot[tid] = sm.expert_slot[tid];
  if (tid < K) {
    g_slot_expert[tid] = sm.slot_expert[tid];
    g_stamp[tid] = sm.stamp[tid];
  }
  if (tid == 0) *g_clock = clock;

  // per-pair slot and wave
#pragma unroll 4
  for (int p = tid; p < P; p += NT) {
    const int pos = sm.pos[ids[p]];
    dev.slot_ids[p] = sm.order_s[pos];
    dev.wave_of[p] = pos / K;
  }
  // CSR offsets of the pairs of each expert, in wave order
  int total;
  const int c = tid < D ? sm.cnt[sm.order_e[tid]] : 0;
  const int off = block_exscan<NT>(c, sm.warp, &total);
  if (tid < E) dev.pair_off[tid] = tid < D ? off : P;
  if (tid == 0) dev.pair_off[E] = P;
  if (tid < D) {
    dev.order_expert[tid] = sm.order_e[tid];
    dev.order_slot[tid] = sm.order_s[tid];
  }
  if (tid == 0) {
    dev.counts[0] = D;
    dev.counts[1] = nH;
    dev.counts[2] = n_waves;
    dev.counts[3] = T;
  }
  if (tid < D) sm.cnt[tid] = off;  // from here on: pair offset of order position tid
  __syncthreads();
  *D_out = D;
  *nH_out = nH;
  *nw_out = n_waves;
}

// Publish the plan to pinned host memory: wavefront 0 writes the wave order
// and the header, makes its writes visible at system scope, then stores seq.
// Device-resolved steps pass no header: their plan stays on the device.
template <class SM>
__device__ void publish(const SM& sm, int E, int T, int P, int D, int nH, int n_waves,
                        PlanHdr* hdr, int32_t seq) {
  if (!hdr || threadIdx.x >= kWave) return;
  int32_t* h_order_e = (int32_t*)(hdr + 1);
  int32_t* h_order_s = h_order_e + E;
  int32_t* h_pair_off = h_order_s + E;
  for (int i = threadIdx.x; i < D; i += kWave) {
    h_order_e[i] = sm.order_e[i];
    h_order_s[i] = sm.order_s[i];
    h_pair_off[i] = sm.cnt[i];
  }
  if (threadIdx.x == 0) h_pair_off[D] = P;
  if (threadIdx.x == 0) {
    hdr->num_tokens = T;
    hdr->num_distinct = D;
    hdr->num_hits = nH;
    hdr->num_waves = n_waves;
  }
  __threadfence_system();
  if (threadIdx.x == 0) __hip_atomic_store(&hdr->seq, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

template <int NT>
__global__ __launch_bounds__(NT) void plan_kernel(const int32_t* __restrict__ ids, int P, int T,
                                                  int E, int K, uint8_t* state, StateLayout sl,
                                                  PlanDev dev, PlanHdr* hdr, int32_t seq) {
  __shared__ PlanSmem sm;
  const StateRegs pre = load_state(state, sl, E, K);
  int D, nH, nw;
  plan_body<NT>(ids, P, T, E, K, state, sl, pre, dev, sm, &D, &nH, &nw);
  publish(sm, E, T, P, D, nH, nw, hdr, seq);
}

// Grouping of a small step: wavefronts W0 .. NWV-1 take the order positions
// round robin (wavefront W0 + r takes r, r + NWV - W0, ...) and collect each
// position's pairs by ballots over the step's ids (in LDS), ascending, at the
// CSR offsets the plan left in sm.cnt (indexed by order position).
// wts: the step's router weights by pair index (LDS, or global memory written
// by this workgroup before a barrier); copied into CSR order as pair_w.
template <int NWV, int W0, class SM>
__device__ inline void group_small(const SM& sm, const int32_t* s_ids, const float* wts, int P, int D,
                                   const PlanDev& dev) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  if (wid < W0) return;
  for (int i = wid - W0; i < D; i += NWV - W0) {
    const int e = sm.order_e[i];
    const int base = sm.cnt[i];
    int running = 0;
    for (int c = 0; c < P; c += kWave) {
      const int p = c + lane;
      const bool m = p < P && s_ids[p] == e;
      const unsigned long long mask = __ballot(m);
      if (m) {
        const int q = base + running + __popcll(mask & below);
        dev.pair_list[q] = p;
        dev.pair_pos[p] = q;
        dev.pair_w[q] = wts[p];
      }
      running += __popcll(mask);
    }
  }
}

// Device-resolved steps: accumulate the step counters (steps, distinct
// experts, activations, hits, misses, waves) by no-return atomic adds.
// Threads t0 .. t0 + 5 issue the six adds.
__device__ inline void add_dstats(long long* dstats, int T, int P, int D, int nH, int nw, int t0) {
  const int t = (int)threadIdx.x - t0;
  if (dstats && t >= 0 && t < 6 && T > 0) {
    const long long v[6] = {1, D, P, nH, D - nH, nw};
    __hip_atomic_fetch_add(dstats + t, v[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Decode-sized steps (T <= 64, T * k <= kSmallPairs): router, slot plan and
// grouping in one workgroup, one launch.
constexpr int kSmallPairs = 2048;

// dstats, if given (device-resolved steps), accumulates the step counters on
// the device: steps, distinct experts, activations, hits, misses, waves.
template <int NT, int NJ>
__global__ __launch_bounds__(NT) void route_plan_small_kernel(const float* __restrict__ logits, int T,
                                                              int E, int k, int K, uint8_t* state,
                                                              StateLayout sl, PlanDev dev,
                                                              PlanHdr* hdr, int32_t seq,
                                                              long long* dstats) {
  constexpr int NWV = NT / kWave;
  __shared__ PlanSmem sm;
  __shared__ int32_t s_ids[kSmallPairs];
  __shared__ float s_z[NWV][MOE_MAX_TOP_K];
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int P = T * k;
  const StateRegs pre = load_state(state, sl, E, K);
  // the router's per-token LDS borrows the victim-key array (unused until the plan)
  unsigned long long* pk = sm.vkey + 0;
  const int per_wave = MOE_MAX_EXPERTS / NWV;
  if (E < per_wave) {
    for (int t = wid; t < T; t += NWV)
      route_token<NJ>(logits + (size_t)t * E, E, k, lane, pk + wid * per_wave, s_z[wid],
                      s_ids + t * k, dev.weights + (size_t)t * k);
  } else if (wid == 0) {
    for (int t = 0; t < T; ++t)
      route_token<NJ>(logits + (size_t)t * E, E, k, lane, pk, s_z[0], s_ids + t * k,
                      dev.weights + (size_t)t * k);
  }
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += NT) dev.ids[p] = s_ids[p];
  int D, nH, nw;
  plan_body<NT>(s_ids, P, T, E, K, state, sl, pre, dev, sm, &D, &nH, &nw);
  group_small<NWV, 0>(sm, s_ids, dev.weights, P, D, dev);
  add_dstats(dstats, T, P, D, nH, nw, 0);
  publish(sm, E, T, P, D, nH, nw, hdr, seq);
}

// ------------------------------------------------------------------ small steps, one planning wavefront
// The same router, plan and grouping as route_plan_small_kernel, for tables of
// E <= 64 * NJ experts (so K <= E slots fit 64 * NJ too). The plan is the
// serial part of a decode step, so it runs in wavefront 0 alone: lane l owns
// experts l + 64 j and slots l + 64 j, hit and miss ranks come from ballots
// and population counts, the CSR offsets from a wavefront scan, and the only
// synchronisation inside the plan is between the lanes of one wavefront.
// The other wavefronts route tokens before it and group pairs after it.

// Inclusive prefix sum over the 64 lanes.
__device__ inline int wave_incl_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// One token routed by all NWV wavefronts (single-token steps): each
// wavefront ranks the token's packed logits against one NWV-th of them, the
// partial ranks meet in LDS, and wavefront 0 lists the selection and computes
// the weights exactly as route_token does.
template <int NJ, int NWV>
__device__ inline void route_token_split(const float* __restrict__ z, int E, int k, int lane, int wid,
                                         unsigned long long* pk, int* rank_part, float* zs,
                                         int32_t* ids_out, float* w_out) {
  unsigned long long mine[NJ];
  float zv[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) zv[j] = z[min(lane + kWave * j, E - 1)];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + kWave * j;
    mine[j] = ~0ull;
    if (e < E) {
      mine[j] = pack_logit(zv[j], e);
      if (wid == 0) pk[e] = mine[j];
    } else {
      zv[j] = 0.f;
    }
  }
  if ((E & 1) && wid == 0 && lane == 0) pk[E] = 0ull;
  lds_barrier();
  const int n2 = (E + 1) >> 1;
  const int per = (n2 + NWV - 1) / NWV;
  const int u0 = wid * per, u1 = min(n2, u0 + per);
  int rank[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) rank[j] = 0;
  const ulonglong2* pk2 = (const ulonglong2*)pk;
#pragma unroll 4
  for (int u = u0; u < u1; ++u) {
    const ulonglong2 v = pk2[u];
#pragma unroll
    for (int j = 0; j < NJ; ++j) rank[j] += (v.x > mine[j] ? 1 : 0) + (v.y > mine[j] ? 1 : 0);
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + kWave * j;
    if (e < E) rank_part[wid * (kWave * NJ) + e] = rank[j];
  }
  lds_barrier();
  if (wid != 0) return;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + kWave * j;
    if (e < E) {
      int r = 0;
#pragma unroll
      for (int w = 0; w < NWV; ++w) r += rank_part[w * (kWave * NJ) + e];
      if (r < k) {
        ids_out[r] = e;
        zs[r] = zv[j];
      }
    }
  }
  wave_lds_sync();
  const float zr = lane < k ? zs[lane] : 0.f;
  const float zmax = zs[0];
  const float ex = lane < k ? __expf(zr - zmax) : 0.f;
  const float sum = wave_sum(ex);
  if (lane < k) w_out[lane] = ex / sum;
  wave_lds_sync();
}

// The table state a planning lane owns, loaded at kernel start.
template <int NJ>
struct LaneState {
  int expert_slot[NJ], slot_expert[NJ];
  long long stamp[NJ], clock;
};

template <int NJ>
__device__ inline LaneState<NJ> load_lane_state(const uint8_t* state, const StateLayout& sl, int E, int K) {
  const int lane = threadIdx.x & (kWave - 1);
  LaneState<NJ> r;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int i = lane + kWave * j;
    r.expert_slot[j] = i < E ? ((const int32_t*)(state + sl.expert_slot))[i] : -1;
    r.slot_expert[j] = i < K ? ((const int32_t*)(state + sl.slot_expert))[i] : -1;
    r.stamp[j] = i < K ? ((const long long*)(state + sl.stamp))[i] : 0;
  }
  r.clock = *(const long long*)(state + sl.clock);
  return r;
}

// The slot plan of plan_body, run by one wavefront (wavefront 0). ids: the
// step's P routed ids in LDS. Leaves in LDS what the grouping and the publish
// read: order_e / order_s by wave-order position, pos by expert, cnt by
// position (CSR offsets), and D, nH, n_waves in warp[0..2]; the table state
// and offsets for the stores in `out`. It issues no global memory access.
// Each lane keeps its slots' expert and stamp in registers. Two facts of the
// plan keep the LDS traffic small: the slots a wave protects are, in wave 0,
// exactly the slots of the hits (every hit is in wave 0 and no miss is resident
// when its wave starts) and, in later waves, none; and a hit keeps the slot it
// had at the start of the step during wave 0.
// LDS of the one-wavefront route and plan for tables of E <= 64 * NJ experts
// (and K <= E slots): per expert, per wave-order position, the router's
// scratch (four wavefronts' packed logits) shared with the victim keys.
template <int NJ>
struct WavePlanSmem {
  static constexpr int N = kWave * NJ;
  int cnt[N];
  int pos[N];
  int order_e[N];
  int order_s[N];
  int expert_slot[N];
  int cpos[N];
  __attribute__((aligned(16))) unsigned long long vkey[4 * N];
  int warp[4];
};

// What plan_wave leaves in registers for plan_wave_store.
template <int NJ>
struct PlanOut {
  int se[NJ], off[NJ];
  long long st[NJ], clock;
};

template <int NJ, class SM>
__device__ void plan_wave(const int32_t* ids, int P, int E, int K, const LaneState<NJ>& pre,
                          SM& sm, PlanOut<NJ>& out) {
  const int lane = threadIdx.x & (kWave - 1);
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int se[NJ];
  long long st[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int i = lane + kWave * j;
    se[j] = pre.slot_expert[j];
    st[j] = pre.stamp[j];
    if (i < E) {
      sm.cnt[i] = 0;
      sm.expert_slot[i] = pre.expert_slot[j];
    }
  }
  wave_lds_sync();
  for (int p = lane; p < P; p += kWave) atomicAdd(&sm.cnt[ids[p]], 1);
  wave_lds_sync();

  // routed count of each owned expert; whether each owned slot holds a routed
  // (hence hit) expert
  int c[NJ];
  bool hit_slot[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int i = lane + kWave * j;
    c[j] = i < E ? sm.cnt[i] : 0;
    hit_slot[j] = i < K && se[j] >= 0 && sm.cnt[se[j]] > 0;
  }
  // referenced experts: residents (hits) first, then missing ones, each ascending
  unsigned long long hm[NJ], mm[NJ];
  int nH = 0, nM = 0, hb[NJ], mb[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const bool hit = c[j] > 0 && pre.expert_slot[j] >= 0;
    hm[j] = __ballot(hit);
    mm[j] = __ballot(c[j] > 0 && !hit);
    hb[j] = nH;
    mb[j] = nM;
    nH += __popcll(hm[j]);
    nM += __popcll(mm[j]);
  }
  const int D = nH + nM;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + kWave * j;
    const bool hit = (hm[j] >> lane) & 1, miss = (mm[j] >> lane) & 1;
    const int pos = hit ? hb[j] + __popcll(hm[j] & below)
                        : (miss ? nH + mb[j] + __popcll(mm[j] & below) : -1);
    if (e < E) sm.pos[e] = pos;
    if (pos >= 0) {
      sm.order_e[pos] = e;
      sm.cpos[pos] = c[j];
      if (hit) sm.order_s[pos] = pre.expert_slot[j];
    }
  }
  const int n_waves = (D + K - 1) / K;
  long long clock = pre.clock;
  wave_lds_sync();

  for (int w = 0; w < n_waves; ++w) {
    clock += 1;
    const int lo = w * K;
    const int hi = min(lo + K, D);
    const int m_lo = max(lo, nH);
    const int nm = hi - m_lo;
    unsigned long long key[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int s = lane + kWave * j;
      key[j] = ~0ull;
      if (s < K) {
        if (w == 0 && hit_slot[j]) st[j] = clock;  // protected: a hit of this wave
        else key[j] = victim_key(st[j], s, false);
        sm.vkey[s] = key[j];
      }
    }
    if ((K & 1) && lane == 0) sm.vkey[K] = ~0ull;  // pads the pairwise reads; never below a key
    wave_lds_sync();
    if (nm > 0) {
      int rank[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) rank[j] = 0;
      const ulonglong2* v2 = (const ulonglong2*)sm.vkey;
      const int n2 = (K + 1) >> 1;
#pragma unroll 4
      for (int u = 0; u < n2; ++u) {
        const ulonglong2 v = v2[u];
#pragma unroll
        for (int j = 0; j < NJ; ++j) rank[j] += (v.x < key[j] ? 1 : 0) + (v.y < key[j] ? 1 : 0);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int s = lane + kWave * j;
        if (s < K && key[j] != ~0ull && rank[j] < nm) {
          const int q = m_lo + rank[j];
          const int e_new = sm.order_e[q];
          if (se[j] >= 0) sm.expert_slot[se[j]] = -1;
          sm.expert_slot[e_new] = s;
          se[j] = e_new;
          st[j] = clock;
          sm.order_s[q] = s;
        }
      }
    }
    wave_lds_sync();  // the next wave rewrites vkey; the write-back reads expert_slot
  }

  // CSR offsets over the wave order (the stores wait for plan_wave_store)
  int carry = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int i = lane + kWave * j;
    out.off[j] = P;
    if (kWave * j < D) {  // uniform: positions past D need no scan
      const int cj = i < D ? sm.cpos[i] : 0;
      const int inc = wave_incl_scan(cj);
      out.off[j] = carry + inc - cj;
      carry += __shfl(inc, kWave - 1, kWave);
    }
    out.se[j] = se[j];
    out.st[j] = st[j];
  }
  out.clock = clock;
  if (lane == 0) {
    sm.warp[0] = D;
    sm.warp[1] = nH;
    sm.warp[2] = n_waves;
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int i = lane + kWave * j;
    if (i < D) sm.cnt[i] = out.off[j];  // from here on: CSR offset of order position i
  }
}

// The global stores of plan_wave (same wavefront, after the workgroup has
// passed the barrier that follows the plan): the table state (with_state),
// the wave order with its slots, the CSR offsets and the counters
// (with_order). Issued together with the per-pair stores of the other
// wavefronts, so their latencies overlap.
template <int NJ, class SM>
__device__ void plan_wave_store(const PlanOut<NJ>& out, int P, int T, int E, int K, uint8_t* state,
                                const StateLayout& sl, const PlanDev& dev, const SM& sm, int D,
                                int nH, int n_waves, bool with_state = true, bool with_order = true) {
  int32_t* g_slot_expert = (int32_t*)(state + sl.slot_expert);
  int32_t* g_expert_slot = (int32_t*)(state + sl.expert_slot);
  long long* g_stamp = (long long*)(state + sl.stamp);
  long long* g_clock = (long long*)(state + sl.clock);
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int i = lane + kWave * j;
    if (with_state) {
      if (i < E) g_expert_slot[i] = sm.expert_slot[i];
      if (i < K) {
        g_slot_expert[i] = out.se[j];
        g_stamp[i] = out.st[j];
      }
    }
    if (with_order) {
      if (i < E) dev.pair_off[i] = i < D ? out.off[j] : P;
      if (i < D) {
        dev.order_expert[i] = sm.order_e[i];
        dev.order_slot[i] = sm.order_s[i];
      }
    }
  }
  if (lane == 0) {
    if (with_state) *g_clock = out.clock;
    if (with_order) {
      dev.pair_off[E] = P;
      dev.counts[0] = D;
      dev.counts[1] = nH;
      dev.counts[2] = n_waves;
      dev.counts[3] = T;
    }
  }
}

// ------------------------------------------------------------------ small steps, one launch
// Router, one-wavefront plan and grouping of a decode-sized step (E <= 256).
//
// route_plan_wave_kernel (PAGE_IN = false): one workgroup; the plan is stored
// and, for host-driven steps, published to the host.
//
// route_plan_page_in_kernel (PAGE_IN = true; device-resolved single-wave steps, [PE] "What happens with
// more than one request?": the single wave is the step a graph can capture;
// "TL;DR": only the routed experts that are not resident are copied in):
// kPageInBlocks workgroups each route and plan the step from the same inputs,
// so each holds the same plan in its LDS, and each then copies its share of
// the missed records from the device-mapped host store into their slots: no
// second launch and no exchange between workgroups. Workgroup 0 stores the
// plan, the pairs and the counters. The table state may be rewritten only once
// every workgroup has read it: each takes a ticket from a counter after its
// plan (which has consumed the state), and the workgroup holding the last
// ticket of the launch stores the new state. The counter grows by the grid
// size per launch, so "last" is a ticket that is one below a multiple of it.
constexpr int kPageInBlocks = 64;
constexpr int kCopyUnroll = 4;
constexpr int kPageInPairs = 256;  // a device-resolved step: T * top_k <= K <= E <= 256

// vblock / nblocks: this workgroup's index among the nblocks workgroups that
// route, plan and page in the step (PAGE_IN), which may be a part of a larger
// launch; PM: the most pairs (T * top_k) a step may have.
template <int NJ, bool PAGE_IN, int PM>
__device__ void route_plan_body(const float* __restrict__ logits, int T, int E, int k, int K, uint8_t* state,
                                const StateLayout& sl, const PlanDev& dev, PlanHdr* hdr, int32_t seq,
                                long long* dstats, unsigned long long* ticket, const uint8_t* __restrict__ host,
                                uint8_t* __restrict__ slots, size_t stride, int vblock, int nblocks,
                                size_t cp_len) {
  constexpr int NT = 256, NWV = NT / kWave;
  __shared__ WavePlanSmem<NJ> sm;
  __shared__ int32_t s_ids[PM];
  __shared__ float s_z[NWV][MOE_MAX_TOP_K];
  __shared__ int s_rank[NWV * kWave * NJ];
  __shared__ float s_w[PM];
  __shared__ int s_last;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int P = T * k;
  LaneState<NJ> pre;
  if (wid == 0) pre = load_lane_state<NJ>(state, sl, E, K);
  // Ids and weights stay in LDS until the plan is done: a global store issued
  // before it would make the plan's first use of the table state wait for the
  // store as well (loads and stores share one counter). The router's per-token
  // LDS borrows the victim-key array (unused until the plan).
  if (T == 1) {
    route_token_split<NJ, NWV>(logits, E, k, lane, wid, sm.vkey, s_rank, s_z[0], s_ids, s_w);
  } else {
    for (int t = wid; t < T; t += NWV)
      route_token<NJ>(logits + (size_t)t * E, E, k, lane, sm.vkey + wid * (kWave * NJ), s_z[wid],
                      s_ids + t * k, s_w + t * k);
  }
  lds_barrier();
  PlanOut<NJ> out;
  if (wid == 0) {
    plan_wave<NJ>(s_ids, P, E, K, pre, sm, out);
    if (PAGE_IN && lane == 0) {
      const unsigned long long tk =
          __hip_atomic_fetch_add(ticket, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = (tk + 1) % nblocks == 0;
    }
  }
  lds_barrier();
  const int D = sm.warp[0], nH = sm.warp[1], nw = sm.warp[2];
  const bool lead = !PAGE_IN || vblock == 0;  // stores the plan, pairs and counters
  const bool last = !PAGE_IN || s_last != 0;      // stores the table state
  // wavefront 0 stores the plan while wavefronts 1 .. NWV-1 store the pairs
  if (wid == 0 && (lead || last)) plan_wave_store<NJ>(out, P, T, E, K, state, sl, dev, sm, D, nH, nw, last, lead);
  if (lead) {
    if (wid > 0) {  // per-pair id, weight, slot and wave
      for (int p = (int)threadIdx.x - kWave; p < P; p += NT - kWave) {
        const int e = s_ids[p];
        const int pos = sm.pos[e];
        dev.ids[p] = e;
        dev.weights[p] = s_w[p];
        dev.slot_ids[p] = sm.order_s[pos];
        dev.wave_of[p] = pos / K;
      }
    }
    group_small<NWV, 1>(sm, s_ids, s_w, P, D, dev);
    add_dstats(dstats, T, P, D, nH, nw, kWave);
  }
  if constexpr (PAGE_IN) {
    // this workgroup's share of the first cp_len bytes of every missed record
    // (the single wave's order positions nH .. D-1; the rest, if any, is
    // copied by the next launch)
    for (int m = nH; m < D; ++m)
      copy_record_share<NT, kCopyUnroll>(host + (size_t)sm.order_e[m] * stride, slots + (size_t)sm.order_s[m] * stride,
                                         cp_len, vblock, nblocks);
  } else {
    publish(sm, E, T, P, D, nH, nw, hdr, seq);
  }
}

template <int NJ>
__global__ __launch_bounds__(256) void route_plan_wave_kernel(const float* __restrict__ logits, int T, int E,
                                                              int k, int K, uint8_t* state, StateLayout sl,
                                                              PlanDev dev, PlanHdr* hdr, int32_t seq,
                                                              long long* dstats) {
  route_plan_body<NJ, false, kSmallPairs>(logits, T, E, k, K, state, sl, dev, hdr, seq, dstats, nullptr,
                                          nullptr, nullptr, 0, 0, 1, 0);
}

// cp_len: bytes of each missed record copied (the record stride for a whole
// page-in, 0 to route and plan only).
template <int NJ>
__global__ __launch_bounds__(256) void route_plan_page_in_kernel(const float* __restrict__ logits, int T,
                                                                 int E, int k, int K, uint8_t* state,
                                                                 StateLayout sl, PlanDev dev, long long* dstats,
                                                                 unsigned long long* ticket,
                                                                 const uint8_t* __restrict__ host,
                                                                 uint8_t* __restrict__ slots, size_t stride,
                                                                 size_t cp_len) {
  route_plan_body<NJ, true, kPageInPairs>(logits, T, E, k, K, state, sl, dev, nullptr, 0, dstats, ticket, host,
                                          slots, stride, blockIdx.x, gridDim.x, cp_len);
}

// One launch of a stack's device-resolved steps with lookahead ([PE] "TL;DR":
// the expert math stays on the GPU while experts cross PCIe), three groups of
// workgroups: 0 .. kPageInBlocks-1 copy the first n.cp_len bytes of each
// record that the NEXT layer's plan (stored by an earlier launch) pages in
// (the down launch that follows copies the rest); the next nroute route and
// plan the layer AFTER the next one exactly as route_plan_page_in_kernel
// does, without copying, so that its copies can start at the beginning of the
// next layer's up launch; the others run THIS layer's up projection exactly
// as ffn_up_kernel does (its gx x experts grid numbered row by row). The
// copies and the routing run beside this layer's math in one queue; the
// launch's end orders them before this layer's down projection and the next
// layer's up projection.
template <int F, int NJ, int RPW, int NJR>
__global__ __launch_bounds__(256) void up_route_next_kernel(FfnArgs a, int gx, NextStep n, NextStep r,
                                                            int nroute) {
  const int b = blockIdx.x;
  if (b < kPageInBlocks) {
    const int D = n.dev.counts[0], nH = n.dev.counts[1];
    for (int m = nH; m < D; ++m) {
      const int e = n.dev.order_expert[m], sl = n.dev.order_slot[m];
      if (e < 0 || e >= n.E || sl < 0 || sl >= n.K) continue;  // never produced by the plan
      copy_record_share<256, kCopyUnroll>(n.host + (size_t)e * n.stride, n.slots + (size_t)sl * n.stride,
                                          n.cp_len, b, kPageInBlocks);
    }
    return;
  }
  if (b < kPageInBlocks + nroute) {
    route_plan_body<NJR, true, kPageInPairs>(r.logits, r.T, r.E, r.k, r.K, r.state, r.sl, r.dev, nullptr, 0,
                                             r.dstats, r.ticket, r.host, r.slots, r.stride, b - kPageInBlocks,
                                             nroute, 0);
    return;
  }
  const int u = b - kPageInBlocks - nroute;
  gemv::ffn_up_body<F, NJ, RPW, uint16_t>(a, u % gx, u / gx);
}

template <int F, int NJR>
hipError_t up_route_next_nj(const FfnArgs& a, const NextStep& n, const NextStep* r, hipStream_t s) {
  constexpr int kRPW = gemv::rpw<F>();
  const int nj = (a.H / gemv::Fmt<F>::CV1 + kWave - 1) / kWave;
  const int gx = (a.I + 4 * kRPW - 1) / (4 * kRPW);
  const int nroute = r ? kPageInBlocks : 0;
  const NextStep rr = r ? *r : n;
  const dim3 grid(kPageInBlocks + nroute + gx * a.n_exp), block(256);
  switch (nj) {
    case 1: launch_k(up_route_next_kernel<F, 1, kRPW, NJR>, grid, block, s, a.ev0, a.ev1, a, gx, n, rr, nroute); break;
    case 2: launch_k(up_route_next_kernel<F, 2, kRPW, NJR>, grid, block, s, a.ev0, a.ev1, a, gx, n, rr, nroute); break;
    case 4: launch_k(up_route_next_kernel<F, 4, kRPW, NJR>, grid, block, s, a.ev0, a.ev1, a, gx, n, rr, nroute); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int F>
hipError_t up_route_next_fmt(const FfnArgs& a, const NextStep& n, const NextStep* r, hipStream_t s) {
  if (n.E <= 64) return up_route_next_nj<F, 1>(a, n, r, s);
  if (n.E <= 128) return up_route_next_nj<F, 2>(a, n, r, s);
  return up_route_next_nj<F, 4>(a, n, r, s);
}

// ------------------------------------------------------------------ grouping
// One workgroup per position i of the wave order: a stable compaction of the
// pair indices routed to its expert, in ascending order (so the list, and
// every later summation order, is deterministic). Thread t owns 64 consecutive
// pairs of each round of 256 x 64: a 64-bit match mask, a workgroup exclusive
// scan of the match counts, then each thread writes its matches in order.
constexpr int kGroupThreads = 256;

__global__ __launch_bounds__(kGroupThreads) void group_kernel(const int32_t* __restrict__ ids, int P,
                                                              PlanDev dev) {
  __shared__ int s_warp[kGroupThreads / kWave + 1];
  const int i = blockIdx.x;
  const int D = dev.counts[0];
  if (i >= D) return;  // uniform over the workgroup
  const int e = dev.order_expert[i];
  int running = dev.pair_off[i];
  for (int r0 = 0; r0 < P; r0 += kGroupThreads * 64) {
    const int p0 = r0 + threadIdx.x * 64;
    unsigned long long m = 0;
    if (p0 + 64 <= P) {
#pragma unroll
      for (int j = 0; j < 64; j += 4) {
        const int4 v = *(const int4*)(ids + p0 + j);  // p0 + j is a multiple of 4
        m |= (unsigned long long)(v.x == e) << j | (unsigned long long)(v.y == e) << (j + 1) |
             (unsigned long long)(v.z == e) << (j + 2) | (unsigned long long)(v.w == e) << (j + 3);
      }
    } else {
      for (int j = 0; p0 + j < P && j < 64; ++j) m |= (unsigned long long)(ids[p0 + j] == e) << j;
    }
    int total;
    int q = running + block_exscan<kGroupThreads>(__popcll(m), s_warp, &total);
    while (m) {
      const int p = p0 + __ffsll((long long)m) - 1;
      m &= m - 1;
      dev.pair_list[q] = p;
      dev.pair_pos[p] = q;
      dev.pair_w[q] = dev.weights[p];
      ++q;
    }
    running += total;
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

// Unit-gain RMSNorm, one workgroup per token row (staged in LDS, then the
// shared norm routine, then written out).
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const uint16_t* x, uint16_t* a, int H) {
  extern __shared__ uint4 row[];
  __shared__ float red[4];
  const int nx16 = H / 8;
  const uint4* src = (const uint4*)(x + (size_t)blockIdx.x * H);
  for (int c = threadIdx.x; c < nx16; c += kNormThreads) row[c] = src[c];
  __syncthreads();
  rmsnorm_row_lds(row, nx16, H, red);
  uint4* dst = (uint4*)(a + (size_t)blockIdx.x * H);
  for (int c = threadIdx.x; c < nx16; c += kNormThreads) dst[c] = row[c];
}

}  // namespace

hipError_t launch_rmsnorm(const uint16_t* x, uint16_t* a, int T, int H, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  rmsnorm_kernel<<<T, kNormThreads, (size_t)H * 2, s>>>(x, a, H);
  return hipGetLastError();
}

hipError_t launch_router(const float* logits, int T, int E, int k, int32_t* ids, float* weights,
                         hipStream_t s, hipEvent_t ev0) {
  if (T <= 0) return hipSuccess;
  const dim3 g((T + 3) / 4), b(256);
  if (E <= 64) launch_k(router_kernel<1>, g, b, s, ev0, nullptr, logits, T, E, k, ids, weights);
  else if (E <= 128) launch_k(router_kernel<2>, g, b, s, ev0, nullptr, logits, T, E, k, ids, weights);
  else if (E <= 256) launch_k(router_kernel<4>, g, b, s, ev0, nullptr, logits, T, E, k, ids, weights);
  else if (E <= 512) launch_k(router_kernel<8>, g, b, s, ev0, nullptr, logits, T, E, k, ids, weights);
  else launch_k(router_kernel<16>, g, b, s, ev0, nullptr, logits, T, E, k, ids, weights);
  return hipGetLastError();
}

hipError_t launch_plan(const int32_t* ids, int T, int k, int E, int K, void* state, PlanDev dev,
                       PlanHdr* host_hdr_dev, int32_t seq, hipStream_t s) {
  const StateLayout sl = state_layout(E, K);
  // the per-pair loops dominate for many pairs: use the widest block then
  if (E <= 256 && T * k <= 4096)
    plan_kernel<256><<<1, 256, 0, s>>>(ids, T * k, T, E, K, (uint8_t*)state, sl, dev, host_hdr_dev, seq);
  else
    plan_kernel<1024><<<1, 1024, 0, s>>>(ids, T * k, T, E, K, (uint8_t*)state, sl, dev, host_hdr_dev, seq);
  return hipGetLastError();
}

bool route_small_ok(int T, int k) { return T <= MOE_MAX_GEMV_TOKENS && T * k <= kSmallPairs; }

hipError_t launch_route_plan_small(const float* logits, int T, int E, int k, int K, void* state,
                                   PlanDev dev, PlanHdr* host_hdr_dev, int32_t seq, hipStream_t s,
                                   hipEvent_t ev0, hipEvent_t ev1, long long* dstats) {
  const StateLayout sl = state_layout(E, K);
  uint8_t* st = (uint8_t*)state;
#define MOE_SMALL(NT, NJ)                                                                   \
  launch_k(route_plan_small_kernel<NT, NJ>, dim3(1), dim3(NT), s, ev0, ev1, logits, T, E, k, K, st, \
           sl, dev, host_hdr_dev, seq, dstats)
#define MOE_WAVE(NJ)                                                                         \
  launch_k(route_plan_wave_kernel<NJ>, dim3(1), dim3(256), s, ev0, ev1, logits, T, E, k, K, st, sl, dev, \
           host_hdr_dev, seq, dstats)
  if (E <= 64) MOE_WAVE(1);
  else if (E <= 128) MOE_WAVE(2);
  else if (E <= 256) MOE_WAVE(4);
  else if (E <= 512) MOE_SMALL(1024, 8);
  else MOE_SMALL(1024, 16);
#undef MOE_SMALL
#undef MOE_WAVE
  return hipGetLastError();
}

bool route_page_in_ok(int E) { return E <= 256; }

bool up_route_next_ok(int fmt, int H, int E, int P) {
  if (E > 256 || P > kPageInPairs) return false;
  int cv1 = 0;
  switch (fmt) {
    case MOE_FMT_BF16: cv1 = 8; break;
    case MOE_FMT_FP8_E4M3_B128: cv1 = 16; break;
    case MOE_FMT_INT4_ASYM_G128:
    case MOE_FMT_MXFP4_B32: cv1 = 32; break;
    default: return false;
  }
  const int nj = (H / cv1 + kWave - 1) / kWave;
  return nj == 1 || nj == 2 || nj == 4;
}

hipError_t launch_up_route_next(const FfnArgs& a, const NextStep& n, const NextStep* r, hipStream_t s) {
  if (a.n_exp <= 0 || !up_route_next_ok(a.fmt, a.H, n.E, n.T * n.k)) return hipErrorInvalidValue;
  if (r && (r->E != n.E || !up_route_next_ok(a.fmt, a.H, r->E, r->T * r->k))) return hipErrorInvalidValue;
  switch (a.fmt) {
    case MOE_FMT_BF16: return up_route_next_fmt<MOE_FMT_BF16>(a, n, r, s);
    case MOE_FMT_FP8_E4M3_B128: return up_route_next_fmt<MOE_FMT_FP8_E4M3_B128>(a, n, r, s);
    case MOE_FMT_INT4_ASYM_G128: return up_route_next_fmt<MOE_FMT_INT4_ASYM_G128>(a, n, r, s);
    case MOE_FMT_MXFP4_B32: return up_route_next_fmt<MOE_FMT_MXFP4_B32>(a, n, r, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_route_plan_page_in(const float* logits, int T, int E, int k, int K, void* state, PlanDev dev,
                                     long long* dstats, unsigned long long* ticket, const uint8_t* host_store_dev,
                                     uint8_t* slots, size_t stride, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1,
                                     size_t cp_len) {
  if (T * k > kPageInPairs) return hipErrorInvalidValue;
  cp_len = cp_len < stride ? cp_len / 16 * 16 : stride;
  const StateLayout sl = state_layout(E, K);
  uint8_t* st = (uint8_t*)state;
#define MOE_FUSED(NJ)                                                                                    \
  launch_k(route_plan_page_in_kernel<NJ>, dim3(kPageInBlocks), dim3(256), s, ev0, ev1, logits, T, E, k, K, st, \
           sl, dev, dstats, ticket, host_store_dev, slots, stride, cp_len)
  if (E <= 64) MOE_FUSED(1);
  else if (E <= 128) MOE_FUSED(2);
  else if (E <= 256) MOE_FUSED(4);
  else return hipErrorInvalidValue;
#undef MOE_FUSED
  return hipGetLastError();
}

hipError_t launch_group(const int32_t* ids, int T, int k, int E, PlanDev dev, hipStream_t s,
                        hipEvent_t ev1) {
  if (T <= 0) return hipSuccess;
  launch_k(group_kernel, dim3(E < T * k ? E : T * k), dim3(kGroupThreads), s, nullptr, ev1, ids, T * k, dev);
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
