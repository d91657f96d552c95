// Internal declarations of libmoepage (not part of the ABI).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#include "moepage.h"

namespace moepage {

// Byte offsets of the per-layer table state (see moe_state_bytes).
struct StateLayout {
  size_t slot_expert, expert_slot, stamp, clock, total;
};

inline size_t align8(size_t v) { return (v + 7) & ~size_t(7); }

inline StateLayout state_layout(int E, int K) {
  StateLayout s;
  s.slot_expert = 0;
  s.expert_slot = align8(s.slot_expert + sizeof(int32_t) * (size_t)K);
  s.stamp = align8(s.expert_slot + sizeof(int32_t) * (size_t)E);
  s.clock = s.stamp + sizeof(int64_t) * (size_t)K;
  s.total = s.clock + sizeof(int64_t);
  return s;
}

// Header of the host-visible plan (pinned, mapped, coherent). The slot-plan
// kernel writes the header fields and the arrays that follow it (wave order,
// slot of each, CSR pair offsets over the wave order),
// then publishes `seq` with a system-scope release store; the host waits for
// seq to reach the value it expects.
struct PlanHdr {
  int32_t seq;
  int32_t num_tokens;
  int32_t num_distinct;
  int32_t num_hits;
  int32_t num_waves;
  int32_t pad[3];
  // int32_t order_expert[E]; int32_t order_slot[E]; int32_t pair_off[E + 1];
};

// Device-side arrays of a plan.
struct PlanDev {
  int32_t* ids;          // [T*k]
  float* weights;        // [T*k]
  int32_t* slot_ids;     // [T*k]
  int32_t* wave_of;      // [T*k]
  int32_t* order_expert; // [E] experts in wave order
  int32_t* order_slot;   // [E] slot of each during its wave
  int32_t* pair_off;     // [E+1] CSR offsets over wave order
  int32_t* pair_list;    // [T*k] pair index t*k+j, grouped by expert, ascending
  int32_t* pair_pos;     // [T*k] inverse of pair_list: CSR position of pair t*k+j
  float* pair_w;         // [T*k] router weight of the pair at each CSR position
  int32_t* counts;       // [4]: num_distinct, num_hits, num_waves, num_tokens
};

// Format traits shared by host validation and launch code.
__host__ __device__ inline int fmt_elem_bits(int fmt) {
  switch (fmt) {
    case MOE_FMT_F32: return 32;
    case MOE_FMT_BF16: return 16;
    case MOE_FMT_FP8_E4M3_B128: return 8;
    case MOE_FMT_INT4_ASYM_G128: return 4;
    case MOE_FMT_MXFP4_B32: return 4;
  }
  return 0;
}

// Byte offsets of the sections of one expert record.
struct RecLayout {
  size_t w13, wd, s13, sd, z13, zd, payload, stride;
};

__host__ __device__ inline RecLayout rec_layout(int fmt, int H, int I) {
  RecLayout r{};
  size_t n13 = (size_t)2 * I * H, nd = (size_t)H * I;
  int bits = fmt_elem_bits(fmt);
  r.w13 = 0;
  r.wd = n13 * bits / 8;
  size_t end = r.wd + nd * bits / 8;
  r.s13 = r.sd = r.z13 = r.zd = end;
  if (fmt == MOE_FMT_FP8_E4M3_B128) {
    r.s13 = end;
    r.sd = r.s13 + sizeof(float) * (size_t)(2 * I / 128) * (H / 128);
    end = r.sd + sizeof(float) * (size_t)(H / 128) * (I / 128);
  } else if (fmt == MOE_FMT_INT4_ASYM_G128) {
    size_t g13 = (size_t)2 * I * (H / 128), gd = (size_t)H * (I / 128);
    r.s13 = end;
    r.sd = r.s13 + 2 * g13;
    r.z13 = r.sd + 2 * gd;
    r.zd = r.z13 + 2 * g13;
    end = r.zd + 2 * gd;
  } else if (fmt == MOE_FMT_MXFP4_B32) {
    r.s13 = end;                                   // E8M0 bytes, one per 32 weights
    r.sd = r.s13 + (size_t)2 * I * (H / 32);
    end = r.sd + (size_t)H * (I / 32);
    r.z13 = r.zd = end;
  }
  r.payload = end;
  r.stride = (end + 255) / 256 * 256;
  return r;
}

// ---------------------------------------------------------------- launchers

// Launch a kernel; when timing events are given they are stamped by the
// dispatch itself (start and end of the kernel's execution on the stream).
template <typename K, typename... Args>
inline void launch_k(K kernel, dim3 grid, dim3 block, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1,
                     Args... args) {
  if (ev0 || ev1)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev0, ev1, 0, args...);
  else
    kernel<<<grid, block, 0, s>>>(args...);
}

// ev0 / ev1: optional timing events stamped at the start / end of the kernel.
hipError_t launch_router(const float* logits, int T, int E, int k, int32_t* ids, float* weights,
                         hipStream_t s, hipEvent_t ev0);

hipError_t launch_plan(const int32_t* ids, int T, int k, int E, int K, void* state,
                       PlanDev dev, PlanHdr* host_hdr_dev, int32_t seq, hipStream_t s);

hipError_t launch_group(const int32_t* ids, int T, int k, int E, PlanDev dev, hipStream_t s,
                        hipEvent_t ev1);

// Router + slot plan + grouping in one launch, for decode-sized steps.
bool route_small_ok(int T, int k);
hipError_t launch_route_plan_small(const float* logits, int T, int E, int k, int K, void* state,
                                   PlanDev dev, PlanHdr* host_hdr_dev, int32_t seq, hipStream_t s,
                                   hipEvent_t ev0, hipEvent_t ev1, long long* dstats = nullptr);
// Device-resolved single-wave step, route and page-in in one launch (E <= 256):
// every workgroup plans the step, workgroup 0 stores the plan and counters,
// the last to finish planning (by the ticket counter, a multiple of the grid
// size between launches) stores the table state, and all copy their share of
// the missed records from the device-mapped host store into the slots.
bool route_page_in_ok(int E);
hipError_t launch_route_plan_page_in(const float* logits, int T, int E, int k, int K, void* state, PlanDev dev,
                                     long long* dstats, unsigned long long* ticket, const uint8_t* host_store_dev,
                                     uint8_t* slots, size_t stride, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1,
                                     size_t cp_len = ~(size_t)0);
// Device-resolved page-in of wave `wave` of a plan: copies the records of the
// misses among wave order positions [wave * K, (wave + 1) * K), i.e. positions
// max(counts[1], wave * K) .. min(counts[0], (wave + 1) * K) - 1, from the
// device-mapped host store into their slots (none for a wave past the step's).
hipError_t launch_page_in_device(const uint8_t* host_store_dev, uint8_t* slots, size_t stride,
                                 const PlanDev& dev, int E, int K, hipStream_t s, hipEvent_t ev0,
                                 hipEvent_t ev1, int wave = 0);

struct FfnArgs {
  int fmt, E, k, H, I, K;
  size_t stride;
  const uint8_t* slots;
  const int32_t* order_slot;
  const int32_t* pair_off;
  const int32_t* pair_list;
  const float* weights;
  const float* pair_w;  // router weight by CSR position (pair_list order)
  int o_lo, n_exp;     // wave's range in wave order
  int T;
  const void* x;       // [T][H]
  float* out;          // [T][H]
  int accumulate;      // 0: write out, 1: add to out
  float* h;            // GEMV scratch fp32 [T*k][I], indexed by CSR position
  uint16_t* hb;        // GEMM scratch bf16 [T*k][I], high part of h
  uint16_t* hb_lo;     // GEMM scratch bf16 [T*k][I], low part of h
  float* y;            // GEMM scratch fp32 [T*k][H]
  int max_rows;        // upper bound on pairs of one expert in this wave (GEMM)
  const int32_t* n_dev; // optional (device-resolved steps): the step's number of distinct
                       // experts D, read on the device; the launch then covers wave-order
                       // positions o_lo .. min(o_lo + n_exp, D) - 1 (none if D <= o_lo)
  uint16_t* x_res;     // optional: the launch that completes out also applies the
                       // stack residual x_res = bf16_rne(x_res + out), bf16 [T][H]
  int res_last;        // with x_res and n_dev: only the launch that holds the step's last
                       // expert (o_lo < D <= o_lo + n_exp) applies it
  int norm;            // GEMV path, bf16 activations: the up kernel applies the unit-gain
                       // RMSNorm to each staged activation row (a stack layer's input)
  // optional (GEMM path, quantised formats): the wave's records dequantised to
  // the bf16 record layout, expert o at wbase + (o - o_lo) * wstride
  const uint8_t* wbase;
  size_t wstride;
  hipEvent_t ev0, ev1; // optional timing events for the next launch
};

hipError_t launch_ffn_up(const FfnArgs& a, hipStream_t s);

// A layer of a stack whose device-resolved route and page-in (as
// launch_route_plan_page_in) run in extra workgroups of an earlier layer's
// launches.
struct NextStep {
  const float* logits;
  int T, E, k, K;
  uint8_t* state;
  StateLayout sl;
  PlanDev dev;
  long long* dstats;
  unsigned long long* ticket;
  const uint8_t* host;
  uint8_t* slots;
  size_t stride;
  size_t cp_len;  // bytes of each missed record copied by the up launch; the down launch copies the rest
};
// Whether a layer of this format, hidden size, E and pairs per step can take
// the merged launch (E <= 256, pairs <= 256, the shapes the up kernel is built for).
bool up_route_next_ok(int fmt, int H, int E, int P);
// This layer's up projection, with extra workgroups that copy the first
// n.cp_len bytes of every record the next layer's plan (already stored)
// misses and, with r, workgroups that route and plan the layer r (route only).
hipError_t launch_up_route_next(const FfnArgs& a, const NextStep& n, const NextStep* r, hipStream_t s);
// This layer's down projection, with extra workgroups that copy bytes
// [n.cp_len, n.stride) of every record the next layer's plan (already stored
// by the up launch) misses.
hipError_t launch_ffn_down_copy_next(const FfnArgs& a, const NextStep& n, hipStream_t s);
hipError_t launch_ffn_down(const FfnArgs& a, hipStream_t s);
bool ffn_shape_supported(int fmt, int H, int I);

// Expands the records of wave-order positions [o_lo, o_lo + n_exp) from the
// layer's format into bf16 records (rec_layout(BF16)) at dst + p * dst_stride.
hipError_t launch_dequant_bf16(const FfnArgs& a, uint8_t* dst, size_t dst_stride, hipStream_t s);

hipError_t launch_gemm_up(const FfnArgs& a, hipStream_t s);
hipError_t launch_gemm_down(const FfnArgs& a, hipStream_t s);
hipError_t launch_combine(const FfnArgs& a, const int32_t* pair_pos, const int32_t* wave_of, int wave,
                          hipStream_t s);
bool gemm_shape_supported(int H, int I);
// Whether the grouped GEMMs read this format's records in their slots (bf16,
// FP8, and int4 and MXFP4 with H <= 2048 and I <= 1024) rather than bf16
// expansions.
bool gemm_reads_record(int fmt, int H, int I);

hipError_t launch_residual(const uint16_t* x_in, const float* out, uint16_t* x_out, int64_t n,
                           hipStream_t s);

// Unit-gain RMSNorm of T bf16 rows of H values (H a multiple of 8), x -> a.
hipError_t launch_rmsnorm(const uint16_t* x, uint16_t* a, int T, int H, hipStream_t s);

}  // namespace moepage
