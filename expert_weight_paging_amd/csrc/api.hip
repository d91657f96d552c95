// C ABI of libmoepage: layer and plan handles, the plan readback, the copy
// engine and the wave sequencing around the kernels.
//
// [PE] = "Running an MoE Model Larger Than Your VRAM: SGLang Paged Experts, the
// PCIe Math, and the 4-Request Cliff".
#include <immintrin.h>

#include <algorithm>
#include <chrono>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "internal.h"

using namespace moepage;

namespace {

thread_local std::string g_err;

moe_status fail(moe_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

#define HIP_TRY(expr)                                                                  \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess)                                                              \
      return fail(MOE_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_));     \
  } while (0)

struct TimerRec {
  hipEvent_t a, b;
  int cls;
  double bytes, flops;
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace of moe_step_device_static: the plan arrays and the GEMV scratch of
// one device-resolved step, in a fixed device array instead of memory the
// library allocates. Each GPU holds its own copy until the process ends. In
// host code `scratch` only names the symbol; its device address on each GPU
// is taken once (hipGetSymbolAddress, at the first moe_layer_init on that
// device, with the device current) and only that address is handed to
// kernels.
constexpr size_t kStaticScratchBytes = MOE_STATIC_WORKSPACE_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

// Resolves the scratch array's address on the current device (once per device).
moe_status resolve_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return MOE_OK;  // the static entry point refuses such a layer
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (g_scratch_ptr[device]) return MOE_OK;
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr)
    return fail(MOE_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
  g_scratch_ptr[device] = (uint8_t*)ptr;
  return MOE_OK;
}

// Offsets of a device-resolved step's arrays in one workspace (the same
// arrays moe_plan_create allocates, sized for P = T * top_k pairs).
struct StepWs {
  size_t ids, w, sid, wo, oe, os, po, pl, pp, pw, cnt, h, total;
};
StepWs step_workspace(int E, int P, int I) {
  StepWs o{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t r = off;
    off = align_up(off + bytes, 256);
    return r;
  };
  o.ids = take(4 * (size_t)P);
  o.w = take(4 * (size_t)P);
  o.sid = take(4 * (size_t)P);
  o.wo = take(4 * (size_t)P);
  o.oe = take(4 * (size_t)E);
  o.os = take(4 * (size_t)E);
  o.po = take(4 * ((size_t)E + 1));
  o.pl = take(4 * (size_t)P);
  o.pp = take(4 * (size_t)P);
  o.pw = take(4 * (size_t)P);
  o.cnt = take(16);
  o.h = take(sizeof(float) * (size_t)P * I);
  o.total = off;
  return o;
}

}  // namespace

struct moe_layer {
  int E, k, H, I, K, fmt;
  int device;                     // HIP device current at init (where the buffers live)
  RecLayout rl;
  size_t stride;
  const uint8_t* host_store;
  const uint8_t* host_store_dev;  // device alias of the host store (null if not mapped)
  long long* dstats;              // device-resolved steps' counters (steps, refs, activations,
                                  // hits, misses, waves; [6]: the route-and-page-in launch's
                                  // ticket counter), device memory
  bool dev_steps;                 // a device-resolved step has been enqueued
  bool dev_pending;               // ... and no host-mode route has waited for it yet
  uint8_t* slots;
  uint8_t* state;
  hipStream_t compute, copy, route;
  hipEvent_t ev_fwd_done, ev_copied, ev_routed;
  hipEvent_t ev_copied_up;        // page_in(w): the gate/up parts of the wave's records are in (before ev_copied)
  hipEvent_t ev_victims_free;     // recorded by forward(w) once the slots page_in(w + 1) overwrites are read
  hipEvent_t ev_victims_up_free;  // ... once their gate/up parts are read (the up projection is done)
  int victims_free_wave;          // the w of that forward in the current step, or -1
  bool fwd_recorded, copy_recorded;
  int initial_fill;
  moe_stats stats;
  // sequencing of the current step
  const moe_plan* cur_plan;
  int next_page, next_fwd, n_waves;
  // timing
  bool timing;
  std::vector<TimerRec> pending;
  std::vector<hipEvent_t> pool;
  moe_timing acc;
};

struct moe_plan {
  const moe_layer* layer;
  int max_tokens, max_pairs;
  void* dev_block;
  PlanDev dev;
  PlanHdr* hdr;       // host pointer
  PlanHdr* hdr_dev;   // device alias of the same pinned memory
  int32_t seq;
  float* h;           // GEMV scratch
  uint16_t* hb;       // GEMM scratch (h high part)
  uint16_t* hb_lo;    // GEMM scratch (h low part)
  float* y;           // GEMM scratch
  uint8_t* wdq;       // GEMM scratch, quantised formats: the wave's records as bf16
  uint16_t* xn;       // GEMM scratch: the normalised activations of a stack layer [T][H] bf16
  int gemv_pairs;     // capacity of h in pairs
  hipEvent_t ev_consumed;
  bool consumed_recorded;
  moe_plan_info info;
  bool valid;
  bool dev_routed;    // last routed by a device-resolved step (host view not updated)
  int dev_tokens;     // its token count
};

namespace {

moe_status get_event(moe_layer* L, hipEvent_t* ev) {
  if (!L->pool.empty()) {
    *ev = L->pool.back();
    L->pool.pop_back();
    return MOE_OK;
  }
  HIP_TRY(hipEventCreate(ev));
  return MOE_OK;
}

moe_status timer_begin(moe_layer* L, hipStream_t s, TimerRec* t) {
  if (!L->timing) return MOE_OK;
  moe_status st = get_event(L, &t->a);
  if (st) return st;
  st = get_event(L, &t->b);
  if (st) return st;
  HIP_TRY(hipEventRecord(t->a, s));
  return MOE_OK;
}

// Kernel timers: the two events are handed to the launch, which stamps them at
// the kernel's start and end.
moe_status timer_events(moe_layer* L, TimerRec* t) {
  t->a = t->b = nullptr;
  if (!L->timing) return MOE_OK;
  moe_status st = get_event(L, &t->a);
  if (st) return st;
  return get_event(L, &t->b);
}

void timer_push(moe_layer* L, TimerRec* t, int cls, double bytes, double flops) {
  if (!L->timing) return;
  t->cls = cls;
  t->bytes = bytes;
  t->flops = flops;
  L->pending.push_back(*t);
}

moe_status timer_end(moe_layer* L, hipStream_t s, TimerRec* t, int cls, double bytes,
                     double flops) {
  if (!L->timing) return MOE_OK;
  HIP_TRY(hipEventRecord(t->b, s));
  t->cls = cls;
  t->bytes = bytes;
  t->flops = flops;
  L->pending.push_back(*t);
  return MOE_OK;
}

void init_state_host(const moe_layer* L, std::vector<uint8_t>& buf) {
  const StateLayout sl = state_layout(L->E, L->K);
  buf.assign(sl.total, 0);
  int32_t* se = (int32_t*)(buf.data() + sl.slot_expert);
  int32_t* es = (int32_t*)(buf.data() + sl.expert_slot);
  int64_t* st = (int64_t*)(buf.data() + sl.stamp);
  int64_t* clk = (int64_t*)(buf.data() + sl.clock);
  for (int e = 0; e < L->E; ++e) es[e] = -1;
  for (int s = 0; s < L->K; ++s) {
    se[s] = L->initial_fill ? s : -1;
    st[s] = L->initial_fill ? 0 : -1;
    if (L->initial_fill) es[s] = s;
  }
  *clk = 0;
}

moe_status restore_initial(moe_layer* L) {
  std::vector<uint8_t> buf;
  init_state_host(L, buf);
  HIP_TRY(hipMemcpy(L->state, buf.data(), buf.size(), hipMemcpyHostToDevice));
  if (L->initial_fill)
    HIP_TRY(hipMemcpy(L->slots, L->host_store, (size_t)L->K * L->stride, hipMemcpyHostToDevice));
  L->cur_plan = nullptr;
  L->next_page = L->next_fwd = L->n_waves = 0;
  L->victims_free_wave = -1;
  return MOE_OK;
}

bool is_pinned(const void* p) {
  hipPointerAttribute_t attr;
  std::memset(&attr, 0, sizeof(attr));
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return attr.type == hipMemoryTypeHost;
}

// Every byte of [p, p + n) lies in page-locked host memory: walks the range
// allocation by allocation (each allocation's extent from the runtime), so a
// range whose ends are pinned but whose middle is not (two allocations with a
// gap between them) is refused. Where the runtime gives no extent, every
// 4 KiB page is checked.
bool range_pinned(const uint8_t* p, size_t n) {
  const uintptr_t end = (uintptr_t)p + n;
  uintptr_t cur = (uintptr_t)p;
  while (cur < end) {
    if (!is_pinned((const void*)cur)) return false;
    void* base = nullptr;
    size_t size = 0;
    uintptr_t next = 0;
    if (hipPointerGetAttribute(&base, HIP_POINTER_ATTRIBUTE_RANGE_START_ADDR, (hipDeviceptr_t)cur) ==
            hipSuccess &&
        hipPointerGetAttribute(&size, HIP_POINTER_ATTRIBUTE_RANGE_SIZE, (hipDeviceptr_t)cur) == hipSuccess &&
        (uintptr_t)base <= cur && (uintptr_t)base + size > cur) {
      next = (uintptr_t)base + size;
    } else {
      (void)hipGetLastError();
      next = (cur | 4095) + 1;  // next 4 KiB page
    }
    cur = next;
  }
  return is_pinned(p + n - 1);
}

// Weight bytes of the gate/up and the down part of one record.
double up_weight_bytes(const moe_layer* L) {
  const RecLayout& r = L->rl;
  double b = (double)(r.wd - r.w13);
  if (L->fmt == MOE_FMT_FP8_E4M3_B128) b += (double)(r.sd - r.s13);
  if (L->fmt == MOE_FMT_INT4_ASYM_G128) b += (double)(r.sd - r.s13) + (double)(r.zd - r.z13);
  if (L->fmt == MOE_FMT_MXFP4_B32) b += (double)(r.sd - r.s13);
  return b;
}
double down_weight_bytes(const moe_layer* L) {
  const RecLayout& r = L->rl;
  double b = (double)(r.s13 - r.wd);
  if (L->fmt == MOE_FMT_FP8_E4M3_B128) b += (double)(r.payload - r.sd);
  if (L->fmt == MOE_FMT_INT4_ASYM_G128) b += (double)(r.z13 - r.sd) + (double)(r.payload - r.zd);
  if (L->fmt == MOE_FMT_MXFP4_B32) b += (double)(r.payload - r.sd);
  return b;
}

moe_status run_ffn(moe_layer* L, const PlanDev& dev, float* h, uint16_t* hb, uint16_t* hb_lo,
                   float* y, int o_lo, int n_exp, int n_pairs, int T, const void* x, float* out,
                   int accumulate, const int32_t* pair_pos, const int32_t* wave_of, int wave,
                   int max_rows, bool combine, uint16_t* x_res = nullptr,
                   const int32_t* n_dev = nullptr, uint8_t* wdq = nullptr, int norm = 0,
                   const NextStep* next = nullptr, const NextStep* route2 = nullptr, int res_last = 0,
                   hipEvent_t after_up = nullptr, hipEvent_t before_down = nullptr);

moe_status self_check(moe_layer* L);

}  // namespace

namespace {
// Does nothing: its timed duration is the floor of every timed launch.
__global__ void empty_kernel() {}

// A plain streaming read for moe_read_probe: every thread loads its four
// 16-byte chunks up front (consecutive threads read consecutive chunks), then
// folds them; nothing is stored unless the fold hits a sentinel value.
__global__ __launch_bounds__(512) void read_probe_kernel(const uint4* __restrict__ p, size_t n16,
                                                         uint32_t* sink) {
  const size_t base = (size_t)blockIdx.x * 2048 + threadIdx.x;
  uint4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const size_t i = base + (size_t)u * 512;
    v[u] = i < n16 ? p[i] : make_uint4(0u, 0u, 0u, 0u);
  }
  uint32_t s = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) s += v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (s == 0x9E3779B9u) sink[0] = s;
}
}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }

size_t moe_record_bytes(int32_t format, int32_t hidden, int32_t intermediate) {
  if (format < MOE_FMT_F32 || format > MOE_FMT_MXFP4_B32) return 0;
  if (hidden <= 0 || intermediate <= 0) return 0;
  if (!ffn_shape_supported(format, hidden, intermediate)) return 0;
  return rec_layout(format, hidden, intermediate).stride;
}

size_t moe_state_bytes(int32_t num_experts, int32_t num_slots) {
  if (num_experts <= 0 || num_slots <= 0) return 0;
  return state_layout(num_experts, num_slots).total;
}

int32_t moe_slots_for_budget(int32_t format, int32_t hidden, int32_t intermediate, int32_t num_experts,
                             int32_t layers, int64_t budget_bytes) {
  const size_t rec = moe_record_bytes(format, hidden, intermediate);
  if (rec == 0 || num_experts < 1 || layers < 1 || budget_bytes < 0) {
    (void)fail(MOE_ERR_INVALID_ARG, "unsupported shape, num_experts or layers < 1, or negative budget");
    return MOE_ERR_INVALID_ARG;
  }
  const uint64_t per_slot = (uint64_t)rec * (uint64_t)layers;  // one slot in every layer
  const uint64_t k = (uint64_t)budget_bytes / per_slot;
  return (int32_t)std::min<uint64_t>(k, (uint64_t)num_experts);
}

moe_status moe_preflight(int32_t layers, int32_t experts, int32_t top_k, double expert_mb, int32_t K,
                         double link_gbps, double tok_s, double kv_bytes_per_token,
                         moe_preflight_result* out) {
  if (!out) return fail(MOE_ERR_INVALID_ARG, "null output");
  if (layers < 1 || experts < 1 || top_k < 1 || K < 1 || K > experts)
    return fail(MOE_ERR_INVALID_ARG, "layers, experts, top_k and K must be >= 1, K <= experts");
  if (!(expert_mb > 0) || !(link_gbps > 0) || !(tok_s > 0) || !(kv_bytes_per_token > 0))
    return fail(MOE_ERR_INVALID_ARG, "expert_mb, link_gbps, tok_s and KV bytes must be positive");
  moe_preflight_result r;
  r.slot_mb = expert_mb * layers;
  r.kv_tokens_per_slot = r.slot_mb * 1e6 / kv_bytes_per_token;
  r.batch_cap = K / top_k;
  r.all_miss_gb_per_token = layers * top_k * expert_mb / 1e3;
  r.max_miss = link_gbps / (tok_s * r.all_miss_gb_per_token);
  r.random_miss = 1.0 - (double)K / experts;
  r.reuse_implied = r.max_miss < 0.8 * r.random_miss ? 1 : 0;
  *out = r;
  return MOE_OK;
}

void* moe_host_alloc(size_t bytes) {
  void* p = nullptr;
  hipError_t e = hipHostMalloc(&p, bytes, hipHostMallocDefault);
  if (e != hipSuccess) {
    g_err = std::string("hipHostMalloc: ") + hipGetErrorString(e);
    return nullptr;
  }
  return p;
}

void moe_host_free(void* p) {
  if (p) (void)hipHostFree(p);
}

moe_status moe_layer_init(const moe_layer_desc* d, void* compute_stream, void* copy_stream,
                          void* route_stream, moe_layer** out) {
  if (!d || !out) return fail(MOE_ERR_INVALID_ARG, "null descriptor or output");
  *out = nullptr;
  if (d->num_experts < 1 || d->num_experts > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_INVALID_ARG, "num_experts must be in 1..1024");
  if (d->top_k < 1 || d->top_k > d->num_experts || d->top_k > MOE_MAX_TOP_K)
    return fail(MOE_ERR_INVALID_ARG, "top_k must be in 1..min(E, 32)");
  if (d->num_slots < 1 || d->num_slots > d->num_experts)
    return fail(MOE_ERR_INVALID_ARG, "num_slots K must be in 1..E");
  if (d->format < MOE_FMT_F32 || d->format > MOE_FMT_MXFP4_B32)
    return fail(MOE_ERR_FORMAT, "unknown expert format");
  if (!ffn_shape_supported(d->format, d->hidden, d->intermediate))
    return fail(MOE_ERR_FORMAT, "hidden/intermediate not supported for this format");
  const RecLayout rl = rec_layout(d->format, d->hidden, d->intermediate);
  if (d->record_bytes != rl.stride)
    return fail(MOE_ERR_FORMAT, "record_bytes does not match the format's record stride (" +
                                    std::to_string(rl.stride) + ")");
  if (!d->host_store || !d->slot_store || !d->state)
    return fail(MOE_ERR_INVALID_ARG, "null host_store, slot_store or state");
  if (((uintptr_t)d->slot_store & 255) || ((uintptr_t)d->state & 7))
    return fail(MOE_ERR_INVALID_ARG, "slot_store must be 256-byte and state 8-byte aligned");
  const uint8_t* hs = (const uint8_t*)d->host_store;
  if (!range_pinned(hs, (size_t)d->num_experts * rl.stride))
    return fail(MOE_ERR_NOT_PINNED, "host_store is not page-locked host memory over its whole range");
  if (d->self_check && d->num_slots < 2)
    return fail(MOE_ERR_INVALID_ARG, "self_check places each expert in two different slots: needs K >= 2");

  moe_layer* L = new (std::nothrow) moe_layer();
  if (!L) return fail(MOE_ERR_INVALID_ARG, "out of host memory");
  L->E = d->num_experts;
  L->k = d->top_k;
  L->H = d->hidden;
  L->I = d->intermediate;
  L->K = d->num_slots;
  L->fmt = d->format;
  L->rl = rl;
  L->stride = rl.stride;
  L->host_store = hs;
  L->slots = (uint8_t*)d->slot_store;
  L->state = (uint8_t*)d->state;
  L->compute = (hipStream_t)compute_stream;
  L->copy = (hipStream_t)copy_stream;
  L->route = (hipStream_t)route_stream;
  L->initial_fill = d->initial_fill ? 1 : 0;
  L->device = -1;
  L->fwd_recorded = L->copy_recorded = false;
  std::memset(&L->stats, 0, sizeof(L->stats));
  std::memset(&L->acc, 0, sizeof(L->acc));
  L->timing = false;
  moe_status st = MOE_OK;
  auto bail = [&](moe_status s) {
    moe_layer_destroy(L);
    return s;
  };
  if (hipEventCreateWithFlags(&L->ev_fwd_done, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&L->ev_copied, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&L->ev_routed, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&L->ev_victims_free, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&L->ev_copied_up, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&L->ev_victims_up_free, hipEventDisableTiming) != hipSuccess)
    return bail(fail(MOE_ERR_HIP, "hipEventCreate failed"));
  // device alias of the host store, for device-resolved steps (none if unmapped)
  void* hs_dev = nullptr;
  if (hipHostGetDevicePointer(&hs_dev, (void*)hs, 0) == hipSuccess) L->host_store_dev = (const uint8_t*)hs_dev;
  else (void)hipGetLastError();
  if (hipGetDevice(&L->device) != hipSuccess) return bail(fail(MOE_ERR_HIP, "hipGetDevice failed"));
  if ((st = resolve_scratch(L->device))) return bail(st);
  if (hipMalloc((void**)&L->dstats, 8 * sizeof(long long)) != hipSuccess ||
      hipMemset(L->dstats, 0, 8 * sizeof(long long)) != hipSuccess)
    return bail(fail(MOE_ERR_HIP, "device counters allocation failed"));
  if (d->self_check) {
    st = self_check(L);
    if (st) return bail(st);
  }
  st = restore_initial(L);
  if (st) return bail(st);
  *out = L;
  return MOE_OK;
}

void moe_layer_destroy(moe_layer* L) {
  if (!L) return;
  (void)hipStreamSynchronize(L->compute);
  (void)hipStreamSynchronize(L->copy);
  (void)hipStreamSynchronize(L->route);
  if (L->ev_fwd_done) (void)hipEventDestroy(L->ev_fwd_done);
  if (L->ev_copied) (void)hipEventDestroy(L->ev_copied);
  if (L->ev_routed) (void)hipEventDestroy(L->ev_routed);
  if (L->ev_victims_free) (void)hipEventDestroy(L->ev_victims_free);
  if (L->ev_copied_up) (void)hipEventDestroy(L->ev_copied_up);
  if (L->ev_victims_up_free) (void)hipEventDestroy(L->ev_victims_up_free);
  if (L->dstats) (void)hipFree(L->dstats);

  for (auto& t : L->pending) {
    (void)hipEventDestroy(t.a);
    (void)hipEventDestroy(t.b);
  }
  for (auto e : L->pool) (void)hipEventDestroy(e);
  delete L;
}

moe_status moe_layer_reset(moe_layer* L) {
  if (!L) return fail(MOE_ERR_INVALID_ARG, "null layer");
  HIP_TRY(hipStreamSynchronize(L->compute));
  HIP_TRY(hipStreamSynchronize(L->copy));
  HIP_TRY(hipStreamSynchronize(L->route));
  return restore_initial(L);
}

moe_status moe_plan_create(const moe_layer* L, int32_t max_tokens, moe_plan** out) {
  if (!L || !out) return fail(MOE_ERR_INVALID_ARG, "null layer or output");
  *out = nullptr;
  if (max_tokens < 1) return fail(MOE_ERR_INVALID_ARG, "max_tokens must be >= 1");
  const bool gemm = max_tokens > MOE_MAX_GEMV_TOKENS;
  if (gemm && (L->fmt == MOE_FMT_F32 || !gemm_shape_supported(L->H, L->I)))
    return fail(MOE_ERR_INVALID_ARG,
                "more than 64 tokens per forward needs a bf16, FP8, int4 or MXFP4 layer with H and I "
                "multiples of 128");
  moe_plan* p = new (std::nothrow) moe_plan();
  if (!p) return fail(MOE_ERR_INVALID_ARG, "out of host memory");
  std::memset(p, 0, sizeof(*p));
  p->layer = L;
  p->max_tokens = max_tokens;
  p->max_pairs = max_tokens * L->k;
  const size_t P = (size_t)p->max_pairs, E = (size_t)L->E;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  const size_t o_ids = take(4 * P), o_w = take(4 * P), o_sid = take(4 * P), o_wo = take(4 * P),
               o_oe = take(4 * E), o_os = take(4 * E), o_po = take(4 * (E + 1)),
               o_pl = take(4 * P), o_pp = take(4 * P), o_pw = take(4 * P), o_cnt = take(16);
  p->gemv_pairs = (int)std::min<size_t>(P, (size_t)MOE_MAX_GEMV_TOKENS * L->k);
  const size_t o_h = take(sizeof(float) * (size_t)p->gemv_pairs * L->I);
  size_t o_hb = 0, o_hl = 0, o_y = 0, o_xn = 0;
  size_t o_wq = 0;
  if (gemm) {
    o_hb = take(2 * P * L->I);
    o_hl = take(2 * P * L->I);
    o_y = take(4 * P * L->H);
    o_xn = take(2 * (size_t)max_tokens * L->H);
    // a wave holds at most min(K, E) experts; those of shapes the GEMMs do
    // not read in place (4-bit formats past the LDS scale region) are each
    // expanded to a bf16 record
    if (!gemm_reads_record(L->fmt, L->H, L->I))
      o_wq = take((size_t)std::min(L->K, L->E) * rec_layout(MOE_FMT_BF16, L->H, L->I).stride);
  }
  auto cleanup = [&](moe_status s) {
    moe_plan_destroy(p);
    return s;
  };
  if (hipMalloc(&p->dev_block, off) != hipSuccess) return cleanup(fail(MOE_ERR_HIP, "hipMalloc plan"));
  uint8_t* b = (uint8_t*)p->dev_block;
  p->dev.ids = (int32_t*)(b + o_ids);
  p->dev.weights = (float*)(b + o_w);
  p->dev.slot_ids = (int32_t*)(b + o_sid);
  p->dev.wave_of = (int32_t*)(b + o_wo);
  p->dev.order_expert = (int32_t*)(b + o_oe);
  p->dev.order_slot = (int32_t*)(b + o_os);
  p->dev.pair_off = (int32_t*)(b + o_po);
  p->dev.pair_list = (int32_t*)(b + o_pl);
  p->dev.pair_pos = (int32_t*)(b + o_pp);
  p->dev.pair_w = (float*)(b + o_pw);
  p->dev.counts = (int32_t*)(b + o_cnt);
  p->h = (float*)(b + o_h);
  p->hb = gemm ? (uint16_t*)(b + o_hb) : nullptr;
  p->hb_lo = gemm ? (uint16_t*)(b + o_hl) : nullptr;
  p->y = gemm ? (float*)(b + o_y) : nullptr;
  p->xn = gemm ? (uint16_t*)(b + o_xn) : nullptr;
  p->wdq = (gemm && !gemm_reads_record(L->fmt, L->H, L->I)) ? b + o_wq : nullptr;
  const size_t hbytes = sizeof(PlanHdr) + sizeof(int32_t) * (3 * E + 1);
  if (hipHostMalloc((void**)&p->hdr, hbytes, hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess)
    return cleanup(fail(MOE_ERR_HIP, "hipHostMalloc plan header"));
  std::memset(p->hdr, 0, hbytes);
  if (hipHostGetDevicePointer((void**)&p->hdr_dev, p->hdr, 0) != hipSuccess)
    return cleanup(fail(MOE_ERR_HIP, "hipHostGetDevicePointer"));
  if (hipEventCreateWithFlags(&p->ev_consumed, hipEventDisableTiming) != hipSuccess)
    return cleanup(fail(MOE_ERR_HIP, "hipEventCreate"));
  *out = p;
  return MOE_OK;
}

void moe_plan_destroy(moe_plan* p) {
  if (!p) return;
  if (p->consumed_recorded) (void)hipEventSynchronize(p->ev_consumed);
  if (p->ev_consumed) (void)hipEventDestroy(p->ev_consumed);
  if (p->dev_block) (void)hipFree(p->dev_block);
  if (p->hdr) (void)hipHostFree(p->hdr);
  delete p;
}

namespace {
moe_status route_impl(moe_layer* L, const float* logits, int32_t T, moe_plan* p, hipEvent_t after,
                      hipStream_t on = nullptr);
}

moe_status moe_route(moe_layer* L, const float* logits, int32_t T, moe_plan* p) {
  return route_impl(L, logits, T, p, nullptr);
}

namespace {
// `after`, if given, is an event the route stream waits for before routing;
// `on`, if given, replaces the layer's route stream for this step.
moe_status route_impl(moe_layer* L, const float* logits, int32_t T, moe_plan* p, hipEvent_t after,
                      hipStream_t on) {
  if (!L || !p) return fail(MOE_ERR_INVALID_ARG, "null layer or plan");
  const hipStream_t rs = on ? on : L->route;
  if (p->layer != L) return fail(MOE_ERR_INVALID_ARG, "plan was created for another layer");
  if (T < 0 || T > p->max_tokens) return fail(MOE_ERR_INVALID_ARG, "num_tokens out of 0..max_tokens");
  if (T > 0 && !logits) return fail(MOE_ERR_INVALID_ARG, "null logits");
  if (L->cur_plan && L->next_fwd < L->n_waves)
    return fail(MOE_ERR_STATE, "previous step of this layer has waves not yet forwarded");

  if (p->consumed_recorded && rs != L->compute) HIP_TRY(hipStreamWaitEvent(rs, p->ev_consumed, 0));
  // A device-resolved step of this layer may still update the table state on
  // the compute stream, also one replayed from a captured graph (whose
  // launches the library does not see): once this layer has had device steps,
  // the route waits for everything enqueued on the compute stream so far.
  if (L->dev_steps && rs != L->compute) {
    HIP_TRY(hipEventRecord(L->ev_fwd_done, L->compute));
    L->fwd_recorded = true;
    HIP_TRY(hipStreamWaitEvent(rs, L->ev_fwd_done, 0));
  }
  L->dev_pending = false;
  if (after) HIP_TRY(hipStreamWaitEvent(rs, after, 0));
  TimerRec tr{};
  moe_status st = timer_events(L, &tr);
  if (st) return st;
  const int32_t seq = ++p->seq;
  if (route_small_ok(T, L->k)) {
    HIP_TRY(launch_route_plan_small(logits, T, L->E, L->k, L->K, L->state, p->dev, p->hdr_dev, seq,
                                    rs, tr.a, tr.b));
  } else {
    HIP_TRY(launch_router(logits, T, L->E, L->k, p->dev.ids, p->dev.weights, rs, tr.a));
    HIP_TRY(launch_plan(p->dev.ids, T, L->k, L->E, L->K, L->state, p->dev, p->hdr_dev, seq, rs));
    HIP_TRY(launch_group(p->dev.ids, T, L->k, L->E, p->dev, rs, tr.b));
  }
  if (T > 0) timer_push(L, &tr, MOE_T_ROUTE, 0.0, 0.0);
  else if (L->timing) {
    L->pool.push_back(tr.a);
    L->pool.push_back(tr.b);
  }
  HIP_TRY(hipEventRecord(L->ev_routed, rs));
  // The one host synchronisation of a layer-step: wait until the slot-plan
  // kernel has published the plan into pinned host memory.
  volatile int32_t* flag = &p->hdr->seq;
  auto t0 = std::chrono::steady_clock::now();
  long spins = 0;
  while (__atomic_load_n(flag, __ATOMIC_ACQUIRE) != seq) {
    _mm_pause();
    if (++spins % 4096 == 0) {
      hipError_t q = hipStreamQuery(rs);
      if (q != hipSuccess && q != hipErrorNotReady)
        return fail(MOE_ERR_HIP, std::string("route kernels failed: ") + hipGetErrorString(q));
      if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(60))
        return fail(MOE_ERR_TIMEOUT, "slot plan did not become host-visible within 60 s");
      if (spins > (1L << 20)) std::this_thread::yield();
    }
  }
  const PlanHdr& h = *p->hdr;
  p->info.num_tokens = h.num_tokens;
  p->info.num_distinct = h.num_distinct;
  p->info.num_hits = h.num_hits;
  p->info.num_misses = h.num_distinct - h.num_hits;
  p->info.num_waves = h.num_waves;
  p->valid = true;
  p->dev_routed = false;
  if (T > 0) {
    L->stats.steps += 1;
    L->stats.refs += h.num_distinct;
    L->stats.activations += (int64_t)T * L->k;
    L->stats.hits += h.num_hits;
    L->stats.misses += h.num_distinct - h.num_hits;
    L->stats.waves += h.num_waves;
    L->stats.bytes_paged += (int64_t)(h.num_distinct - h.num_hits) * (int64_t)L->stride;
  }
  L->n_waves = h.num_waves;
  L->next_page = L->next_fwd = 0;
  L->victims_free_wave = -1;
  L->cur_plan = h.num_waves > 0 ? p : nullptr;
  return MOE_OK;
}

}  // namespace

moe_status moe_plan_get_info(const moe_plan* p, moe_plan_info* out) {
  if (!p || !out) return fail(MOE_ERR_INVALID_ARG, "null plan or output");
  if (!p->valid) return fail(MOE_ERR_STATE, "plan has not been routed");
  *out = p->info;
  return MOE_OK;
}

moe_status moe_plan_get_wave(const moe_plan* p, int32_t w, moe_wave_info* out) {
  if (!p || !out) return fail(MOE_ERR_INVALID_ARG, "null plan or output");
  if (!p->valid) return fail(MOE_ERR_STATE, "plan has not been routed");
  if (w < 0 || w >= p->info.num_waves) return fail(MOE_ERR_INVALID_ARG, "wave out of range");
  const int K = p->layer->K, D = p->info.num_distinct, nH = p->info.num_hits;
  const int lo = w * K, hi = std::min(lo + K, D), mlo = std::max(lo, nH);
  const int32_t* oe = (const int32_t*)(p->hdr + 1);
  const int32_t* os = oe + p->layer->E;
  out->num_experts = hi - lo;
  out->num_misses = hi - mlo;
  out->experts = oe + lo;
  out->slots = os + lo;
  out->miss_experts = oe + mlo;
  out->miss_slots = os + mlo;
  return MOE_OK;
}

moe_status moe_plan_read(const moe_plan* p, int32_t* ids, float* weights, int32_t* slot_ids,
                         int32_t* wave_of) {
  if (!p) return fail(MOE_ERR_INVALID_ARG, "null plan");
  if (!p->valid && !p->dev_routed) return fail(MOE_ERR_STATE, "plan has not been routed");
  const moe_layer* L = p->layer;
  HIP_TRY(hipStreamSynchronize(p->dev_routed ? L->compute : L->route));
  const size_t n = (size_t)(p->dev_routed ? p->dev_tokens : p->info.num_tokens) * L->k;
  if (n == 0) return MOE_OK;
  if (ids) HIP_TRY(hipMemcpy(ids, p->dev.ids, 4 * n, hipMemcpyDeviceToHost));
  if (weights) HIP_TRY(hipMemcpy(weights, p->dev.weights, 4 * n, hipMemcpyDeviceToHost));
  if (slot_ids) HIP_TRY(hipMemcpy(slot_ids, p->dev.slot_ids, 4 * n, hipMemcpyDeviceToHost));
  if (wave_of) HIP_TRY(hipMemcpy(wave_of, p->dev.wave_of, 4 * n, hipMemcpyDeviceToHost));
  return MOE_OK;
}

namespace {
// Byte ranges of a record: what the up projection reads (W13 and its scales /
// zero points) and the rest (W_d, its tables and the padding up to the stride).
struct RecParts {
  int n_up = 0, n_rest = 0;
  size_t up_lo[3], up_hi[3], rest_lo[4], rest_hi[4];
};
// Whether page_in of a step of T tokens copies the missed records in two parts
// (gate/up first): only for the grouped GEMMs that read records in place, whose
// copies are long enough to hide the up GEMM; on the GEMV path the extra DMA
// calls cost more host time than the overlap saves.
bool split_page_in(const moe_layer* L, int T) {
  return T > MOE_MAX_GEMV_TOKENS && gemm_reads_record(L->fmt, L->H, L->I);
}

RecParts record_parts(const moe_layer* L) {
  const RecLayout& r = L->rl;
  RecParts q;
  auto up = [&](size_t lo, size_t hi) {
    if (hi > lo) { q.up_lo[q.n_up] = lo; q.up_hi[q.n_up] = hi; ++q.n_up; }
  };
  up(r.w13, r.wd);
  if (L->fmt == MOE_FMT_FP8_E4M3_B128 || L->fmt == MOE_FMT_MXFP4_B32 || L->fmt == MOE_FMT_INT4_ASYM_G128)
    up(r.s13, r.sd);
  if (L->fmt == MOE_FMT_INT4_ASYM_G128) up(r.z13, r.zd);
  size_t at = 0;  // the rest: the gaps between the up ranges (ascending) up to the stride
  for (int i = 0; i <= q.n_up; ++i) {
    const size_t lo = at, hi = i < q.n_up ? q.up_lo[i] : L->stride;
    if (hi > lo) { q.rest_lo[q.n_rest] = lo; q.rest_hi[q.n_rest] = hi; ++q.n_rest; }
    if (i < q.n_up) at = q.up_hi[i];
  }
  return q;
}
}  // namespace

moe_status moe_page_in(moe_layer* L, const moe_plan* p, int32_t w) {
  if (!L || !p) return fail(MOE_ERR_INVALID_ARG, "null layer or plan");
  if (L->cur_plan != p) return fail(MOE_ERR_STATE, "plan is not this layer's current step");
  if (w != L->next_page || w != L->next_fwd)
    return fail(MOE_ERR_STATE, "waves must be paged in in order, each after the previous forward");
  moe_wave_info wi;
  moe_status st = moe_plan_get_wave(p, w, &wi);
  if (st) return st;
  // A victim slot may still be read by the previous forward of this layer.
  // When that forward computed the experts in this wave's victim slots first,
  // only that part is waited for, in two steps: a slot's gate/up part may be
  // overwritten once their up projection is done, the rest once their down
  // projection is.
  const bool victims = w > 0 && L->victims_free_wave == w - 1;
  const bool split = split_page_in(L, p->info.num_tokens);
  if (victims) HIP_TRY(hipStreamWaitEvent(L->copy, split ? L->ev_victims_up_free : L->ev_victims_free, 0));
  else if (L->fwd_recorded) HIP_TRY(hipStreamWaitEvent(L->copy, L->ev_fwd_done, 0));
  TimerRec tr{};
  st = timer_begin(L, L->copy, &tr);
  if (st) return st;
  for (int i = 0; i < wi.num_misses; ++i) {
    const int e = wi.miss_experts[i], s = wi.miss_slots[i];
    if (e < 0 || e >= L->E || s < 0 || s >= L->K)
      return fail(MOE_ERR_STATE, "corrupt miss list");
  }
  // With split, the missed records' gate/up parts are copied first and the
  // rest second, so the forward's up projection of the missed experts waits
  // only for the first part ([PE] "TL;DR": experts cross PCIe while the math
  // runs). Each part is one strided DMA copy per run of misses that is
  // contiguous in both stores (expert e + 1 into slot s + 1 after e into s):
  // fewer, larger copies keep the link busier than one per record, and a
  // strided copy of a run moves as fast as one contiguous copy of it
  // (measured on MI355X: 56.2 against 56.3 GB/s for 36 bf16 records).
  RecParts parts;
  if (split) {
    parts = record_parts(L);
  } else {
    parts.n_up = 1;
    parts.up_lo[0] = 0;
    parts.up_hi[0] = L->stride;
  }
  auto copy_ranges = [&](int nr, const size_t* lo, const size_t* hi) -> moe_status {
    for (int i = 0; i < wi.num_misses;) {
      const int e = wi.miss_experts[i], s = wi.miss_slots[i];
      int n = 1;
      while (i + n < wi.num_misses && wi.miss_experts[i + n] == e + n && wi.miss_slots[i + n] == s + n) ++n;
      uint8_t* dst = L->slots + (size_t)s * L->stride;
      const uint8_t* src = L->host_store + (size_t)e * L->stride;
      for (int j = 0; j < nr; ++j) {
        if (n == 1)
          HIP_TRY(hipMemcpyAsync(dst + lo[j], src + lo[j], hi[j] - lo[j], hipMemcpyHostToDevice, L->copy));
        else
          HIP_TRY(hipMemcpy2DAsync(dst + lo[j], L->stride, src + lo[j], L->stride, hi[j] - lo[j], (size_t)n,
                                   hipMemcpyHostToDevice, L->copy));
      }
      i += n;
    }
    return MOE_OK;
  };
  if ((st = copy_ranges(parts.n_up, parts.up_lo, parts.up_hi))) return st;
  if (split) {
    HIP_TRY(hipEventRecord(L->ev_copied_up, L->copy));
    if (victims) HIP_TRY(hipStreamWaitEvent(L->copy, L->ev_victims_free, 0));
    if ((st = copy_ranges(parts.n_rest, parts.rest_lo, parts.rest_hi))) return st;
  }
  st = timer_end(L, L->copy, &tr, MOE_T_PAGE_IN, (double)wi.num_misses * L->stride, 0.0);
  if (st) return st;
  HIP_TRY(hipEventRecord(L->ev_copied, L->copy));
  L->copy_recorded = true;
  L->next_page = w + 1;
  return MOE_OK;
}

namespace {
moe_status forward_impl(moe_layer* L, const moe_plan* p, int32_t w, const void* x, float* out,
                        uint16_t* x_res, int norm = 0);
}

moe_status moe_forward(moe_layer* L, const moe_plan* p, int32_t w, const void* x, float* out) {
  return forward_impl(L, p, w, x, out, nullptr);
}

namespace {
// The part of wave w's positions [o_lo, o_lo + n_exp) that reads the slots
// wave w + 1 pages into: the shortest prefix or suffix of the range that holds
// all of them, as [*v_lo, *v_lo + *v_n); *v_n = 0 if there are none, n_exp if
// they span the range.
void victims_first(const moe_layer* L, const moe_plan* p, int w, int o_lo, int n_exp, int* v_lo, int* v_n) {
  const int K = L->K, D = p->info.num_distinct, nH = p->info.num_hits;
  const int32_t* os = (const int32_t*)(p->hdr + 1) + L->E;  // slot of each wave-order position
  const int lo1 = (w + 1) * K, hi1 = std::min(lo1 + K, D), m1 = std::max(lo1, nH);
  std::vector<char> victim((size_t)K, 0);
  for (int i = m1; i < hi1; ++i)
    if (os[i] >= 0 && os[i] < K) victim[(size_t)os[i]] = 1;
  int first = -1, last = -1;
  for (int o = o_lo; o < o_lo + n_exp; ++o) {
    const int sl = os[o];
    if (sl >= 0 && sl < K && victim[(size_t)sl]) {
      if (first < 0) first = o;
      last = o;
    }
  }
  *v_lo = o_lo;
  *v_n = n_exp;
  if (first < 0) {
    *v_n = 0;
    return;
  }
  const int pre = last - o_lo + 1, suf = o_lo + n_exp - first;
  if (pre <= suf) {
    *v_n = pre;
  } else {
    *v_lo = first;
    *v_n = suf;
  }
}

// x_res, if given, receives the stack residual bf16_rne(x_res + out) from the
// kernel that completes out (only on a step's last wave). norm: x is a stack
// layer's residual stream and the experts read its unit-gain RMSNorm (GEMV
// path: computed by the up kernels; GEMM path: by a norm kernel into the
// plan's workspace before wave 0).
moe_status forward_impl(moe_layer* L, const moe_plan* p, int32_t w, const void* x, float* out,
                        uint16_t* x_res, int norm) {
  if (!L || !p) return fail(MOE_ERR_INVALID_ARG, "null layer or plan");
  if (L->cur_plan != p) return fail(MOE_ERR_STATE, "plan is not this layer's current step");
  if (w != L->next_fwd || L->next_page != w + 1)
    return fail(MOE_ERR_STATE, "forward(w) must follow page_in(w)");
  const int T = p->info.num_tokens;
  if (!x || !out) return fail(MOE_ERR_INVALID_ARG, "null x or out");
  if (((uintptr_t)x & 15) || ((uintptr_t)out & 15))
    return fail(MOE_ERR_INVALID_ARG, "x and out must be 16-byte aligned");
  HIP_TRY(hipStreamWaitEvent(L->compute, L->ev_routed, 0));
  if (norm && T > MOE_MAX_GEMV_TOKENS) {
    if (!p->xn) return fail(MOE_ERR_STATE, "plan has no normalisation workspace");
    if (w == 0) HIP_TRY(launch_rmsnorm((const uint16_t*)x, p->xn, T, L->H, L->compute));
    x = p->xn;
    norm = 0;
  }
  const int K = L->K, D = p->info.num_distinct, nH = p->info.num_hits;
  const int o_lo = w * K, n_exp = std::min(K, D - o_lo);
  // The wave order lists the experts that were resident first: they can be
  // computed while the wave's misses are still being copied; only the missed
  // experts wait for the copy ([SRV]-style overlap of transfer and compute).
  const int n_res = std::max(0, std::min(nH, o_lo + n_exp) - o_lo);
  moe_plan* pm = const_cast<moe_plan*>(p);
  const int32_t* hoff = (const int32_t*)(p->hdr + 1) + 2 * L->E;  // CSR offsets, host copy
  auto pairs_in = [&](int lo, int n) { return hoff[lo + n] - hoff[lo]; };
  const bool gemm = T > MOE_MAX_GEMV_TOKENS;
  // Whether to split is decided from the plan alone on the GEMV path, where the
  // two launches add into out in a different order than one launch does: a
  // wave with both resident and missed experts is always split, so a step's
  // bits never depend on how far its copies had got. On the GEMM path the
  // split only changes which launch fills an expert's rows of y, and the
  // combine sums them in a fixed order, so there the split is taken only while
  // the copies are still in flight (it costs extra launches).
  const bool copies_pending =
      n_res < n_exp && L->copy_recorded &&
      (!gemm || hipEventQuery(L->ev_copied) == hipErrorNotReady);
  // With split, page_in(w) copied the missed records' gate/up parts first: the
  // up projection waits for those, the down projection for the rest.
  const bool split = split_page_in(L, T);
  hipEvent_t up_ready = split ? L->ev_copied_up : L->ev_copied;
  hipEvent_t down_ready = split ? L->ev_copied : nullptr;
  moe_status st;
  if (n_res > 0 && copies_pending) {
    st = run_ffn(L, p->dev, p->h, p->hb, p->hb_lo, p->y, o_lo, n_res, pairs_in(o_lo, n_res), T, x, out,
                 w > 0, p->dev.pair_pos, p->dev.wave_of, w, T, /*combine=*/false, nullptr, nullptr, p->wdq, norm);
    if (st) return st;
    HIP_TRY(hipStreamWaitEvent(L->compute, up_ready, 0));
    st = run_ffn(L, p->dev, p->h, p->hb, p->hb_lo, p->y, o_lo + n_res, n_exp - n_res,
                 pairs_in(o_lo + n_res, n_exp - n_res), T, x, out, w > 0 || !gemm, p->dev.pair_pos,
                 p->dev.wave_of, w, T, /*combine=*/gemm, x_res, nullptr, p->wdq, norm, nullptr, nullptr, 0,
                 nullptr, down_ready);
    if (st) return st;
  } else {
    if (!L->copy_recorded) down_ready = nullptr;
    if (L->copy_recorded) HIP_TRY(hipStreamWaitEvent(L->compute, up_ready, 0));
    // Victims first (GEMM path): when the next wave pages experts into slots
    // this wave reads, the experts in those slots are computed first, and the
    // next wave's copies start while the rest of this wave computes. The
    // combine after both parts sums in the same fixed order, so the result is
    // bitwise the same as one launch.
    int v_lo = o_lo, v_n = n_exp;
    if (gemm && w + 1 < p->info.num_waves) victims_first(L, p, w, o_lo, n_exp, &v_lo, &v_n);
    if (v_n == 0) {  // the next wave's copies touch none of this wave's slots
      if (split) HIP_TRY(hipEventRecord(L->ev_victims_up_free, L->compute));
      HIP_TRY(hipEventRecord(L->ev_victims_free, L->compute));
      L->victims_free_wave = w;
    }
    if (v_n > 0 && v_n < n_exp) {
      const int r_lo = v_lo == o_lo ? o_lo + v_n : o_lo, r_n = n_exp - v_n;
      // the victims' up projection marks their gate/up parts free, their down
      // projection the rest
      st = run_ffn(L, p->dev, p->h, p->hb, p->hb_lo, p->y, v_lo, v_n, pairs_in(v_lo, v_n), T, x, out, w > 0,
                   p->dev.pair_pos, p->dev.wave_of, w, T, /*combine=*/false, nullptr, nullptr, p->wdq, norm,
                   nullptr, nullptr, 0, split ? L->ev_victims_up_free : nullptr, down_ready);
      if (st) return st;
      HIP_TRY(hipEventRecord(L->ev_victims_free, L->compute));
      L->victims_free_wave = w;
      st = run_ffn(L, p->dev, p->h, p->hb, p->hb_lo, p->y, r_lo, r_n, pairs_in(r_lo, r_n), T, x, out, w > 0,
                   p->dev.pair_pos, p->dev.wave_of, w, T, /*combine=*/gemm, x_res, nullptr, p->wdq, norm);
    } else {
      st = run_ffn(L, p->dev, p->h, p->hb, p->hb_lo, p->y, o_lo, n_exp, pairs_in(o_lo, n_exp), T, x, out,
                   w > 0, p->dev.pair_pos, p->dev.wave_of, w, T, /*combine=*/gemm, x_res, nullptr, p->wdq, norm,
                   nullptr, nullptr, 0, nullptr, down_ready);
    }
    if (st) return st;
  }
  HIP_TRY(hipEventRecord(L->ev_fwd_done, L->compute));
  L->fwd_recorded = true;
  HIP_TRY(hipEventRecord(pm->ev_consumed, L->compute));
  pm->consumed_recorded = true;
  L->next_fwd = w + 1;
  if (L->next_fwd == L->n_waves) L->cur_plan = nullptr;
  return MOE_OK;
}
}  // namespace

moe_status moe_rmsnorm_bf16(const void* x, void* a, int32_t T, int32_t H, void* stream) {
  if (T < 0 || H < 8 || (H & 7) || (T > 0 && (!x || !a)))
    return fail(MOE_ERR_INVALID_ARG, "bad norm arguments (H must be a positive multiple of 8)");
  if (((uintptr_t)x & 15) || ((uintptr_t)a & 15))
    return fail(MOE_ERR_INVALID_ARG, "x and a must be 16-byte aligned");
  if ((size_t)H * 2 > 64 * 1024) return fail(MOE_ERR_INVALID_ARG, "H above 32768");
  HIP_TRY(launch_rmsnorm((const uint16_t*)x, (uint16_t*)a, T, H, (hipStream_t)stream));
  return MOE_OK;
}

moe_status moe_residual_bf16(const void* x_in, const float* out, void* x_out, int64_t n,
                             void* stream) {
  if (n < 0 || (n > 0 && (!x_in || !out || !x_out)))
    return fail(MOE_ERR_INVALID_ARG, "bad residual arguments");
  if (((uintptr_t)x_in & 7) || ((uintptr_t)x_out & 7) || ((uintptr_t)out & 15))
    return fail(MOE_ERR_INVALID_ARG, "x must be 8-byte and out 16-byte aligned");
  HIP_TRY(launch_residual((const uint16_t*)x_in, out, (uint16_t*)x_out, n, (hipStream_t)stream));
  return MOE_OK;
}

moe_status moe_stack_forward(moe_layer* const* layers, moe_plan* const* plans, int32_t n,
                             const float* logits, int32_t T, void* x, float* out, int32_t lookahead) {
  if (!layers || !plans || n < 1) return fail(MOE_ERR_INVALID_ARG, "need n_layers >= 1 layers and plans");
  if (T < 0 || (T > 0 && (!logits || !x || !out))) return fail(MOE_ERR_INVALID_ARG, "bad buffers");
  const moe_layer* L0 = layers[0];
  if (!L0) return fail(MOE_ERR_INVALID_ARG, "null layer");
  for (int l = 0; l < n; ++l) {
    const moe_layer* L = layers[l];
    if (!L || !plans[l] || plans[l]->layer != L)
      return fail(MOE_ERR_INVALID_ARG, "layer/plan " + std::to_string(l) + " missing or mismatched");
    if (L->E != L0->E || L->k != L0->k || L->H != L0->H || L->fmt != L0->fmt ||
        L->compute != L0->compute)
      return fail(MOE_ERR_INVALID_ARG, "stack layers must share E, top_k, H, format and compute stream");
    if (T > plans[l]->max_tokens) return fail(MOE_ERR_INVALID_ARG, "T exceeds a plan's max_tokens");
  }
  if (L0->fmt == MOE_FMT_F32) return fail(MOE_ERR_FORMAT, "the stack residual is bf16");
  if (T == 0) return MOE_OK;
  const size_t lstride = (size_t)T * L0->E;
  hipStream_t cs = L0->compute;
  moe_status st = MOE_OK;
  auto run = [&]() -> moe_status {
    moe_status r = route_impl(layers[0], logits, T, plans[0], nullptr);
    if (r) return r;
    if (lookahead) {
      r = moe_page_in(layers[0], plans[0], 0);
      if (r) return r;
    }
    for (int l = 0; l < n; ++l) {
      moe_layer* L = layers[l];
      moe_plan* P = plans[l];
      if (lookahead && l + 1 < n) {
        r = route_impl(layers[l + 1], logits + (l + 1) * lstride, T, plans[l + 1], nullptr);
        if (r) return r;
        r = moe_page_in(layers[l + 1], plans[l + 1], 0);
        if (r) return r;
      }
      const int nw = P->info.num_waves;
      for (int w = 0; w < nw; ++w) {
        if (w > 0 || !lookahead) {
          r = moe_page_in(L, P, w);
          if (r) return r;
        }
        // the kernel that completes the last wave's out also applies the residual
        r = forward_impl(L, P, w, x, out, w == nw - 1 ? (uint16_t*)x : nullptr, /*norm=*/1);
        if (r) return r;
      }
      if (!lookahead && l + 1 < n) {
        // strict order: layer l+1 is routed on the compute stream, behind the
        // residual, with no cross-stream hand-over
        r = route_impl(layers[l + 1], logits + (l + 1) * lstride, T, plans[l + 1], nullptr, cs);
        if (r) return r;
      }
    }
    return MOE_OK;
  };
  st = run();
  return st;
}

namespace {

bool stream_capturing(hipStream_t s) {
  hipStreamCaptureStatus c = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &c) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return c != hipStreamCaptureStatusNone;
}

// Waves a device-resolved step of T tokens may need: its distinct experts
// (at most min(T * top_k, E)) in chunks of K.
constexpr int kMaxDeviceWaves = 16;
int device_waves(const moe_layer* L, int T) {
  const int D = std::min(T * L->k, L->E);
  return (D + L->K - 1) / L->K;
}

// Device-resolved step that may need more than one wave ([PE] "What happens
// with more than one request?": each wave pages in its misses, then computes
// its experts; the plan is the host-driven one): one launch routes and plans
// every wave, then, for each wave w the step may have, a kernel page-in of
// w's misses and w's FFN over wave-order positions w * K .., all on the
// compute stream, so wave w + 1's copies follow wave w's math (they may
// overwrite its slots). Launches for waves the step does not have find no
// work (the counts are read on the device). Wave 0 writes out and later waves
// add to it; the stack residual is applied by the launch holding the step's
// last expert.
moe_status step_device_waves(moe_layer* L, const PlanDev& dev, float* h, const float* logits, int32_t T,
                             const void* x, float* out, uint16_t* x_res, int nw, int norm) {
  const hipStream_t cs = L->compute;
  TimerRec tr{};
  moe_status st = timer_events(L, &tr);
  if (st) return st;
  if (launch_route_plan_small(logits, T, L->E, L->k, L->K, L->state, dev, nullptr, 0, cs, tr.a, tr.b,
                              L->dstats) != hipSuccess)
    return fail(MOE_ERR_HIP, "route launch failed");
  timer_push(L, &tr, MOE_T_ROUTE, 0.0, 0.0);
  for (int w = 0; w < nw; ++w) {
    TimerRec tc{};
    if ((st = timer_events(L, &tc))) return st;
    if (launch_page_in_device(L->host_store_dev, L->slots, L->stride, dev, L->E, L->K, cs, tc.a, tc.b, w) !=
        hipSuccess)
      return fail(MOE_ERR_HIP, "page-in launch failed");
    timer_push(L, &tc, MOE_T_PAGE_IN, 0.0, 0.0);
    st = run_ffn(L, dev, h, nullptr, nullptr, nullptr, w * L->K, L->K, T * L->k, T, x, out, w > 0, nullptr,
                 nullptr, 0, T, false, x_res, dev.counts, nullptr, norm, nullptr, nullptr, /*res_last=*/1);
    if (st) return st;
  }
  return MOE_OK;
}

moe_status step_device_check(const moe_layer* L, const moe_plan* p, int32_t T) {
  if (!L || !p) return fail(MOE_ERR_INVALID_ARG, "null layer or plan");
  if (p->layer != L) return fail(MOE_ERR_INVALID_ARG, "plan was created for another layer");
  if (T < 1 || T > p->max_tokens || T > MOE_MAX_GEMV_TOKENS)
    return fail(MOE_ERR_INVALID_ARG, "num_tokens must be in 1..min(max_tokens, 64)");
  if (!route_small_ok(T, L->k)) return fail(MOE_ERR_INVALID_ARG, "too many pairs for one route launch");
  if (device_waves(L, T) > kMaxDeviceWaves)
    return fail(MOE_ERR_INVALID_ARG, "the step may need more than " + std::to_string(kMaxDeviceWaves) +
                                         " waves (T * top_k far above K)");
  if (!L->host_store_dev) return fail(MOE_ERR_STATE, "host store is not mapped into the device");
  if (L->cur_plan) return fail(MOE_ERR_STATE, "a host-driven step of this layer is unfinished");
  return MOE_OK;
}

// Device-resolved step: route + plan (kept on the device, counters in
// dstats) and the kernel page-in of the misses on stream `ps`, then the expert
// FFN (expert count read on the device) and the optional stack residual on the
// compute stream. With ps != compute the host records L->ev_copied on ps and
// the compute stream waits for it (under capture the pair becomes a graph
// dependency). A step that may need several waves runs step_device_waves, all
// on the compute stream.
moe_status step_device_core(moe_layer* L, const PlanDev& dev, float* h, const float* logits, int32_t T,
                            const void* x, float* out, uint16_t* x_res, hipStream_t ps, bool cap,
                            bool no_timers, int norm = 0) {
  const hipStream_t cs = L->compute;
  const bool timing = L->timing;
  if (cap || no_timers) L->timing = false;  // dispatch-stamped events are not captured
  moe_status st = MOE_OK;
  const int nw = device_waves(L, T);
  if (nw > 1) {
    st = step_device_waves(L, dev, h, logits, T, x, out, x_res, nw, norm);
  } else do {
    TimerRec tr{}, tc{};
    if (ps == cs && route_page_in_ok(L->E)) {
      // one launch routes, plans and pages in (timed as the page-in; its ticket
      // counter is the layer's device counter 6)
      if ((st = timer_events(L, &tc))) break;
      if (launch_route_plan_page_in(logits, T, L->E, L->k, L->K, L->state, dev, L->dstats,
                                    (unsigned long long*)(L->dstats + 6), L->host_store_dev, L->slots,
                                    L->stride, ps, tc.a, tc.b) != hipSuccess) {
        st = fail(MOE_ERR_HIP, "route and page-in launch failed");
        break;
      }
      timer_push(L, &tc, MOE_T_PAGE_IN, 0.0, 0.0);
    } else {
      if ((st = timer_events(L, &tr)) || (st = timer_events(L, &tc))) break;
      if (launch_route_plan_small(logits, T, L->E, L->k, L->K, L->state, dev, nullptr, 0, ps, tr.a, tr.b,
                                  L->dstats) != hipSuccess) {
        st = fail(MOE_ERR_HIP, "route launch failed");
        break;
      }
      timer_push(L, &tr, MOE_T_ROUTE, 0.0, 0.0);
      if (launch_page_in_device(L->host_store_dev, L->slots, L->stride, dev, L->E, L->K, ps, tc.a, tc.b) !=
          hipSuccess) {
        st = fail(MOE_ERR_HIP, "page-in launch failed");
        break;
      }
      // bytes are not known on the host here; moe_layer_stats has the misses
      timer_push(L, &tc, MOE_T_PAGE_IN, 0.0, 0.0);
    }
    if (ps != cs && (hipEventRecord(L->ev_copied, ps) != hipSuccess ||
                     hipStreamWaitEvent(cs, L->ev_copied, 0) != hipSuccess)) {
      st = fail(MOE_ERR_HIP, "hand-over from the copy stream failed");
      break;
    }
    // at most min(T * top_k, E) experts; exactly top_k for one token
    const int n_max = std::min(T * L->k, L->E);
    st = run_ffn(L, dev, h, nullptr, nullptr, nullptr, 0, n_max, T * L->k, T, x, out, 0, nullptr,
                 nullptr, 0, T, false, x_res, dev.counts, nullptr, norm);
  } while (0);
  L->timing = timing;
  if (st) return st;
  if (!cap) {  // ordering for later host-driven calls on other streams
    HIP_TRY(hipEventRecord(L->ev_fwd_done, cs));
    L->fwd_recorded = true;
  }
  L->dev_steps = true;
  L->dev_pending = true;
  return MOE_OK;
}

// Device-resolved step with a plan's arrays (step_device_core), then the
// plan's consumption event.
moe_status step_device_impl(moe_layer* L, moe_plan* p, const float* logits, int32_t T, const void* x,
                            float* out, uint16_t* x_res, hipStream_t ps, bool cap, int norm = 0) {
  moe_status st = step_device_core(L, p->dev, p->h, logits, T, x, out, x_res, ps, cap, false, norm);
  if (st) return st;
  if (!cap) {
    HIP_TRY(hipEventRecord(p->ev_consumed, L->compute));
    p->consumed_recorded = true;
  }
  p->valid = false;
  p->dev_routed = true;
  p->dev_tokens = T;
  return MOE_OK;
}

}  // namespace

moe_status moe_step_device(moe_layer* L, moe_plan* p, const float* logits, int32_t T, const void* x,
                           float* out, void* x_res) {
  moe_status st = step_device_check(L, p, T);
  if (st) return st;
  if (!logits || !x || !out) return fail(MOE_ERR_INVALID_ARG, "null logits, x or out");
  if (((uintptr_t)x & 15) || ((uintptr_t)out & 15) || ((uintptr_t)x_res & 7))
    return fail(MOE_ERR_INVALID_ARG, "x and out must be 16-byte aligned, x_res 8-byte aligned");
  if (x_res && L->fmt == MOE_FMT_F32) return fail(MOE_ERR_FORMAT, "the stack residual is bf16");
  return step_device_impl(L, p, logits, T, x, out, (uint16_t*)x_res, L->compute,
                          stream_capturing(L->compute));
}

moe_status moe_step_device_static(moe_layer* L, const float* logits, int32_t T, const void* x, float* out,
                                  void* x_res) {
  if (!L) return fail(MOE_ERR_INVALID_ARG, "null layer");
  if (T < 1 || T > MOE_MAX_GEMV_TOKENS) return fail(MOE_ERR_INVALID_ARG, "num_tokens must be in 1..64");
  if ((int64_t)T * L->k > L->K)
    return fail(MOE_ERR_INVALID_ARG, "T * top_k exceeds K: the step may need more than one wave");
  if (!route_small_ok(T, L->k)) return fail(MOE_ERR_INVALID_ARG, "too many pairs for one route launch");
  if (!L->host_store_dev) return fail(MOE_ERR_STATE, "host store is not mapped into the device");
  if (L->cur_plan) return fail(MOE_ERR_STATE, "a host-driven step of this layer is unfinished");
  if (!logits || !x || !out) return fail(MOE_ERR_INVALID_ARG, "null logits, x or out");
  if (((uintptr_t)x & 15) || ((uintptr_t)out & 15) || ((uintptr_t)x_res & 7))
    return fail(MOE_ERR_INVALID_ARG, "x and out must be 16-byte aligned, x_res 8-byte aligned");
  if (x_res && L->fmt == MOE_FMT_F32) return fail(MOE_ERR_FORMAT, "the stack residual is bf16");
  const StepWs ws = step_workspace(L->E, T * L->k, L->I);
  if (ws.total > kStaticScratchBytes)
    return fail(MOE_ERR_INVALID_ARG, "step needs " + std::to_string(ws.total) +
                                         " bytes of workspace, more than the fixed " +
                                         std::to_string(kStaticScratchBytes));
  uint8_t* b = (L->device >= 0 && L->device < kMaxDevices) ? g_scratch_ptr[L->device] : nullptr;
  if (!b) return fail(MOE_ERR_STATE, "no workspace address for the layer's device");
  // Every array below is written by the route kernel before it is read in
  // the same step, so nothing needs clearing between calls.
  PlanDev dev{};
  dev.ids = (int32_t*)(b + ws.ids);
  dev.weights = (float*)(b + ws.w);
  dev.slot_ids = (int32_t*)(b + ws.sid);
  dev.wave_of = (int32_t*)(b + ws.wo);
  dev.order_expert = (int32_t*)(b + ws.oe);
  dev.order_slot = (int32_t*)(b + ws.os);
  dev.pair_off = (int32_t*)(b + ws.po);
  dev.pair_list = (int32_t*)(b + ws.pl);
  dev.pair_pos = (int32_t*)(b + ws.pp);
  dev.pair_w = (float*)(b + ws.pw);
  dev.counts = (int32_t*)(b + ws.cnt);
  return step_device_core(L, dev, (float*)(b + ws.h), logits, T, x, out, (uint16_t*)x_res, L->compute,
                          stream_capturing(L->compute), /*no_timers=*/true);
}

moe_status moe_step_token_waves(moe_layer* L, moe_plan* p, const float* logits, int32_t T, const void* x,
                                float* out, void* x_res) {
  if (!L || !p) return fail(MOE_ERR_INVALID_ARG, "null layer or plan");
  const int G = std::min({L->K / L->k, p->max_tokens, (int)MOE_MAX_GEMV_TOKENS});
  if (G < 1) return fail(MOE_ERR_INVALID_ARG, "K < top_k: no group of tokens fits one wave");
  if (T < 1) return fail(MOE_ERR_INVALID_ARG, "num_tokens must be >= 1");
  if (!logits || !x || !out) return fail(MOE_ERR_INVALID_ARG, "null logits, x or out");
  if (((uintptr_t)x & 15) || ((uintptr_t)out & 15) || ((uintptr_t)x_res & 7))
    return fail(MOE_ERR_INVALID_ARG, "x and out must be 16-byte aligned, x_res 8-byte aligned");
  if (x_res && L->fmt == MOE_FMT_F32) return fail(MOE_ERR_FORMAT, "the stack residual is bf16");
  moe_status st = step_device_check(L, p, std::min(G, T));
  if (st) return st;
  const size_t xe = L->fmt == MOE_FMT_F32 ? 4 : 2, H = (size_t)L->H;
  const bool cap = stream_capturing(L->compute);
  // consecutive groups of G tokens, one device-resolved single-wave step each,
  // in token order on the compute stream (every group reuses the plan buffers)
  for (int32_t t0 = 0; t0 < T; t0 += G) {
    const int32_t n = std::min(G, T - t0);
    st = step_device_impl(L, p, logits + (size_t)t0 * L->E, n, (const uint8_t*)x + t0 * H * xe,
                          out + t0 * H, x_res ? (uint16_t*)x_res + t0 * H : nullptr, L->compute, cap);
    if (st) return st;
  }
  return MOE_OK;
}

moe_status moe_stack_forward_device(moe_layer* const* layers, moe_plan* const* plans, int32_t n,
                                    const float* logits, int32_t T, void* x, float* out,
                                    int32_t lookahead) {
  if (!layers || !plans || n < 1) return fail(MOE_ERR_INVALID_ARG, "need n_layers >= 1 layers and plans");
  if (!logits || !x || !out) return fail(MOE_ERR_INVALID_ARG, "bad buffers");
  if (((uintptr_t)x & 15) || ((uintptr_t)out & 15))
    return fail(MOE_ERR_INVALID_ARG, "x and out must be 16-byte aligned");
  const moe_layer* L0 = layers[0];
  if (!L0) return fail(MOE_ERR_INVALID_ARG, "null layer");
  for (int l = 0; l < n; ++l) {
    const moe_layer* L = layers[l];
    moe_status st = step_device_check(L, plans[l], T);
    if (st) return fail(st, "layer " + std::to_string(l) + ": " + g_err);
    if (L->E != L0->E || L->k != L0->k || L->H != L0->H || L->fmt != L0->fmt ||
        L->compute != L0->compute)
      return fail(MOE_ERR_INVALID_ARG, "stack layers must share E, top_k, H, format and compute stream");
  }
  if (L0->fmt == MOE_FMT_F32) return fail(MOE_ERR_FORMAT, "the stack residual is bf16");
  if (lookahead && !(route_page_in_ok(L0->E) && up_route_next_ok(L0->fmt, L0->H, L0->E, T * L0->k)))
    return fail(MOE_ERR_INVALID_ARG, "lookahead needs E <= 256, T * top_k <= 256 and an up kernel of this shape");
  for (int l = 0; lookahead && l < n; ++l)
    if (device_waves(layers[l], T) > 1)
      return fail(MOE_ERR_INVALID_ARG, "lookahead needs single-wave steps (T * top_k <= K)");
  const size_t lstride = (size_t)T * L0->E;
  const hipStream_t cs = L0->compute;
  const bool cap = stream_capturing(cs);
  if (!lookahead) {
    for (int l = 0; l < n; ++l) {
      moe_status st = step_device_impl(layers[l], plans[l], logits + l * lstride, T, x, out, (uint16_t*)x, cs,
                                       cap, /*norm=*/1);
      if (st) return st;
    }
    return MOE_OK;
  }
  // Lookahead, one stream: layer 0 is routed and paged in alone and layer 1
  // routed; then, for every layer l, one launch runs l's up projection, copies
  // the first half of each record l + 1 misses and routes l + 2, and one runs
  // l's down projection and residual and copies the second halves ([PE]
  // "TL;DR": the experts of the next layer cross PCIe while this layer's math
  // runs; routing a layer before its copies are due keeps the router off the
  // copies' path). Valid only when the router logits do not depend on the
  // previous layers' outputs (given in advance), the caller's promise.
  auto next_of = [&](int l) {
    moe_layer* M = layers[l];
    moe_plan* q = plans[l];
    NextStep ns{};
    ns.logits = logits + l * lstride;
    ns.T = T;
    ns.E = M->E;
    ns.k = M->k;
    ns.K = M->K;
    ns.state = M->state;
    ns.sl = state_layout(M->E, M->K);
    ns.dev = q->dev;
    ns.dstats = M->dstats;
    ns.ticket = (unsigned long long*)(M->dstats + 6);
    ns.host = M->host_store_dev;
    ns.slots = M->slots;
    ns.stride = M->stride;
    // the up launch copies the first half of each missed record, the down
    // launch the rest (16-byte pieces; the stride is a multiple of 256)
    ns.cp_len = M->stride / 2 / 16 * 16;
    return ns;
  };
  std::vector<bool> timing(n);
  for (int l = 0; l < n; ++l) {
    timing[l] = layers[l]->timing;
    if (cap) layers[l]->timing = false;  // dispatch-stamped events are not captured
  }
  moe_status st = MOE_OK;
  {
    moe_layer* M = layers[0];
    TimerRec tc{};
    if ((st = timer_events(M, &tc)) == MOE_OK) {
      if (launch_route_plan_page_in(logits, T, M->E, M->k, M->K, M->state, plans[0]->dev, M->dstats,
                                    (unsigned long long*)(M->dstats + 6), M->host_store_dev, M->slots, M->stride,
                                    cs, tc.a, tc.b) != hipSuccess)
        st = fail(MOE_ERR_HIP, "route and page-in launch failed");
      else
        timer_push(M, &tc, MOE_T_PAGE_IN, 0.0, 0.0);
    }
  }
  if (!st && n > 1) {  // layer 1: routed and planned only; layer 0's launches copy it
    moe_layer* M = layers[1];
    if (launch_route_plan_page_in(logits + lstride, T, M->E, M->k, M->K, M->state, plans[1]->dev, M->dstats,
                                  (unsigned long long*)(M->dstats + 6), M->host_store_dev, M->slots, M->stride, cs,
                                  nullptr, nullptr, 0) != hipSuccess)
      st = fail(MOE_ERR_HIP, "route launch failed");
  }
  for (int l = 0; l < n && !st; ++l) {
    moe_layer* L = layers[l];
    moe_plan* p = plans[l];
    NextStep ns{}, rs{};
    if (l + 1 < n) ns = next_of(l + 1);
    if (l + 2 < n) rs = next_of(l + 2);
    const int n_max = std::min(T * L->k, L->E);
    st = run_ffn(L, p->dev, p->h, nullptr, nullptr, nullptr, 0, n_max, T * L->k, T, x, out, 0, nullptr, nullptr, 0,
                 T, false, (uint16_t*)x, p->dev.counts, nullptr, /*norm=*/1, l + 1 < n ? &ns : nullptr,
                 l + 2 < n ? &rs : nullptr);
  }
  for (int l = 0; l < n; ++l) layers[l]->timing = timing[l];
  if (st) return st;
  for (int l = 0; l < n; ++l) {
    moe_layer* L = layers[l];
    moe_plan* p = plans[l];
    if (!cap) {  // ordering for later host-driven calls on other streams
      HIP_TRY(hipEventRecord(L->ev_fwd_done, cs));
      L->fwd_recorded = true;
      HIP_TRY(hipEventRecord(p->ev_consumed, cs));
      p->consumed_recorded = true;
    }
    L->dev_steps = true;
    L->dev_pending = true;
    p->valid = false;
    p->dev_routed = true;
    p->dev_tokens = T;
  }
  return MOE_OK;
}

moe_status moe_layer_stats(const moe_layer* L, moe_stats* out) {
  if (!L || !out) return fail(MOE_ERR_INVALID_ARG, "null layer or output");
  *out = L->stats;
  if (L->dev_steps) {  // add the device-resolved steps' counters
    long long d[8];
    HIP_TRY(hipStreamSynchronize(L->compute));
    HIP_TRY(hipMemcpy(d, L->dstats, sizeof(d), hipMemcpyDeviceToHost));
    out->steps += d[0];
    out->refs += d[1];
    out->activations += d[2];
    out->hits += d[3];
    out->misses += d[4];
    out->waves += d[5];
    out->bytes_paged += d[4] * (int64_t)L->stride;
  }
  return MOE_OK;
}

moe_status moe_layer_get_state(moe_layer* L, int32_t* slot_expert, int32_t* expert_slot,
                               int64_t* stamp, int64_t* clock) {
  if (!L) return fail(MOE_ERR_INVALID_ARG, "null layer");
  HIP_TRY(hipStreamSynchronize(L->route));
  const StateLayout sl = state_layout(L->E, L->K);
  std::vector<uint8_t> buf(sl.total);
  HIP_TRY(hipMemcpy(buf.data(), L->state, sl.total, hipMemcpyDeviceToHost));
  if (slot_expert) std::memcpy(slot_expert, buf.data() + sl.slot_expert, 4 * (size_t)L->K);
  if (expert_slot) std::memcpy(expert_slot, buf.data() + sl.expert_slot, 4 * (size_t)L->E);
  if (stamp) std::memcpy(stamp, buf.data() + sl.stamp, 8 * (size_t)L->K);
  if (clock) std::memcpy(clock, buf.data() + sl.clock, 8);
  return MOE_OK;
}

moe_status moe_timing_enable(moe_layer* L, int32_t enable) {
  if (!L) return fail(MOE_ERR_INVALID_ARG, "null layer");
  L->timing = enable != 0;
  return MOE_OK;
}

moe_status moe_timing_read(moe_layer* L, moe_timing* out) {
  if (!L || !out) return fail(MOE_ERR_INVALID_ARG, "null layer or output");
  for (auto& t : L->pending) {
    HIP_TRY(hipEventSynchronize(t.b));
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, t.a, t.b));
    L->acc.count[t.cls] += 1;
    L->acc.ms[t.cls] += ms;
    L->acc.bytes[t.cls] += t.bytes;
    L->acc.flops[t.cls] += t.flops;
    L->pool.push_back(t.a);
    L->pool.push_back(t.b);
  }
  L->pending.clear();
  *out = L->acc;
  std::memset(&L->acc, 0, sizeof(L->acc));
  return MOE_OK;
}

moe_status moe_read_probe(void* stream, void* buf, size_t buf_bytes, size_t bytes, int32_t reps,
                          double* us) {
  if (!us || !buf) return fail(MOE_ERR_INVALID_ARG, "null buffer or output");
  if (reps < 1 || reps > 10000) return fail(MOE_ERR_INVALID_ARG, "reps must be in 1..10000");
  if (bytes < 16 || bytes % 16 || ((uintptr_t)buf & 255) || buf_bytes < 2 * bytes)
    return fail(MOE_ERR_INVALID_ARG, "bytes must be a positive multiple of 16 and at most half of a "
                                     "256-byte aligned buffer");
  const size_t n16 = bytes / 16;
  const size_t nwg = (n16 + 2047) / 2048;
  if (nwg > 0x7FFFFFFFu) return fail(MOE_ERR_INVALID_ARG, "read too large");
  // each launch starts one read's length plus 64 MB further on (wrapping), so
  // what it reads was not read by the launches just before
  const size_t hop = (bytes + 255) / 256 * 256 + ((size_t)64 << 20);
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t a = nullptr, b = nullptr;
  moe_status st = MOE_OK;
  std::vector<double> t;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
    st = fail(MOE_ERR_HIP, "event creation failed");
  } else {
    size_t off = 0;
    for (int r = 0; r <= reps && !st; ++r) {  // launch 0 warms up, untimed
      if (off + bytes > buf_bytes) off = 0;
      hipExtLaunchKernelGGL(read_probe_kernel, dim3((unsigned)nwg), dim3(512), 0, s, a, b, 0,
                            (const uint4*)((const uint8_t*)buf + off), n16, (uint32_t*)buf);
      off += hop;
      float ms = 0.f;
      if (hipGetLastError() != hipSuccess || hipEventSynchronize(b) != hipSuccess ||
          hipEventElapsedTime(&ms, a, b) != hipSuccess)
        st = fail(MOE_ERR_HIP, "read-probe timing failed");
      else if (r > 0)
        t.push_back(ms * 1e3);
    }
    if (!st) {
      std::sort(t.begin(), t.end());
      *us = t[t.size() / 2];
    }
  }
  if (a) (void)hipEventDestroy(a);
  if (b) (void)hipEventDestroy(b);
  return st;
}

moe_status moe_timing_floor(void* stream, int32_t reps, double* us) {
  if (!us) return fail(MOE_ERR_INVALID_ARG, "null output");
  if (reps < 1 || reps > 10000) return fail(MOE_ERR_INVALID_ARG, "reps must be in 1..10000");
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t a = nullptr, b = nullptr;
  moe_status st = MOE_OK;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
    st = fail(MOE_ERR_HIP, "event creation failed");
  } else {
    double total = 0.0;
    for (int r = 0; r <= reps && !st; ++r) {  // launch 0 warms up, untimed
      hipExtLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, s, a, b, 0);
      float ms = 0.f;
      if (hipGetLastError() != hipSuccess || hipEventSynchronize(b) != hipSuccess ||
          hipEventElapsedTime(&ms, a, b) != hipSuccess)
        st = fail(MOE_ERR_HIP, "empty-kernel timing failed");
      else if (r > 0)
        total += ms;
    }
    if (!st) *us = total * 1e3 / reps;
  }
  if (a) (void)hipEventDestroy(a);
  if (b) (void)hipEventDestroy(b);
  return st;
}

}  // extern "C"

namespace {

// Expert FFN over wave-order positions [o_lo, o_lo + n_exp). GEMV path: the
// down kernel writes (or, with accumulate, adds to) out. GEMM path: the two
// grouped GEMMs fill y for those experts' pairs; with combine, the combine
// kernel then adds the whole wave's pairs into out.
moe_status run_ffn(moe_layer* L, const PlanDev& dev, float* h, uint16_t* hb, uint16_t* hb_lo,
                   float* y, int o_lo, int n_exp, int n_pairs, int T, const void* x, float* out,
                   int accumulate, const int32_t* pair_pos, const int32_t* wave_of, int wave,
                   int max_rows, bool combine, uint16_t* x_res, const int32_t* n_dev,
                   uint8_t* wdq, int norm, const NextStep* next, const NextStep* route2, int res_last,
                   hipEvent_t after_up, hipEvent_t before_down) {
  FfnArgs a{};
  a.norm = norm;
  a.res_last = res_last;
  a.n_dev = n_dev;
  a.fmt = L->fmt;
  a.E = L->E;
  a.k = L->k;
  a.H = L->H;
  a.I = L->I;
  a.K = L->K;
  a.stride = L->stride;
  a.slots = L->slots;
  a.order_slot = dev.order_slot;
  a.pair_off = dev.pair_off;
  a.pair_list = dev.pair_list;
  a.weights = dev.weights;
  a.pair_w = dev.pair_w;
  a.o_lo = o_lo;
  a.n_exp = n_exp;
  a.T = T;
  a.x = x;
  a.out = out;
  a.accumulate = accumulate;
  a.h = h;
  a.hb = hb;
  a.hb_lo = hb_lo;
  a.y = y;
  a.max_rows = max_rows;
  const double xb = (L->fmt == MOE_FMT_F32 ? 4.0 : 2.0);
  // pairs of this wave are not known on the host; count the weight bytes
  // (exact) and bound the activation bytes by all pairs of the step
  const double up_b = n_exp * up_weight_bytes(L);
  const double dn_b = n_exp * down_weight_bytes(L);
  const double flop_up = 2.0 * 2.0 * L->I * (double)L->H * n_pairs;
  const double flop_dn = 2.0 * (double)L->H * L->I * n_pairs;
  (void)xb;
  moe_status st;
  if (T <= MOE_MAX_GEMV_TOKENS) {
    TimerRec t1{}, t2{};
    if ((st = timer_events(L, &t1)) || (st = timer_events(L, &t2))) return st;
    a.ev0 = t1.a;
    a.ev1 = t1.b;
    if (next) {
      // the launch also routes and pages in the next layer; its length is
      // mostly that layer's copies, so it is timed with the page-ins
      HIP_TRY(launch_up_route_next(a, *next, route2, L->compute));
      timer_push(L, &t1, MOE_T_PAGE_IN, 0.0, 0.0);
    } else {
      HIP_TRY(launch_ffn_up(a, L->compute));
      timer_push(L, &t1, MOE_T_FFN_UP, up_b, flop_up);
    }
    // optional: mark the up projection done / wait for the down weights
    if (after_up) HIP_TRY(hipEventRecord(after_up, L->compute));
    if (before_down) HIP_TRY(hipStreamWaitEvent(L->compute, before_down, 0));
    a.ev0 = t2.a;
    a.ev1 = t2.b;
    a.x_res = x_res;  // the down kernel completes out
    if (next) {  // ... and copies the rest of the next layer's missed records
      HIP_TRY(launch_ffn_down_copy_next(a, *next, L->compute));
      timer_push(L, &t2, MOE_T_PAGE_IN, 0.0, 0.0);
    } else {
      HIP_TRY(launch_ffn_down(a, L->compute));
      timer_push(L, &t2, MOE_T_FFN_DOWN, dn_b, flop_dn);
    }
  } else {
    TimerRec t1{}, t2{}, t3{};
    // 4-bit experts past the GEMMs' LDS scale region: the wave's records are
    // expanded to bf16 first; otherwise the GEMMs read the records in place
    // (weights widened in registers)
    if (!gemm_reads_record(L->fmt, L->H, L->I)) {
      if (!wdq) return fail(MOE_ERR_STATE, "plan has no dequantisation scratch");
      const size_t ws = rec_layout(MOE_FMT_BF16, L->H, L->I).stride;
      HIP_TRY(launch_dequant_bf16(a, wdq, ws, L->compute));
      a.wbase = wdq;
      a.wstride = ws;
    }
    if ((st = timer_events(L, &t1)) || (st = timer_events(L, &t2))) return st;
    a.ev0 = t1.a;
    a.ev1 = t1.b;
    HIP_TRY(launch_gemm_up(a, L->compute));
    timer_push(L, &t1, MOE_T_GEMM_UP, up_b, flop_up);
    if (after_up) HIP_TRY(hipEventRecord(after_up, L->compute));
    if (before_down) HIP_TRY(hipStreamWaitEvent(L->compute, before_down, 0));
    a.ev0 = t2.a;
    a.ev1 = t2.b;
    HIP_TRY(launch_gemm_down(a, L->compute));
    timer_push(L, &t2, MOE_T_GEMM_DOWN, dn_b, flop_dn);
    if (combine) {
      if ((st = timer_events(L, &t3))) return st;
      a.ev0 = t3.a;
      a.ev1 = t3.b;
      a.x_res = x_res;  // the combine completes out
      HIP_TRY(launch_combine(a, pair_pos, wave_of, wave, L->compute));
      timer_push(L, &t3, MOE_T_COMBINE, 0.0, 0.0);
    }
  }
  return MOE_OK;
}

// Startup independence check ([PE] "Can paging change the model's outputs?":
// at startup one more chunk of experts is re-run and the check fails if
// experts got mixed). Pages up to four experts into two different slot
// permutations and requires each expert's output to be bitwise identical in
// both and different from every other expert's output.
moe_status self_check(moe_layer* L) {
  const int n = std::min(std::min(L->K, L->E), 4);
  const int H = L->H, I = L->I;
  const size_t xsz = (L->fmt == MOE_FMT_F32 ? 4 : 2) * (size_t)H;
  std::vector<uint8_t> xh(xsz);
  for (int i = 0; i < H; ++i) {
    const float v = 0.5f * (float)((i * 37) % 17 - 8) / 8.f;
    if (L->fmt == MOE_FMT_F32) std::memcpy(&xh[4 * i], &v, 4);
    else {
      uint32_t b;
      std::memcpy(&b, &v, 4);
      const uint16_t hbits = (uint16_t)(b >> 16);
      std::memcpy(&xh[2 * i], &hbits, 2);
    }
  }
  // scratch: x, out[2][n][H], h[I], and a one-pair plan per launch
  size_t off = 0;
  auto take = [&](size_t b) {
    size_t o = off;
    off = align_up(off + b, 256);
    return o;
  };
  const size_t o_x = take(xsz), o_out = take(sizeof(float) * 2 * n * H), o_h = take(sizeof(float) * I),
               o_os = take(4), o_po = take(8), o_pl = take(4), o_w = take(4);
  void* blk = nullptr;
  HIP_TRY(hipMalloc(&blk, off));
  uint8_t* b = (uint8_t*)blk;
  moe_status result = MOE_OK;
  std::vector<float> outs(2 * (size_t)n * H);
  do {
    const int32_t po[2] = {0, 1}, pl = 0;
    const float one = 1.f;
    if (hipMemcpy(b + o_x, xh.data(), xsz, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(b + o_po, po, 8, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(b + o_pl, &pl, 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(b + o_w, &one, 4, hipMemcpyHostToDevice) != hipSuccess) {
      result = fail(MOE_ERR_HIP, "self-check setup copy failed");
      break;
    }
    PlanDev dev{};
    dev.order_slot = (int32_t*)(b + o_os);
    dev.pair_off = (int32_t*)(b + o_po);
    dev.pair_list = (int32_t*)(b + o_pl);
    dev.weights = (float*)(b + o_w);
    dev.pair_w = dev.weights;  // the one pair is at CSR position 0
    const bool timing = L->timing;
    L->timing = false;
    for (int perm = 0; perm < 2 && !result; ++perm) {
      for (int i = 0; i < n && !result; ++i) {
        // second placement: every expert shifted by ceil(K / 2) slots (mod K),
        // a different slot for each expert whenever K >= 2 (checked at init)
        const int slot = perm == 0 ? i : (i + (L->K + 1) / 2) % L->K;
        if (hipMemcpy(L->slots + (size_t)slot * L->stride, L->host_store + (size_t)i * L->stride,
                      L->stride, hipMemcpyHostToDevice) != hipSuccess ||
            hipMemcpy(b + o_os, &slot, 4, hipMemcpyHostToDevice) != hipSuccess) {
          result = fail(MOE_ERR_HIP, "self-check page-in failed");
          break;
        }
        float* o = (float*)(b + o_out) + ((size_t)perm * n + i) * H;
        // the one-pair plan addresses token 0 as pair 0 (k may exceed 1: pair 0 / k == 0)
        result = run_ffn(L, dev, (float*)(b + o_h), nullptr, nullptr, nullptr, 0, 1, 1, 1, b + o_x,
                         o, 0, nullptr, nullptr, 0, 1, false);
        if (!result && hipStreamSynchronize(L->compute) != hipSuccess)
          result = fail(MOE_ERR_HIP, "self-check forward failed");
      }
    }
    L->timing = timing;
    if (result) break;
    if (hipMemcpy(outs.data(), b + o_out, sizeof(float) * outs.size(), hipMemcpyDeviceToHost) != hipSuccess) {
      result = fail(MOE_ERR_HIP, "self-check readback failed");
      break;
    }
    for (int i = 0; i < n && !result; ++i) {
      if (std::memcmp(&outs[(size_t)i * H], &outs[((size_t)n + i) * H], sizeof(float) * H) != 0)
        result = fail(MOE_ERR_SELFCHECK, "expert " + std::to_string(i) +
                                             " gives different outputs from two different slots");
      for (int j = 0; j < i && !result; ++j)
        if (std::memcmp(&outs[(size_t)i * H], &outs[(size_t)j * H], sizeof(float) * H) == 0)
          result = fail(MOE_ERR_SELFCHECK, "experts " + std::to_string(j) + " and " +
                                               std::to_string(i) + " give identical outputs");
    }
  } while (0);
  (void)hipFree(blk);
  return result;
}

}  // namespace
