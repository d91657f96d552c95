/*
 * moepage.h -- C ABI of the Paged Experts hot path on AMD MI355X (gfx950).
 *
 * Sources, cited by title and section:
 *   [PE]  "Running an MoE Model Larger Than Your VRAM: SGLang Paged Experts,
 *         the PCIe Math, and the 4-Request Cliff" (post on the sgl-project
 *         feed page).
 *   [LRU] "Locality of reference helped 94GB Qwen3.8-Flash-Next runs at 68
 *         tok/s on one RTX 5090" (post on the same page).
 *
 * The scheme ([PE] "TL;DR", "What does Paged Experts actually do?"): every MoE
 * layer keeps K of its E experts in a slot table in GPU memory and all E in
 * pinned host memory; a step copies in only the routed experts that are not
 * resident (least recently used out), then runs the expert math on the GPU.
 *
 * One layer-step is:
 *   moe_route(layer, logits, T, plan)             router + slot plan; returns
 *                                                  once the plan is host-visible
 *   for w in 0 .. plan.num_waves-1:
 *     moe_page_in(layer, plan, w)                  async copies, copy stream
 *     moe_forward(layer, plan, w, x, out)          async expert FFN, compute stream
 *
 * Conventions for every call:
 *   - Returns MOE_OK (0) or a negative moe_status; nothing throws or aborts
 *     across the ABI. moe_last_error() gives a message for the calling thread.
 *   - Pointers marked "device" are HIP device pointers (torch CUDA tensors);
 *     "host" are CPU pointers. Streams are hipStream_t passed as void*;
 *     NULL means the null stream.
 *   - The caller owns every buffer it passes and both/all streams. The library
 *     owns only the opaque handles and what moe_plan_create allocates.
 *   - A layer handle and the plans used with it are used by one host thread
 *     at a time.
 *   - There is never a silent fallback: unsupported shapes or formats fail at
 *     init ([PE] "A rollout checklist": rejection at startup is the good
 *     failure).
 */
#ifndef MOEPAGE_H
#define MOEPAGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* bad shape, pointer, wave index or size limit   */
  MOE_ERR_NOT_PINNED = -2,  /* host store is not page-locked host memory       */
  MOE_ERR_FORMAT = -3,      /* unknown format or record size mismatch          */
  MOE_ERR_HIP = -4,         /* a HIP runtime call failed                        */
  MOE_ERR_SELFCHECK = -5,   /* slot-independence check at init failed           */
  MOE_ERR_STATE = -6,       /* calls out of order (page-in/forward vs plan)     */
  MOE_ERR_TIMEOUT = -7      /* the plan did not become host-visible in time     */
} moe_status;

/* Expert weight formats ([PE] "What does Paged Experts actually do?": bf16,
 * block-FP8 and GPTQ-style int4 experts; MXFP4 is among the formats it lists
 * for the follow-up work). Record layout of one expert, in this
 * order (reduction dimension contiguous in every matrix):
 *   W13 = [W_gate; W_up]  2I x H      W_d  H x I
 *   MOE_FMT_F32            : float32 weights
 *   MOE_FMT_BF16           : bfloat16 weights
 *   MOE_FMT_FP8_E4M3_B128  : OCP e4m3fn codes, then float32 scales per 128x128
 *                            tile: W13 [2I/128][H/128], W_d [H/128][I/128];
 *                            w = decode(q) * scale (weight-only)
 *   MOE_FMT_INT4_ASYM_G128 : 8 codes per uint32 along the reduction dim (low
 *                            nibble = lower index), then float16 scales W13
 *                            [2I][H/128], W_d [H][I/128], then float16 zeros
 *                            in the same shapes; w = (q - z) * s
 *   MOE_FMT_MXFP4_B32      : OCP microscaling FP4: E2M1 codes, two per byte
 *                            (low nibble = lower index), then one E8M0 scale
 *                            byte per 32 weights along the reduction dim:
 *                            W13 [2I][H/32], W_d [H][I/32];
 *                            w = e2m1(q) * 2^(scale - 127)
 * All per-expert tensors live in the one record, so one page-in moves all of
 * them ([PE] "Can paging change the model's outputs?": a tensor left unpaged
 * makes a paged-in expert run with another expert's values). The record
 * stride is the payload rounded up to 256 bytes. */
typedef enum moe_format {
  MOE_FMT_F32 = 0,
  MOE_FMT_BF16 = 1,
  MOE_FMT_FP8_E4M3_B128 = 2,
  MOE_FMT_INT4_ASYM_G128 = 3,
  MOE_FMT_MXFP4_B32 = 4
} moe_format;

/* Limits of this implementation (checked at init). */
#define MOE_MAX_EXPERTS 1024        /* E                                      */
#define MOE_MAX_TOP_K 32            /* top_k                                  */
#define MOE_MAX_GEMV_TOKENS 64      /* tokens per forward on the GEMV path (f32: the limit) */

/* Record stride in bytes for a format and shape, or 0 if unsupported. */
size_t moe_record_bytes(int32_t format, int32_t hidden, int32_t intermediate);

/* Bytes of the per-layer slot-table state buffer (device). Layout:
 * int32 slot_expert[K], int32 expert_slot[E], int64 stamp[K], int64 clock,
 * each array starting on an 8-byte boundary. */
size_t moe_state_bytes(int32_t num_experts, int32_t num_slots);

/* Slots per layer for a device-memory budget, the same K in every layer
 * ([LRU] "How to use it": the expert cache is sized as one memory budget;
 * [PE] "What does a resident slot cost in context length?": a slot costs its
 * record bytes in each MoE layer): the largest K <= num_experts with
 * K * layers * moe_record_bytes(format, hidden, intermediate) <= budget_bytes.
 * Host-only. Returns K >= 0, or MOE_ERR_INVALID_ARG for an unsupported
 * format/shape, num_experts or layers < 1, or a negative budget. */
int32_t moe_slots_for_budget(int32_t format, int32_t hidden, int32_t intermediate,
                             int32_t num_experts, int32_t layers, int64_t budget_bytes);

/* Preflight arithmetic ([PE] "A preflight script before you turn it on"),
 * host-only. Inputs: MoE layers, experts per layer, top_k, per-expert MB
 * (1e6 bytes), slots K, a measured host-link GB/s, a measured decode tok/s and
 * the KV-cache bytes per token. */
typedef struct moe_preflight_result {
  double slot_mb;                /* expert_mb * layers: one slot in every layer   */
  double kv_tokens_per_slot;     /* slot bytes / KV bytes per token               */
  int32_t batch_cap;             /* K / top_k: the largest batch that is one wave */
  double all_miss_gb_per_token;  /* layers * top_k * expert_mb / 1e3              */
  double max_miss;               /* link GB/s / (tok/s * all-miss GB per token):
                                    the highest miss rate the speed allows        */
  double random_miss;            /* 1 - K / E: the miss rate without reuse        */
  int32_t reuse_implied;         /* max_miss < 0.8 * random_miss                  */
} moe_preflight_result;

/* MOE_ERR_INVALID_ARG for a null out, layers, experts, top_k or K < 1, K > E,
 * or a non-positive expert_mb, link_gbps, tok_s or kv_bytes_per_token. */
moe_status moe_preflight(int32_t layers, int32_t experts, int32_t top_k, double expert_mb,
                         int32_t num_slots, double link_gbps, double tok_s,
                         double kv_bytes_per_token, moe_preflight_result* out);

typedef struct moe_layer_desc {
  int32_t num_experts;   /* E, 1..MOE_MAX_EXPERTS                              */
  int32_t top_k;         /* k, 1..min(E, MOE_MAX_TOP_K)                        */
  int32_t hidden;        /* H                                                  */
  int32_t intermediate;  /* I                                                  */
  int32_t num_slots;     /* K, 1..E ([PE] "What does Paged Experts actually do?")*/
  int32_t format;        /* moe_format                                          */
  size_t record_bytes;   /* must equal moe_record_bytes(format, H, I)          */
  const void* host_store;/* host, pinned, [E][record_bytes]; caller-owned; must
                            outlive the handle ([PE] "What does Paged Experts
                            actually do?": the pinned store holds every expert) */
  void* slot_store;      /* device, [K][record_bytes]; caller-owned              */
  void* state;           /* device, moe_state_bytes(E, K); caller-owned          */
  int32_t initial_fill;  /* 0: empty table; 1: experts 0..K-1 copied into slots
                            0..K-1 (stamp 0) at init and at reset                */
  int32_t self_check;    /* 1: run the slot-independence check at init (K >= 2)  */
} moe_layer_desc;

typedef struct moe_layer moe_layer;
typedef struct moe_plan moe_plan;

/* Create a layer. Validates the descriptor; verifies with
 * hipPointerGetAttributes that host_store is page-locked host memory
 * (MOE_ERR_NOT_PINNED otherwise); initialises the state buffer (synchronously)
 * and, with initial_fill, copies experts 0..K-1 into the slots.
 *   compute_stream: expert FFN kernels
 *   copy_stream:    page-in copies (hipMemcpyAsync, pinned host -> slot)
 *   route_stream:   router and slot-plan kernels (may equal compute_stream)
 * With self_check, pages a few experts into two different slot permutations
 * and requires bitwise-identical per-expert outputs and distinct outputs
 * across experts ([PE] "Can paging change the model's outputs?": the startup
 * independence check); MOE_ERR_SELFCHECK on failure. */
moe_status moe_layer_init(const moe_layer_desc* desc, void* compute_stream,
                          void* copy_stream, void* route_stream, moe_layer** out);

/* Restore the initial table (empty, or experts 0..K-1 when initial_fill),
 * synchronously, after the layer's streams have drained ([PE] "What does
 * Paged Experts actually do?": the K resident slots start empty or hold the
 * first K experts; this returns a layer to that state between runs).
 * Statistics are kept. MOE_ERR_INVALID_ARG for a null layer, MOE_ERR_HIP if a
 * synchronisation or copy fails. */
moe_status moe_layer_reset(moe_layer* layer);
void moe_layer_destroy(moe_layer* layer);

/* Create a plan for up to max_tokens tokens per route call with this layer.
 * Allocates small device arrays (ids, weights, slot map, grouping), the
 * pinned host-visible plan and the FFN workspace; with max_tokens above
 * MOE_MAX_GEMV_TOKENS the GEMM workspace too (for int4 and MXFP4 layers
 * with H > 2048 or I > 1024 it includes min(K, E) bf16 records, 6 * H * I
 * bytes each). Errors:
 * MOE_ERR_INVALID_ARG (max_tokens < 1; more than MOE_MAX_GEMV_TOKENS tokens
 * on an f32 layer or with H or I not a multiple of 128), MOE_ERR_HIP. */
moe_status moe_plan_create(const moe_layer* layer, int32_t max_tokens, moe_plan** out);
void moe_plan_destroy(moe_plan* plan);

/* Route T tokens and plan the step.
 *   logits: device, float32 [T][E], row-major
 * Router: top_k largest logits compared as float32, equal logits to the
 * smaller id, listed by descending logit; weights are the softmax renormalised
 * over the selected k ([PE] "What does Paged Experts actually do?").
 * Slot plan: distinct routed experts D; residents first, then missing ones,
 * each ascending; waves are consecutive chunks of K of that order, so a step
 * is one wave exactly when |D| <= K ([PE] "What happens with more than one
 * request?"). Per wave the clock ticks; victims are slots whose expert is not
 * in the wave, empty first, then oldest stamp, ties to the lower slot; the
 * i-th missing expert (ascending id) takes the i-th victim ([PE] "TL;DR":
 * least recently used out; [LRU] "The fix").
 * Kernels run on route_stream; they wait for the plan's previous forward. The
 * call returns once the plan is host-visible (the one host synchronisation of
 * a layer-step). T may be 0 (no waves). T <= max_tokens. */
moe_status moe_route(moe_layer* layer, const float* logits, int32_t num_tokens, moe_plan* plan);

typedef struct moe_plan_info {
  int32_t num_tokens;
  int32_t num_distinct;   /* |D|                          */
  int32_t num_hits;       /* resident at the start        */
  int32_t num_misses;     /* experts paged in, all waves  */
  int32_t num_waves;      /* ceil(|D| / K)                */
} moe_plan_info;

typedef struct moe_wave_info {
  int32_t num_experts;             /* experts in this wave                   */
  int32_t num_misses;              /* of which paged in                      */
  const int32_t* experts;          /* host, [num_experts], wave order        */
  const int32_t* slots;            /* host, [num_experts], slot of each      */
  const int32_t* miss_experts;     /* host, [num_misses] = tail of experts   */
  const int32_t* miss_slots;       /* host, [num_misses] = tail of slots     */
} moe_wave_info;

/* Host views of the last routed plan (valid until the next moe_route). */
moe_status moe_plan_get_info(const moe_plan* plan, moe_plan_info* out);
moe_status moe_plan_get_wave(const moe_plan* plan, int32_t wave, moe_wave_info* out);

/* Copy the plan's per-(token, j) arrays to host buffers (synchronous; for
 * checking): ids int32 [T][k], weights float32 [T][k], slot of each pair
 * during its wave int32 [T][k], wave of each pair int32 [T][k]. Any pointer
 * may be NULL. */
moe_status moe_plan_read(const moe_plan* plan, int32_t* ids, float* weights,
                         int32_t* slot_ids, int32_t* wave_of);

/* Page in the misses of one wave ([PE] "What does Paged Experts actually
 * do?": only the routed experts that are not resident are copied from the
 * pinned host store into slots; "What happens with more than one request?":
 * every wave has its own page-in; "Can paging change the model's outputs?":
 * the whole record moves, so no per-expert tensor is left behind): each
 * miss's whole host record -> its slot by hipMemcpyAsync (misses that are consecutive in both stores, expert e + 1 into
 * slot s + 1 after e into s, share one copy), on copy_stream, after the
 * layer's previous forward has finished
 * (a victim slot may still be read by it). Waves are paged in and computed in
 * order: page_in(w) requires forward(w-1) to have been issued.
 * Errors: MOE_ERR_INVALID_ARG (null layer or plan), MOE_ERR_STATE (plan not
 * this layer's current step, wave out of order, corrupt miss list),
 * MOE_ERR_HIP (a copy could not be enqueued). */
moe_status moe_page_in(moe_layer* layer, const moe_plan* plan, int32_t wave);

/* Expert math of one wave on compute_stream, after that wave's page-in
 * ([PE] "What does Paged Experts actually do?": once a wave's experts are in
 * their slots the MoE computation runs over the slots; its output for a token
 * is the router-weighted sum of its top_k SwiGLU experts, 3 matrices of H x I
 * each as "Why is it fast when experts keep crossing PCIe?" sizes them):
 *   x:   device, [T][H], float32 for MOE_FMT_F32 else bfloat16
 *   out: device, float32 [T][H]; wave 0 writes it, later waves add to it
 * out[t] = sum over (t, j) in this wave of w_tj * W_d (SiLU(W_gate x_t) *
 * (W_up x_t)), reading each expert from its slot. For T <= MOE_MAX_GEMV_TOKENS
 * the weights are streamed once per wave (GEMV path); with more tokens the
 * token-grouped bf16 MFMA GEMM runs (H and I multiples of 128): FP8 records,
 * and int4 and MXFP4 records with H <= 2048 and I <= 1024, are read in place
 * and widened to bf16 in registers; larger int4 and MXFP4 shapes are first
 * expanded to bf16 in the plan's workspace (either way each weight is its
 * dequantised value in fp32 rounded to nearest even); f32 layers are limited
 * to the GEMV path.
 * A wave with both resident and missed experts is computed in two launches on
 * the GEMV path (residents first, while the copies are in flight), decided
 * from the plan alone, so results are bitwise reproducible.
 * Errors: MOE_ERR_INVALID_ARG (null or misaligned x/out), MOE_ERR_STATE
 * (forward without its page-in, out of order), MOE_ERR_HIP. */
moe_status moe_forward(moe_layer* layer, const moe_plan* plan, int32_t wave,
                       const void* x, float* out);

/* Unit-gain RMSNorm of bf16 hidden states, the input of every layer of a
 * stack: a[t][i] = bf16_rne(x[t][i] / sqrt(mean_i(x[t][i]^2) + MOE_RMS_EPS))
 * (float32 arithmetic, fixed summation order). The pages run Qwen3-30B-A3B
 * ([PE] "What does Paged Experts actually do?"), whose MoE block reads the
 * residual stream through an RMSNorm; with no trained weights here its gain
 * is one. x and a: device bf16 [T][H], 16-byte aligned, may alias; H a
 * multiple of 8. Runs on the given stream. MOE_ERR_INVALID_ARG for bad
 * sizes, pointers or alignment. */
#define MOE_RMS_EPS 1e-6f
moe_status moe_rmsnorm_bf16(const void* x, void* a, int32_t num_tokens, int32_t hidden, void* stream);

/* Residual of a stack of MoE layers (attention omitted):
 * x_out[i] = bf16_rne(float(x_in[i]) + out[i]) for i < n; x_in and x_out are
 * device bf16 (may alias), out device float32. Runs on the given stream. */
moe_status moe_residual_bf16(const void* x_in, const float* out, void* x_out,
                             int64_t n, void* stream);

/* A batch through a stack of paged MoE layers, attention omitted: for each
 * layer l, a = moe_rmsnorm_bf16(x), out = MoE_l(a) and then
 * x = bf16_rne(x + out), in place (on the GEMV path the norm is computed
 * inside the first expert kernel, with the same bits as moe_rmsnorm_bf16).
 *   layers, plans: n_layers handles (plan l created for layer l with
 *                  max_tokens >= T); all layers share E, top_k, H, format and
 *                  the compute stream
 *   logits:        device, float32 [n_layers][T][E]
 *   x:             device, bf16 [T][H], updated in place
 *   out:           device, float32 [T][H], scratch
 *   lookahead:     0 = strict order (layer l+1 is routed after layer l's
 *                  residual, on the compute stream's timeline); 1 = layer l+1
 *                  is routed and its first wave paged in while layer l
 *                  computes, so its copies overlap layer l's math ([PE] "TL;DR":
 *                  the expert math stays on the GPU while experts cross PCIe).
 *                  Lookahead is only valid when the router input of layer l+1
 *                  does not depend on layer l's output (e.g. logits computed
 *                  in advance), which is the caller's promise.
 * Host-synchronous per layer (each moe_route waits for its plan); the GPU
 * work is asynchronous. */
moe_status moe_stack_forward(moe_layer* const* layers, moe_plan* const* plans, int32_t n_layers,
                             const float* logits, int32_t num_tokens, void* x, float* out,
                             int32_t lookahead);

/* Device-resolved step: the graph-capturable path ([PE] "What happens with
 * more than one request?": a step whose experts fit in the slots is one wave,
 * the case a graph can capture; a larger step runs several waves, each paging
 * in its misses before it computes). Routes the T tokens, plans the step,
 * pages the misses in and runs the experts, all on the layer's compute stream,
 * with the plan kept on the device: the miss list is read by a copy kernel
 * from device memory and the records are read from the host store through its
 * device mapping, so there is no host synchronisation and no allocation, and
 * the call may be captured in a HIP graph (timers are skipped while the
 * stream captures). When T * top_k > K the step may need several waves: one
 * launch plans them all, then for each wave the step may have (up to
 * ceil(min(T * top_k, E) / K)) a page-in launch and the FFN launches follow
 * in order; launches for waves the step turns out not to have find no work.
 *   logits: device float32 [T][E]; x: device bf16 [T][H] (fp32 for the f32
 *           format); out: device float32 [T][H], overwritten (16-byte aligned)
 *   x_res:  NULL, or device bf16 [T][H] that receives bf16_rne(x_res + out)
 *           (the stack residual; may alias x)
 * Requirements: 1 <= T <= min(max_tokens, MOE_MAX_GEMV_TOKENS), at most 16
 * possible waves (ceil(min(T * top_k, E) / K) <= 16); a host store that is mapped
 * into the device (moe_host_alloc memory is); no unfinished host-driven step
 * of the layer. Results (plan arrays, table state, out) are the same as a
 * host-driven step; the plan's host view is not updated (moe_plan_get_info
 * and moe_plan_get_wave return MOE_ERR_STATE until the next moe_route;
 * moe_plan_read reads the device arrays), and the layer counters of these
 * steps are kept on the device and added by moe_layer_stats. Errors:
 * MOE_ERR_INVALID_ARG (sizes, pointers, alignment), MOE_ERR_STATE (unmapped
 * store, unfinished host step), MOE_ERR_FORMAT (x_res on an f32 layer),
 * MOE_ERR_HIP. A later host-driven moe_route of the layer waits for all work
 * enqueued on the compute stream by then; replays of a captured graph must
 * therefore be launched on the compute stream (or be ordered before the
 * route by the caller). */
moe_status moe_step_device(moe_layer* layer, moe_plan* plan, const float* logits,
                           int32_t num_tokens, const void* x, float* out, void* x_res);

/* moe_step_device without a plan, for callers that cannot allocate device
 * memory while they run (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the step's plan arrays and FFN scratch
 * (ids, weights, slot map, grouping, h) live in one fixed device array of
 * MOE_STATIC_WORKSPACE_BYTES per GPU, compiled into the library and held
 * until the process ends, instead of in a moe_plan. The call allocates
 * nothing (no hipMalloc, no event creation; timers are skipped) and enqueues
 * the same kernels as moe_step_device, so out, the table state and the
 * counters are the same.
 *   logits, x, out, x_res: as moe_step_device
 * Requirements: as moe_step_device with T * top_k <= K (one wave), and a workspace of
 * 11 arrays (4 * T * top_k or 4 * E bytes each, 256-byte aligned) plus
 * 4 * T * top_k * I bytes of h within MOE_STATIC_WORKSPACE_BYTES
 * (MOE_ERR_INVALID_ARG beyond it). Every call on one GPU shares that GPU's
 * array and leaves its contents behind: calls that overlap on one GPU (two
 * streams, two threads, two layers in flight at once) race and give wrong
 * results; successive calls on one stream are fine. Nothing in the array
 * needs to start at zero. */
#define MOE_STATIC_WORKSPACE_BYTES (4u << 20)
moe_status moe_step_device_static(moe_layer* layer, const float* logits, int32_t num_tokens,
                                  const void* x, float* out, void* x_res);

/* Token-partitioned waves: a batch larger than one wave allows, served as
 * consecutive groups of G = min(K / top_k, max_tokens, MOE_MAX_GEMV_TOKENS)
 * tokens, each group one device-resolved single-wave step (moe_step_device on
 * tokens [g*G, g*G + G) of logits, x, out and x_res), in token order on the
 * compute stream, with no host synchronisation ([PE] "What happens with more
 * than one request?": a decode batch of up to K // top_k requests is one
 * wave, the captured case; larger batches need several waves, each with its
 * own page-in). Against moe_route's expert-partitioned waves this pages an
 * expert shared by two groups once per group if it was evicted in between
 * (never fewer page-ins, often more), but needs no host round trip.
 *   logits: device float32 [T][E]; x: device bf16 [T][H] (fp32 for the f32
 *           format); out: device float32 [T][H], overwritten; x_res: NULL or
 *           device bf16 [T][H] (as in moe_step_device)
 * Requirements: T >= 1, K >= top_k, and the moe_step_device requirements
 * for the first group. The plan's device arrays afterwards describe the last
 * group. Errors: as moe_step_device; a failure leaves the groups before it
 * enqueued. */
moe_status moe_step_token_waves(moe_layer* layer, moe_plan* plan, const float* logits,
                                int32_t num_tokens, const void* x, float* out, void* x_res);

/* moe_stack_forward through device-resolved steps: for each layer l,
 * moe_rmsnorm_bf16(x -> a) and moe_step_device(layer l, plan l, logits[l], T,
 * a, out, x_res = x), with the norm computed inside the up kernel (no extra
 * launch, the same bits) and no host synchronisation (capturable). Same requirements per layer as
 * moe_step_device; logits device float32 [n_layers][T][E]; x bf16 [T][H]
 * updated in place; out float32 [T][H] holds the last layer's MoE output.
 *   lookahead: 0 = each layer routed, paged in and computed in turn;
 *              1 = layer 0 is routed and paged in alone and layer 1 routed,
 *              then for every layer l one launch runs l's up projection while
 *              extra workgroups of it copy the first half of each record
 *              layer l + 1 misses and route layer l + 2, and one launch runs
 *              l's down projection and residual while extra workgroups copy
 *              the second halves ([PE] "TL;DR": the next experts cross PCIe
 *              while the expert math runs; a layer is routed one launch pair
 *              before its copies, so they start with the launch); everything
 *              stays on the compute stream (no cross-stream hand-over), so a
 *              captured token is one straight chain of launches. Needs E <= 256
 *              and T * top_k <= 256. Like moe_stack_forward's lookahead this is
 *              valid only when the router logits do not depend on the previous
 *              layers' outputs (given in advance), the caller's promise. */
moe_status moe_stack_forward_device(moe_layer* const* layers, moe_plan* const* plans,
                                    int32_t n_layers, const float* logits, int32_t num_tokens,
                                    void* x, float* out, int32_t lookahead);

typedef struct moe_stats {
  int64_t steps;        /* moe_route calls with T > 0                          */
  int64_t refs;         /* sum of distinct experts per step                    */
  int64_t activations;  /* sum of T * top_k                                    */
  int64_t hits;         /* sum of resident-at-start distinct experts           */
  int64_t misses;       /* experts paged in                                    */
  int64_t waves;        /* sum of waves                                        */
  int64_t bytes_paged;  /* misses * record_bytes                               */
} moe_stats;

/* Per-layer counters ([LRU] "The fix": the hit rate is reported at exit;
 * [PE] "Why is it fast ...": only a counter inside the engine gives the real
 * miss rate). */
moe_status moe_layer_stats(const moe_layer* layer, moe_stats* out);

/* Synchronous copy of the table state to host buffers (any may be NULL):
 * slot_expert int32 [K], expert_slot int32 [E], stamp int64 [K], clock
 * ([PE] "TL;DR" and [LRU] "The fix": which expert each slot holds and when it
 * was last used decide the least-recently-used victim; exported so that a
 * caller can check the table against a reference). Waits for the layer's
 * route and compute streams. MOE_ERR_INVALID_ARG for a null layer,
 * MOE_ERR_HIP if the copy fails. */
moe_status moe_layer_get_state(moe_layer* layer, int32_t* slot_expert, int32_t* expert_slot,
                               int64_t* stamp, int64_t* clock);

/* Kernel timing with HIP events on the streams the work runs on. */
typedef enum moe_timer {
  MOE_T_ROUTE = 0,     /* router + slot plan + grouping kernels              */
  MOE_T_FFN_UP = 1,    /* GEMV path, gate/up + SiLU kernel                    */
  MOE_T_FFN_DOWN = 2,  /* GEMV path, down projection + weighted combine       */
  MOE_T_GEMM_UP = 3,   /* GEMM path, grouped gate/up GEMM + SiLU              */
  MOE_T_GEMM_DOWN = 4, /* GEMM path, grouped down GEMM                        */
  MOE_T_COMBINE = 5,   /* GEMM path, weighted top-k combine                   */
  MOE_T_PAGE_IN = 6,   /* one wave's page-in copies                           */
  MOE_T_COUNT = 7
} moe_timer;

typedef struct moe_timing {
  int64_t count[MOE_T_COUNT];    /* timed launches                            */
  double ms[MOE_T_COUNT];        /* summed event-measured duration            */
  double bytes[MOE_T_COUNT];     /* summed algorithmic bytes (weights read for
                                    the FFN/GEMM classes, bytes copied for
                                    page-in)                                  */
  double flops[MOE_T_COUNT];     /* summed algorithmic flops                  */
} moe_timing;

/* enable != 0 starts recording events around each timed launch (adds host
 * overhead); moe_timing_read waits for them, returns the sums since the last
 * read and clears them. */
moe_status moe_timing_enable(moe_layer* layer, int32_t enable);
moe_status moe_timing_read(moe_layer* layer, moe_timing* out);

/* Floor of the figures above: the average duration the same dispatch-stamped
 * events report for an empty one-workgroup kernel, over `reps` (1..10000)
 * launches on `stream` (a hipStream_t; NULL = default stream). It is the
 * part of every timed launch that does not depend on the kernel's work (the
 * dispatch and the cache actions at kernel boundaries). Synchronous; *us
 * receives microseconds. MOE_ERR_INVALID_ARG for a null us or reps out of
 * range, MOE_ERR_HIP if a launch or event call fails. */
moe_status moe_timing_floor(void* stream, int32_t reps, double* us);

/* Reference for the FFN launches' durations: the median duration, by the same
 * dispatch-stamped events, of one launch of a plain streaming read of `bytes`
 * bytes (16 per lane, every load issued before any is used, nothing stored),
 * over `reps` (1..10000) launches on `stream`, each reading a different part
 * of the caller's device buffer `buf` of buf_bytes (each launch starts the
 * read's length plus 64 MB past the previous one, wrapping): with buf_bytes
 * several times the 256 MB last-level cache every read comes from HBM, as in
 * the caches-cold decode pass. bytes: a positive multiple of 16, at most
 * buf_bytes / 2; buf 256-byte aligned; its first 4 bytes may be overwritten.
 * Synchronous; *us receives microseconds. MOE_ERR_INVALID_ARG for bad sizes
 * or pointers, MOE_ERR_HIP if a launch or event call fails. */
moe_status moe_read_probe(void* stream, void* buf, size_t buf_bytes, size_t bytes, int32_t reps,
                          double* us);

/* Page-locked host memory for expert stores (hipHostMalloc), and its release. */
void* moe_host_alloc(size_t bytes);
void moe_host_free(void* p);

/* Message of the last failing call on this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOEPAGE_H */
