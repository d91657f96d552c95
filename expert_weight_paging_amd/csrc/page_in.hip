// Device-resolved page-in: a kernel copies the missed experts' records from
// the host store (page-locked and mapped into the GPU's address space) into
// their slots, reading the miss list the slot-plan kernel left on the device.
//
// [PE] ("Running an MoE Model Larger Than Your VRAM: SGLang Paged Experts, the
// PCIe Math, and the 4-Request Cliff"), "What happens with more than one
// request?": a step whose distinct experts fit in the slots is one wave, and
// that single wave is the case a graph can capture. With the miss list
// resolved on the device, route, page-in and expert math of such a step are
// enqueued without the host reading the plan, so no host synchronisation sits
// between them and the sequence can be captured in a HIP graph. The copy moves
// the same bytes as the host-issued DMA copies ([PE] "TL;DR": only routed,
// non-resident experts cross the link, whole records).
//
// Reads of mapped host memory travel over PCIe; 64 workgroups with four
// 16-byte loads in flight per thread keep the link as busy as the DMA engines
// (measured on MI355X: 50 to 57 GB/s for 2.5 to 75 MB), while leaving the
// other CUs free.
#include "copy.h"
#include "internal.h"

namespace moepage {

namespace {

constexpr int kCopyBlocks = 64;
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(kCopyThreads) void page_in_kernel(const uint8_t* __restrict__ host,
                                                               uint8_t* __restrict__ slots,
                                                               size_t stride,
                                                               const int32_t* __restrict__ order_expert,
                                                               const int32_t* __restrict__ order_slot,
                                                               const int32_t* __restrict__ counts, int E,
                                                               int K, int wave) {
  // the misses of this wave, in wave order: positions wave * K .. of the
  // order that come after the hits (all hits are in wave 0)
  const int D = counts[0], nH = counts[1];
  const int m0 = max(nH, wave * K), m1 = min(D, (wave + 1) * K);
  for (int m = m0; m < m1; ++m) {
    const int e = order_expert[m], s = order_slot[m];
    if (e < 0 || e >= E || s < 0 || s >= K) continue;  // never produced by the plan
    copy_record_share<kCopyThreads, kCopyUnroll>(host + (size_t)e * stride, slots + (size_t)s * stride, stride,
                                                 blockIdx.x, gridDim.x);
  }
}

}  // namespace

hipError_t launch_page_in_device(const uint8_t* host_store_dev, uint8_t* slots, size_t stride,
                                 const PlanDev& dev, int E, int K, hipStream_t s, hipEvent_t ev0,
                                 hipEvent_t ev1, int wave) {
  launch_k(page_in_kernel, dim3(kCopyBlocks), dim3(kCopyThreads), s, ev0, ev1, host_store_dev, slots,
           stride, (const int32_t*)dev.order_expert, (const int32_t*)dev.order_slot,
           (const int32_t*)dev.counts, E, K, wave);
  return hipGetLastError();
}

}  // namespace moepage
