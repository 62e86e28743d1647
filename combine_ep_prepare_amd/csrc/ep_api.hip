// ep_api.hip -- the C ABI of include/ep.h: argument validation, handle
// layout and kernel launches. Stateless apart from a per-device cache of the
// architecture check and compute-unit count, and the static scratch array of
// ep_prepare_static with its per-device address.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <cstring>

#include "ep.h"
#include "ep_internal.h"

using namespace epmi;

namespace {

constexpr int64_t kInt32Limit = (int64_t)1 << 31;
constexpr int kMaxDevices = 64;

// 0 = unknown, 1 = gfx950, 2 = other architecture; then the CU count.
std::atomic<int> g_dev_kind[kMaxDevices];
std::atomic<int> g_dev_cus[kMaxDevices];

// Device address of `scratch` (below) on each device, 0 until looked up.
std::atomic<uintptr_t> g_scratch_addr[kMaxDevices];

static_assert(EP_PREPARE_STATIC_SCRATCH_BYTES % 256 == 0, "whole 256-byte blocks");

}  // namespace

// ep_prepare_static's scratch: prepare's per-unit histograms and bad-id flags
// (up to EP_PREPARE_STATIC_SCRATCH_BYTES), in place of the handle's scratch
// region. Each device holds its own copy until the process ends. In host code
// this name is only a stand-in for the device array: its device address comes
// from hipGetSymbolAddress, once per device (static_scratch below).
static __device__ __align__(256) int32_t scratch[EP_PREPARE_STATIC_SCRATCH_BYTES / 4];

namespace {

// The current device's address of `scratch`, looked up on the first call on
// that device with the device current.
ep_status_t static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return EP_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return EP_ERR_DEVICE;
  uintptr_t a = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (a == 0) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return EP_ERR_HIP;
    a = reinterpret_cast<uintptr_t>(p);
    g_scratch_addr[dev].store(a, std::memory_order_release);
  }
  *out = reinterpret_cast<void*>(a);
  return EP_OK;
}

ep_status_t check_layout(const ep_layout_t* L) {
  if (!L) return EP_ERR_NULL;
  if (L->recv_capacity < 0 || L->recv_capacity >= kInt32Limit) return EP_ERR_CAPACITY;
  if (L->num_tokens < 0 || L->num_tokens >= kInt32Limit) return EP_ERR_SHAPE;
  if (L->topk < 1 || L->topk > kMaxTopk) return EP_ERR_SHAPE;
  if (L->num_experts < 1 || L->num_experts > kMaxExperts) return EP_ERR_SHAPE;
  if (L->alignment < 1) return EP_ERR_SHAPE;
  if (L->dtype != EP_DTYPE_BF16 && L->dtype != EP_DTYPE_FP16 && L->dtype != EP_DTYPE_FP32)
    return EP_ERR_SHAPE;
  if ((L->flags & ~(uint32_t)(EP_LAYOUT_NO_PAD_FILL | EP_LAYOUT_ZERO_TAIL)) != 0)
    return EP_ERR_SHAPE;
  if (L->hidden < 8 || L->hidden % 8 != 0 || L->hidden >= kInt32Limit) return EP_ERR_SHAPE;
  const int64_t routes = L->num_tokens * (int64_t)L->topk;
  const int64_t worst = routes + (int64_t)L->num_experts * ((int64_t)L->alignment - 1);
  if (routes >= kInt32Limit || worst >= kInt32Limit) return EP_ERR_SHAPE;
  return EP_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks that the current device is gfx950 (once per device) and returns its
// compute-unit count.
ep_status_t current_device(int* num_cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return EP_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return EP_ERR_DEVICE;
  int kind = g_dev_kind[dev].load(std::memory_order_acquire);
  if (kind == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return EP_ERR_HIP;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    kind = ok ? 1 : 2;
    g_dev_kind[dev].store(kind, std::memory_order_release);
  }
  if (kind != 1) return EP_ERR_DEVICE;
  *num_cus = g_dev_cus[dev].load(std::memory_order_relaxed);
  return EP_OK;
}

Dims dims_of(const ep_layout_t* L, int32_t num_units) {
  Dims d;
  d.T = L->num_tokens;
  d.K = L->topk;
  d.E = L->num_experts;
  d.A = L->alignment;
  d.num_units = num_units;
  d.cap = L->recv_capacity;
  d.H = L->hidden;
  const int64_t esize = L->dtype == EP_DTYPE_FP32 ? 4 : 2;
  d.V = L->hidden * esize / 16;
  d.dtype = L->dtype;
  d.fill_pads = (L->flags & EP_LAYOUT_NO_PAD_FILL) ? 0 : 1;
  d.zero_tail = (L->flags & EP_LAYOUT_ZERO_TAIL) ? 1 : 0;
  return d;
}

// Common host-side checks of the payload ops; fills the dims and the handle
// view. The device check comes after each op's own pointer checks.
ep_status_t payload_common(const ep_layout_t* L, const void* handle_mem, size_t handle_bytes,
                           Dims* d, HandleView* hv) {
  ep_status_t st = check_layout(L);
  if (st != EP_OK) return st;
  if (!handle_mem) return EP_ERR_NULL;
  const HandleLayout hl =
      handle_layout(L->num_tokens, L->topk, L->num_experts, L->recv_capacity);
  if (handle_bytes < hl.maps_bytes) return EP_ERR_HANDLE_SIZE;
  if (!aligned16(handle_mem)) return EP_ERR_ALIGN;
  *d = dims_of(L, hl.num_units);
  *hv = handle_view(const_cast<void*>(handle_mem), hl);
  return EP_OK;
}

}  // namespace

extern "C" {

int64_t ep_recv_capacity_worst(int64_t num_tokens, int32_t topk, int32_t num_experts,
                               int32_t alignment) {
  if (num_tokens < 0 || topk < 1 || num_experts < 1 || alignment < 1) return -1;
  if (num_tokens >= kInt32Limit) return -1;
  const int64_t per_token = topk < num_experts ? topk : num_experts;
  return num_tokens * per_token + (int64_t)num_experts * ((int64_t)alignment - 1);
}

size_t ep_handle_mem_size(const ep_layout_t* layout) {
  if (check_layout(layout) != EP_OK) return 0;
  return handle_layout(layout->num_tokens, layout->topk, layout->num_experts,
                       layout->recv_capacity)
      .bytes;
}

ep_status_t ep_handle_regions(const ep_layout_t* layout, ep_handle_regions_t* out) {
  ep_status_t st = check_layout(layout);
  if (st != EP_OK) return st;
  if (!out) return EP_ERR_NULL;
  const HandleLayout hl = handle_layout(layout->num_tokens, layout->topk,
                                        layout->num_experts, layout->recv_capacity);
  out->status = hl.header + offsetof(HandleHeader, status);
  out->counts = hl.counts;
  out->offsets = hl.offsets;
  out->slot = hl.slot;
  out->row_src = hl.row_src;
  out->runs = hl.runs;
  out->bytes = hl.bytes;
  out->maps_bytes = hl.maps_bytes;
  out->stream_live = hl.header + offsetof(HandleHeader, stream_live);
  out->run_units = hl.header + offsetof(HandleHeader, run_units);
  out->run_list_entries = (size_t)run_stream_cap(hl.num_units);
  return EP_OK;
}

ep_status_t ep_prepare(const ep_layout_t* layout, const int64_t* topk_idx,
                       int32_t* token_counts, int32_t* expert_offsets, void* handle_mem,
                       size_t handle_bytes, hipStream_t stream) {
  ep_status_t st = check_layout(layout);
  if (st != EP_OK) return st;
  if (!token_counts || !handle_mem) return EP_ERR_NULL;
  if (layout->num_tokens > 0 && !topk_idx) return EP_ERR_NULL;
  const HandleLayout hl =
      handle_layout(layout->num_tokens, layout->topk, layout->num_experts,
                    layout->recv_capacity);
  if (handle_bytes < hl.bytes) return EP_ERR_HANDLE_SIZE;
  if (!aligned16(handle_mem)) return EP_ERR_ALIGN;
  int num_cus = 0;
  st = current_device(&num_cus);
  if (st != EP_OK) return st;
  const Dims d = dims_of(layout, hl.num_units);
  const HandleView hv = handle_view(handle_mem, hl);
  if (launch_prepare(d, hv, topk_idx, token_counts, expert_offsets, num_cus, stream) !=
      hipSuccess)
    return EP_ERR_HIP;
  return EP_OK;
}

ep_status_t ep_prepare_static(const ep_layout_t* layout, const int64_t* topk_idx,
                              int32_t* token_counts, int32_t* expert_offsets, void* handle_mem,
                              size_t handle_bytes, hipStream_t stream) {
  ep_status_t st = check_layout(layout);
  if (st != EP_OK) return st;
  if (!token_counts || !handle_mem) return EP_ERR_NULL;
  if (layout->num_tokens > 0 && !topk_idx) return EP_ERR_NULL;
  const HandleLayout hl =
      handle_layout(layout->num_tokens, layout->topk, layout->num_experts,
                    layout->recv_capacity);
  if (handle_bytes < hl.maps_bytes) return EP_ERR_HANDLE_SIZE;
  if (scratch_bytes(hl.num_units, layout->num_experts) > EP_PREPARE_STATIC_SCRATCH_BYTES)
    return EP_ERR_SCRATCH;
  if (!aligned16(handle_mem)) return EP_ERR_ALIGN;
  int num_cus = 0;
  st = current_device(&num_cus);
  if (st != EP_OK) return st;
  void* sp = nullptr;
  st = static_scratch(&sp);
  if (st != EP_OK) return st;
  const Dims d = dims_of(layout, hl.num_units);
  HandleView hv = handle_view(handle_mem, hl);
  // the histograms and flags go to the static array instead of the handle;
  // the hist kernel writes every entry before the slot kernel reads it, so
  // nothing there has to start at zero
  hv.unit_hist = static_cast<int32_t*>(sp);
  hv.unit_flags = reinterpret_cast<int32_t*>(static_cast<char*>(sp) +
                                             scratch_hist_bytes(hl.num_units, d.E));
  if (launch_prepare(d, hv, topk_idx, token_counts, expert_offsets, num_cus, stream) !=
      hipSuccess)
    return EP_ERR_HIP;
  return EP_OK;
}

ep_status_t ep_dispatch(const ep_layout_t* layout, const void* handle_mem,
                        size_t handle_bytes, const void* tokens,
                        const float* topk_weights, void* recv_tokens,
                        float* recv_topk_weights, hipStream_t stream) {
  Dims d;
  HandleView hv;
  int num_cus = 0;
  ep_status_t st = payload_common(layout, handle_mem, handle_bytes, &d, &hv);
  if (st != EP_OK) return st;
  // A buffer with no element may be NULL: tokens/topk_weights when T == 0,
  // recv_tokens/recv_topk_weights when recv_capacity == 0.
  const bool rows = d.cap > 0, toks = d.T > 0;
  if ((rows && !recv_tokens) || (toks && !tokens)) return EP_ERR_NULL;
  if (rows && toks && (topk_weights == nullptr) != (recv_topk_weights == nullptr))
    return EP_ERR_NULL;
  if (!aligned16(tokens) || !aligned16(recv_tokens)) return EP_ERR_ALIGN;
  st = current_device(&num_cus);
  if (st != EP_OK) return st;
  if (launch_run_rows(d, hv, tokens, topk_weights, recv_tokens, recv_topk_weights, num_cus,
                      stream) != hipSuccess)
    return EP_ERR_HIP;
  return EP_OK;
}

ep_status_t ep_combine(const ep_layout_t* layout, const void* handle_mem,
                       size_t handle_bytes, const void* expert_out, void* result,
                       hipStream_t stream) {
  Dims d;
  HandleView hv;
  int num_cus = 0;
  ep_status_t st = payload_common(layout, handle_mem, handle_bytes, &d, &hv);
  if (st != EP_OK) return st;
  if ((d.T > 0 && !result) || (d.cap > 0 && !expert_out)) return EP_ERR_NULL;
  if (!aligned16(expert_out) || !aligned16(result)) return EP_ERR_ALIGN;
  st = current_device(&num_cus);
  if (st != EP_OK) return st;
  if (launch_reduce_rows(d, hv, expert_out, nullptr, nullptr, result, nullptr, num_cus,
                         stream) != hipSuccess)
    return EP_ERR_HIP;
  return EP_OK;
}

ep_status_t ep_dispatch_bwd(const ep_layout_t* layout, const void* handle_mem,
                            size_t handle_bytes, const void* grad,
                            const float* g_recv_topk_weights, void* grad_tokens,
                            float* grad_topk_weights, hipStream_t stream) {
  Dims d;
  HandleView hv;
  int num_cus = 0;
  ep_status_t st = payload_common(layout, handle_mem, handle_bytes, &d, &hv);
  if (st != EP_OK) return st;
  if ((d.T > 0 && !grad_tokens) || (d.cap > 0 && !grad)) return EP_ERR_NULL;
  if (!aligned16(grad) || !aligned16(grad_tokens)) return EP_ERR_ALIGN;
  st = current_device(&num_cus);
  if (st != EP_OK) return st;
  if (launch_reduce_rows(d, hv, grad, nullptr, g_recv_topk_weights, grad_tokens,
                         grad_topk_weights, num_cus, stream) != hipSuccess)
    return EP_ERR_HIP;
  return EP_OK;
}

ep_status_t ep_combine_bwd(const ep_layout_t* layout, const void* handle_mem,
                           size_t handle_bytes, const void* grad, void* grad_expert_out,
                           hipStream_t stream) {
  Dims d;
  HandleView hv;
  int num_cus = 0;
  ep_status_t st = payload_common(layout, handle_mem, handle_bytes, &d, &hv);
  if (st != EP_OK) return st;
  if ((d.cap > 0 && !grad_expert_out) || (d.T > 0 && !grad)) return EP_ERR_NULL;
  if (!aligned16(grad) || !aligned16(grad_expert_out)) return EP_ERR_ALIGN;
  st = current_device(&num_cus);
  if (st != EP_OK) return st;
  if (launch_run_rows(d, hv, grad, nullptr, grad_expert_out, nullptr, num_cus, stream) !=
      hipSuccess)
    return EP_ERR_HIP;
  return EP_OK;
}

ep_status_t ep_combine_weighted(const ep_layout_t* layout, const void* handle_mem,
                                size_t handle_bytes, const void* expert_out,
                                const float* recv_topk_weights, void* result,
                                hipStream_t stream) {
  Dims d;
  HandleView hv;
  int num_cus = 0;
  ep_status_t st = payload_common(layout, handle_mem, handle_bytes, &d, &hv);
  if (st != EP_OK) return st;
  if ((d.T > 0 && !result) || (d.cap > 0 && (!expert_out || !recv_topk_weights)))
    return EP_ERR_NULL;
  if (!aligned16(expert_out) || !aligned16(result)) return EP_ERR_ALIGN;
  st = current_device(&num_cus);
  if (st != EP_OK) return st;
  // a non-null weight pointer selects the weighted sum; with no received
  // rows there is nothing to weight and the unweighted kernel writes zeros
  const float* rw = (d.cap > 0) ? recv_topk_weights : nullptr;
  if (launch_reduce_rows(d, hv, expert_out, rw, nullptr, result, nullptr, num_cus, stream) !=
      hipSuccess)
    return EP_ERR_HIP;
  return EP_OK;
}

ep_status_t ep_combine_weighted_bwd(const ep_layout_t* layout, const void* handle_mem,
                                    size_t handle_bytes, const void* grad,
                                    const void* expert_out, const float* recv_topk_weights,
                                    void* grad_expert_out, float* grad_recv_topk_weights,
                                    hipStream_t stream) {
  Dims d;
  HandleView hv;
  int num_cus = 0;
  ep_status_t st = payload_common(layout, handle_mem, handle_bytes, &d, &hv);
  if (st != EP_OK) return st;
  if (d.T > 0 && !grad) return EP_ERR_NULL;
  if (d.cap > 0) {
    if (!grad_expert_out || !recv_topk_weights) return EP_ERR_NULL;
    if (grad_recv_topk_weights && !expert_out) return EP_ERR_NULL;
  }
  if (!aligned16(grad) || !aligned16(expert_out) || !aligned16(grad_expert_out))
    return EP_ERR_ALIGN;
  st = current_device(&num_cus);
  if (st != EP_OK) return st;
  if (launch_weighted_bwd(d, hv, grad, expert_out, recv_topk_weights, grad_expert_out,
                          grad_recv_topk_weights, num_cus, stream) != hipSuccess)
    return EP_ERR_HIP;
  return EP_OK;
}

ep_status_t ep_read_status(const void* handle_mem, uint32_t* host_out, hipStream_t stream) {
  if (!handle_mem || !host_out) return EP_ERR_NULL;
  if (!aligned16(handle_mem)) return EP_ERR_ALIGN;
  int num_cus = 0;
  ep_status_t st = current_device(&num_cus);
  if (st != EP_OK) return st;
  const HandleHeader* h = static_cast<const HandleHeader*>(handle_mem);
  if (hipMemcpyAsync(host_out, &h->status, sizeof(uint32_t), hipMemcpyDeviceToHost, stream) !=
      hipSuccess)
    return EP_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return EP_ERR_HIP;
  return EP_OK;
}

const char* ep_status_str(ep_status_t status) {
  switch (status) {
    case EP_OK: return "ok";
    case EP_ERR_NULL: return "a required pointer is NULL";
    case EP_ERR_SHAPE: return "a layout size is out of range";
    case EP_ERR_ALIGN: return "a payload or handle pointer is not 16-byte aligned";
    case EP_ERR_HANDLE_SIZE: return "handle_bytes is below ep_handle_mem_size(layout)";
    case EP_ERR_CAPACITY: return "recv_capacity is negative or not below 2^31";
    case EP_ERR_DEVICE: return "the current device is not gfx950";
    case EP_ERR_HIP: return "a HIP call or kernel launch failed";
    case EP_ERR_SCRATCH:
      return "the layout needs more prepare scratch than ep_prepare_static's static buffer holds";
  }
  return "unknown ep_status_t";
}

}  // extern "C"
