// Backward entry point that allocates nothing.
//
// mmdit_attn_bwd_noalloc runs the recompute backward of mmdit_attn_bwd with
// its workspace (D = rowsum(dO * O) and the gain-gradient partials; fp32
// plans also their dQ-hat / dK-hat accumulators) in a device array owned by
// the library, for callers that cannot call hipMalloc (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation). The caller
// still passes every input and output.
//
// The array is a file-scope __device__ object, so every GPU that loads the
// library holds its own copy, at its own address, until the process ends. In
// host code its name is only a handle: the device address comes from
// hipGetSymbolAddress, looked up once per device (with that device current)
// and kept; kernels only ever receive that address.
//
// Nothing in the workspace needs to start at zero: the dQ kernel writes D for
// every query before the dK/dV kernel reads it, every workgroup writes its
// gain partials (idle block-map slots write zeros), and the fp32 path writes
// every row of its accumulators before reading it. Every call on one GPU uses the same array, so two
// calls in flight at once on one GPU (on different streams, or from
// different threads without ordering) race and give wrong results.
#include <mutex>

#include "internal.h"

namespace mmdit {

static __device__ __align__(256) unsigned char scratch[MMDIT_NOALLOC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_scratch[kMaxDevices];
hipError_t g_lookup[kMaxDevices];

// Device address of this device's copy of `scratch`.
mmdit_status scratch_address(int dev, void **out) {
  std::call_once(g_once[dev], [dev] {
    void *ptr = nullptr;
    g_lookup[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch[dev] = ptr;
  });
  if (g_lookup[dev] != hipSuccess || g_scratch[dev] == nullptr)
    return fail(MMDIT_ERR_HIP, "hipGetSymbolAddress of the backward scratch failed on device %d: %s", dev,
                hipGetErrorString(g_lookup[dev]));
  *out = g_scratch[dev];
  return MMDIT_OK;
}

mmdit_status attn_bwd_noalloc(const mmdit_plan *plan, const void *blob, const mmdit_bwd_args *a, void *stream) {
  if (!plan) return fail(MMDIT_ERR_INVALID_ARG, "plan must not be NULL");
  if (!a) return fail(MMDIT_ERR_INVALID_ARG, "args must not be NULL");
  if (a->stages & MMDIT_STAGE_BWD_STORE_DS)
    return fail(MMDIT_ERR_UNSUPPORTED,
                "the allocation-free backward runs the recompute mode only (the stored dS takes ~2*H*sum(L^2) bytes)");
  if (plan->bwd_workspace_bytes > MMDIT_NOALLOC_WORKSPACE_BYTES)
    return fail(MMDIT_ERR_BUFFER_TOO_SMALL,
                "this pack's backward workspace (%llu bytes) exceeds the allocation-free entry point's %llu bytes",
                (unsigned long long)plan->bwd_workspace_bytes,
                (unsigned long long)MMDIT_NOALLOC_WORKSPACE_BYTES);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MMDIT_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MMDIT_ERR_UNSUPPORTED, "device %d is beyond the %d this entry point serves", dev, kMaxDevices);
  if (stream) {  // the scratch used is the current device's: the stream must be on it
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) return fail(MMDIT_ERR_HIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
    if (sdev != dev)
      return fail(MMDIT_ERR_INVALID_ARG, "the stream belongs to device %d, not the current device %d", (int)sdev,
                  dev);
  }
  void *ws = nullptr;
  mmdit_status st = scratch_address(dev, &ws);
  if (st) return st;
  // Exactly the recompute workspace: the stored-dS mode is never chosen.
  return attn_bwd(plan, blob, a, ws, plan->bwd_workspace_bytes, stream);
}

}  // namespace
}  // namespace mmdit

extern "C" mmdit_status mmdit_attn_bwd_noalloc(const mmdit_plan *plan, const void *plan_blob_dev,
                                               const mmdit_bwd_args *args, void *hip_stream) {
  mmdit::clear_error();
  try {
    return mmdit::attn_bwd_noalloc(plan, plan_blob_dev, args, hip_stream);
  } catch (...) {
    return mmdit::fail(MMDIT_ERR_INVALID_ARG, "allocation-free backward failed on the host");
  }
}
