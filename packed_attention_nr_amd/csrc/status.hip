// The per-device fault word of the library's kernels and its query.
//
// A kernel that finds, before reading anything else of it, that the device
// blob it was given is not the one the host plan describes (the blob header's
// fingerprint differs from the plan's) ORs MMDIT_DEVICE_FAULT_STALE_BLOB into
// this word and exits without writing anything. The word is a file-scope
// __device__ object, one per GPU; in host code its name is only a handle, and
// its device address comes from hipGetSymbolAddress (once per device, with
// that device current). mmdit_device_faults reads and clears it.
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "internal.h"

namespace mmdit {

static __device__ __align__(16) uint32_t fault_word;

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
uint32_t *g_word[kMaxDevices];
hipError_t g_lookup[kMaxDevices];

mmdit_status current_device(void *stream, int *dev_out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MMDIT_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MMDIT_ERR_UNSUPPORTED, "device %d is beyond the %d the library serves", dev, kMaxDevices);
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) return fail(MMDIT_ERR_HIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
    if (sdev != dev)
      return fail(MMDIT_ERR_INVALID_ARG, "the stream belongs to device %d, not the current device %d", (int)sdev,
                  dev);
  }
  *dev_out = dev;
  return MMDIT_OK;
}
}  // namespace

// Test hook for the launch-failure path: with MMDIT_FAULT_INJECT=launch in the
// environment, the entry points that launch the method's kernels fail where
// they would launch (after their argument checks, before any HIP call) with
// MMDIT_ERR_HIP and a message naming the hook; unset (or any other value), it
// does nothing. The variable is read on every call, so a test can set and
// clear it within one process.
mmdit_status injected_launch_fault() {
  const char *v = std::getenv("MMDIT_FAULT_INJECT");
  if (v && std::strcmp(v, "launch") == 0)
    return fail(MMDIT_ERR_HIP, "kernel launch failed: fault injected by MMDIT_FAULT_INJECT=launch (test hook)");
  return MMDIT_OK;
}

mmdit_status device_fault_word(void *stream, uint32_t **word) {
  int dev = -1;
  mmdit_status st = current_device(stream, &dev);
  if (st) return st;
  std::call_once(g_once[dev], [dev] {
    void *ptr = nullptr;
    g_lookup[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(fault_word));
    g_word[dev] = static_cast<uint32_t *>(ptr);
  });
  if (g_lookup[dev] != hipSuccess || !g_word[dev])
    return fail(MMDIT_ERR_HIP, "hipGetSymbolAddress of the fault word failed on device %d: %s", dev,
                hipGetErrorString(g_lookup[dev]));
  *word = g_word[dev];
  return MMDIT_OK;
}

static mmdit_status device_faults(uint32_t *flags, void *stream) {
  if (!flags) return fail(MMDIT_ERR_INVALID_ARG, "flags must not be NULL");
  uint32_t *word = nullptr;
  mmdit_status st = device_fault_word(stream, &word);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  static const uint32_t zero = 0;
  uint32_t got = 0;
  hipError_t e = hipMemcpyAsync(&got, word, sizeof(got), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(word, &zero, sizeof(zero), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(MMDIT_ERR_HIP, "reading the fault word failed: %s", hipGetErrorString(e));
  *flags = got;
  return MMDIT_OK;
}

}  // namespace mmdit

extern "C" mmdit_status mmdit_device_faults(uint32_t *flags, void *hip_stream) {
  mmdit::clear_error();
  try {
    return mmdit::device_faults(flags, hip_stream);
  } catch (...) {
    return mmdit::fail(MMDIT_ERR_INVALID_ARG, "fault query failed on the host");
  }
}
