// Measurement probes (context for the rooflines, not part of the method): a
// dense loop of bf16 matrix instructions that gives the throughput the chip
// sustains on them and its core clock under that load, and a streaming copy
// that gives the HBM bandwidth a plain read-once / write-once kernel reaches.
//
// Every wave runs `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16
// (32,768 FLOP each) on register operands, so nothing but the matrix pipes
// limits it. Wave 0 of each workgroup records the core clock counter
// (s_memtime) and the constant 100 MHz counter (s_memrealtime) at its start
// and end; their ratio is the core clock the workgroup ran at.
#include "device.h"
#include "internal.h"
#include "../../include/mmdit_probe.h"

namespace mmdit {

__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, uint64_t *clocks, float *sums) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (bf16)(1e-3f * (float)(lane + j));
    b[j] = (bf16)(1e-3f * (float)(lane - j));
  }
  f32x16 c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) c[k][i] = 0.f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = mfma32(a, b, c[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[k][i];
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    uint64_t *o = clocks + 4 * (uint64_t)blockIdx.x;
    o[0] = t0;
    o[1] = t1;
    o[2] = r0;
    o[3] = r1;
    sums[blockIdx.x] = s;  // keeps the matrix work live
  }
}

// Streaming copy: each thread moves four 16-byte words per step, all four
// loads issued before the stores, grid-stride over the buffer; n16 = number
// of 16-byte words.
__global__ __launch_bounds__(256) void copy_kernel(const u32x4 *src, u32x4 *dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256 * 4;
  for (int64_t i = (int64_t)blockIdx.x * 1024 + threadIdx.x; i < n16; i += stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + 256 * u < n16) v[u] = __builtin_nontemporal_load(src + i + 256 * u);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + 256 * u < n16) __builtin_nontemporal_store(v[u], dst + i + 256 * u);
  }
}

}  // namespace mmdit

extern "C" mmdit_status mmdit_probe_copy(const void *src, void *dst, uint64_t bytes, int32_t blocks,
                                         void *hip_stream) {
  mmdit::clear_error();
  if (!src || !dst || (reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(dst) & 15u) ||
      bytes % 16 || blocks < 1)
    return mmdit::fail(MMDIT_ERR_INVALID_ARG,
                       "src and dst must be 16-byte aligned device pointers, bytes a multiple of 16, blocks >= 1");
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  if (s0 < d0 + bytes && d0 < s0 + bytes) return mmdit::fail(MMDIT_ERR_INVALID_ARG, "src and dst overlap");
  hipLaunchKernelGGL(mmdit::copy_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(hip_stream),
                     static_cast<const mmdit::u32x4 *>(src), static_cast<mmdit::u32x4 *>(dst), (int64_t)(bytes / 16));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return mmdit::fail(MMDIT_ERR_HIP, "probe launch failed: %s", hipGetErrorString(e));
  return MMDIT_OK;
}

extern "C" mmdit_status mmdit_probe_mfma(int32_t blocks, int32_t iters, uint64_t *clocks, float *sums,
                                         void *hip_stream) {
  mmdit::clear_error();
  if (blocks < 1 || iters < 1) return mmdit::fail(MMDIT_ERR_INVALID_ARG, "blocks and iters must be >= 1");
  if (!clocks || (reinterpret_cast<uintptr_t>(clocks) & 15u))
    return mmdit::fail(MMDIT_ERR_INVALID_ARG, "clocks must be a non-NULL 16-byte aligned device pointer");
  if (!sums) return mmdit::fail(MMDIT_ERR_INVALID_ARG, "sums must be a non-NULL device pointer");
  hipLaunchKernelGGL(mmdit::mfma_loop_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(hip_stream), (int)iters, clocks, sums);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return mmdit::fail(MMDIT_ERR_HIP, "probe launch failed: %s", hipGetErrorString(e));
  return MMDIT_OK;
}
