/*
 * mmdit_probe.h - measurement probe of libmmdit (context for the rooflines
 * the benchmark reports; not part of the attention method or its ABI
 * contract).
 */
#ifndef MMDIT_PROBE_H
#define MMDIT_PROBE_H

#include <stdint.h>

#include "mmdit.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Launch `blocks` workgroups of 256 threads (4 waves) on hip_stream (NULL =
 * default); every wave runs `iters` rounds of 8 independent bf16
 * 32x32x16 matrix instructions (32,768 FLOP each) on register operands, so
 * one launch does blocks * 4 * iters * 8 * 32768 FLOP. Thread 0 of workgroup
 * b writes {core clock counter at its start, at its end, 100 MHz real-time
 * counter at its start, at its end} to clocks[4b .. 4b+3] (device memory,
 * uint64, 16-byte aligned, caller-owned); (end - start) of the first over the
 * second, times 100 MHz, is the core clock the workgroup ran at. It also
 * writes its wave 0's sum of the results to sums[b] (device float, so that
 * the work cannot be optimised away). Enqueues only; errors: INVALID_ARG
 * (blocks or iters < 1, clocks NULL or misaligned, sums NULL), HIP (launch
 * failure). */
mmdit_status mmdit_probe_mfma(int32_t blocks, int32_t iters, uint64_t *clocks, float *sums,
                              void *hip_stream);

/* Copy `bytes` (a multiple of 16) from src to dst (device, 16-byte aligned,
 * not overlapping) with `blocks` workgroups of 256 threads, each thread
 * moving four 16-byte words per grid-stride step with non-temporal loads and
 * stores: the HBM bandwidth of a plain streaming kernel. Enqueues only;
 * errors: INVALID_ARG, HIP. */
mmdit_status mmdit_probe_copy(const void *src, void *dst, uint64_t bytes, int32_t blocks, void *hip_stream);

/* Stream nsrc source buffers into ndst destination buffers at once, `bytes`
 * (a positive multiple of 16) each: srcs and dsts are HOST arrays of device
 * pointers (16-byte aligned, no two buffers overlapping); `blocks`
 * workgroups of 256 threads, each thread loading `unroll` (1 or 2) 16-byte
 * words of every source per grid-stride step with non-temporal accesses
 * before storing to every destination. dsts[w] receives the XOR of the
 * sources' words with w added to the first 32-bit component of each word
 * (so the result can be checked). With ndst = 0 the loads are folded into a
 * value written to *sink (a device uint32, required then) only in a case no
 * input here produces. Supported (nsrc, ndst): (1,0) read-only, (1,1) copy,
 * (2,1), (2,2) (the QK prologue's mix) and (4,2) (the adaLN backward's).
 * Moved bytes = (nsrc + ndst) * bytes. Enqueues only; errors: INVALID_ARG
 * (unsupported mix or unroll, NULL, misaligned or overlapping buffers),
 * HIP. */
mmdit_status mmdit_probe_streams(const void *const *srcs, int32_t nsrc, void *const *dsts, int32_t ndst,
                                 uint64_t bytes, int32_t blocks, int32_t unroll, uint32_t *sink, void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* MMDIT_PROBE_H */
