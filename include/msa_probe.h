/* msa_probe.h -- measurement probes of the GPU itself, beside the method's entry points.
 *
 * They measure the two hardware denominators the rooflines of the method's kernels are read
 * against, on the GPU at hand: the rate at which a large buffer streams in from HBM, and the
 * rate of bf16 matrix-core work with no memory traffic. They compute nothing of the method.
 * Same conventions as msa.h: device pointers, caller-owned buffers, work enqueued on the
 * caller's hipStream_t (passed as void*, NULL = the null stream), validation errors returned
 * before anything is enqueued, MSA_ERR_HIP for a failed launch. */
#ifndef MSA_PROBE_H
#define MSA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "msa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` bytes at `buf` (16-byte aligned, bytes a positive multiple of 16):
 * 2048 workgroups of 256 threads, eight 16-byte loads in flight per thread, grid-stride order.
 * A fold of each thread's data goes to sink[0 .. 2048 * 256 - 1] (524288 floats, 2 MiB) so
 * no load can be dropped.
 * The caller times the launch (HIP events on the stream) and divides bytes by the time. */
msa_status msa_probe_hbm_read(const void* buf, size_t bytes, float* sink, void* stream);

/* bf16 matrix-core rate: `workgroups` workgroups of 4 waves, each wave running `iters` rounds of
 * four independent v_mfma_f32_32x32x16_bf16 on register operands (32768 FLOP each), so
 * FLOP = workgroups * 4 * iters * 4 * 32768. One float per wave goes to
 * sink[0 .. 4 * workgroups - 1]. workgroups in 1 .. 65535, iters >= 1. */
msa_status msa_probe_mfma_bf16(float* sink, int32_t workgroups, int32_t iters, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MSA_PROBE_H */
