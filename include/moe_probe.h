/*
 * moe_probe.h -- measurement probes of the MoE layer library (not part of the
 * layer): the measured peaks its kernels are reported against next to the
 * published ones.  "Why MoE on RTX 5090 falls short: a bandwidth measurement"
 * (news.malakhovai.ru) reports achieved bandwidth against a measured one and
 * bandwidth as a function of the bytes one kernel reads on cold data; these
 * two kernels are the MI355X counterparts.
 *
 * Return codes as moe.h: 0 ok, -1 NULL pointer, -2 size out of range,
 * -4 misaligned (16 bytes), -6 HIP launch failure.  Work is enqueued on
 * `stream` (hipStream_t, NULL = default stream); time it with events.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a multiple of 16, >= 16) of device memory `buf` once with
 * 16-byte loads from ceil(bytes / 64 KiB) work-groups (at most 8192; each
 * reads one contiguous share) and stores one 32-bit fold per work-group into
 * `sink` (device, at least 8192 * 4 bytes). */
int moe_probe_read(const void* buf, size_t bytes, void* sink, void* stream);

/* One work-group of four waves per compute unit, each wave issuing `iters`
 * rounds of 8 independent 32x32x16 bf16 MFMAs on register operands.  Writes
 * the flops of the launch to *flops (host) and one float per thread to
 * `sink` (device, at least 256 * 4 * number of compute units bytes). */
int moe_probe_mfma_bf16(int32_t iters, void* sink, double* flops /* host */, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
