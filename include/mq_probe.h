/*
 * mq_probe.h — calibration probes, C ABI of libmq_probe.so (a library of its
 * own, loaded by the benchmark only; not part of libmq.so).
 *
 * Not part of the method: they measure what this GPU delivers, so that the
 * kernels' roofline fractions can be read against measured references as
 * well as against the published peaks.  Each call enqueues one kernel on
 * `stream`; the caller times it (events around the call).  Workgroups have
 * 256 threads.  Status codes are mq.h's.
 *
 * mq_probe_stream — reads the `bytes` bytes at src once, 16 bytes per lane
 *   per load (each wave load is 1 KB of one contiguous range, eight loads in
 *   flight per lane), and writes the XOR of each lane's words to
 *   sink[workgroups * 256] (uint32) so that no read can be skipped.
 *   src 16-byte aligned, bytes a positive multiple of 16, workgroups >= 1.
 * mq_probe_mfma — each wave runs `iters` rounds of eight independent
 *   v_mfma_f32_16x16x32_bf16 on register operands (16384 flop each; no
 *   memory traffic; random bf16 operands that change every MFMA) and writes
 *   one float per thread to sink[workgroups * 256].  Work = workgroups * 4 *
 *   iters * 8 * 16384 flop.  iters >= 1.
 * Errors: MQ_ERR_INVALID for a NULL pointer or an argument outside the
 *   ranges above (checked before any HIP call); MQ_ERR_HIP if the launch
 *   fails.
 */
#ifndef MQ_PROBE_H
#define MQ_PROBE_H

#include "mq.h"

#ifdef __cplusplus
extern "C" {
#endif

mq_status mq_probe_stream(const void* src, int64_t bytes, uint32_t* sink, int32_t workgroups,
                          void* stream);
mq_status mq_probe_mfma(int32_t iters, float* sink, int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MQ_PROBE_H */
