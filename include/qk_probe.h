/*
 * qk_probe.h — measurement helper exported by libqk.so next to the C ABI of
 * qk.h: the HBM read rate a plain streaming kernel reaches, so that GEMV
 * throughput can be compared with an achievable ceiling in the same run
 * (the roofline's peak stays the published 8 TB/s), and a plain copy of
 * known size whose hardware counters calibrate the HBM byte counters taken
 * on the GEMV kernels. Neither is part of the GEMV path.
 */
#ifndef QK_PROBE_H
#define QK_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads every byte of buf[0..bytes) once (bytes a multiple of 16, buf
 * 16-byte aligned device memory) and writes one XOR digest per workgroup
 * into out[0..min(out_len, 8*CUs)). Enqueued on `stream`; returns 0, -1 for a
 * bad argument (nothing launched) or -5 for a launch error. */
int qk_probe_read(const void *buf, int64_t bytes, uint32_t *out, int64_t out_len, void *stream);

/* Copies bytes from src to dst (device memory, both 16-byte aligned, bytes a
 * multiple of 16, not overlapping) with a plain grid-stride kernel: every
 * byte is read once and written once. Enqueued on `stream`; returns 0, -1
 * for a bad argument (nothing launched) or -5 for a launch error. */
int qk_probe_copy(const void *src, void *dst, int64_t bytes, void *stream);


#ifdef __cplusplus
}
#endif

#endif /* QK_PROBE_H */
