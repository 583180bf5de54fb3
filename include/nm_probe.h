/*
 * nm_probe.h -- measurement helpers of libnmprobe.so (not part of the method, and not
 * exported by libnmsparse): the achievable ceilings of the machine at hand, reported
 * beside the nominal peaks.  Same conventions as nm.h (device pointers, enqueue-only).
 *   nm_probe_sink_bytes   bytes of the device sink both probes write.
 *   nm_probe_read         one streaming read of `bytes` (a multiple of 16; of 16384 for
 *                         mode 2) at buf; buf and sink 16-byte aligned.  mode 0: 16-byte
 *                         loads at a grid stride, 4 in flight per lane; 1: one contiguous
 *                         block per workgroup, 16 loads in flight per lane; 2: direct-to-LDS
 *                         16-byte loads, contiguous 16 KiB chunks per wave.
 *   nm_probe_mfma         `iters` rounds of 16 independent bf16 16x16x32 matrix instructions
 *                         per wave on register operands; nm_probe_mfma_flops(iters) gives the
 *                         FLOPs one launch performs.
 * Both only enqueue work on `stream`; time them with events on that stream.
 */
#ifndef NM_PROBE_H
#define NM_PROBE_H

#include "nm.h"

#ifdef __cplusplus
extern "C" {
#endif

int64_t nm_probe_sink_bytes(void);
nm_status nm_probe_read(const void* buf, int64_t bytes, void* sink, int mode, void* stream);
int64_t nm_probe_mfma_flops(int64_t iters);
nm_status nm_probe_mfma(int64_t iters, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NM_PROBE_H */
