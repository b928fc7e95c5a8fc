/*
 * csa2_probe.h -- measurement support of the CSA2 library (not part of the
 * method): a read-only streaming kernel that gives the practical HBM read
 * ceiling on the device, against which the decode kernels (almost all reads)
 * are compared beside the datasheet peak.
 */
#ifndef CSA2_PROBE_H
#define CSA2_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "csa2.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read n_bytes (a multiple of 16, 16-byte aligned device memory) once with
 * 16-byte loads from `blocks` workgroups of 256 threads; nothing is written
 * except, in practice never, one word of sink (device, 1024 uint32). */
csa2_status csa2_stream_read(const void *p, size_t n_bytes, uint32_t *sink, int32_t blocks, void *stream);

#ifdef __cplusplus
}
#endif
#endif
