/*
 * csa2_probe.h -- measurement and testing support of the CSA2 library (not
 * part of the method): a read-only streaming kernel that gives the practical
 * HBM read ceiling on the device, against which the decode kernels (almost
 * all reads) are compared beside the datasheet peak; and the choice between
 * the library's two attention kernels, so that tests cover both and timings
 * compare them.
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

/* Attention kernel of csa2_sparse_attend, csa2_sparse_attend_noalloc and
 * csa2_layer_step, for the calls that follow (process-wide; both kernels give
 * the same results to rounding and use the same workspace):
 *   CSA2_ATTEND_AUTO (0)  by the work per workgroup: the paired-wave kernel
 *                         when the busiest workgroup takes at least 3 units of
 *                         128 positions, the eight-wave kernel otherwise;
 *   CSA2_ATTEND_SEG  (1)  the eight-wave kernel (each unit's rows shared by
 *                         eight waves through LDS);
 *   CSA2_ATTEND_PAIR (2)  the paired-wave kernel (each pair of waves its own
 *                         32 positions of a unit).
 * The initial choice is AUTO, or what the environment variable
 * CSA2_ATTEND_KERNEL (auto, seg, pair) names. Returns CSA2_EINVAL for any
 * other value. Not synchronised with calls in flight on other threads. */
#define CSA2_ATTEND_AUTO 0
#define CSA2_ATTEND_SEG 1
#define CSA2_ATTEND_PAIR 2
csa2_status csa2_set_attend_kernel(int32_t kernel);

#ifdef __cplusplus
}
#endif
#endif
