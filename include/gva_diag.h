/*
 * gva_diag.h - measurement aid of the GVA library (not part of the method's interface).
 *
 * The decode is bound by HBM reads, so its roofline needs the rate at which this part streams
 * reads in practice, beside the 8 TB/s figure on the data sheet. gva_diag_stream_read is the
 * plainest kernel that moves bytes from HBM to the compute units: every lane issues 16-byte
 * non-temporal loads (each load instruction reading 1 KiB of consecutive bytes), several in
 * flight, over a contiguous buffer, and folds them into one word per work-group so that the
 * loads cannot be dropped.
 */
#ifndef GVA_DIAG_H_
#define GVA_DIAG_H_

#include <stddef.h>
#include <stdint.h>

#include "gva.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes at `src` (device, 16-byte aligned, bytes a multiple of 16) once, with
 * `work_groups` work-groups of 256 lanes (1 .. 65536) in a grid-stride loop, each lane keeping
 * `in_flight` 16-byte loads outstanding (1, 2, 4 or 8). Writes the XOR of everything a
 * work-group read to sink[work-group id] (device uint32 [work_groups]). Asynchronous on stream;
 * argument errors return GVA_ERR_INVALID_ARG before any launch. */
gva_status gva_diag_stream_read(const void *src, size_t bytes, int32_t work_groups,
                                int32_t in_flight, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GVA_DIAG_H_ */
