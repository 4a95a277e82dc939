/*
 * bf16delta_probe.h -- measurement aids of the libbf16delta benchmark, built
 * as their own library (libbf16delta_probe.so) beside the product library.
 * They are not steps of the method: they time the memory access patterns of
 * the main kernels with nothing else, so that those kernels can be compared
 * against what the pattern itself costs on the device, beside the published
 * HBM peak.  Conventions (status codes, streams, device pointers) are those
 * of bf16delta.h.
 */
#ifndef BF16DELTA_PROBE_H
#define BF16DELTA_PROBE_H

#include "bf16delta.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads the first 8192 * floor(n / 8192) elements of a, and of b unless b is
 * NULL, with the encoder's whole-block access pattern (one workgroup per
 * 8192-element block, 16-byte loads, the blocks split into one contiguous
 * range per XCD as the main kernels take them; with b, non-temporal loads as
 * the encoder's, and without it plain loads as the apply pass's) and does
 * nothing else, so that
 * its time is the read ceiling of that pattern: the "achievable" figure that
 * kernel times are compared against, beside the published HBM peak.  a and b
 * are device pointers to at least n elements each, 16-byte aligned; sink is 8
 * bytes of device memory, written only when a fold of the data equals key
 * (the store keeps the loads from being removed).  Enqueued on stream.
 * Returns BF16D_EINVAL for a NULL a or sink, a misaligned pointer or more
 * than 2^31 - 1 blocks; BF16D_EHIP if the launch fails; else BF16D_OK. */
int bf16d_probe_read(const uint16_t *a, const uint16_t *b, uint64_t n, uint64_t *sink,
                     uint64_t key, hipStream_t stream);

/* Measurement aid (not a step of the method): the traffic of an in-place
 * apply with nothing else.  Reads the first 8192 * floor(n / 8192) elements
 * of w with the apply pass's whole-block pattern (in the same block order as
 * bf16d_probe_read) and writes back, unchanged, every 16-byte chunk c
 * (elements 8c .. 8c + 7) whose bit (c & 31) of dirty[c >> 5] is set, so
 * that, given the chunks a delta changes, its time is the cost of applying
 * that delta's traffic in place through the simplest kernel (a reference
 * point, not a strict lower bound).  w: device, 16-byte aligned, n elements,
 * left as it was; dirty: device, 4-byte aligned, at least 32 * floor(n /
 * 8192) words; sink as in bf16d_probe_read.  No other work may write w
 * meanwhile.  Returns BF16D_EINVAL for a NULL or misaligned pointer or more
 * than 2^31 - 1 blocks; BF16D_EHIP if the launch fails; else BF16D_OK. */
int bf16d_probe_inplace(uint16_t *w, uint64_t n, const uint32_t *dirty, uint64_t *sink,
                        uint64_t key, hipStream_t stream);

/* Measurement aid: the in-place apply's writes with nothing else.  Writes
 * (a pattern, not data) every 16-byte chunk c of the first 8192 *
 * floor(n / 8192) elements of w whose bit (c & 31) of dirty[c >> 5] is set,
 * in the blocks' XCD-aware order, and reads nothing from w: beside
 * bf16d_probe_read of the same elements, its time shows how much of the
 * in-place traffic is the scattered writes of the changed chunks.  w:
 * device, 16-byte aligned, n elements, overwritten at the marked chunks (a
 * scratch array); dirty as in bf16d_probe_inplace.  Returns BF16D_EINVAL for
 * a NULL or misaligned pointer or more than 2^31 - 1 blocks; BF16D_EHIP if
 * the launch fails; else BF16D_OK. */
int bf16d_probe_write(uint16_t *w, uint64_t n, const uint32_t *dirty, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* BF16DELTA_PROBE_H */
