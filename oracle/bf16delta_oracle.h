/*
 * bf16delta_oracle.h -- TEST INFRASTRUCTURE ONLY.
 *
 * The plain, slow, single-threaded CPU oracle of the bf16delta_v1 lossless
 * BF16 weight-delta format.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the GPU library never does, and
 * the two implementations share no code, header, table or helper.
 *
 * What the method computes (sources, cited by page title and section):
 *  - "GPU-accelerated Weight Teleportation", section "Delta update algebra":
 *    the delta of two checkpoints is their bitwise XOR, and the receiver gets
 *    the new weights back by XOR-ing that mask onto the old ones; no floating
 *    point is involved, so the work is done on raw 16-bit patterns.
 *  - "Every byte counts: ARCv3 and the case for cross-region RL", section
 *    "Deep dive into ARCv3" and the figure "How ARCv3 encodes a block of
 *    weights": every changed element is classified by which bfloat16 fields
 *    changed; unchanged elements cost nothing, mantissa-only changes carry
 *    only their mantissa bits, and the rare exponent/sign changes are packed
 *    in a stream of their own with all their changed fields together; the
 *    receiver applies both streams to the previous checkpoint and checks the
 *    result against a checksum of the trainer's weights.
 *  - same page, section "Using ARCv3": delta_compress(src, dst) returns the
 *    compressed diff and a checksum; delta_decompress(src, diff, checksum)
 *    returns weights bit-for-bit equal to dst.
 *
 * The pages fix no wire format, block size, position index or checksum
 * algorithm; the readings taken here (block of 8192 elements, per-block
 * descriptor, bitmap-or-gap position segment, 7-bit mantissa XOR fields with
 * 0 as the escape into the 16-bit rare stream, SplitMix64-based sum checksum)
 * are this project's own format, "bf16delta_v1".
 *
 * Status codes are plain integers; they mirror the library's contract but
 * are defined here independently.
 */
#ifndef BF16DELTA_ORACLE_H
#define BF16DELTA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define REF_OK        0
#define REF_EINVAL    1
#define REF_ECAPACITY 2
#define REF_EFORMAT   3
#define REF_ECHECKSUM 4
#define REF_EVERSION  7

typedef struct ref_result {
    uint64_t payload_bytes;   /* bytes written, or bytes required on REF_ECAPACITY */
    uint64_t checksum;        /* checksum of dst */
    uint64_t n_changed;       /* elements whose XOR is non-zero */
    uint64_t n_rare;          /* elements whose XOR touches the exponent or sign */
    uint64_t n_bitmap_blocks; /* blocks whose position segment is a bitmap */
} ref_result;

/* SplitMix64 finaliser (exposed so the tests can pin it to published values). */
uint64_t bf16d_ref_mix64(uint64_t z);

/* Checksum of n bf16 patterns (host memory). */
uint64_t bf16d_ref_checksum(const uint16_t *w, uint64_t n);

/* Upper bound on the payload of an n-element tensor. */
uint64_t bf16d_ref_max_payload_bytes(uint64_t n);

/* Encode the delta src -> dst into payload[0 .. capacity). */
int bf16d_ref_compress(const uint16_t *src, const uint16_t *dst, uint64_t n,
                       uint8_t *payload, uint64_t capacity, ref_result *res);

/* Apply payload onto weights (old -> new) in place; weights end new on
 * REF_OK and bit-exactly old on every other status.  Reads version-1 and
 * version-2 payloads; the binding of a version-2 payload is not checked. */
int bf16d_ref_decompress(uint16_t *weights, uint64_t n, const uint8_t *payload,
                         uint64_t payload_bytes, uint64_t checksum);

/* Version 2 ("GPU-accelerated Weight Teleportation", section "Eval, fault
 * tolerance, and resuming from trained checkpoints", and the NeMo
 * Delta-Compressed Refit summary: absolute overwrites beside XOR masks,
 * retry-safe versioning with a joint commit).  The 64 bytes of the version-1
 * header (with version = 2) are followed by u64 base_version, u64
 * target_version, u32 flags, u32 0, u64 0; the descriptor table starts at
 * byte 96.  flags bit 0 (overwrite): every changed element carries its new
 * value as a 16-bit word right after the position segment (no mantissa
 * segment; the descriptor's r equals c), and applying it sets the element to
 * that value.  Records are otherwise those of version 1. */
#define REF_FLAG_OVERWRITE 1u
int bf16d_ref_compress_v2(const uint16_t *src, const uint16_t *dst, uint64_t n,
                          uint64_t base_version, uint64_t target_version, uint32_t flags,
                          uint8_t *payload, uint64_t capacity, ref_result *res);

/* Apply a version-1 or version-2 payload.  version (may be NULL) is the
 * receiver's version word: a version-2 payload whose base differs returns
 * REF_EVERSION with nothing touched; on REF_OK it becomes the target.  An
 * overwrite payload is built and checked in a copy and written only when the
 * checksum matches, so the weights end new on REF_OK and untouched
 * otherwise, whatever mix of old and new values they held at the changed
 * positions. */
int bf16d_ref_decompress_v2(uint16_t *weights, uint64_t n, const uint8_t *payload,
                            uint64_t payload_bytes, uint64_t checksum, uint64_t *version);

#ifdef __cplusplus
}
#endif
#endif
