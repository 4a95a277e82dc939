/*
 * bf16delta.h -- C ABI of libbf16delta: lossless delta compression of BF16
 * checkpoints on AMD Instinct MI355X (gfx950).
 *
 * The operation.  Sources are cited by page title and section:
 *  - "GPU-accelerated Weight Teleportation", section "Delta update algebra":
 *    the delta between two checkpoints is the bitwise XOR of their bit
 *    patterns, and the receiver rebuilds the new weights by XOR-ing that mask
 *    onto the old ones.  The work is bitwise, with no floating point.
 *  - "Every byte counts: ARCv3 and the case for cross-region RL", section
 *    "Deep dive into ARCv3" and the figure "How ARCv3 encodes a block of
 *    weights":
 *    - each changed element is classified as mantissa-only or as an
 *      exponent/sign change;
 *    - unchanged elements cost nothing;
 *    - mantissa-only changes carry only their mantissa bits;
 *    - the rare exponent/sign changes are packed in a stream of their own;
 *    - the receiver applies both streams to the previous checkpoint and
 *      checks the result against a checksum of the trainer's weights.
 *  - same page, section "Using ARCv3": compress(src, dst) returns the
 *    compressed diff and a checksum; decompress(src, diff, checksum)
 *    returns weights equal to dst bit for bit.
 *  - "A strong baseline with Blackwell-native DE" (Weight Teleportation):
 *    the XOR is applied in place in HBM by one launch that reads a plan
 *    prepared on the CPU.  Here the plan is the job table passed to
 *    bf16d_compress / bf16d_decompress.
 *
 * Wire format "bf16delta_v1".  The pages fix no format; this one is the
 * project's own and is not ARCv3's.
 *   - Elements are 16-bit patterns, in blocks of BF16D_BLOCK_ELEMS = 8192
 *     (the last block may be shorter).
 *   - Header, 64 bytes, little-endian:
 *       magic "BF16DXOR", u32 version = 1, u32 block_elems = 8192, u64 n,
 *       u64 n_changed, u64 n_rare, u64 pos_bytes, u64 mant_bytes,
 *       u64 rare_bytes.
 *   - Then one u32 descriptor per block:
 *       c | r << 14 | code << 28
 *     c counts changed elements, r counts exponent/sign ("rare") changes.
 *     code 0..13 means a gap list of width `code`; 15 means a bitmap;
 *     14 is invalid.
 *   - Then one record per block, in block order, with no padding between
 *     records:
 *       position segment : either c gap fields of `code` bits or one bit per
 *                          element, whichever is smaller (a tie goes to the
 *                          gap list)
 *       mantissa segment : c fields of 7 bits, each the mantissa XOR, or 0
 *                          for an exponent/sign change
 *       rare segment     : r u16 words, the full XOR of every exponent/sign
 *                          change
 *     Bit fields are packed LSB-first and each segment is zero-padded to a
 *     byte.
 *   - Checksum of the new weights:
 *       checksum = mix64(S ^ n)
 *       S        = sum over k of mix64(W_k ^ (k+1) * 0x9E3779B97F4A7C15)
 *                  mod 2^64
 *     W_k is the little-endian u64 of elements 4k..4k+3; missing elements
 *     are 0.  mix64 is the SplitMix64 finaliser.
 *
 * Conventions shared by every entry point:
 *   - The caller owns every buffer.  The library allocates no device memory
 *     and keeps no state between calls; the one exception is the static
 *     scratch of bf16d_decompress_noalloc, a fixed array in the library's
 *     device code.
 *   - src, dst, weights, payload and workspace are device pointers and must
 *     be 16-byte aligned.
 *   - `results` must be memory the device can write: device memory, or
 *     pinned host memory.  It may not overlap any buffer the call writes.
 *   - `stream` is a HIP stream; NULL means the null stream.  All device work
 *     is enqueued on it, and results[] is valid once the stream has
 *     completed.
 *   - Element counts and byte sizes (n, capacity, payload_bytes) are at
 *     most 2^62; larger values are refused with BF16D_EINVAL.
 *   - The return value reports only errors the host can detect before
 *     enqueueing anything:
 *       BF16D_EINVAL  bad pointer, alignment, size, overlap, or a workspace
 *                     that is too small;
 *       BF16D_EHIP    a HIP runtime call failed.
 *     Errors found on the device land in results[i].status.
 *   - Calls that share a workspace, payload or weight buffer must not
 *     overlap in time (for example, on two streams).
 */
#ifndef BF16DELTA_H
#define BF16DELTA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BF16D_OK        0  /* success */
#define BF16D_EINVAL    1  /* invalid arguments (host-detected; nothing enqueued) */
#define BF16D_ECAPACITY 2  /* compress: payload larger than capacity; required size reported */
#define BF16D_EFORMAT   3  /* decompress: malformed or mismatched payload; weights end old */
#define BF16D_ECHECKSUM 4  /* decompress: rebuilt weights fail the checksum; weights end old */
#define BF16D_EHIP      5  /* a HIP runtime call failed */
#define BF16D_ECODEC    6  /* codec race: the frame's codec library is not available here */
#define BF16D_EVERSION  7  /* decompress: the receiver's version is not the payload's base;
                              nothing touched */

#define BF16D_BLOCK_ELEMS    8192
#define BF16D_HEADER_BYTES   64
#define BF16D_FORMAT_VERSION 1
#define BF16D_FORMAT_VERSION_BOUND 2   /* version-2 payloads: bound to versions */
#define BF16D_HEADER_BYTES_BOUND   96
#define BF16D_BIND_OVERWRITE       1u  /* version 2: records carry absolute values */

/* Per-job outcome, written by the device. 48 bytes. */
typedef struct bf16d_result {
    int32_t  status;          /* BF16D_OK, BF16D_ECAPACITY, BF16D_EFORMAT or BF16D_ECHECKSUM */
    uint32_t reserved;
    uint64_t payload_bytes;   /* compress: bytes written, or bytes required on ECAPACITY;
                                 decompress: the payload length given */
    uint64_t checksum;        /* compress: checksum of dst; decompress: checksum of the
                                 weights after the apply pass (before any rollback), or 0
                                 if the payload was rejected before applying */
    uint64_t n_changed;       /* elements whose XOR is non-zero */
    uint64_t n_rare;          /* elements whose XOR touches the exponent or the sign */
    uint64_t n_bitmap_blocks; /* blocks whose position segment is a bitmap */
} bf16d_result;

/* One tensor to compress.
 *   src, dst : device, 16-byte aligned, n elements each.  They are read only
 *              and may be the same buffer; they may be NULL when n == 0.
 *   payload  : device, 16-byte aligned, capacity bytes.  It must not overlap
 *              src or dst.
 *   capacity : room in payload.  bf16d_max_payload_bytes(n) always suffices.
 *              If it is too small, the status is BF16D_ECAPACITY, the
 *              required size is reported, nothing is written at or beyond
 *              capacity, and the bytes below it are unspecified. */
typedef struct bf16d_compress_job {
    const uint16_t *src;
    const uint16_t *dst;
    uint64_t        n;
    uint8_t        *payload;
    uint64_t        capacity;
} bf16d_compress_job;

/* One tensor to rebuild in place.
 *   weights       : device, 16-byte aligned, n elements.  It holds the old
 *                   weights on entry, and the new ones on BF16D_OK.  On any
 *                   other status it holds the old ones bit for bit (XOR is
 *                   its own inverse, so the pass is undone).
 *   payload       : device, 16-byte aligned, payload_bytes bytes.  It must
 *                   not overlap weights.  It may be NULL only when
 *                   payload_bytes is 0; such a payload is too short, and the
 *                   status is BF16D_EFORMAT.
 *   checksum      : the value returned by compress for this tensor. */
typedef struct bf16d_decompress_job {
    uint16_t      *weights;
    uint64_t       n;
    const uint8_t *payload;
    uint64_t       payload_bytes;
    uint64_t       checksum;
} bf16d_decompress_job;

/* Upper bound on the bytes of an n-element payload.  Per block it is:
 * a bitmap-sized position segment, with every element changed and rare. */
uint64_t bf16d_max_payload_bytes(uint64_t n);

/* Workspace bytes that suffice for any batch of `count` jobs totalling
 * total_n elements, in either direction.  For compress this includes a 2 KiB
 * record slot per 8192-element block (12.5 % of the weights). */
size_t bf16d_workspace_bytes(uint64_t total_n, uint32_t count);

/* Compress workspace with record slots of slot_bytes per block (a multiple
 * of 16 from 16 to 2048; 0 is returned for any other value).  Compress uses
 * the largest slot (up to 2048 bytes, in steps of 16) that the workspace it
 * is given holds, so a caller short of memory passes less: with 256-byte
 * slots the workspace is about 1.9 % of the weights.  A block's record
 * (its position, mantissa and rare segments) that does not fit its slot is
 * staged at the tail of the job's payload buffer instead, in the room between
 * the final payload and `capacity`; one that finds no room there is encoded
 * a second time from the weights, which reads that block again.  The payload
 * bytes are the same either way; only the time differs.  With small slots,
 * bytes of the payload buffer from payload_bytes up to capacity are
 * unspecified after the call. */
size_t bf16d_compress_workspace_bytes(uint64_t total_n, uint32_t count, uint32_t slot_bytes);

/* Compress `count` tensors in one batched pass: old = src, new = dst.
 * The job array is host memory.  It is copied into the workspace before
 * the call returns, so it may be freed right after.  results[i] receives
 * job i's outcome.  All jobs share one launch per kernel; each job gets its
 * own payload and checksum. */
int bf16d_compress(const bf16d_compress_job *jobs, uint32_t count,
                   void *workspace, size_t workspace_bytes,
                   bf16d_result *results, hipStream_t stream);

/* Apply `count` payloads in place in one batched pass.  Per job, one of:
 *   - a bad header or descriptor table: BF16D_EFORMAT, weights untouched;
 *   - a malformed block record: BF16D_EFORMAT, pass undone, weights old;
 *   - a checksum mismatch: BF16D_ECHECKSUM, pass undone, weights old;
 *   - BF16D_OK, weights new. */
int bf16d_decompress(const bf16d_decompress_job *jobs, uint32_t count,
                     void *workspace, size_t workspace_bytes,
                     bf16d_result *results, hipStream_t stream);

/* Events recorded on the call's stream immediately before and after the main
 * kernel of a call (compress: the encode kernel, which reads both
 * checkpoints; decompress: the apply kernel, which rewrites the weights).
 * They let a caller time that kernel alone.  The caller owns the events,
 * which must be created with timing enabled; either may be NULL. */
typedef struct bf16d_events {
    hipEvent_t before;
    hipEvent_t after;
} bf16d_events;

/* bf16d_compress / bf16d_decompress plus kernel events (`events` may be
 * NULL, which is exactly the plain call). */
int bf16d_compress_ex(const bf16d_compress_job *jobs, uint32_t count,
                      void *workspace, size_t workspace_bytes,
                      bf16d_result *results, hipStream_t stream,
                      const bf16d_events *events);
int bf16d_decompress_ex(const bf16d_decompress_job *jobs, uint32_t count,
                        void *workspace, size_t workspace_bytes,
                        bf16d_result *results, hipStream_t stream,
                        const bf16d_events *events);

/* Allocation-free decompress, for callers that cannot allocate device
 * memory (tight serving loops, harnesses that forbid allocation): the same
 * call as bf16d_decompress, with the same kernels, statuses, rollback and
 * argument checks, but its workspace is the library's own scratch instead of
 * a caller buffer.  The caller still passes the jobs (weights and payloads)
 * and `results`.
 *
 * The scratch is a static device array of BF16D_NOALLOC_SCRATCH_BYTES
 * (64 MiB) per GPU.  Every GPU the library runs on holds its own copy until
 * the process ends; its address is taken on the first call made on each
 * device.  A batch fits when its decompress workspace layout does, which
 * needs at most
 *   81 bytes per 8192-element block + 224 bytes per job + 8 KiB.
 * All 291 tensors of a 7B-shaped checkpoint (822,593 blocks) fit in one
 * call; larger batches must be split (by layer, for example).  A batch that
 * does not fit returns BF16D_EINVAL with nothing enqueued.
 *
 * `stream` must belong to the current device (NULL: the current device's
 * null stream); otherwise BF16D_EINVAL.  The job table is copied from host
 * memory before the call returns, as in bf16d_decompress.  Calls share
 * their GPU's scratch, so two calls that overlap in time on one GPU (for
 * example on two streams) race and give undefined results; calls in one
 * stream's order are safe.  Each call clears what it needs cleared (with a
 * kernel, not a memset), so the contents left by the previous call do not
 * matter.  This call allocates no device memory.  It is not meant for HIP
 * graph capture: its job table goes up with an asynchronous copy from a host
 * buffer that the call frees before it returns. */
#define BF16D_NOALLOC_SCRATCH_BYTES (64u << 20)
int bf16d_decompress_noalloc(const bf16d_decompress_job *jobs, uint32_t count,
                             bf16d_result *results, hipStream_t stream);

/* Verify-first decompress: the apply of bf16d_decompress split in two
 * passes, so that the weights are never touched by a payload that fails.
 * The first pass decodes every record and checks it, and sums the checksum
 * of the would-be result (old weights XOR the mask) without storing
 * anything; only jobs that pass (BF16D_OK) are then written, by a second
 * pass that decodes the record again and reads, XORs and stores only the
 * 16-byte chunks that change.  On BF16D_EFORMAT and BF16D_ECHECKSUM the
 * weights are untouched (bf16d_decompress rolls them back instead, which
 * ends with the same bits but writes them twice meanwhile).  It moves more
 * bytes than the single in-place pass: the changed chunks are read twice
 * and the payload decoded twice.  Arguments, statuses and results are those
 * of bf16d_decompress_ex (events bracket the first pass's kernel).  NeMo-DCR
 * summary: an update left placed wrongly or half-applied is unusable. */
int bf16d_decompress_verified(const bf16d_decompress_job *jobs, uint32_t count,
                              void *workspace, size_t workspace_bytes, bf16d_result *results,
                              hipStream_t stream, const bf16d_events *events);

/* Single-tensor forms of the two calls above, named after the pages'
 * delta_compress(src, dst) -> (payload, checksum) and
 * delta_decompress(src, payload, checksum) -> dst ("Every byte counts:
 * ARCv3 and the case for cross-region RL", section "Using ARCv3").
 * delta_decompress rebuilds dst in src_inout, in place. */
int bf16d_delta_compress(const uint16_t *src, const uint16_t *dst, uint64_t n,
                         uint8_t *payload, uint64_t capacity,
                         void *workspace, size_t workspace_bytes,
                         bf16d_result *result, hipStream_t stream);

int bf16d_delta_decompress(uint16_t *src_inout, uint64_t n,
                           const uint8_t *payload, uint64_t payload_bytes,
                           uint64_t checksum,
                           void *workspace, size_t workspace_bytes,
                           bf16d_result *result, hipStream_t stream);

/* Version-2 payloads: bound to versions, optionally with absolute values.
 *
 * "GPU-accelerated Weight Teleportation", section "Eval, fault tolerance,
 * and resuming from trained checkpoints": deltas are also kept against
 * versions other than the previous one (the last evaluated version, the
 * engines' base version), so a receiver must be able to tell which version a
 * payload applies to.  The NeMo Delta-Compressed Refit summary: changes that
 * cannot be carried as XOR masks travel as absolute overwrites, partial
 * writes are retried through overwrites, and a joint commit binds the
 * installed weights to the version the next delta is made from.
 *
 * Format version 2: the 64 header bytes of version 1 with version = 2, then
 *   u64 base_version, u64 target_version, u32 flags, u32 0, u64 0
 * (96 bytes); the descriptor table starts at byte 96.  Records are those of
 * version 1, except with flags & BF16D_BIND_OVERWRITE: then every changed
 * element (old != new) carries its new value as a little-endian u16 right
 * after the position segment, there is no mantissa segment, the
 * descriptor's r equals c, and the header counts mant_bytes = 0 and
 * rare_bytes = 2 * n_changed.  Applying an overwrite record sets each listed
 * element to its value, so the result is the new tensor whatever mix of old
 * and new values the listed elements held: a retry after a partial write.
 * A version-2 payload is at most bf16d_max_payload_bytes(n) + 32 bytes. */
typedef struct bf16d_binding {
    uint64_t base_version;    /* the version the receiver's weights must hold */
    uint64_t target_version;  /* the version they hold after the apply */
    uint32_t flags;           /* 0 or BF16D_BIND_OVERWRITE */
    uint32_t reserved;        /* 0 */
} bf16d_binding;

/* bf16d_compress writing version-2 payloads: bindings[i] (host array) for
 * job i.  Results are those of bf16d_compress; for an overwrite payload
 * n_rare counts its words (= n_changed).  Returns BF16D_EINVAL for a NULL
 * bindings array, unknown flags or a non-zero reserved field. */
int bf16d_compress_bound(const bf16d_compress_job *jobs, const bf16d_binding *bindings,
                         uint32_t count, void *workspace, size_t workspace_bytes,
                         bf16d_result *results, hipStream_t stream);

/* bf16d_decompress with the receiver's version words.
 *   versions : device memory, 8-byte aligned, count u64: versions[i] is the
 *              version tensor i holds.  May be NULL: then no binding is
 *              checked.  It may not overlap the weights, payloads or
 *              workspace.
 * Per job, on top of bf16d_decompress:
 *   - a version-2 payload whose base_version differs from versions[i]:
 *     BF16D_EVERSION, weights and versions[i] untouched (a malformed header
 *     or descriptor table still reports BF16D_EFORMAT first);
 *   - BF16D_OK for a version-2 payload: versions[i] = target_version,
 *     written together with the weights; on any other status it is kept;
 *   - a version-1 payload leaves versions[i] alone.
 * An overwrite payload ends with the weights new on BF16D_OK and exactly as
 * they were before the call (partly written or not) on any other status.
 * When the workspace has room beyond the call's own layout for an undo area
 * of one byte per payload byte (bf16d_workspace_bytes leaves it for any
 * sparse delta), it is applied in place in one pass and each replaced value
 * is kept in the undo area; a job that fails is then restored from it.
 * Without that room it is verified first (its checksum is that of the
 * would-be result) and written after, which reads and decodes the payload
 * twice.  This holds in bf16d_decompress too.  bf16d_decompress and the
 * streamed and remapped calls read version-2 payloads too, without checking
 * the binding (the streamed call and the prepared remapped call always
 * verify overwrite payloads first). */
int bf16d_decompress_bound(const bf16d_decompress_job *jobs, uint64_t *versions, uint32_t count,
                           void *workspace, size_t workspace_bytes, bf16d_result *results,
                           hipStream_t stream);

/* Remapped apply: the new weights land on a physical layout that differs
 * from the logical tensor the payload was made from.
 *
 * "GPU-accelerated Weight Teleportation", sections "A strong baseline with
 * Blackwell-native DE" and "Working with low-precision RL": fused kernels
 * may keep weights in a reordered physical layout (for example gate and up
 * projections paired in groups of 64 rows); the XOR mask is remapped the
 * same way through address metadata prepared on the CPU, and one launch
 * applies it to the whole model.  Here that metadata is a list of segments
 * per tensor.
 *
 * Logical elements [first, first + count) of a tensor live at dst[0, count).
 *   first  : a multiple of BF16D_BLOCK_ELEMS (8192): segments are
 *            block-granular, so each block of the payload lands in one
 *            place.  Gate/up pairing in groups of 64 rows qualifies whenever
 *            a row holds at least 128 elements.
 *   count  : elements; every segment but the tensor's last must hold a
 *            multiple of 8192.
 *   dst    : device, 16-byte aligned.
 * The segments of a tensor must follow one another (segment k + 1 starts
 * where segment k ends), start at 0 and cover exactly n elements.  The
 * checksum is that of the logical tensor, as compress computed it. */
typedef struct bf16d_segment {
    uint64_t  first;
    uint64_t  count;
    uint16_t *dst;
} bf16d_segment;

/* The segments of one tensor (host memory).  count == 0 means no remap: the
 * job's weights pointer is used as in bf16d_decompress.  With count > 0 the
 * job's weights pointer must be NULL. */
typedef struct bf16d_remap {
    const bf16d_segment *segments;
    uint32_t             count;
} bf16d_remap;

/* Workspace bytes that suffice for a remapped decompress of `count` jobs
 * totalling total_n elements and total_segments segments. */
size_t bf16d_workspace_bytes_remapped(uint64_t total_n, uint32_t count,
                                      uint64_t total_segments);

/* bf16d_decompress with remaps[j] for job j (remaps may be NULL: no remap).
 * Statuses, rollback and argument errors are those of bf16d_decompress; the
 * segments' physical ranges are the weights that are written, and they may
 * not overlap one another, a payload or the workspace. */
int bf16d_decompress_remapped(const bf16d_decompress_job *jobs, const bf16d_remap *remaps,
                              uint32_t count, void *workspace, size_t workspace_bytes,
                              bf16d_result *results, hipStream_t stream);

/* Remapped apply with the layout prepared once.
 *
 * A receiver that applies a delta at every step onto the same remapped layout
 * can check and upload that layout once ("GPU-accelerated Weight
 * Teleportation", section "Working with low-precision RL": the address
 * metadata is prepared on the CPU for the layout, which does not change
 * between steps).  bf16d_remap_prepare checks the segments as
 * bf16d_decompress_remapped does (block-aligned, in order, covering each
 * tensor, no two physical ranges overlapping) and writes:
 *   plan      : host memory, bf16d_remap_plan_bytes(count, total_segments)
 *               bytes, owned by the caller: the jobs' (weights, n) and the
 *               sorted physical ranges;
 *   block_map : device memory, 8-byte aligned, bf16d_remap_map_bytes(sum
 *               of n, count) bytes, owned by the caller: the address of
 *               every 8192-element block's first weight, uploaded on
 *               `stream` (the host copy is staged before the call returns).
 * Only the jobs' weights and n are read (payload fields are ignored).
 * Returns BF16D_EINVAL for an invalid layout or short buffers, BF16D_EHIP
 * if the upload fails.
 *
 * bf16d_decompress_remapped_prepared then applies payloads onto that layout:
 * `jobs` must be the prepared jobs in the same order with the same weights
 * (NULL for a remapped tensor) and n; their payloads and checksums may
 * differ at every call.  Each call checks its payloads, workspace and
 * results against each other and against the prepared ranges (a binary
 * search each), and reads each block's place from block_map; nothing about
 * the layout is uploaded or searched again.  The workspace needs
 * bf16d_workspace_bytes(sum of n, count) bytes.  Statuses, rollback and the
 * other errors are those of bf16d_decompress.  The plan and the map must
 * stay unchanged while calls that use them run, and the physical buffers
 * must be the ones prepared. */
size_t bf16d_remap_plan_bytes(uint32_t count, uint64_t total_segments);
size_t bf16d_remap_map_bytes(uint64_t total_n, uint32_t count);
int bf16d_remap_prepare(const bf16d_decompress_job *jobs, const bf16d_remap *remaps,
                        uint32_t count, void *plan, size_t plan_bytes, uint64_t *block_map,
                        size_t map_bytes, hipStream_t stream);
int bf16d_decompress_remapped_prepared(const bf16d_decompress_job *jobs, uint32_t count,
                                       const void *plan, const uint64_t *block_map,
                                       void *workspace, size_t workspace_bytes,
                                       bf16d_result *results, hipStream_t stream);

/* Streamed receiver: payloads in host memory, applied layer by layer.
 *
 * The double-buffered pipeline of "GPU-accelerated Weight Teleportation",
 * sections "Overlapping DE and SM" and "Assembling the weight teleporter":
 * the payloads wait in host memory, and the model is streamed through two
 * device slots, one group of tensors (a layer) at a time, so that the copy
 * of one group overlaps the in-place apply of the previous one and only two
 * groups' payloads are ever on the device.  Here the copies are host-to-
 * device DMA transfers on the copy streams, the applies are
 * bf16d_decompress calls on `compute`, and the slots form a ring of `slots`
 * (two or more): with two,
 * every copy waits for the apply just before it, so each cross-stream wait
 * lands on the copies' critical path; three give the copies one group of
 * slack.
 *
 * One tensor of such a call:
 *   weights       : device, 16-byte aligned, n elements (as in
 *                   bf16d_decompress_job).
 *   payload       : host memory, payload_bytes bytes.  Pinned memory
 *                   (hipHostMalloc, or a pinned torch tensor) lets the copy
 *                   run asynchronously; pageable memory is correct but makes
 *                   the copies synchronous with the host.  It must stay valid
 *                   and unchanged until `compute` has completed the call.
 *   checksum      : as in bf16d_decompress_job. */
typedef struct bf16d_stream_job {
    uint16_t      *weights;
    uint64_t       n;
    const uint8_t *payload;
    uint64_t       payload_bytes;
    uint64_t       checksum;
} bf16d_stream_job;

/* Apply `count` host-resident payloads in place, streamed in `groups`
 * groups.  Group g holds jobs [group_end[g-1], group_end[g]) (group_end[-1]
 * is 0); group_end must increase strictly and end at count.
 *   staging      : device, 16-byte aligned, slots * slot_bytes bytes: slot k
 *                  at staging + k * slot_bytes.  slot_bytes must be a
 *                  multiple of 16, and 2 <= slots <= 64.  Group g's payloads
 *                  are packed into slot g % slots, each at a 16-byte
 *                  boundary; every group must fit.  The copy of group g
 *                  waits for the apply of group g - slots.
 *   workspace    : device, 16-byte aligned, at least
 *                  bf16d_workspace_bytes(sum of n, count) bytes (enough
 *                  with or without the extra lane); one workspace serves
 *                  every group, each lane's groups in its stream order.
 *   results      : results[j] for job j, as in bf16d_decompress.
 *   compute      : stream of the applies; the call's work on the copy streams
 *                  starts only after the work enqueued on `compute` before
 *                  the call, and results are valid once `compute` has
 *                  completed.
 *   copy         : copy_streams streams (1 to 8, host array) for the copies;
 *                  group g's copy goes on copy[g % copy_streams].  Each
 *                  host-to-device transfer has a fixed cost of its own
 *                  (about 10 us, more with the event that follows it), which
 *                  two streams hide behind each other's transfers.  A copy
 *                  stream may equal `compute` (that makes the pipeline
 *                  serial).
 *   lanes        : n_lanes (0 or 1) more compute streams (host array; NULL
 *                  when n_lanes is 0).  Group g's apply runs on `compute`
 *                  when g % (1 + n_lanes) == 0, else on lanes[g % (1 +
 *                  n_lanes) - 1], each lane with a workspace region of its
 *                  own, so that one group's short set-up and check kernels
 *                  overlap another group's apply.  The lanes start after the
 *                  work enqueued on `compute` before the call, and `compute`
 *                  waits for them at its end.  A lane should be a stream of
 *                  its own (neither `compute` nor a copy stream).
 *                  All streams must be of the same device.
 * Consecutive payloads of a group that lie in host memory exactly as they are
 * packed in the slot (each at the next 16-byte boundary after the previous
 * one) are copied with a single transfer, padding included.
 * Returns BF16D_EINVAL (nothing enqueued) for bad arguments, BF16D_EHIP if a
 * runtime call fails.  Per-job statuses and the weights' final state are
 * those of bf16d_decompress; a failed job does not affect the others. */
int bf16d_decompress_streamed(const bf16d_stream_job *jobs, uint32_t count,
                              const uint32_t *group_end, uint32_t groups,
                              void *staging, size_t slot_bytes, uint32_t slots,
                              void *workspace, size_t workspace_bytes,
                              bf16d_result *results, hipStream_t compute,
                              const hipStream_t *copy, uint32_t copy_streams,
                              const hipStream_t *lanes, uint32_t n_lanes);

/* Codec race (host only): general-purpose compression of payloads.
 *
 * "Every byte counts: ARCv3 and the case for cross-region RL", section "Deep
 * dive into ARCv3": on top of the structured encoding, every tensor's output
 * is compressed by several general-purpose algorithms running in parallel on
 * the CPU, and the smallest result is kept.  The pages name no codec.  Here
 * the candidates are the caller's list of (codec, level) pairs drawn from
 * zstd, LZ4, LZ4-HC, zlib, Brotli and xz; their runtime libraries
 * (libzstd.so.1, liblz4.so.1, libz.so.1, libbrotlienc.so.1 /
 * libbrotlidec.so.1, liblzma.so.5) are opened on first use, so a host without
 * one of them only loses that codec.  These calls touch no GPU.
 *
 * Frame, little-endian:
 *   magic "BF16DRC1", u32 codec, i32 level, u64 raw_bytes, u64 raw_hash,
 *   then the body: the codec's standard output for the raw bytes (zstd
 *   frame, LZ4 block, zlib stream, Brotli stream, xz stream), or the raw
 *   bytes themselves for BF16D_CODEC_STORED.
 *   raw_hash = mix64(S ^ raw_bytes), S = sum mod 2^64 of
 *   mix64(W_k ^ (k + 1) * 0x9E3779B97F4A7C15) over the little-endian u64
 *   words W_k of the raw bytes, the last one zero-padded (the construction of
 *   the weights' checksum, over bytes).
 * Levels: zstd -5..22; LZ4 acceleration 1..65537; LZ4-HC 1..12; zlib 1..9;
 * Brotli quality 0..11 (window 2^22); xz preset 0..6 (CRC32 check).
 * LZ4 and LZ4-HC take inputs below 0x7E000000 bytes; larger inputs skip
 * them. */
#define BF16D_CODEC_STORED 0
#define BF16D_CODEC_ZSTD   1
#define BF16D_CODEC_LZ4    2
#define BF16D_CODEC_LZ4HC  3
#define BF16D_CODEC_ZLIB   4
#define BF16D_CODEC_BROTLI 5
#define BF16D_CODEC_XZ     6
#define BF16D_RACE_FRAME_HEADER 32

/* One candidate of the race. */
typedef struct bf16d_codec {
    uint32_t codec;
    int32_t  level;
} bf16d_codec;

/* One buffer to compress or decompress.  All pointers are host memory.
 *   in, in_bytes      : the input (race_compress: a payload; race_decompress:
 *                       a frame).  in may be NULL when in_bytes is 0.
 *   out, out_capacity : the output buffer, owned by the caller; it must not
 *                       overlap in.
 *   out_bytes         : written by the call: bytes stored in out.
 *   codec, level      : written by the call: the frame's codec and level.
 *   status            : written by the call: BF16D_OK or, for
 *                       race_decompress, the job's error. */
typedef struct bf16d_race_job {
    const uint8_t *in;
    uint64_t       in_bytes;
    uint8_t       *out;
    uint64_t       out_capacity;
    uint64_t       out_bytes;
    uint32_t       codec;
    int32_t        level;
    int32_t        status;
    uint32_t       reserved;
} bf16d_race_job;

/* 1 if the codec's runtime library could be opened on this host (the stored
 * codec always is), else 0. */
int bf16d_codec_available(uint32_t codec);

/* Frame bytes that always suffice for a raw input of `bytes`: the header plus
 * the input (a frame never exceeds the stored one). */
uint64_t bf16d_race_bound(uint64_t bytes);

/* Race the candidates over every job's input and keep, per job, the smallest
 * frame.  The stored frame always takes part and wins ties; among codecs a
 * tie goes to the earlier candidate, so the result does not depend on thread
 * timing.  Jobs and candidates run on `threads` host threads (0: one per
 * hardware thread; at most 1024), largest inputs first.
 * out_capacity must be at least bf16d_race_bound(in_bytes).  Returns
 * BF16D_EINVAL, with nothing written, for a NULL array or pointer, a short
 * output, an unknown codec, a level out of range, a codec that is not
 * available, or more than 64 candidates.  Otherwise every job ends BF16D_OK:
 * a codec that fails simply loses. */
int bf16d_race_compress(bf16d_race_job *jobs, uint32_t count,
                        const bf16d_codec *candidates, uint32_t n_candidates,
                        uint32_t threads);

/* Read a frame's header: raw size, codec and level (any of the out-pointers
 * may be NULL).  Returns BF16D_EFORMAT for a short frame, a bad magic or an
 * unknown codec, else BF16D_OK. */
int bf16d_race_frame_info(const uint8_t *frame, uint64_t frame_bytes, uint64_t *raw_bytes,
                          uint32_t *codec, int32_t *level);

/* Decode every job's frame into its output, on `threads` host threads as
 * above.  Per job: BF16D_EFORMAT for a malformed frame, a body the codec
 * rejects, or a decoded size other than the header's; BF16D_ECAPACITY if
 * out_capacity is below the raw size (nothing written); BF16D_ECODEC if the
 * codec's library is not available; BF16D_EFORMAT also when the decoded
 * bytes fail raw_hash; else BF16D_OK with out_bytes = raw size.
 * The bytes of out are unspecified after an error.  Returns BF16D_EINVAL for
 * a NULL array or a NULL pointer with a non-zero size, else BF16D_OK. */
int bf16d_race_decompress(bf16d_race_job *jobs, uint32_t count, uint32_t threads);

/* Human-readable name of a status code (static storage). */
const char *bf16d_status_string(int status);

/* Wire-format version this library reads and writes (1). */
int bf16d_format_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BF16DELTA_H */
