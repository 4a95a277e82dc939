// internal.hpp -- shared definitions of the libbf16delta HIP kernels and the
// host code that launches them (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "bf16delta.h"

namespace bf16d {

// ---- format constants (bf16delta_v1) ---------------------------------------
constexpr uint32_t kBlock = BF16D_BLOCK_ELEMS;            // elements per block
constexpr uint32_t kHeader = BF16D_HEADER_BYTES;          // header bytes (version 1)
// version 2: the version-1 header fields, then the binding block
// (u64 base_version, u64 target_version, u32 flags, u32 0, u64 0)
constexpr uint32_t kHeaderBound = BF16D_HEADER_BYTES_BOUND;   // 96
constexpr uint32_t kFlagOverwrite = BF16D_BIND_OVERWRITE;     // records carry new values
constexpr uint32_t kCodeBitmap = 15;
constexpr uint32_t kCodeInvalid = 14;
constexpr uint32_t kExpSign = 0xFF80u;                   // sign + exponent bits of a bf16
constexpr uint32_t kMant = 0x007Fu;                      // mantissa bits
// largest record of one block: bitmap-sized position segment + 7 bits and a
// rare word for every element
constexpr uint32_t kMaxRecord = kBlock / 8 + (7 * kBlock) / 8 + 2 * kBlock;   // 24576
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr uint32_t kMagicLo = 0x36314642u;               // "BF16"
constexpr uint32_t kMagicHi = 0x524F5844u;               // "DXOR"

// ---- launch shape -------------------------------------------------------------
constexpr uint32_t kThreads = 256;                       // 4 waves of 64
constexpr uint32_t kWaves = kThreads / 64;
constexpr uint32_t kChunks = kBlock / 8;                 // 16-byte chunks per block
constexpr uint32_t kChunksPerThread = kChunks / kThreads;   // 4
constexpr uint32_t kDescPerThread = 8;
constexpr uint32_t kDescTile = kThreads * kDescPerThread;   // descriptors per scan tile
// compress: the largest record built in LDS and staged for the place
// kernel (2 KiB); larger records are encoded a second time straight into the
// payload.  Each tile has a workspace slot of `slot_bytes` (a multiple of
// 16, from 16 to kSlot: the caller's workspace decides); a staged record
// that does not fit its slot goes to the payload buffer's tail instead.
constexpr uint32_t kSlot = 2048;
constexpr uint32_t kMinSlot = 16;
// Staging at the payload's tail: up to kStageWays stacks per job, each with
// its own counter (block b uses stack b % ways), so that the blocks of one
// large tensor do not all wait on one atomic.  The stacks take chunks of up
// to kStageChunk bytes from the top of the buffer down, in turn (chunk i of
// stack k is the (i * ways + k)-th from the top), so that the staged records
// stay together at the top, above the final payload where possible.
constexpr uint32_t kStageWays = 32;
constexpr uint32_t kStageChunk = 8192;
constexpr uint32_t kStageTries = 4;   // a range that crosses a chunk's end is abandoned

// ---- decoupled look-back status words ---------------------------------------
// bits 62..63: 0 = not yet published, 1 = tile aggregate, 2 = inclusive prefix
constexpr uint64_t kFlagAggregate = 1ull << 62;
constexpr uint64_t kFlagPrefix = 2ull << 62;
constexpr uint64_t kValueMask = (1ull << 62) - 1;

// Pointers into the caller's buffers, as device code sees them: global memory
// (address space 1), so that accesses compile to global rather than flat
// instructions and wait only on the vector-memory counter.  Host code sees
// plain pointers of the same size.
#if defined(__HIP_DEVICE_COMPILE__)
#define BF16D_GMEM __attribute__((address_space(1)))
#else
#define BF16D_GMEM
#endif

// ---- device-side job tables (copied into the workspace by the host) ---------
struct alignas(64) CompressJob {
    BF16D_GMEM const uint16_t *src;
    BF16D_GMEM const uint16_t *dst;
    uint64_t n;
    BF16D_GMEM uint8_t *payload;
    uint64_t capacity;
    uint64_t block0;   // first global tile index of this job
    uint64_t nb;       // blocks of this job
    uint32_t hdr;      // header bytes: kHeader (version 1) or kHeaderBound (version 2)
    uint32_t flags;    // version 2: kFlagOverwrite or 0
    uint64_t base_version, target_version;   // version 2 binding
};

enum JobState : uint32_t { kStateReady = 1, kStateRejected = 2, kStateVersion = 3 };

// one segment of a remapped tensor: logical elements [first, first + count)
// live at dst (first is block-aligned)
struct alignas(32) RemapSegment {
    uint64_t first, count;
    BF16D_GMEM uint16_t *dst;
    uint64_t pad;
};

struct alignas(64) DecompressJob {
    BF16D_GMEM uint16_t *weights;
    uint64_t n;
    BF16D_GMEM const uint8_t *payload;
    uint64_t payload_bytes;
    uint64_t checksum;
    uint64_t block0;   // first global tile index
    uint64_t nb;       // blocks
    uint64_t dtile0;   // first global descriptor-scan tile index
    BF16D_GMEM const RemapSegment *segs;   // remapped: the job's segments; else nullptr
    uint32_t nsegs;             // 0: no remap, the weights pointer is used
    BF16D_GMEM uint64_t *version;   // the receiver's version word, or nullptr
    uint32_t verify_first;      // XOR records: verified before anything is written
    // overwrite records: an undo area laid out like the job's records (the
    // old value of a record's j-th change at record offset + 2j), or nullptr
    // (then an overwrite job is verified first and written after)
    BF16D_GMEM uint8_t *undo;
};

// per-job device state of a decompress call (zeroed by the setup kernel)
struct alignas(64) DecompressState {
    unsigned long long sum_c, sum_r, sum_pos, sum_mant, sum_rare, n_bitmap;
    uint32_t desc_bad;     // a descriptor failed its checks
    uint32_t state;        // JobState, set by the prepare kernel
    uint32_t block_bad;    // a block record failed its checks
    uint32_t rollback;     // the apply pass must be undone
    uint32_t commit;       // overwrite payload verified: the commit pass writes it
    uint32_t hdr;          // header bytes of the payload (set by the prepare kernel)
    uint32_t ow;           // an overwrite payload
    uint32_t bound;        // a version-2 payload
    uint32_t undo;         // overwrite, written in place with an undo log (set by prepare)
    long long undo_delta;  // undo area minus the start of the job's records (bytes)
};

// decompress: everything the apply pass needs about one tile, gathered once
// by the plan kernel so that a workgroup starts with a single (scalar) load
struct alignas(32) ApplyPlan {
    BF16D_GMEM uint16_t *w;          // first weight of the block
    BF16D_GMEM const uint8_t *rec;   // first byte of the block's record
    uint32_t desc;        // the block's descriptor
    uint32_t len_room;    // block length (bits 0..13; 0 = skip the tile) | payload bytes
                          // left from `rec`, capped at 2^16 - 1 (bits 14..29) |
                          // kPlanVerifyFirst (bit 30): an XOR record verified before
                          // it is written | kPlanOverwrite (bit 31): an overwrite record
    uint32_t job;
    uint32_t block;       // block index within the job
};
static_assert(sizeof(ApplyPlan) == 32, "ApplyPlan is two 16-byte words");
constexpr uint32_t kPlanOverwrite = 1u << 31;
constexpr uint32_t kPlanVerifyFirst = 1u << 30;
// with kPlanOverwrite, the same bit: an overwrite record written in place
// with an undo log (instead of verified first)
constexpr uint32_t kPlanUndo = kPlanVerifyFirst;
constexpr uint32_t kRoomCap = (1u << 16) - 1;   // above any record window (24 KiB + 15)

// per-job sums (zeroed at the start of a call), accumulated with one atomic
// per job and scan tile of 2048 blocks: the checksum sum S (both directions,
// from the per-wave partials) and, for compress, the header totals.  (One
// atomic per wave and tile, straight from the main kernels, contends on the
// few addresses and measured much slower.)
struct alignas(64) JobSums {
    unsigned long long csum, c, r, pos, mant, nbm;
    unsigned long long pad;
    unsigned long long P;       // compress: payload bytes, written by finalize
};

// compress: where one tile's record goes, written by the offsets kernel for
// the place kernel
struct alignas(16) PlaceEntry {
    BF16D_GMEM uint8_t *dst;   // first byte of the record in the payload
    uint32_t len;              // bytes to copy: 0 if none (empty, re-encoded elsewhere,
                               // or past the capacity), else cut at the capacity
    uint32_t staged;           // 1: the record waits at the payload's tail, and the
                               // slot holds its address; 0: the record is in the slot
};
constexpr uint32_t kStaged = 1;
static_assert(sizeof(PlaceEntry) == 16, "PlaceEntry is one 16-byte word");

struct alignas(64) Control {
    uint32_t ticket;          // (unused) dynamic tile ids
    uint32_t dticket;         // dynamic tile ids for the descriptor-scan look-back
    uint32_t any_rollback;    // decompress: some job must be rolled back
    uint32_t overflow_count;  // compress: tiles whose record exceeded a slot
    uint32_t any_commit;      // decompress: some overwrite payload is to be written
    uint32_t scan_done;       // workgroups of the descriptor/offset scan that have finished
    uint32_t sum_done;        // decompress: workgroups of the checksum sum that have finished
    uint32_t any_commit_xor;  // decompress: some job verified first is to be written
    uint32_t pad[8];
};

// Set-up of a batched call in one launch: zero fills and tile -> job maps.
struct SetupArgs {
    uint32_t *zero[3];            // ranges to clear (may be null)
    uint64_t zero_words[3];
    const uint64_t *start[2];     // job start tables of the maps
    uint32_t *map[2];             // map[m][t] = j with start[m][j] <= t < start[m][j + 1]
    uint64_t *status[2];          // cleared alongside map[m] (may be null)
    uint64_t tiles[2];
    uint32_t count;
};

// Workspace layout, computed identically by every entry point.
struct Layout {
    size_t control, jobs, block_start, dtile_start, tile_job, status, partial, sums, desc,
        dtile_job, dstatus, state, slots, overflow, stage, plan, total;
    uint32_t slot_bytes;   // compress: the record slot of each tile
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline Layout make_layout(uint64_t tiles, uint64_t dtiles, uint32_t count, bool compress,
                          uint32_t slot_bytes = kSlot) {
    Layout l{};
    l.slot_bytes = compress ? slot_bytes : 0;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    size_t job_bytes = sizeof(CompressJob) > sizeof(DecompressJob) ? sizeof(CompressJob)
                                                                  : sizeof(DecompressJob);
    l.control = take(sizeof(Control));
    l.jobs = take(job_bytes * count);
    l.block_start = take(8 * (size_t(count) + 1));
    l.dtile_start = take(8 * (size_t(count) + 1));
    l.tile_job = take(4 * tiles);
    l.status = take(8 * tiles);     // record offsets
    l.partial = take(8 * kWaves * tiles);   // per-wave checksum partial sums of each tile
    l.sums = take(sizeof(JobSums) * size_t(count));   // per-job sums (atomic)
    l.desc = take(4 * tiles);       // compress: descriptor copies
    l.dtile_job = take(4 * dtiles);
    l.dstatus = take(8 * dtiles);
    l.state = take(sizeof(DecompressState) * size_t(count));
    l.slots = take(compress ? size_t(slot_bytes) * tiles : 0);   // compress: record slots
    l.overflow = take(compress ? 4 * tiles : 0);              // compress: overflowing tiles
    // compress: bytes taken in each part of each job's tail staging
    l.stage = take(compress ? 8 * size_t(kStageWays) * count : 0);
    // per-tile plan: compress, where each record goes (PlaceEntry); decompress, ApplyPlan
    l.plan = take(compress ? sizeof(PlaceEntry) * tiles : sizeof(ApplyPlan) * tiles);
    l.total = off;
    return l;
}

// ---- device helpers ------------------------------------------------------------

// SplitMix64 finaliser (Steele, Lea and Flood, OOPSLA 2014; Stafford's Mix13).
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z;
}

// Relaxed device-scope loads and stores.  They order nothing: a reader only
// relies on the single word it reads.  The look-back status words carry
// their flag and their value in one 64-bit word for exactly that reason (a
// reader that sees the flag sees the value that came with it).
__device__ __forceinline__ uint64_t ld_relaxed_agent(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_agent(const unsigned long long *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Workgroup b of a launch runs on XCD b % 8 (workgroups are dispatched to
// the XCDs in turn).  A one-workgroup-per-tile kernel maps b to a tile so
// that each XCD takes a contiguous range (XCD x: q + (x < r) tiles from
// x*q + min(x, r), q = tiles / 8, r = tiles % 8): neighbouring tiles, and
// the lines of per-tile tables they share, stay in one L2.  A bijection on
// [0, tiles) whatever the dispatch order.
__device__ __forceinline__ uint64_t xcd_tile(uint64_t b, uint64_t tiles) {
    const uint64_t q = tiles >> 3, r = tiles & 7, x = b & 7, y = b >> 3;
    return x * q + (x < r ? x : r) + y;
}

// Counts the workgroups of a grid as they finish; true in the last one.
// Workgroups hand results to it only through device-scope atomics, which the
// last workgroup reads with device-scope loads.  `dep` is the XOR of the
// values the calling thread's atomics returned (0 in threads that made
// none): the count waits for them to come back, so they are done before the
// last workgroup can look.  Every thread must call it (it contains barriers).
//
// Why this is safe without a fence.  The ordering comes from the hardware,
// not from the HIP memory model: with relaxed atomics only, the model itself
// would not order the sums before the count (that would take a release on
// the count and an acquire in the last workgroup).  On gfx950 a
// device-scope atomic is performed at the device's coherence point, and a
// returning atomic has been performed there once its value is back in a
// register.  The asm below makes the count's increment depend on those
// values, so every sum this workgroup adds is at the coherence point before
// its increment is issued.  The last workgroup's loads are device-scope
// (they read the coherence point, not a stale L2 line) and are issued after
// its own increment returned the final count, i.e. after every other
// workgroup's increment, and so after every sum.  Only atomics cross
// workgroups here; plain stores would need a real release.  The fence this
// avoids is not free on this chip: a device-scope release writes back the
// XCD's L2 and an acquire invalidates it, in every workgroup (0.14 ms per
// call on the 7B-shaped decompress, measured).
__device__ __forceinline__ bool last_workgroup(uint32_t *done, uint64_t dep) {
    __shared__ bool s_last;
    asm volatile("" ::"v"(dep) : "memory");
    __syncthreads();
    if (threadIdx.x == 0)
        s_last = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 gridDim.x - 1;
    __syncthreads();
    return s_last;
}
__device__ __forceinline__ void st_agent(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}
// The value lane 0 holds, as a wave-uniform (scalar) value, read where the
// whole wave is active: a value the wave has just reduced can then be stored
// by one lane without the reduction moving into that lane's branch.
__device__ __forceinline__ uint32_t first_lane(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}
__device__ __forceinline__ uint64_t first_lane(uint64_t v) {
    return (uint64_t)first_lane((uint32_t)v) | (uint64_t)first_lane((uint32_t)(v >> 32)) << 32;
}
__device__ __forceinline__ unsigned long long first_lane(unsigned long long v) {
    return first_lane((uint64_t)v);
}

// Block-wide sum over kThreads threads; every thread gets the total.
// s_tmp needs kWaves entries.  Contains two barriers.
template <typename T>
__device__ __forceinline__ T block_sum(T v, T *s_tmp) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const T w = first_lane(wave_sum(v));
    if (lane == 0) s_tmp[wave] = w;
    __syncthreads();
    T t = 0;
#pragma unroll
    for (int w2 = 0; w2 < (int)kWaves; ++w2) t += s_tmp[w2];
    __syncthreads();
    return t;
}

// Block-wide exclusive prefix sum in thread order; `total` receives the sum.
template <typename T>
__device__ __forceinline__ T block_exclusive_sum(T v, T *s_tmp, T &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    T inc = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        T o = __shfl_up(inc, d, 64);
        if (lane >= d) inc += o;
    }
    if (lane == 63) s_tmp[wave] = inc;
    __syncthreads();
    T before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < (int)kWaves; ++w) {
        if (w < wave) before += s_tmp[w];
        all += s_tmp[w];
    }
    __syncthreads();
    total = all;
    return before + inc - v;
}

// ---- wave64 DPP scans (GFX9 row_shr / row_bcast / wave_shr) -------------------
// Inclusive scans over the 64 lanes of a wave in 6 DPP-fused ALU ops.
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ uint32_t dpp_src(uint32_t v) {
    // lanes without a source (or outside row_mask) read 0, the identity of add and unsigned max
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, kRowMask, 0xf, false);
}
__device__ __forceinline__ uint32_t wave_incl_add(uint32_t v) {
    v += dpp_src<0x111>(v);          // row_shr:1
    v += dpp_src<0x112>(v);          // row_shr:2
    v += dpp_src<0x114>(v);          // row_shr:4
    v += dpp_src<0x118>(v);          // row_shr:8
    v += dpp_src<0x142, 0xa>(v);     // row_bcast:15 into rows 1 and 3
    v += dpp_src<0x143, 0xc>(v);     // row_bcast:31 into rows 2 and 3
    return v;
}
__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t wave_incl_max(uint32_t v) {
    v = umax32(v, dpp_src<0x111>(v));
    v = umax32(v, dpp_src<0x112>(v));
    v = umax32(v, dpp_src<0x114>(v));
    v = umax32(v, dpp_src<0x118>(v));
    v = umax32(v, dpp_src<0x142, 0xa>(v));
    v = umax32(v, dpp_src<0x143, 0xc>(v));
    return v;
}
// inclusive scans within each row of 16 lanes
__device__ __forceinline__ uint32_t row_incl_add(uint32_t v) {
    v += dpp_src<0x111>(v);
    v += dpp_src<0x112>(v);
    v += dpp_src<0x114>(v);
    v += dpp_src<0x118>(v);
    return v;
}
__device__ __forceinline__ uint32_t row_incl_max(uint32_t v) {
    v = umax32(v, dpp_src<0x111>(v));
    v = umax32(v, dpp_src<0x112>(v));
    v = umax32(v, dpp_src<0x114>(v));
    v = umax32(v, dpp_src<0x118>(v));
    return v;
}
// Cross-lane reads (readlane_u32, lane63, the DPP scans) belong in control
// flow that the whole wave executes.  Inside a branch only some lanes take
// (`if (lane == 0)`), the compiler may compute the operand for the active
// lanes only, and the read then returns another lane's stale value: take the
// value before the branch and use it inside.
__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, uint32_t lane) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, (int)lane);
}
// value of the previous lane (0 for lane 0)
__device__ __forceinline__ uint32_t wave_shr1(uint32_t v) { return dpp_src<0x138>(v); }
// value of the previous lane, `fill` for lane 0 (one DPP move, no lane test)
__device__ __forceinline__ uint32_t wave_shr1_fill(uint32_t v, uint32_t fill) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)fill, (int)v, 0x138, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t lane63(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Decoupled look-back by one wave over the status words of tiles
// [first, tile): returns the sum of their values (the exclusive prefix of
// `tile`).  Each lane reads kLookDepth words per round, so one round trip
// covers 64 * kLookDepth predecessors.  A tile publishes its aggregate
// before it looks back, and a workgroup only waits on tiles claimed before
// its own, whose holders are running; so every wait ends.  Tiles below
// `first` read as an empty inclusive prefix.
constexpr int kLookDepth = 4;

__device__ __forceinline__ uint64_t look_back(uint64_t *status, uint64_t tile, uint64_t first) {
    const int lane = threadIdx.x & 63;
    uint64_t excl = 0;
    int64_t pred = (int64_t)tile - 1;
    for (;;) {
        uint64_t v[kLookDepth];
#pragma unroll
        for (int k = 0; k < kLookDepth; ++k) {
            const int64_t idx = pred - lane - 64 * k;   // distance 1 + lane + 64k
            v[k] = idx >= (int64_t)first ? ld_relaxed_agent(&status[idx]) : kFlagPrefix;
        }
        // wait only for the entries nearer than the nearest inclusive prefix
        // seen so far; re-pick that prefix after every reload
        int stop_k, stop_lane;
        for (;;) {
            stop_k = kLookDepth;
            stop_lane = 63;
#pragma unroll
            for (int k = kLookDepth - 1; k >= 0; --k) {
                const uint64_t m = __ballot((v[k] >> 62) == 2);
                if (m) {
                    stop_k = k;
                    stop_lane = __ffsll((unsigned long long)m) - 1;
                }
            }
            bool pending = false;
#pragma unroll
            for (int k = 0; k < kLookDepth; ++k)
                pending |= (k < stop_k || (k == stop_k && lane < stop_lane)) && (v[k] >> 62) == 0;
            if (__ballot(pending) == 0) break;
            __builtin_amdgcn_s_sleep(1);
#pragma unroll
            for (int k = 0; k < kLookDepth; ++k) {
                const int64_t idx = pred - lane - 64 * k;
                if ((k < stop_k || (k == stop_k && lane < stop_lane)) && (v[k] >> 62) == 0)
                    v[k] = ld_relaxed_agent(&status[idx]);
            }
        }
        uint64_t mine = 0;
#pragma unroll
        for (int k = 0; k < kLookDepth; ++k)
            if (k < stop_k || (k == stop_k && lane <= stop_lane)) mine += v[k] & kValueMask;
        excl += first_lane(wave_sum(mine));   // wave-uniform, whatever the caller's branch
        if (stop_k < kLookDepth) return excl;
        pred -= 64 * kLookDepth;
    }
}

__device__ __forceinline__ uint32_t bit_length(uint32_t v) { return v ? 32u - __clz(v) : 0u; }

// OR `width` (<= 16) bits of `value` into an LDS bit stream at `bitpos`.
__device__ __forceinline__ void lds_or_bits(uint32_t *s, uint32_t bitpos, uint32_t value,
                                            uint32_t width) {
    if (value == 0) return;
    const uint32_t d = bitpos >> 5, sh = bitpos & 31;
    atomicOr(&s[d], value << sh);
    if (sh + width > 32) atomicOr(&s[d + 1], value >> (32 - sh));
}

// Read `width` (<= 32) bits at `bitpos` of an LDS bit stream.
__device__ __forceinline__ uint32_t lds_get_bits(const uint32_t *s, uint32_t bitpos,
                                                 uint32_t width) {
    const uint32_t d = bitpos >> 5, sh = bitpos & 31;
    const uint64_t v = (uint64_t)s[d] | ((uint64_t)s[d + 1] << 32);
    const uint64_t mask = (width >= 32) ? 0xFFFFFFFFull : ((1ull << width) - 1);
    return (uint32_t)((v >> sh) & mask);
}

// 8-bit mask of the non-zero 16-bit halves of a 16-byte chunk: bit s is set
// iff element s (low half of dword s/2 for even s, high half for odd s) != 0.
__device__ __forceinline__ uint32_t nz2(uint32_t w) {
    // bit 15 of each half: its low 15 bits are non-zero, or bit 15 itself is set
    return (((w & 0x7FFF7FFFu) + 0x7FFF7FFFu) | w) & 0x80008000u;
}
__device__ __forceinline__ uint32_t nonzero_halves(const uint4 &v) {
    // halves of dword d land on bits 2d (low) and 2d+16 (high) ...
    const uint32_t m = (nz2(v.x) >> 15) | (nz2(v.y) >> 13) | (nz2(v.z) >> 11) | (nz2(v.w) >> 9);
    // ... then bits 16..22 move down next to their even partners
    return (m & 0x55u) | ((m >> 15) & 0xAAu);
}
// Per 16-bit half: min(half, 1), i.e. 1 where the half is non-zero.  Written
// as the packed-integer instruction itself: the compiler would otherwise turn
// the min into two compares and two selects per dword.
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t w, uint32_t ones) {
    uint32_t r;
    asm("v_pk_min_u16 %0, %1, %2" : "=v"(r) : "v"(w), "v"(ones));
    return r;
}
// 8-bit element-order mask of the non-zero halves of (v & mask).
__device__ __forceinline__ uint32_t nonzero8(const uint4 &v, uint32_t mask) {
    const uint32_t ones = 0x00010001u;
    // low halves (elements 0,2,4,6) land on bits 0,2,4,6; high halves on 16,18,20,22
    const uint32_t s = pk_min_u16(v.x & mask, ones) | (pk_min_u16(v.y & mask, ones) << 2) |
                       (pk_min_u16(v.z & mask, ones) << 4) | (pk_min_u16(v.w & mask, ones) << 6);
    return (s & 0x55u) | ((s >> 15) & 0xAAu);
}
__device__ __forceinline__ uint4 and4(const uint4 &v, uint32_t m) {
    return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// Element s (0..7) of a 16-byte chunk held as uint4.
__device__ __forceinline__ uint32_t chunk_elem(const uint4 &v, int s) {
    uint32_t w = (s < 2) ? v.x : (s < 4) ? v.y : (s < 6) ? v.z : v.w;
    return (s & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// A 16-byte load of data that is read once and never written: marked
// non-temporal (`nt`), so the lines of a checkpoint streamed through the
// caches do not stay there at the cost of other data.  On the 7B-shaped
// workload the encoder runs 2-5 % faster this way, and a read-only probe of
// the same pattern 8 %.  Not for a pass that writes back what it reads: the
// in-place apply measured 29 % slower with it.
__device__ __forceinline__ uint4 load_stream16(BF16D_GMEM const void *p) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<BF16D_GMEM const v4u *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// A 16-byte store of data that this kernel will not read again, marked
// non-temporal.  The encoder's record stores take it: with the checkpoint
// loads also non-temporal, they made the encoder 3-5 % faster on the
// 7B-shaped workload when it runs right after a decompress, as in a
// benchmark step (with plain loads the same stores measured no faster).
__device__ __forceinline__ void store_stream16(void *p, const uint4 &q) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    v4u v;
    v.x = q.x;
    v.y = q.y;
    v.z = q.z;
    v.w = q.w;
    __builtin_nontemporal_store(v, reinterpret_cast<v4u *>(p));
}

// Load 8 bf16 patterns at p, of which the first `valid` (<= 8) exist.
__device__ __forceinline__ uint4 load_chunk(BF16D_GMEM const uint16_t *p, uint32_t valid) {
    if (valid >= 8) return *reinterpret_cast<BF16D_GMEM const uint4 *>(p);
    uint32_t w[4] = {0, 0, 0, 0};
    for (uint32_t s = 0; s < valid; ++s) w[s >> 1] |= (uint32_t)p[s] << (16 * (s & 1));
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Checksum terms of one chunk of new weights starting at element index e
// (a multiple of 8) of which `valid` exist: words k = e/4 and e/4+1.
__device__ __forceinline__ uint64_t chunk_checksum(const uint4 &v, uint64_t e, uint32_t valid) {
    uint64_t acc = 0;
    const uint64_t k = e >> 2;
    if (valid > 0) acc += mix64(((uint64_t)v.y << 32 | v.x) ^ ((k + 1) * kGamma));
    if (valid > 4) acc += mix64(((uint64_t)v.w << 32 | v.z) ^ ((k + 2) * kGamma));
    return acc;
}

}  // namespace bf16d

// ---- kernel launchers (defined in the .hip files) ------------------------------
namespace bf16d {
// host side of a decompress call (api.hip): checks the jobs and lays out the
// job table; decompress_table writes the bytes [l.jobs, l.dtile_start +
// 8 * (count + 1)) of the workspace as they must be uploaded
struct DecompressPrep {
    std::vector<uint64_t> bstart, dstart;   // first tile / descriptor tile of each job
    uint64_t tiles = 0, dtiles = 0;
};
// `mapped`: the weights' places come from a prepared block map, so the jobs'
// weights pointers are not checked here (the prepared call checks them
// against its plan instead)
int decompress_prep(const bf16d_decompress_job *jobs, uint32_t count, DecompressPrep &p,
                    const bf16d_remap *remaps = nullptr, bool mapped = false);
size_t decompress_table_bytes(const Layout &l, uint32_t count);
void decompress_table(const bf16d_decompress_job *jobs, uint32_t count, const DecompressPrep &p,
                      const Layout &l, uint8_t *out, bool verify_first = false);

// workgroups of a persistent kernel: as many as fit on the device at once
uint32_t persistent_grid(const void *kernel, uint64_t tiles, size_t dynamic_lds = 0);
void launch_setup(const SetupArgs &a, hipStream_t stream);
hipError_t launch_compress(const Layout &l, uint8_t *ws, uint32_t count, uint64_t tiles,
                           uint64_t dtiles, bf16d_result *results, hipStream_t stream,
                           const bf16d_events *events, bool any_overwrite);
// block_map (may be null): the physical address of each tile's first weight,
// prepared once for a remapped layout (bf16d_remap_prepare)
hipError_t launch_decompress(const Layout &l, uint8_t *ws, uint32_t count, uint64_t tiles,
                             uint64_t dtiles, bf16d_result *results, hipStream_t stream,
                             const bf16d_events *events, const uint64_t *block_map = nullptr,
                             bool verify_first = false);
}  // namespace bf16d
