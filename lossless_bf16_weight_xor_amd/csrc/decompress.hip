// decompress.hip -- in-place BF16 delta decoder for gfx950.
//
// The receiver rebuilds the new weights by XOR-ing the decoded mask onto the
// old ones in HBM ("GPU-accelerated Weight Teleportation", sections "Delta
// update algebra" and "A strong baseline with Blackwell-native DE").  It
// then checks them against the trainer's checksum ("Every byte counts: ARCv3
// and the case for cross-region RL", section "Deep dive into ARCv3").
//
// Kernels of one batched call, in stream order (six launches):
//   setup     : clears the call's state and builds the descriptor-tile -> job
//               map.
//   desc_scan : validates every descriptor and builds the block offset table
//               (the exclusive sum of record sizes within each job).  It uses
//               the same decoupled look-back as the encoder, over tiles of
//               2048 descriptors.  Its last workgroup then checks each job's
//               header against the arguments and the descriptor sums; a job
//               that fails is rejected before any weight is touched.
//   plan      : one entry per block: its weight and record addresses.
//   apply     : one workgroup per 8192-element block.  The block's old
//               weights are loaded into registers first, so HBM latency
//               overlaps the decode; occupancy (up to 6 workgroups per CU)
//               hides the rest.  The record is staged in LDS and
//               decoded into a dense 16 KiB XOR tile in LDS, checking that it
//               is canonical.  Then old ^ tile is formed, only the changed
//               16-byte chunks are written back, and the checksum terms of
//               the result are accumulated.
//   sum       : adds up each job's checksum terms; its last workgroup
//               compares every job's checksum and writes the results.
//   fixup     : the apply pass again, for the failed jobs only (XOR is its
//               own inverse, so this restores the old weights exactly) and for
//               verified overwrite payloads; it exits at once when there is
//               neither.
//
// Version-2 payloads ("GPU-accelerated Weight Teleportation", section "Eval,
// fault tolerance, and resuming from trained checkpoints"; the NeMo
// Delta-Compressed Refit summary): the header check refuses a payload whose
// base version is not the receiver's, before anything is touched, and the
// checksum step moves the receiver's version word to the target together
// with the weights.  An overwrite payload carries absolute values, which
// applying again cannot undo, so the apply kernel only verifies it (the
// checksum of the would-be result, no stores) and the fix-up pass writes it
// once verified: the weights end new, or untouched.
#include "internal.hpp"

namespace bf16d {


__device__ __forceinline__ uint32_t block_length(uint64_t n, uint64_t b) {
    const uint64_t left = n - b * kBlock;
    return left < kBlock ? (uint32_t)left : kBlock;
}

// ------------------------------------------------------------------ prepare ---
// Job j's header against its arguments and its descriptor sums (read with
// device-scope loads: the scan's last workgroup runs this right after the
// other workgroups' atomics).
__device__ void prepare_job(const DecompressJob *__restrict__ jobs,
                            DecompressState *__restrict__ state, uint32_t j) {
    const DecompressJob job = jobs[j];
    DecompressState *st = &state[j];
    const unsigned long long sum_c = ld_agent(&st->sum_c), sum_r = ld_agent(&st->sum_r),
                             sum_pos = ld_agent(&st->sum_pos),
                             sum_mant = ld_agent(&st->sum_mant);
    const uint32_t desc_bad = ld_agent(&st->desc_bad);
    bool ok = job.payload_bytes >= kHeader;
    bool bound = false, ow = false, wrong_version = false;
    uint32_t hdr = kHeader;
    if (ok) {
        BF16D_GMEM const uint32_t *h = reinterpret_cast<BF16D_GMEM const uint32_t *>(job.payload);
        BF16D_GMEM const uint64_t *h64 = reinterpret_cast<BF16D_GMEM const uint64_t *>(job.payload);
        bound = h[2] == BF16D_FORMAT_VERSION_BOUND;
        hdr = bound ? kHeaderBound : kHeader;
        ok = h[0] == kMagicLo && h[1] == kMagicHi && (bound || h[2] == BF16D_FORMAT_VERSION) &&
             job.payload_bytes >= hdr;
        if (ok && bound) {   // the binding block: known flags, zero reserved words
            ok = (h[20] & ~kFlagOverwrite) == 0 && h[21] == 0 && h64[11] == 0;
            ow = (h[20] & kFlagOverwrite) != 0;
        }
        ok = ok && h[3] == kBlock && h64[2] == job.n && job.payload_bytes >= hdr + 4 * job.nb &&
             desc_bad == 0 && sum_c == h64[3] && sum_r == h64[4] && sum_pos == h64[5] &&
             sum_mant == h64[6] && 2 * sum_r == h64[7] &&
             hdr + 4 * job.nb + sum_pos + sum_mant + 2 * sum_r == job.payload_bytes;
        // the binding: a version-2 payload applies only to its base version
        wrong_version = ok && bound && job.version && *job.version != h64[8];
    }
    st->hdr = hdr;
    st->ow = ow;
    st->bound = bound;
    st->undo = ow && job.undo != nullptr;
    st->undo_delta = st->undo ? (long long)((uintptr_t)job.undo -
                                            (uintptr_t)(job.payload + hdr + 4 * job.nb))
                              : 0;
    st->state = !ok ? kStateRejected : (wrong_version ? kStateVersion : kStateReady);
}

// ---------------------------------------------------------------- desc_scan ---
__global__ __launch_bounds__(kThreads) void desc_scan_kernel(
    const DecompressJob *__restrict__ jobs, const uint32_t *__restrict__ dtile_job,
    uint64_t *__restrict__ dstatus, uint64_t *__restrict__ offsets,
    DecompressState *__restrict__ state, Control *__restrict__ ctrl, uint32_t count) {
    __shared__ uint32_t s_tmp32[kWaves];
    __shared__ unsigned long long s_tmp64[kWaves];
    __shared__ uint32_t s_dt;
    __shared__ uint64_t s_excl;
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    if (tid == 0)
        s_dt = __hip_atomic_fetch_add(&ctrl->dticket, 1u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint64_t dt = s_dt;
    const uint32_t j = dtile_job[dt];
    const DecompressJob job = jobs[j];
    const uint64_t ld = dt - job.dtile0;
    // header size and record kind, read before the header is validated (the
    // header check rejects the job if they were wrong)
    uint32_t hdr = kHeader;
    bool ow = false;
    if (job.payload_bytes >= kHeaderBound) {
        BF16D_GMEM const uint32_t *h = reinterpret_cast<BF16D_GMEM const uint32_t *>(job.payload);
        if (h[2] == BF16D_FORMAT_VERSION_BOUND) {
            hdr = kHeaderBound;
            ow = (h[20] & kFlagOverwrite) != 0;
        }
    }
    const bool table_ok = job.payload_bytes >= hdr + 4 * job.nb;

    uint32_t lens[kDescPerThread];
    uint32_t mine = 0, bad = table_ok ? 0u : 1u;
    unsigned long long c_sum = 0, r_sum = 0, pos_sum = 0, mant_sum = 0, nbm = 0;
#pragma unroll
    for (uint32_t k = 0; k < kDescPerThread; ++k) {
        const uint64_t d = ld * kDescTile + kDescPerThread * tid + k;
        lens[k] = 0;
        if (!table_ok || d >= job.nb) continue;
        const uint32_t desc =
            *reinterpret_cast<BF16D_GMEM const uint32_t *>(job.payload + hdr + 4 * d);
        const uint32_t L = block_length(job.n, d);
        const uint32_t c = desc & 0x3FFFu, r = (desc >> 14) & 0x3FFFu, code = desc >> 28;
        uint32_t pb;
        if (code == kCodeBitmap) {
            pb = (L + 7) / 8;
            bad |= (c == 0);
        } else {
            pb = (c * code + 7) / 8;
            bad |= (code == kCodeInvalid) | (c == 0 && code != 0) | (pb > (L + 7) / 8);
        }
        bad |= (c > L) | (r > c) | (ow & (r != c));   // overwrite: one word per change
        const uint32_t mb = ow ? 0u : (7 * c + 7) / 8;
        lens[k] = pb + mb + 2 * r;
        mine += lens[k];
        c_sum += c;
        r_sum += r;
        pos_sum += pb;
        mant_sum += mb;
        nbm += code == kCodeBitmap;
    }

    uint32_t tile_total;
    uint32_t excl = block_exclusive_sum(mine, s_tmp32, tile_total);
    if (tid == 0) st_agent(&dstatus[dt], (ld == 0 ? kFlagPrefix : kFlagAggregate) | tile_total);
    if (wave == 0) {
        const uint64_t e = (ld == 0) ? 0 : look_back(dstatus, dt, job.dtile0);
        if (lane == 0) {
            if (ld != 0) st_agent(&dstatus[dt], kFlagPrefix | (e + tile_total));
            s_excl = e;
        }
    }
    __syncthreads();
    if (table_ok) {
        uint64_t off = s_excl + excl;
#pragma unroll
        for (uint32_t k = 0; k < kDescPerThread; ++k) {
            const uint64_t d = ld * kDescTile + kDescPerThread * tid + k;
            if (d < job.nb) offsets[job.block0 + d] = off;
            off += lens[k];
        }
    }
    c_sum = block_sum(c_sum, s_tmp64);
    r_sum = block_sum(r_sum, s_tmp64);
    pos_sum = block_sum(pos_sum, s_tmp64);
    mant_sum = block_sum(mant_sum, s_tmp64);
    nbm = block_sum(nbm, s_tmp64);
    const uint32_t any_bad = __syncthreads_or(bad);
    uint64_t dep = 0;
    if (tid == 0) {
        DecompressState *st = &state[j];
        dep = atomicAdd(&st->sum_c, c_sum) ^ atomicAdd(&st->sum_r, r_sum) ^
              atomicAdd(&st->sum_pos, pos_sum) ^ atomicAdd(&st->sum_mant, mant_sum) ^
              atomicAdd(&st->n_bitmap, nbm);
        if (any_bad) dep ^= atomicOr(&st->desc_bad, 1u);
    }
    // the last workgroup to finish checks every job's header against the sums
    if (last_workgroup(&ctrl->scan_done, dep))
        for (uint32_t jj = tid; jj < count; jj += kThreads) prepare_job(jobs, state, jj);
}

// For calls without descriptors (every tensor empty); otherwise the scan's
// last workgroup prepares the jobs.
__global__ void prepare_kernel(const DecompressJob *__restrict__ jobs,
                               DecompressState *__restrict__ state, uint32_t count) {
    const uint32_t j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j < count) prepare_job(jobs, state, j);
}

// --------------------------------------------------------------------- plan ---
// One thread per tile: gathers the tile's weight and record addresses and its
// descriptor, so that an apply workgroup starts from one load.  Tiles of jobs
// that were rejected get length 0 and are skipped.
__global__ void plan_kernel(const DecompressJob *__restrict__ jobs,
                            const DecompressState *__restrict__ state,
                            const uint64_t *__restrict__ start, uint32_t count,
                            const uint64_t *__restrict__ offsets, ApplyPlan *__restrict__ plan,
                            const uint64_t *__restrict__ block_map, uint64_t tiles) {
    for (uint64_t t = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; t < tiles;
         t += (uint64_t)gridDim.x * blockDim.x) {
        uint32_t lo = 0, hi = count;   // invariant: start[lo] <= t < start[hi]
        while (hi - lo > 1) {
            const uint32_t mid = (lo + hi) >> 1;
            if (start[mid] <= t) lo = mid; else hi = mid;
        }
        const DecompressJob &job = jobs[lo];
        ApplyPlan p;
        p.w = nullptr;
        p.rec = nullptr;
        p.desc = 0;
        p.len_room = 0;
        p.job = lo;
        p.block = 0;
        const DecompressState &st = state[lo];
        if (st.state == kStateReady) {
            const uint64_t b = t - job.block0;
            const uint64_t D = st.hdr + 4 * job.nb + offsets[t];
            const uint64_t room = job.payload_bytes - D;   // prepare checked D <= payload_bytes
            if (block_map) {   // a prepared remap: the block's place, looked up once
                p.w = (BF16D_GMEM uint16_t *)(uintptr_t)block_map[t];
            } else if (job.nsegs == 0) {
                p.w = job.weights + b * kBlock;
            } else {   // the segment holding block b (segments are block-aligned)
                const uint64_t e = b * kBlock;
                uint32_t slo = 0, shi = job.nsegs;   // segs[slo].first <= e < segs[shi].first
                while (shi - slo > 1) {
                    const uint32_t mid = (slo + shi) >> 1;
                    if (job.segs[mid].first <= e) slo = mid; else shi = mid;
                }
                p.w = job.segs[slo].dst + (e - job.segs[slo].first);
            }
            p.rec = job.payload + D;
            p.desc = *reinterpret_cast<BF16D_GMEM const uint32_t *>(job.payload + st.hdr + 4 * b);
            p.len_room = block_length(job.n, b) |
                         (uint32_t)(room < kRoomCap ? room : kRoomCap) << 14 |
                         (st.ow ? kPlanOverwrite | (st.undo ? kPlanUndo : 0u)
                                : (job.verify_first ? kPlanVerifyFirst : 0u));
            p.block = (uint32_t)b;
        }
        plan[t] = p;
    }
}

// -------------------------------------------------------------------- apply ---
// The first kStageChunks 16-byte words of the record window (which starts at
// the 16-byte boundary at or before the record) are staged in LDS, one load
// per thread; fields beyond are read from HBM (only dense blocks have such
// long records).
constexpr uint32_t kStageChunks = 244;   // LDS: 16 KiB tile + 3904 + 192 = 20 KiB, 8 workgroups per CU
constexpr uint32_t kStageWords = 4 * kStageChunks;

// Bit reader over a record: window dwords [0, kStageWords - 1) come from LDS,
// later ones from the payload in global memory.
struct RecordBits {
    const uint32_t *lds;        // staged dwords; window byte 0 = win[0]
    BF16D_GMEM const uint8_t *win;   // 16-byte aligned start of the window
    uint32_t room;              // payload bytes from win[0] to the end (capped)
    uint32_t rb0;               // window bit of record bit 0

    __device__ __forceinline__ uint32_t get(uint32_t bitpos, uint32_t width) const {
        const uint32_t wb = rb0 + bitpos;
        const uint32_t d = wb >> 5, sh = wb & 31;
        uint64_t v;
        if (d + 1 < kStageWords) {
            v = (uint64_t)lds[d] | ((uint64_t)lds[d + 1] << 32);
        } else {
            v = 0;
            const uint32_t at = 4 * d;
            for (uint32_t t = 0; t < 8; ++t)
                if (at + t < room) v |= (uint64_t)win[at + t] << (8 * t);
        }
        const uint64_t mask = (width >= 32) ? 0xFFFFFFFFull : ((1ull << width) - 1);
        return (uint32_t)((v >> sh) & mask);
    }

    // `width` (<= 32) bits at `bitpos` of a record that lies wholly in the
    // staged window.
    __device__ __forceinline__ uint32_t get_staged(uint32_t bitpos, uint32_t width) const {
        const uint32_t wb = rb0 + bitpos;
        const uint32_t d = wb >> 5;
        const uint32_t v = __builtin_amdgcn_alignbit(lds[d + 1], lds[d], wb & 31);
        return width >= 32 ? v : v & ((1u << width) - 1);
    }
};

// Bits [pos, pos + 32) of the 96-bit little-endian window w0 | w1 | w2
// (pos < 96; bits past the window read as zero).
__device__ __forceinline__ uint32_t window_bits(uint32_t w0, uint32_t w1, uint32_t w2,
                                                uint32_t pos) {
    if (pos < 32) return __builtin_amdgcn_alignbit(w1, w0, pos);
    if (pos < 64) return __builtin_amdgcn_alignbit(w2, w1, pos - 32);
    return w2 >> (pos - 64);
}

struct ApplyShared {
    uint32_t a[kWaves], b[kWaves], c[kWaves], f[kWaves];
    uint32_t dirty[kChunks / 32];   // sparse tiles: one bit per 16-byte chunk with a change
};

// OR of `v` over the workgroup; also a barrier.  (The library's
// __syncthreads_or would take 256 more bytes of LDS.)
__device__ __forceinline__ uint32_t block_any(uint32_t v, ApplyShared &sa, uint32_t tid) {
    const uint32_t lane = tid & 63, wave = tid >> 6;
    const uint32_t any = __ballot(v != 0) != 0;
    if (lane == 0) sa.f[wave] = any;
    __syncthreads();
    uint32_t out = 0;
#pragma unroll
    for (uint32_t w = 0; w < kWaves; ++w) out |= sa.f[w];
    return out;
}

struct TileGeom {
    uint32_t L, c, r, code, pb, mb, len, lead;
    bool stage;   // this thread stages a 16-byte word of the record window
};

__device__ __forceinline__ TileGeom tile_geom(const ApplyPlan &pe, uint32_t tid) {
    TileGeom g;
    g.L = pe.len_room & 0x3FFFu;
    g.c = pe.desc & 0x3FFFu;
    g.r = (pe.desc >> 14) & 0x3FFFu;
    g.code = pe.desc >> 28;
    g.pb = g.code == kCodeBitmap ? (g.L + 7) / 8 : (g.c * g.code + 7) / 8;
    g.mb = (pe.len_room & kPlanOverwrite) ? 0u : (7 * g.c + 7) / 8;   // overwrite: none
    g.len = g.pb + g.mb + 2 * g.r;
    g.lead = (uint32_t)((uintptr_t)pe.rec & 15);
    g.stage = tid < kStageChunks && 16 * tid < g.lead + g.len;
    return g;
}

// This thread's 16-byte word of a tile's record window.  Every thread loads,
// at an offset clamped to the record's last word and to the last 16 bytes
// that lie wholly inside the payload, under uniform branches only, so that
// the wait before the decode can leave the later weight loads in flight.
// fix_record_word then redoes, byte by byte, the one word that crosses the
// payload's end.
__device__ __forceinline__ uint4 load_record_word(const ApplyPlan &pe, uint32_t tid) {
    const TileGeom g = tile_geom(pe, tid);
    const uint32_t room = g.lead + ((pe.len_room >> 14) & kRoomCap);
    if (g.L == 0 || g.len == 0 || room < 16) return make_uint4(0, 0, 0, 0);
    // threads past the record reload its last word (the same cache line), so
    // the window costs no HBM traffic beyond the record
    const uint32_t last = ((g.lead + g.len + 15) & ~15u) - 16;
    const uint32_t lim0 = (room & ~15u) - 16;
    const uint32_t lim = last < lim0 ? last : lim0;
    const uint32_t off = 16 * tid < lim ? 16 * tid : lim;
    return *reinterpret_cast<BF16D_GMEM const uint4 *>(pe.rec - g.lead + off);
}

__device__ __forceinline__ uint4 fix_record_word(const ApplyPlan &pe, uint4 rv, uint32_t tid) {
    const TileGeom g = tile_geom(pe, tid);
    const uint32_t room = g.lead + ((pe.len_room >> 14) & kRoomCap);
    if (g.L == 0 || !g.stage || 16 * tid + 16 <= room) return rv;
    BF16D_GMEM const uint8_t *win = pe.rec - g.lead;
    uint32_t w[4] = {0, 0, 0, 0};
    for (uint32_t t = 0; t < 16; ++t)
        if (16 * tid + t < room) w[t >> 2] |= (uint32_t)win[16 * tid + t] << (8 * (t & 3));
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// This thread's 4 chunks of old weights.  kFull (a whole block): four
// unconditional 16-byte loads; otherwise (the short last block of a tensor)
// element by element up to L, zero beyond.
template <bool kFull>
__device__ __forceinline__ void load_old(const ApplyPlan &pe, uint4 (&o)[kChunksPerThread],
                                         uint32_t tid) {
    const uint32_t L = pe.len_room & 0x3FFFu;
#pragma unroll
    for (uint32_t i = 0; i < kChunksPerThread; ++i) {
        const uint32_t e0 = 8 * (tid + kThreads * i);
        if (kFull) {
            o[i] = *reinterpret_cast<BF16D_GMEM const uint4 *>(pe.w + e0);
        } else {
            o[i] = make_uint4(0, 0, 0, 0);
            if (e0 < L) o[i] = load_chunk(pe.w + e0, L - e0);
        }
    }
}

__device__ __forceinline__ void stage_record_word(const ApplyPlan &pe, uint4 rv, uint32_t *s_raw,
                                                  uint32_t tid) {
    if (tile_geom(pe, tid).stage) reinterpret_cast<uint4 *>(s_raw)[tid] = rv;
}

// Gap-list decode of a block with at most kFastFields fields per thread
// whose record lies wholly in the staged window: thread t owns fields
// [t*F, t*F + F), reads them from one window of three (gaps) and two
// (mantissas) LDS dwords, keeps them in registers, and writes the XOR of
// every changed element into s_x.  Up to 256 fields, wave 0 does it alone
// (lane t owns [t*F, t*F + F)).  Returns this thread's share of `bad`.
// kOw (an overwrite record): no mantissa fields; every change takes the next
// word, its new value, which goes to s_x as it is.
constexpr uint32_t kFastFields = 4;

//   kDirect: each value is stored straight to its weight (the commit of a
//   verified overwrite record) instead of into s_x.
//   sparse: the tile was not cleared beforehand (a tile of at most 256
//   changes, decoded by wave 0 alone): the wave first zeroes the chunks its
//   positions fall in and marks them in sa.dirty, then stores the values.
//   Within the wave the zeroing stores all come before the value stores, so
//   two positions in one chunk are safe.
//   kUndo (overwrite records): 1 = keep each replaced value (the tile holds
//   the old weights) in undo[j] before the new one goes in; 2 = write undo[j]
//   back (with kDirect: the restore of a failed in-place overwrite).
template <bool kOw, bool kDirect, int kUndo = 0>
__device__ __forceinline__ uint32_t decode_delta_fast(const RecordBits &rb, uint32_t c,
                                                      uint32_t r, uint32_t w, uint32_t L,
                                                      uint32_t mant0, uint32_t rare0,
                                                      uint16_t *s_x, ApplyShared &sa,
                                                      uint32_t tid, BF16D_GMEM uint16_t *wts,
                                                      bool sparse = false,
                                                      BF16D_GMEM uint16_t *undo = nullptr) {
    const uint32_t lane = tid & 63, wave = tid >> 6;
    // A sparse block (at most 256 fields) is decoded by wave 0 alone: its
    // scans stay within the wave, with no exchange of totals between waves
    // and no barrier; the other waves have nothing to do here.
    const bool one = c <= 64 * kFastFields;   // uniform
    if (one && wave != 0) return 0;
    const uint32_t idx = one ? lane : tid, n_threads = one ? 64u : kThreads;
    const uint32_t F = (c + n_threads - 1) / n_threads;
    const uint32_t jb = idx * F < c ? idx * F : c;
    const uint32_t nf = (jb + F < c ? jb + F : c) - jb;
    uint32_t g0 = 0, g1 = 0, g2 = 0, m0 = 0, m1 = 0, gsh = 0, msh = 0;
    if (nf) {
        const uint32_t gb = rb.rb0 + jb * w, mb = rb.rb0 + mant0 + 7 * jb;
        const uint32_t gd = gb >> 5, md = mb >> 5;
        gsh = gb & 31;
        msh = mb & 31;
        g0 = rb.lds[gd];
        g1 = rb.lds[gd + 1];
        g2 = rb.lds[gd + 2];
        if (!kOw) {
            m0 = rb.lds[md];
            m1 = rb.lds[md + 1];
        }
    }
    const uint32_t gmask = (1u << w) - 1;
    uint32_t gk[kFastFields], mk[kFastFields];
    uint32_t sum_g1 = 0, esc = 0, top = 0;
#pragma unroll
    for (uint32_t k = 0; k < kFastFields; ++k) {
        gk[k] = window_bits(g0, g1, g2, gsh + k * w) & gmask;
        const uint32_t mp = msh + 7 * k;
        mk[k] = kOw ? 0u : (mp < 32 ? __builtin_amdgcn_alignbit(m1, m0, mp) : m1 >> (mp - 32)) &
                               kMant;
        if (k < nf) {
            sum_g1 += gk[k] + 1;
            esc += mk[k] == 0;
            top |= w ? gk[k] >> (w - 1) : 1u;   // the field uses its top bit
        }
    }
    // escapes before this lane (esc <= 4): by bit planes of ballots
    const uint64_t e1 = __ballot(esc & 1), e2 = __ballot(esc & 2), e4 = __ballot(esc & 4);
    const uint64_t below = (1ull << lane) - 1;
    const uint32_t e_lane = __popcll(e1 & below) + 2 * __popcll(e2 & below) +
                            4 * __popcll(e4 & below);
    const uint32_t e_wave = __popcll(e1) + 2 * __popcll(e2) + 4 * __popcll(e4);
    const uint32_t inc_g = wave_incl_add(sum_g1);
    const uint32_t top_wave = __ballot(top) != 0;
    const uint32_t tot_g = lane63(inc_g);   // outside the branch below: see lane63
    uint32_t run = inc_g - sum_g1, e = e_lane;
    uint32_t total_g1 = tot_g, esc_total = e_wave, any_top = top_wave;
    if (!one) {   // every wave has fields: add up the waves' totals
        if (lane == 0) {
            sa.a[wave] = tot_g;
            sa.b[wave] = e_wave;
            sa.c[wave] = top_wave;
        }
        __syncthreads();
        total_g1 = esc_total = any_top = 0;
#pragma unroll
        for (uint32_t w2 = 0; w2 < kWaves; ++w2) {
            if (w2 < wave) {
                run += sa.a[w2];
                e += sa.b[w2];
            }
            total_g1 += sa.a[w2];
            esc_total += sa.b[w2];
            any_top |= sa.c[w2];
        }
    }
    uint32_t bad = (total_g1 - 1 >= L) | (esc_total != r) | (any_top == 0);
    if (sparse) {   // uniform; only with `one`, so all of this is wave 0's
        uint32_t r2 = run;
#pragma unroll
        for (uint32_t k = 0; k < kFastFields; ++k) {
            if (k < nf) {
                r2 += gk[k] + 1;
                const uint32_t p = r2 - 1;
                if (p < L) {
                    reinterpret_cast<uint4 *>(s_x)[p >> 3] = make_uint4(0, 0, 0, 0);
                    atomicOr(&sa.dirty[p >> 8], 1u << ((p >> 3) & 31));
                }
            }
        }
    }
#pragma unroll
    for (uint32_t k = 0; k < kFastFields; ++k) {
        if (k < nf) {
            run += gk[k] + 1;
            const uint32_t p = run - 1;
            uint32_t x = mk[k];
            if (x == 0) {
                if (e < r) {
                    x = rb.get_staged(rare0 + 16 * e, 16);
                    if (!kOw) bad |= (x & kExpSign) == 0;
                } else {
                    bad = 1;
                }
                ++e;
            }
            if (p >= L) {
                bad = 1;
            } else if (kDirect) {
                wts[p] = kUndo == 2 ? undo[jb + k] : (uint16_t)x;
            } else {
                if (kUndo == 1) undo[jb + k] = s_x[p];
                s_x[p] = (uint16_t)x;
            }
        }
    }
    return bad;
}

// Decode one tile and XOR it onto the weights.
//   On entry: s_x is all zero and s_raw holds this tile's record window; both
//   were written before this call by this workgroup, and this call's first
//   barrier makes them visible.  On return s_x is all zero again.
//   `next` / `rv_next`: the following tile and this thread's word of its
//   record window, loaded by the caller before this call so that its latency
//   overlaps the decode; it is written to s_raw once this tile's record has
//   been read.
//   kPass: kPassApply (XOR, store, checksum), kPassRollback (XOR again, store,
//   no checksum), kPassVerify (overwrite record: checksum of the result, no
//   store), kPassCommit (overwrite record: store, no checksum),
//   kPassVerifyXor (XOR record, verified first: checksum of old ^ mask, no
//   store), kPassCommitXor (a verified XOR record: each changed chunk's old
//   value loaded only now, XOR, store; no checksum).
//   kPassOwUndo (overwrite record, in place: each replaced value kept in the
//   undo area, result stored and summed), kPassOwRestore (a failed in-place
//   overwrite: the kept values written back; no checksum).
enum : int {
    kPassApply = 0, kPassRollback = 1, kPassVerify = 2, kPassCommit = 3, kPassVerifyXor = 4,
    kPassCommitXor = 5, kPassOwUndo = 6, kPassOwRestore = 7
};

// A tile of at most 256 changes in a gap list that lies wholly in the staged
// window: wave 0 decodes it alone.  In the one-tile-per-workgroup passes it
// is also `sparse`: its LDS tile is not cleared and read back whole, only
// the chunks with changes (marked in a bitmap) are.
__device__ __forceinline__ bool sparse_tile(const TileGeom &g) {
    return g.code != kCodeBitmap && g.c != 0 && g.c <= 64 * kFastFields &&
           g.lead + g.len + 12 <= 4 * kStageWords;
}

//   kSparseOk: the tile is not reused after this call (one tile per
//   workgroup), so a sparse tile may leave s_x dirty.
template <int kPass, bool kSparseOk = false>
__device__ __forceinline__ void finish_tile(const ApplyPlan &pe, const uint4 (&o)[kChunksPerThread],
                                            uint64_t tile, const ApplyPlan &next, uint4 rv_next,
                                            DecompressState *__restrict__ state,
                                            uint64_t *__restrict__ partial, uint16_t *s_x,
                                            uint32_t *s_raw, ApplyShared &sa, uint32_t tid) {
    constexpr bool kOw = kPass == kPassVerify || kPass == kPassCommit || kPass == kPassOwUndo ||
                         kPass == kPassOwRestore;
    constexpr bool kSum = kPass == kPassApply || kPass == kPassVerify || kPass == kPassVerifyXor ||
                          kPass == kPassOwUndo;
    constexpr bool kStore = kPass != kPassVerify && kPass != kPassVerifyXor;
    // a verified XOR record's commit reads only the changed chunks' old values
    constexpr bool kLateOld = kPass == kPassCommitXor;
    // the commit writes each verified value at its position, and the restore
    // each kept value: absolute values need neither the old weights nor the
    // tile
    constexpr bool kDirect = kPass == kPassCommit || kPass == kPassOwRestore;
    constexpr int kUndo = kPass == kPassOwUndo ? 1 : (kPass == kPassOwRestore ? 2 : 0);
    const uint32_t lane = tid & 63, wave = tid >> 6;
    const TileGeom g = tile_geom(pe, tid);
    const uint32_t L = g.L, c = g.c, r = g.r, code = g.code, pb = g.pb, mb = g.mb;
    const bool sparse = kSparseOk && !kOw && sparse_tile(g);   // uniform
    // the tile's undo range: its record's offset within the job's records,
    // in the job's undo area (made even: ranges of neighbouring tiles still
    // do not overlap, as a record of c changes is at least 2c bytes)
    BF16D_GMEM uint16_t *undo = nullptr;
    if (kUndo)
        undo = (BF16D_GMEM uint16_t *)(((uintptr_t)pe.rec + state[pe.job].undo_delta) &
                                       ~(uintptr_t)1);

    RecordBits rb;
    rb.lds = s_raw;
    rb.win = pe.rec - g.lead;
    rb.room = g.lead + ((pe.len_room >> 14) & kRoomCap);
    rb.rb0 = 8 * g.lead;

    // ---- decode the record into s_x, checking that it is canonical ----
    // A block without changes has an empty record (its descriptor was
    // checked): nothing to decode and nothing to write.
    const bool changed = c != 0;
    const uint32_t mant0 = 8 * pb, rare0 = 8 * (pb + mb);
    uint32_t bad = 0;
    if (changed) {
        // overwrite: the tile starts as the current weights, and the decode
        // writes the new values over them
        if (kOw && !kDirect) {
#pragma unroll
            for (uint32_t i = 0; i < kChunksPerThread; ++i)
                reinterpret_cast<uint4 *>(s_x)[tid + kThreads * i] = o[i];
        }
        __syncthreads();   // record staged; s_x clear (overwrite: s_x = the weights)
        if (code != kCodeBitmap && c <= kFastFields * kThreads &&
            g.lead + g.len + 12 <= 4 * kStageWords) {
            bad = decode_delta_fast<kOw, kDirect, kUndo>(rb, c, r, code, L, mant0, rare0, s_x,
                                                         sa, tid, pe.w, sparse, undo);
            if (tid == 0 && 8 * pb > c * code)               // position padding
                bad |= rb.get(c * code, 8 * pb - c * code) != 0;
        } else if (code == kCodeBitmap) {
            // thread t owns bitmap bits [32t, 32t + 32) = elements 32t .. 32t+31
            const uint32_t lo = 32 * tid, seg_end = 8 * pb;
            uint32_t word = 0;
            if (lo < seg_end) {
                word = rb.get(lo, 32);
                if (lo + 32 > seg_end) word &= (1u << (seg_end - lo)) - 1;
            }
            const uint32_t valid_mask =
                lo + 32 <= L ? 0xFFFFFFFFu : (lo >= L ? 0u : (1u << (L - lo)) - 1);
            bad |= (word & ~valid_mask) != 0;               // pad bits must be zero
            word &= valid_mask;
            const uint32_t pop = __popc(word);
            const uint32_t last1 = word ? lo + 32 - __clz(word) : 0;   // last position + 1
            const uint32_t inc_pop = wave_incl_add(pop), inc_last = wave_incl_max(last1);
            const uint32_t tot_pop = lane63(inc_pop), tot_last = lane63(inc_last);
            if (lane == 0) {
                sa.a[wave] = tot_pop;
                sa.b[wave] = tot_last;
            }
            __syncthreads();
            uint32_t rank0 = inc_pop - pop, prev1 = wave_shr1(inc_last), total = 0;
            for (uint32_t w2 = 0; w2 < kWaves; ++w2) {
                if (w2 < wave) {
                    rank0 += sa.a[w2];
                    prev1 = umax32(prev1, sa.b[w2]);
                }
                total += sa.a[w2];
            }
            bad |= total != c;
            // gaps before each set bit, and the escapes among this thread's fields
            uint32_t maxg = 0, esc = 0;
            {
                uint32_t bits = word, jj = rank0, p1 = prev1;
                while (bits) {
                    const uint32_t p = lo + __ffs(bits) - 1;
                    bits &= bits - 1;
                    maxg = umax32(maxg, p - p1);
                    p1 = p + 1;
                    esc += kOw ? 1u : (rb.get(mant0 + 7 * jj, 7) == 0);
                    ++jj;
                }
            }
            const uint32_t inc_esc = wave_incl_add(esc), wmax = lane63(wave_incl_max(maxg));
            const uint32_t tot_esc = lane63(inc_esc);
            __syncthreads();   // sa.a / sa.b reads done
            if (lane == 0) {
                sa.a[wave] = tot_esc;
                sa.c[wave] = wmax;
            }
            __syncthreads();
            uint32_t e = inc_esc - esc, esc_total = 0;
            maxg = 0;
            for (uint32_t w2 = 0; w2 < kWaves; ++w2) {
                if (w2 < wave) e += sa.a[w2];
                esc_total += sa.a[w2];
                maxg = umax32(maxg, sa.c[w2]);
            }
            bad |= esc_total != r;
            bad |= !(pb < (c * bit_length(maxg) + 7) / 8);   // a bitmap only when smaller
            uint32_t bits = word, jj = rank0;
            while (bits) {
                const uint32_t p = lo + __ffs(bits) - 1;
                bits &= bits - 1;
                uint32_t x = kOw ? 0u : rb.get(mant0 + 7 * jj, 7);
                if (x == 0) {
                    if (e < r) {
                        x = rb.get(rare0 + 16 * e, 16);
                        if (!kOw) bad |= (x & kExpSign) == 0;
                    } else {
                        bad = 1;
                    }
                    ++e;
                }
                // a malformed bitmap may set more than c bits: the undo range
                // of the tile holds c entries, so ranks from c on are not kept
                // (nothing of a malformed block is stored) nor restored
                if (kDirect) {
                    if (kUndo != 2)
                        pe.w[p] = (uint16_t)x;
                    else if (jj < c)
                        pe.w[p] = undo[jj];
                } else {
                    if (kUndo == 1 && jj < c) undo[jj] = s_x[p];
                    s_x[p] = (uint16_t)x;
                }
                ++jj;
            }
        } else {
            // gap list of width w: thread t owns fields [t*F, t*F + F)
            const uint32_t w = code;
            const uint32_t F = (c + kThreads - 1) / kThreads;
            const uint32_t jb = tid * F < c ? tid * F : c;
            const uint32_t je = jb + F < c ? jb + F : c;
            uint32_t sum_g1 = 0, esc = 0, maxg = 0;
            for (uint32_t jj = jb; jj < je; ++jj) {
                const uint32_t g = w ? rb.get(jj * w, w) : 0;
                sum_g1 += g + 1;
                maxg = umax32(maxg, g);
                esc += kOw ? 1u : (rb.get(mant0 + 7 * jj, 7) == 0);
            }
            const uint32_t inc_g = wave_incl_add(sum_g1), inc_e = wave_incl_add(esc);
            const uint32_t wmax = lane63(wave_incl_max(maxg));
            const uint32_t tot_g = lane63(inc_g), tot_e = lane63(inc_e);
            if (lane == 0) {
                sa.a[wave] = tot_g;
                sa.b[wave] = tot_e;
                sa.c[wave] = wmax;
            }
            __syncthreads();
            uint32_t run = inc_g - sum_g1, e = inc_e - esc;
            uint32_t total_g1 = 0, esc_total = 0;
            maxg = 0;
            for (uint32_t w2 = 0; w2 < kWaves; ++w2) {
                if (w2 < wave) {
                    run += sa.a[w2];
                    e += sa.b[w2];
                }
                total_g1 += sa.a[w2];
                esc_total += sa.b[w2];
                maxg = umax32(maxg, sa.c[w2]);
            }
            bad |= (c > 0) && (total_g1 - 1 >= L);          // last position inside the block
            bad |= esc_total != r;
            bad |= bit_length(maxg) != w;                    // width is minimal
            for (uint32_t jj = jb; jj < je; ++jj) {
                const uint32_t g = w ? rb.get(jj * w, w) : 0;
                run += g + 1;
                const uint32_t p = run - 1;
                uint32_t x = kOw ? 0u : rb.get(mant0 + 7 * jj, 7);
                if (x == 0) {
                    if (e < r) {
                        x = rb.get(rare0 + 16 * e, 16);
                        if (!kOw) bad |= (x & kExpSign) == 0;
                    } else {
                        bad = 1;
                    }
                    ++e;
                }
                if (p >= L) {
                    bad = 1;
                } else if (kDirect) {
                    pe.w[p] = kUndo == 2 ? undo[jj] : (uint16_t)x;
                } else {
                    if (kUndo == 1) undo[jj] = s_x[p];
                    s_x[p] = (uint16_t)x;
                }
            }
            if (tid == 0 && 8 * pb > c * w)                  // position padding
                bad |= rb.get(c * w, 8 * pb - c * w) != 0;
        }
        if (tid == 0 && 8 * mb > 7 * c)                      // mantissa padding
            bad |= rb.get(mant0 + 7 * c, 8 * mb - 7 * c) != 0;
        bad = block_any(bad, sa, tid);   // s_x complete; every read of s_raw done
    }
    stage_record_word(next, rv_next, s_raw, tid);
    if (kDirect) return;   // the values are written; the tile was not used

    // ---- new = old ^ tile; store only changed chunks; clear the tile ----
    uint64_t acc = 0;
    uint64_t kg = (((uint64_t)pe.block * kBlock >> 2) + 1 + 2 * tid) * kGamma;
    // per-round key step and G as opaque uniform values: kept in SGPRs rather
    // than folded into per-chunk 64-bit constants held in VGPRs
    uint64_t round_kg = (uint64_t)(2 * kThreads) * kGamma, gamma = kGamma;
    asm volatile("" : "+s"(round_kg), "+s"(gamma));
#pragma unroll
    for (uint32_t i = 0; i < kChunksPerThread; ++i) {
        const uint32_t q = tid + kThreads * i;
        const uint32_t e0 = 8 * q;
        const uint32_t valid = e0 < L ? (L - e0 < 8 ? L - e0 : 8) : 0;
        uint4 nw = o[i];
        if (kOw) {   // the tile holds the result itself
            const uint4 t = changed ? reinterpret_cast<const uint4 *>(s_x)[q] : nw;
            const bool dirty = ((t.x ^ nw.x) | (t.y ^ nw.y) | (t.z ^ nw.z) | (t.w ^ nw.w)) != 0;
            if (changed) reinterpret_cast<uint4 *>(s_x)[q] = make_uint4(0, 0, 0, 0);
            if (dirty && !bad) {
                nw = t;
                BF16D_GMEM uint16_t *dstp = pe.w + e0;
                if (!kStore) {
                    // verify: the result is only summed
                } else if (valid == 8) {
                    *reinterpret_cast<BF16D_GMEM uint4 *>(dstp) = nw;
                } else {
                    for (uint32_t s = 0; s < valid; ++s) dstp[s] = (uint16_t)chunk_elem(nw, s);
                }
            }
        } else if (const uint4 t = (changed && (!sparse || ((sa.dirty[q >> 5] >> (q & 31)) & 1u)))
                                       ? reinterpret_cast<const uint4 *>(s_x)[q]
                                       : make_uint4(0, 0, 0, 0);
                   (t.x | t.y | t.z | t.w) != 0) {   // dirty
            if (!kSparseOk) {
                // tid >> 16 is 0; written so the zero is not one more
                // register held across the persistent loop
                const uint32_t z = tid >> 16;
                reinterpret_cast<uint4 *>(s_x)[q] = make_uint4(z, z, z, z);
            }
            if (!bad) {
                BF16D_GMEM uint16_t *dstp = pe.w + e0;
                if (kLateOld) nw = load_chunk(dstp, valid);
                nw = make_uint4(nw.x ^ t.x, nw.y ^ t.y, nw.z ^ t.z, nw.w ^ t.w);
                if (!kStore) {
                    // verified first: the result is only summed
                } else if (valid == 8) {
                    *reinterpret_cast<BF16D_GMEM uint4 *>(dstp) = nw;
                } else {
                    for (uint32_t s = 0; s < valid; ++s) dstp[s] = (uint16_t)chunk_elem(nw, s);
                }
            }
        }
        if (kSum) {
            if (valid > 0) acc += mix64(((uint64_t)nw.y << 32 | nw.x) ^ kg);
            if (valid > 4) acc += mix64(((uint64_t)nw.w << 32 | nw.z) ^ (kg + gamma));
            kg += round_kg;
        }
    }
    if (kSum) {
        acc = first_lane(wave_sum(acc));
        if (lane == 0) partial[kWaves * tile + wave] = acc;
        if (tid == 0 && bad) atomicOr(&state[pe.job].block_bad, 1u);
    }
}

// One step of the persistent pass: tile `pc` (its record already staged in
// s_raw) from its weight loads to its stores, with the next tile's record
// word loaded meanwhile.  Whole blocks and the short last block of a tensor
// are compiled separately (see load_old).
template <int kPass, bool kFull>
__device__ __forceinline__ void pass_step(const ApplyPlan &pc, const ApplyPlan &pn, uint64_t t,
                                          DecompressState *__restrict__ state,
                                          uint64_t *__restrict__ partial, uint16_t *s_x,
                                          uint32_t *s_raw, ApplyShared &sa, uint32_t tid) {
    uint4 o[kChunksPerThread];
    if (kPass == kPassCommit || kPass == kPassOwRestore) {   // writes values only: the
                                                             // old weights are not read
#pragma unroll
        for (uint32_t i = 0; i < kChunksPerThread; ++i) o[i] = make_uint4(0, 0, 0, 0);
    } else {
        load_old<kFull>(pc, o, tid);
    }
    const uint4 rv_next = fix_record_word(pn, load_record_word(pn, tid), tid);
    finish_tile<kPass>(pc, o, t, pn, rv_next, state, partial, s_x, s_raw, sa, tid);
}

// A persistent pass over the tiles (rollback and commit); workgroup g takes tiles
// g, g + G, g + 2G, ...  While a tile is decoded, its old weights and the next tile's
// record word are in flight, and the plan entry of the tile after that has
// been requested; the next tile's record is staged in LDS as soon as this
// one's has been read, so its decode can start at once.  LDS is kept at
// 20 KiB so that 8 workgroups (8 waves per SIMD) fit on a CU.
// It visits the tiles of jobs marked for rollback (an XOR pass again, or, for
// an overwrite payload applied in place, the replaced values written back
// from the undo area) and of overwrite jobs that passed verification (their
// values written); the tile's plan entry says which.
__device__ __forceinline__ void fixup_pass(const ApplyPlan *__restrict__ plan,
                                           DecompressState *__restrict__ state,
                                           uint64_t *__restrict__ partial, uint64_t tiles) {
    __shared__ __attribute__((aligned(16))) uint16_t s_x[kBlock];        // dense XOR tile
    __shared__ __attribute__((aligned(16))) uint32_t s_raw[kStageWords];  // staged record
    __shared__ ApplyShared sa;
    const uint64_t G = gridDim.x;
    uint64_t t = blockIdx.x;
    if (t >= tiles) return;
    ApplyPlan none;
    none.w = nullptr;
    none.rec = nullptr;
    none.desc = none.len_room = none.job = none.block = 0;
    auto fetch = [&](uint64_t u) -> ApplyPlan {
        if (u >= tiles) return none;
        ApplyPlan p = plan[u];
        // XOR records verified first are committed by commit_kernel (the
        // same bit on an overwrite record means an in-place one: restored here)
        if ((p.len_room & (kPlanOverwrite | kPlanVerifyFirst)) == kPlanVerifyFirst) return none;
        if (p.len_room & 0x3FFFu) {
            const DecompressState &st = state[p.job];
            if ((st.rollback | st.commit) == 0) p = none;
        }
        return p;
    };
    for (uint32_t u = threadIdx.x; u < kBlock / 8; u += kThreads)
        reinterpret_cast<uint4 *>(s_x)[u] = make_uint4(0, 0, 0, 0);
    ApplyPlan pc = fetch(t);
    ApplyPlan pn = fetch(t + G);
    {
        const uint32_t tid = threadIdx.x;
        stage_record_word(pc, fix_record_word(pc, load_record_word(pc, tid), tid), s_raw, tid);
    }
    for (;;) {
        // the thread index, opaque to the optimiser once per tile: values
        // derived from it are recomputed per tile instead of being hoisted
        // out of the loop and held in registers
        uint32_t tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const ApplyPlan pnn = fetch(t + 2 * G);
        const uint32_t L = pc.len_room & 0x3FFFu;
        const bool ow = (pc.len_room & kPlanOverwrite) != 0;
        if (L != 0 && ow && (pc.len_room & kPlanUndo))   // a failed in-place overwrite
            pass_step<kPassOwRestore, true>(pc, pn, t, state, partial, s_x, s_raw, sa, tid);
        else if (L == kBlock && ow)
            pass_step<kPassCommit, true>(pc, pn, t, state, partial, s_x, s_raw, sa, tid);
        else if (L == kBlock)
            pass_step<kPassRollback, true>(pc, pn, t, state, partial, s_x, s_raw, sa, tid);
        else if (L != 0 && ow)
            pass_step<kPassCommit, false>(pc, pn, t, state, partial, s_x, s_raw, sa, tid);
        else if (L != 0)
            pass_step<kPassRollback, false>(pc, pn, t, state, partial, s_x, s_raw, sa, tid);
        else   // a skipped tile: nothing reads its record
            stage_record_word(pn, fix_record_word(pn, load_record_word(pn, tid), tid), s_raw, tid);
        t += G;
        if (t >= tiles) break;
        pc = pn;
        pn = pnn;
    }
}

// One tile of the apply pass, from its loads to its stores.  Whole blocks
// and the short last block of a tensor are compiled separately (see
// load_old), so that the wave waits only for the record word before the
// decode while the weight loads stay in flight.
//   kPass: kPassApply, kPassVerify (overwrite record), kPassVerifyXor or
//   kPassCommitXor (which reads no whole block: only the changed chunks,
//   once the record is decoded).
template <bool kFull, int kPass>
__device__ __forceinline__ void apply_one(const ApplyPlan &pe, uint64_t tile,
                                          DecompressState *__restrict__ state,
                                          uint64_t *__restrict__ partial, uint16_t *s_x,
                                          uint32_t *s_raw, ApplyShared &sa) {
    constexpr bool kOw = kPass == kPassVerify || kPass == kPassOwUndo;
    const uint32_t tid = threadIdx.x;
    uint4 rv = load_record_word(pe, tid);
    uint4 o[kChunksPerThread];
    if (kPass == kPassCommitXor) {
#pragma unroll
        for (uint32_t i = 0; i < kChunksPerThread; ++i) o[i] = make_uint4(0, 0, 0, 0);
    } else {
        load_old<kFull>(pe, o, tid);
    }
    rv = fix_record_word(pe, rv, tid);
    if (pe.desc & 0x3FFFu) {   // changed elements: the decode needs a clear tile
        if (!kOw) {   // (an overwrite tile is filled with the weights instead)
            if (sparse_tile(tile_geom(pe, tid))) {   // uniform: only its chunks, marked
                if (tid < kChunks / 32) sa.dirty[tid] = 0;
            } else {
                for (uint32_t u = tid; u < kBlock / 8; u += kThreads)
                    reinterpret_cast<uint4 *>(s_x)[u] = make_uint4(0, 0, 0, 0);
            }
        }
        stage_record_word(pe, rv, s_raw, tid);
    }
    ApplyPlan none;
    none.w = nullptr;
    none.rec = nullptr;
    none.desc = none.len_room = none.job = none.block = 0;
    finish_tile<kPass, true>(pe, o, tile, none, make_uint4(0, 0, 0, 0), state, partial, s_x,
                             s_raw, sa, tid);
}

// The apply pass: one workgroup per tile, 8 workgroups per CU (20 KiB of
// LDS).  Its plan entry is the only load before the record and the old
// weights are requested.  Variants that keep a workgroup for several tiles
// and fetch the next tile's record during the current decode (a persistent
// loop, or 2 and 3 tiles per workgroup) measured slower on the 7B-shaped
// checkpoint: the pass is bound by HBM traffic, not by the decode latency.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
void apply_kernel(const ApplyPlan *__restrict__ plan, DecompressState *__restrict__ state,
                  uint64_t *__restrict__ partial) {
    __shared__ __attribute__((aligned(16))) uint16_t s_x[kBlock];        // dense XOR tile
    __shared__ __attribute__((aligned(16))) uint32_t s_raw[kStageWords];  // staged record
    __shared__ ApplyShared sa;
    const uint64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const ApplyPlan pe = plan[tile];
    const uint32_t L = pe.len_room & 0x3FFFu;
    if ((pe.len_room & (kPlanOverwrite | kPlanUndo)) == (kPlanOverwrite | kPlanUndo)) {
        // overwrite records written in place, the replaced values kept
        if (L == kBlock)
            apply_one<true, kPassOwUndo>(pe, tile, state, partial, s_x, s_raw, sa);
        else if (L != 0)
            apply_one<false, kPassOwUndo>(pe, tile, state, partial, s_x, s_raw, sa);
    } else if (pe.len_room & kPlanOverwrite) {   // overwrite records: verified, written later
        if (L == kBlock)
            apply_one<true, kPassVerify>(pe, tile, state, partial, s_x, s_raw, sa);
        else if (L != 0)
            apply_one<false, kPassVerify>(pe, tile, state, partial, s_x, s_raw, sa);
    } else if (pe.len_room & kPlanVerifyFirst) {   // XOR records verified first
        if (L == kBlock)
            apply_one<true, kPassVerifyXor>(pe, tile, state, partial, s_x, s_raw, sa);
        else if (L != 0)
            apply_one<false, kPassVerifyXor>(pe, tile, state, partial, s_x, s_raw, sa);
    } else if (L == kBlock) {
        apply_one<true, kPassApply>(pe, tile, state, partial, s_x, s_raw, sa);
    } else if (L != 0) {   // 0: the job was rejected
        apply_one<false, kPassApply>(pe, tile, state, partial, s_x, s_raw, sa);
    }
}

// The second pass of a verify-first call: the XOR records of the jobs that
// passed, one workgroup per tile as in the apply pass (so that 8 workgroups
// per CU keep their changed chunks' loads in flight); each changed chunk's
// old value is read only now, XOR-ed and stored.  Exits at once when no job
// of the call passed.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
void commit_kernel(const ApplyPlan *__restrict__ plan, DecompressState *__restrict__ state,
                   const Control *__restrict__ ctrl) {
    __shared__ __attribute__((aligned(16))) uint16_t s_x[kBlock];        // dense XOR tile
    __shared__ __attribute__((aligned(16))) uint32_t s_raw[kStageWords];  // staged record
    __shared__ ApplyShared sa;
    if (ctrl->any_commit_xor == 0) return;
    const uint64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const ApplyPlan pe = plan[tile];
    if ((pe.len_room & (kPlanOverwrite | kPlanVerifyFirst)) != kPlanVerifyFirst ||
        (pe.len_room & 0x3FFFu) == 0)
        return;
    if (state[pe.job].commit == 0) return;   // uniform: the job failed, nothing is written
    apply_one<false, kPassCommitXor>(pe, tile, state, nullptr, s_x, s_raw, sa);
}

// After the finalize step: the rollback of failed XOR jobs (applying the same
// mask again restores the old weights exactly), the restore of failed
// overwrite jobs applied in place (from their undo area) and the writing of
// verified overwrite payloads, in one persistent pass that exits at once when
// there is none of these.  Absolute values cannot be undone by applying them
// twice, so without an undo area they are written only once the whole result
// is known to be right.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
void fixup_kernel(const ApplyPlan *__restrict__ plan, DecompressState *__restrict__ state,
                  const Control *__restrict__ ctrl, uint64_t tiles) {
    if ((ctrl->any_rollback | ctrl->any_commit) == 0) return;
    fixup_pass(plan, state, nullptr, tiles);
}

// ----------------------------------------------------------------- finalize ---
// Job j's checksum comparison, status and result.  The sums are read with
// device-scope loads: the checksum kernel's last workgroup runs this right
// after the other workgroups' atomics.
__device__ void finalize_job(const DecompressJob *__restrict__ jobs,
                             DecompressState *__restrict__ state,
                             const JobSums *__restrict__ sums, Control *__restrict__ ctrl,
                             bf16d_result *__restrict__ results, uint32_t j) {
    const DecompressJob job = jobs[j];
    DecompressState *st = &state[j];
    const bool ready = st->state == kStateReady;
    const unsigned long long S = ld_agent(&sums[j].csum);
    bf16d_result res;
    res.reserved = 0;
    res.payload_bytes = job.payload_bytes;
    if (!ready) {
        res.status = st->state == kStateVersion ? BF16D_EVERSION : BF16D_EFORMAT;
        res.checksum = 0;
        res.n_changed = res.n_rare = res.n_bitmap_blocks = 0;
    } else {
        const uint64_t cs = mix64(S ^ job.n);
        res.status = ld_agent(&st->block_bad) ? BF16D_EFORMAT
                                              : (cs != job.checksum ? BF16D_ECHECKSUM : BF16D_OK);
        res.checksum = cs;
        res.n_changed = st->sum_c;
        res.n_rare = st->sum_r;
        res.n_bitmap_blocks = st->n_bitmap;
        if (st->ow && st->undo) {
            // written in place: a failure restores the kept values
            if (res.status != BF16D_OK) {
                st->rollback = 1;
                atomicOr(&ctrl->any_rollback, 1u);
            }
        } else if (st->ow || job.verify_first) {
            // overwrite, or an XOR job verified first: nothing was written
            // yet; the fix-up pass (overwrite) or the commit pass (XOR)
            // writes it
            if (res.status == BF16D_OK) {
                st->commit = 1;
                atomicOr(st->ow ? &ctrl->any_commit : &ctrl->any_commit_xor, 1u);
            }
        } else if (res.status != BF16D_OK) {
            st->rollback = 1;
            atomicOr(&ctrl->any_rollback, 1u);
        }
        // the joint commit: the version word moves to the target with the weights
        if (res.status == BF16D_OK && st->bound && job.version)
            *job.version = reinterpret_cast<BF16D_GMEM const uint64_t *>(job.payload)[9];
    }
    results[j] = res;
}

// For calls without tiles; otherwise the checksum kernel's last workgroup
// finalizes the jobs.
__global__ __launch_bounds__(kThreads) void decompress_finalize_kernel(
    const DecompressJob *__restrict__ jobs, DecompressState *__restrict__ state,
    const JobSums *__restrict__ sums, Control *__restrict__ ctrl, uint32_t count,
    bf16d_result *__restrict__ results) {
    const uint32_t j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j < count) finalize_job(jobs, state, sums, ctrl, results, j);
}

// ------------------------------------------------------------- checksum sum ---
// The checksum sum S of every job that was applied: one workgroup per 2048
// blocks (the descriptor-scan tiles) sums its blocks' per-wave partials and
// adds them to the job's total with one atomic (exact mod 2^64 in any order).
// The last workgroup to finish then finalizes every job.
__global__ __launch_bounds__(kThreads) void sum_partials_kernel(
    const DecompressJob *__restrict__ jobs, const uint32_t *__restrict__ dtile_job,
    DecompressState *__restrict__ state, const uint64_t *__restrict__ partial,
    JobSums *__restrict__ sums, Control *__restrict__ ctrl, uint32_t count,
    bf16d_result *__restrict__ results) {
    __shared__ unsigned long long s_tmp[kWaves];
    const uint64_t dt = blockIdx.x;
    const uint32_t j = dtile_job[dt];
    uint64_t dep = 0;
    if (state[j].state == kStateReady) {   // uniform; otherwise nothing was applied
        const DecompressJob &job = jobs[j];
        const uint64_t ld = dt - job.dtile0;
        unsigned long long S = 0;
#pragma unroll
        for (uint32_t k = 0; k < kDescPerThread; ++k) {
            const uint64_t b = ld * kDescTile + kDescPerThread * threadIdx.x + k;
            if (b < job.nb)
#pragma unroll
                for (uint32_t w = 0; w < kWaves; ++w)
                    S += partial[kWaves * (job.block0 + b) + w];
        }
        S = block_sum(S, s_tmp);
        if (threadIdx.x == 0) dep = atomicAdd(&sums[j].csum, S);
    }
    if (last_workgroup(&ctrl->sum_done, dep))
        for (uint32_t jj = threadIdx.x; jj < count; jj += kThreads)
            finalize_job(jobs, state, sums, ctrl, results, jj);
}

hipError_t launch_decompress(const Layout &l, uint8_t *ws, uint32_t count, uint64_t tiles,
                             uint64_t dtiles, bf16d_result *results, hipStream_t stream,
                             const bf16d_events *events, const uint64_t *block_map,
                             bool verify_first) {
    auto *ctrl = reinterpret_cast<Control *>(ws + l.control);
    auto *jobs = reinterpret_cast<const DecompressJob *>(ws + l.jobs);
    auto *bstart = reinterpret_cast<const uint64_t *>(ws + l.block_start);
    auto *dstart = reinterpret_cast<const uint64_t *>(ws + l.dtile_start);
    auto *offsets = reinterpret_cast<uint64_t *>(ws + l.status);
    auto *partial = reinterpret_cast<uint64_t *>(ws + l.partial);
    auto *sums = reinterpret_cast<JobSums *>(ws + l.sums);
    auto *dmap = reinterpret_cast<uint32_t *>(ws + l.dtile_job);
    auto *dstatus = reinterpret_cast<uint64_t *>(ws + l.dstatus);
    auto *state = reinterpret_cast<DecompressState *>(ws + l.state);
    auto *plan = reinterpret_cast<ApplyPlan *>(ws + l.plan);

    SetupArgs sa{};
    sa.zero[0] = reinterpret_cast<uint32_t *>(ctrl);
    sa.zero_words[0] = sizeof(Control) / 4;
    sa.zero[1] = reinterpret_cast<uint32_t *>(state);
    sa.zero_words[1] = sizeof(DecompressState) / 4 * (uint64_t)count;
    sa.zero[2] = reinterpret_cast<uint32_t *>(sums);
    sa.zero_words[2] = sizeof(JobSums) / 4 * (uint64_t)count;
    sa.start[0] = dstart;
    sa.map[0] = dmap;
    sa.status[0] = dstatus;
    sa.tiles[0] = dtiles;
    sa.count = count;
    launch_setup(sa, stream);
    if (dtiles)   // its last workgroup also prepares the jobs
        desc_scan_kernel<<<(uint32_t)dtiles, kThreads, 0, stream>>>(jobs, dmap, dstatus, offsets,
                                                                    state, ctrl, count);
    else
        prepare_kernel<<<(count + kThreads - 1) / kThreads, kThreads, 0, stream>>>(jobs, state,
                                                                                   count);
    if (tiles) {
        const uint64_t g = (tiles + kThreads - 1) / kThreads;
        plan_kernel<<<(uint32_t)(g < 4096 ? g : 4096), kThreads, 0, stream>>>(
            jobs, state, bstart, count, offsets, plan, block_map, tiles);
        if (events && events->before && hipEventRecord(events->before, stream) != hipSuccess)
            return hipErrorInvalidValue;
        apply_kernel<<<(uint32_t)tiles, kThreads, 0, stream>>>(plan, state, partial);
        if (events && events->after && hipEventRecord(events->after, stream) != hipSuccess)
            return hipErrorInvalidValue;
        // its last workgroup also finalizes the jobs
        sum_partials_kernel<<<(uint32_t)dtiles, kThreads, 0, stream>>>(
            jobs, dmap, state, partial, sums, ctrl, count, results);
        fixup_kernel<<<persistent_grid((const void *)fixup_kernel, tiles), kThreads, 0, stream>>>(
            plan, state, ctrl, tiles);
        if (verify_first)
            commit_kernel<<<(uint32_t)tiles, kThreads, 0, stream>>>(plan, state, ctrl);
    } else {
        decompress_finalize_kernel<<<(count + kThreads - 1) / kThreads, kThreads, 0, stream>>>(
            jobs, state, sums, ctrl, count, results);
    }
    return hipGetLastError();
}

}  // namespace bf16d
