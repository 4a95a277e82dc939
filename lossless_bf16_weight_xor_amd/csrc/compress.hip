// compress.hip -- BF16 delta encoder for gfx950.
//
// A batch of tensors ("jobs") is one sequence of kernels; a tile is one
// 8192-element block of one job, and the tile-to-job map built by the setup
// kernel turns a tile index into (job, block).
//
// Per tile the encoder:
//   1. loads old and new with 16-byte coalesced loads and forms x = old XOR
//      new.  This is the mask of "GPU-accelerated Weight Teleportation",
//      section "Delta update algebra"; it lives only in registers and LDS
//      and is never stored.
//   2. classifies each element ("Every byte counts: ARCv3 and the case for
//      cross-region RL", section "Deep dive into ARCv3"):
//        x == 0                unchanged
//        (x & 0xFF80) == 0     mantissa-only
//        otherwise             exponent/sign change
//      The checksum terms of the new weights are summed in the same pass.
//   3. scans the changed/rare counts in element order with wave64 DPP
//      scans, and finds the widest gap, which gives the gap-field width and
//      the cheaper position encoding (gap list or bitmap).
//   4. builds the record (position | mantissa | rare segments) in LDS with
//      atomic ORs.  Each field has one owner, so the bytes do not depend on
//      timing.
//
// Placing records needs each record's byte offset: the exclusive sum of the
// sizes of the job's earlier records.  Computing that inside the streaming
// pass would stall it on a cross-workgroup look-back.  So the work is split:
//   setup    : clears the call's sums and builds the tile -> job maps.
//   encode   : one workgroup per tile, no inter-workgroup waits.  Reads old
//              and new once.  Writes each record to a fixed per-tile slot in
//              the workspace if it fits, plus its descriptor and checksum
//              partials.  A record that does not fit its slot but is at most
//              kSlot bytes is staged at the payload buffer's tail (16-byte
//              aligned ranges taken top down with one atomic per record);
//              larger ones, and those that find no room, are listed for
//              re-encoding.
//   offsets  : a decoupled look-back scan (Merrill and Garland, "Single-pass
//              Parallel Prefix Scan with Decoupled Look-back", 2016) over the
//              record sizes of each job: the stream offsets.  It writes
//              the descriptor table, and its last workgroup writes each
//              job's header, checksum and result.
//   place    : each wave copies four tiles' slots to their records' offsets.
//   reencode : for tiles whose record did not fit a slot (dense blocks),
//              encodes again straight into the payload.
//
// A version-2 payload adds a binding block to the header; an overwrite
// payload (its flag set) has no mantissa segment and carries the new value
// of every change as a 16-bit word.  Overwrite tiles take their own compiled
// instances of the same steps.
// The staging costs 2 * (record bytes) of extra traffic, about 2% at a 2%
// change rate.  The slot size is the caller's choice through the workspace
// it passes: kSlot bytes per tile (12.5 % of the weights) keeps every record
// of a sparse delta in the workspace; 256 bytes (1.6 %) keeps the common
// sparse records there and stages the rest in the payload buffer, which
// must then have room for them beyond the final payload, or they are
// encoded again.
#include "internal.hpp"

namespace bf16d {

constexpr uint32_t kPosMantMax = kBlock / 8 + (7 * kBlock) / 8;   // 8192 bytes

// Uniform (per-workgroup) description of one tile.
struct TileRef {
    BF16D_GMEM const uint16_t *src, *dst;   // first element of the tile
    uint64_t b;                  // block index within the job
    uint32_t L;                  // elements in this block
};

__device__ __forceinline__ TileRef tile_ref(const CompressJob &job, uint64_t t) {
    TileRef r;
    r.b = t - job.block0;
    const uint64_t base = r.b * kBlock;
    const uint64_t left = job.n - base;
    r.L = left < kBlock ? (uint32_t)left : kBlock;
    r.src = job.src + base;
    r.dst = job.dst + base;
    return r;
}

// kFull (a whole block): eight unconditional 16-byte loads, all in flight
// at once, marked non-temporal (load_stream16).  Otherwise (the short last
// block of a tensor) element by element up to L, zero beyond.
template <bool kFull>
__device__ __forceinline__ void load_tile(const TileRef &t, uint4 (&o)[kChunksPerThread],
                                          uint4 (&nw)[kChunksPerThread]) {
#pragma unroll
    for (uint32_t i = 0; i < kChunksPerThread; ++i) {
        const uint32_t e0 = 8 * (threadIdx.x + kThreads * i);
        if (kFull) {   // both checkpoints are read once: streamed past the caches
            o[i] = load_stream16(t.src + e0);
            nw[i] = load_stream16(t.dst + e0);
        } else {
            o[i] = make_uint4(0, 0, 0, 0);
            nw[i] = make_uint4(0, 0, 0, 0);
            if (e0 < t.L) {
                o[i] = load_chunk(t.src + e0, t.L - e0);
                nw[i] = load_chunk(t.dst + e0, t.L - e0);
            }
        }
    }
}

// LDS shared by the encoding steps.
struct EncodeShared {
    uint32_t cnt[kChunksPerThread * kWaves];    // [round][wave]: changed | rare << 16
    uint32_t last[kChunksPerThread * kWaves];   // [round][wave]: last changed position + 1
    uint32_t gmax[kWaves];
    uint8_t gap8[256];   // widest gap between set bits of an 8-bit mask (0 if < 2 bits)
    uint64_t stage_at;   // payload offset of a record staged at the tail (0: no room)
};

// Fill sh.gap8 (once per workgroup; the caller synchronises).
__device__ __forceinline__ void init_gap_table(EncodeShared &sh) {
    const uint32_t m = threadIdx.x;   // kThreads == 256
    uint32_t best = 0;
    int prev = -1;
    for (int b = 0; b < 8; ++b) {
        if ((m >> b) & 1) {
            if (prev >= 0) best = umax32(best, (uint32_t)(b - prev - 1));
            prev = b;
        }
    }
    sh.gap8[m] = (uint8_t)best;
}

// Result of classifying and scanning one tile (per thread, except the
// uniform fields c, r, w, code, pb, mb, len, desc).
struct TileCode {
    uint32_t M, R;           // changed / rare flags of this thread: bit 8i+s = slot s of round i
    uint64_t Jb, Kb, Pb;     // per-round bases (16 bits per round): changed rank, rare rank,
                             // previous changed position + 1
    uint64_t acc;            // checksum partial of this thread
    uint32_t c, r, w, code, pb, mb, len, desc;
};

// Per-thread results of classifying a tile, before the scans.
struct TileFlags {
    uint32_t M, R;                          // changed / rare flags, bit 8i+s = slot s of round i
    uint32_t cnt[kChunksPerThread];         // changed | rare << 16 per round
    uint32_t last[kChunksPerThread];        // last changed position + 1 per round (0 = none)
    uint64_t acc;                           // checksum partial
};

// Steps 1-2 for one tile, in registers only: writes x to s_x (each thread
// touches only its own chunks).  After it returns, o/nw are free.
//   kOw (an overwrite payload): s_x gets the new values instead, and every
//   change counts as a word of the word segment (rare flags = changed flags).
template <bool kOw>
__device__ __forceinline__ void classify(const TileRef &t, const uint4 (&o)[kChunksPerThread],
                                         const uint4 (&nw)[kChunksPerThread], uint16_t *s_x,
                                         TileFlags &f) {
    const uint32_t tid = threadIdx.x;
    uint32_t M = 0, R = 0;
    uint64_t acc = 0;
    // (k+1)*G of this thread's first word: word index = tile word + 2*tid + 512*i
    const uint64_t kg0 = ((t.b * kBlock >> 2) + 1 + 2 * tid) * kGamma;
    constexpr uint64_t kRoundKg = (uint64_t)(2 * kThreads) * kGamma;
#pragma unroll
    for (uint32_t i = 0; i < kChunksPerThread; ++i) {
        const uint32_t q = tid + kThreads * i;
        const uint32_t e0 = 8 * q;
        const uint32_t valid = e0 < t.L ? (t.L - e0 < 8 ? t.L - e0 : 8) : 0;
        const uint4 x = make_uint4(o[i].x ^ nw[i].x, o[i].y ^ nw[i].y, o[i].z ^ nw[i].z,
                                   o[i].w ^ nw[i].w);
        reinterpret_cast<uint4 *>(s_x)[q] = kOw ? nw[i] : x;
        const uint64_t kg = kg0 + i * kRoundKg;
        if (valid > 0) acc += mix64(((uint64_t)nw[i].y << 32 | nw[i].x) ^ kg);
        if (valid > 4) acc += mix64(((uint64_t)nw[i].w << 32 | nw[i].z) ^ (kg + kGamma));
        const uint32_t c8 = nonzero8(x, 0xFFFFFFFFu);
        const uint32_t r8 = kOw ? c8 : nonzero8(x, 0xFF80FF80u);
        M |= c8 << (8 * i);
        R |= r8 << (8 * i);
        f.cnt[i] = __popc(c8) | (__popc(r8) << 16);
        f.last[i] = c8 ? e0 + 32 - __clz(c8) : 0;
    }
    f.M = M;
    f.R = R;
    f.acc = acc;
}

// Step 3: scans in element order (round i, then thread, then slot), the
// widest gap and the record layout.  Contains two barriers.  kOw: no
// mantissa segment.
template <bool kOw>
__device__ __forceinline__ void scan(const TileRef &t, const TileFlags &f, EncodeShared &sh,
                                     TileCode &out) {
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t M = f.M;
    const uint32_t(&cnt)[kChunksPerThread] = f.cnt;
    const uint32_t(&last)[kChunksPerThread] = f.last;
    uint32_t inc_cnt[kChunksPerThread], inc_last[kChunksPerThread];
#pragma unroll
    for (uint32_t i = 0; i < kChunksPerThread; ++i) {
        inc_cnt[i] = wave_incl_add(cnt[i]);
        inc_last[i] = wave_incl_max(last[i]);
        const uint32_t tot = lane63(inc_cnt[i]), mx = lane63(inc_last[i]);
        if (lane == 0) {
            sh.cnt[kWaves * i + wave] = tot;
            sh.last[kWaves * i + wave] = mx;
        }
    }
    __syncthreads();
    // the 16 (round, wave) totals in element order, scanned by lanes 0..15 of
    // every wave (one DPP row): exclusive sums and exclusive maxima
    const uint32_t v16 = lane < 16 ? sh.cnt[lane] : 0u, m16 = lane < 16 ? sh.last[lane] : 0u;
    const uint32_t inc16 = row_incl_add(v16), max16 = row_incl_max(m16);
    const uint32_t ex16 = inc16 - v16, exm16 = wave_shr1(max16);   // lane 0 reads 0
    uint64_t Jb = 0, Kb = 0, Pb = 0;
#pragma unroll
    for (uint32_t i = 0; i < kChunksPerThread; ++i) {
        const uint32_t base = readlane_u32(ex16, kWaves * i + wave);
        const uint32_t pbase = readlane_u32(exm16, kWaves * i + wave);
        const uint32_t ex = base + inc_cnt[i] - cnt[i];
        Jb |= (uint64_t)(ex & 0xFFFFu) << (16 * i);
        Kb |= (uint64_t)(ex >> 16) << (16 * i);
        Pb |= (uint64_t)umax32(pbase, wave_shr1(inc_last[i])) << (16 * i);
    }
    const uint32_t run = readlane_u32(inc16, 15);
    const uint32_t c = run & 0xFFFFu, r = run >> 16;

    // widest gap: the gap before each chunk's first change, and the widest
    // gap inside each chunk (table) -> field width -> cheaper encoding
    uint32_t maxgap = 0;
#pragma unroll
    for (uint32_t i = 0; i < kChunksPerThread; ++i) {
        const uint32_t c8 = (M >> (8 * i)) & 0xFFu;
        if (c8) {
            const uint32_t p1 = (uint32_t)(Pb >> (16 * i)) & 0xFFFFu;   // previous change + 1
            const uint32_t first = 8 * (tid + kThreads * i) + __ffs(c8) - 1;
            maxgap = umax32(maxgap, umax32(first - p1, sh.gap8[c8]));
        }
    }
    maxgap = lane63(wave_incl_max(maxgap));
    if (lane == 0) sh.gmax[wave] = maxgap;
    __syncthreads();
    maxgap = umax32(umax32(sh.gmax[0], sh.gmax[1]), umax32(sh.gmax[2], sh.gmax[3]));

    out.M = M;
    out.R = f.R;
    out.Jb = Jb;
    out.Kb = Kb;
    out.Pb = Pb;
    out.acc = f.acc;
    out.c = c;
    out.r = r;
    out.w = bit_length(maxgap);
    const uint32_t delta_bytes = (c * out.w + 7) / 8;
    const uint32_t bitmap_bytes = (t.L + 7) / 8;
    out.code = bitmap_bytes < delta_bytes ? kCodeBitmap : out.w;
    out.pb = out.code == kCodeBitmap ? bitmap_bytes : delta_bytes;
    out.mb = kOw ? 0u : (7 * c + 7) / 8;
    out.len = out.pb + out.mb + 2 * r;
    out.desc = c | (r << 14) | (out.code << 28);
}

// Step 4: OR this thread's fields into a zeroed LDS record.  The rare words
// go in too when kWithRare; otherwise the caller stores them directly.  kOw:
// the words are the new values of every change, and there are no mantissa
// fields.
template <bool kWithRare, bool kOw>
__device__ __forceinline__ void or_fields(uint32_t *s_rec, const uint16_t *s_x,
                                          const TileCode &k) {
    const uint32_t tid = threadIdx.x;
    const uint32_t mant_bit = 8 * k.pb, rare_bit = 8 * (k.pb + k.mb);
    if (k.code == kCodeBitmap) {
#pragma unroll
        for (uint32_t i = 0; i < kChunksPerThread; ++i) {
            const uint32_t q = tid + kThreads * i, c8 = (k.M >> (8 * i)) & 0xFFu;
            if (c8) atomicOr(&s_rec[q >> 2], c8 << (8 * (q & 3)));
        }
    }
    for (uint32_t bits = k.M; bits; bits &= bits - 1) {
        const uint32_t idx = __ffs(bits) - 1, i = idx >> 3, s = idx & 7;
        const uint32_t below = (k.M >> (8 * i)) & ((1u << s) - 1);
        const uint32_t q = tid + kThreads * i;
        const uint32_t j = ((uint32_t)(k.Jb >> (16 * i)) & 0xFFFFu) + __popc(below);
        if (k.code != kCodeBitmap) {
            const uint32_t p1 = below ? 8 * q + 32 - __clz(below)
                                      : (uint32_t)(k.Pb >> (16 * i)) & 0xFFFFu;
            lds_or_bits(s_rec, j * k.w, 8 * q + s - p1, k.w);
        }
        const uint32_t xs = s_x[8 * q + s];
        if (!kOw && !(xs & kExpSign)) {
            lds_or_bits(s_rec, mant_bit + 7 * j, xs & kMant, 7);
        } else if (kWithRare) {
            const uint32_t kk = ((uint32_t)(k.Kb >> (16 * i)) & 0xFFFFu) +
                                __popc((k.R >> (8 * i)) & ((1u << s) - 1));
            lds_or_bits(s_rec, rare_bit + 16 * kk, xs, 16);
        }
    }
}

// ------------------------------------------------------------------ encode ---
// One tile, from its loads to its slot.  Whole blocks and the short last
// block of a tensor are compiled separately, so that all of a whole block's
// loads are in flight together.
template <bool kFull, bool kOw>
__device__ __forceinline__ void encode_one(const TileRef &tr, uint64_t t, uint16_t *s_x,
                                           uint32_t *s_rec, EncodeShared &sh,
                                           uint8_t *__restrict__ slots, uint32_t slot_bytes,
                                           const CompressJob &job,
                                           unsigned long long *__restrict__ stage,
                                           uint32_t *__restrict__ desc_out,
                                           uint64_t *__restrict__ partial,
                                           uint32_t *__restrict__ overflow,
                                           Control *__restrict__ ctrl) {
    const uint32_t tid = threadIdx.x, lane = tid & 63;
    uint4 o[kChunksPerThread], nw[kChunksPerThread];
    load_tile<kFull>(tr, o, nw);
    // while the loads are in flight: clear the record, build the gap table
    for (uint32_t u = tid; u < kSlot / 4 + 4; u += kThreads) s_rec[u] = 0;
    init_gap_table(sh);

    TileFlags f;
    classify<kOw>(tr, o, nw, s_x, f);
    TileCode k;
    scan<kOw>(tr, f, sh, k);   // its barriers also order the clearing above

    const bool fits = k.len <= kSlot;   // built in LDS; larger records are re-encoded
    if (fits) or_fields<true, kOw>(s_rec, s_x, k);
    const uint64_t acc = first_lane(wave_sum(k.acc));
    __syncthreads();

    if (fits) {
        uint8_t *dst = slots + t * slot_bytes;
        if (k.len > slot_bytes) {   // uniform: the record waits at the payload's tail
            // a 16-byte aligned range between the descriptor table and the
            // capacity, in block b's stack (b % ways): the stack's bytes
            // [o, o + room) taken with one atomic, o counting from the top
            // chunk by chunk; a range that crosses a chunk's end is
            // abandoned and another taken, a few times at most, then the
            // record is encoded again instead (nothing ever waits).  Where it
            // lands decides only which record is copied from where, never
            // the payload's bytes.
            if (tid == 0) {
                const uint64_t room = (k.len + 15) & ~15u;
                const uint64_t top = job.capacity & ~15ull;
                const uint64_t floor = (job.hdr + 4 * job.nb + 15) & ~15ull;
                const uint64_t ways = job.nb < kStageWays ? job.nb : kStageWays;
                const uint64_t span = top > floor ? (top - floor) / ways & ~15ull : 0;
                const uint64_t C = span < kStageChunk ? span : kStageChunk;
                const uint64_t w = tr.b % ways;
                uint64_t at = 0;
                for (uint32_t tries = 0; at == 0 && room <= C && tries < kStageTries; ++tries) {
                    const uint64_t o = atomicAdd(&stage[w], room);
                    if (o % C + room > C) continue;   // crosses a chunk's end
                    const uint64_t below = ((o / C) * ways + w + 1) * C;
                    if (below > top - floor) break;   // out of room
                    at = top - below + o % C;
                }
                sh.stage_at = at;
            }
            __syncthreads();
            const uint64_t at = sh.stage_at;
            // the slot keeps where the record is: its address and offset, or
            // a null address when there was no room (the tile is then
            // listed for re-encoding here, and the place kernel skips it)
            if (tid == 0)
                *reinterpret_cast<ulonglong2 *>(dst) = make_ulonglong2(
                    at ? (unsigned long long)(uintptr_t)(job.payload + at) : 0ull, at);
            if (at == 0) {   // no room: encoded again once the offsets are known
                if (tid == 0) overflow[atomicAdd(&ctrl->overflow_count, 1u)] = (uint32_t)t;
                dst = nullptr;
            } else {
                dst = (uint8_t *)(job.payload + at);
            }
        }
        if (dst) {
            uint4 *out = reinterpret_cast<uint4 *>(dst);
            const uint4 *rec = reinterpret_cast<const uint4 *>(s_rec);
            for (uint32_t u = tid; u < (k.len + 15) / 16; u += kThreads)
                store_stream16(out + u, rec[u]);   // read next by the place kernel only
        }
    } else if (tid == 0) {
        overflow[atomicAdd(&ctrl->overflow_count, 1u)] = (uint32_t)t;
    }
    if (lane == 0) partial[kWaves * t + (tid >> 6)] = acc;
    if (tid == 0) desc_out[t] = k.desc;
}

// One workgroup per tile, no inter-workgroup waits.  Occupancy hides the
// load latency: with 54 VGPRs and 18.8 KiB of LDS, eight workgroups fit on a
// CU.  That measured faster than a persistent loop that keeps the next
// tile's loads in registers at half the occupancy.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(6, 8)))
void encode_kernel(const CompressJob *__restrict__ jobs, const uint32_t *__restrict__ tile_job,
                   uint8_t *__restrict__ slots, uint32_t slot_bytes,
                   unsigned long long *__restrict__ stage, uint32_t *__restrict__ desc_out,
                   uint64_t *__restrict__ partial, uint32_t *__restrict__ overflow,
                   Control *__restrict__ ctrl) {
    __shared__ __attribute__((aligned(16))) uint16_t s_x[kBlock];
    __shared__ __attribute__((aligned(16))) uint32_t s_rec[kSlot / 4 + 4];
    __shared__ EncodeShared sh;
    const uint64_t t = xcd_tile(blockIdx.x, gridDim.x);
    const uint32_t j = tile_job[t];
    const CompressJob &job = jobs[j];
    unsigned long long *js = stage + (size_t)kStageWays * j;
    const TileRef tr = tile_ref(job, t);
    if (job.flags & kFlagOverwrite) {   // overwrite payloads: their own instances
        if (tr.L == kBlock)
            encode_one<true, true>(tr, t, s_x, s_rec, sh, slots, slot_bytes, job, js, desc_out,
                                   partial, overflow, ctrl);
        else
            encode_one<false, true>(tr, t, s_x, s_rec, sh, slots, slot_bytes, job, js, desc_out,
                                    partial, overflow, ctrl);
    } else if (tr.L == kBlock) {
        encode_one<true, false>(tr, t, s_x, s_rec, sh, slots, slot_bytes, job, js, desc_out,
                                partial, overflow, ctrl);
    } else {
        encode_one<false, false>(tr, t, s_x, s_rec, sh, slots, slot_bytes, job, js, desc_out,
                                 partial, overflow, ctrl);
    }
}

// ---------------------------------------------------------------- finalize ---
// Job j's header, checksum and result.  The sums are read with device-scope
// loads: the offsets kernel's last workgroup runs this right after the other
// workgroups' atomics.
__device__ void finalize_job(const CompressJob *__restrict__ jobs, JobSums *__restrict__ sums,
                             bf16d_result *__restrict__ results, uint32_t j) {
    const CompressJob job = jobs[j];
    JobSums *js = &sums[j];
    const unsigned long long S = ld_agent(&js->csum), c = ld_agent(&js->c), r = ld_agent(&js->r),
                             pos = ld_agent(&js->pos), mant = ld_agent(&js->mant),
                             nbm = ld_agent(&js->nbm);
    const uint64_t rare = 2 * r;
    const uint64_t P = job.hdr + 4 * job.nb + pos + mant + rare;
    const int status = P <= job.capacity ? BF16D_OK : BF16D_ECAPACITY;
    js->P = P;   // for the place kernel: staged records below P are re-encoded
    if (status == BF16D_OK) {
        BF16D_GMEM uint32_t *h = reinterpret_cast<BF16D_GMEM uint32_t *>(job.payload);
        BF16D_GMEM uint64_t *h64 = reinterpret_cast<BF16D_GMEM uint64_t *>(job.payload);
        h[0] = kMagicLo;
        h[1] = kMagicHi;
        h[2] = job.hdr == kHeaderBound ? BF16D_FORMAT_VERSION_BOUND : BF16D_FORMAT_VERSION;
        h[3] = kBlock;
        h64[2] = job.n;
        h64[3] = c;
        h64[4] = r;
        h64[5] = pos;
        h64[6] = mant;
        h64[7] = rare;
        if (job.hdr == kHeaderBound) {   // the binding block
            h64[8] = job.base_version;
            h64[9] = job.target_version;
            h[20] = job.flags;
            h[21] = 0;
            h64[11] = 0;
        }
    }
    bf16d_result res;
    res.status = status;
    res.reserved = 0;
    res.payload_bytes = P;
    res.checksum = mix64(S ^ job.n);
    res.n_changed = c;
    res.n_rare = r;
    res.n_bitmap_blocks = nbm;
    results[j] = res;
}

// For calls without tiles (every tensor empty); otherwise the offsets
// kernel's last workgroup finalizes the jobs.
__global__ __launch_bounds__(kThreads) void compress_finalize_kernel(
    const CompressJob *__restrict__ jobs, JobSums *__restrict__ sums, uint32_t count,
    bf16d_result *__restrict__ results) {
    const uint32_t j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j < count) finalize_job(jobs, sums, results, j);
}

// ----------------------------------------------------------------- offsets ---
// Record offsets within each job: exclusive sum of record sizes over the
// job's tiles, by tiles of kDescTile descriptors with a decoupled look-back.
__global__ __launch_bounds__(kThreads) void record_offsets_kernel(
    const CompressJob *__restrict__ jobs, const uint32_t *__restrict__ dtile_job,
    const uint64_t *__restrict__ dstart, const uint32_t *__restrict__ desc,
    uint64_t *__restrict__ dstatus, uint64_t *__restrict__ offsets,
    PlaceEntry *__restrict__ place, uint32_t slot_bytes, const uint64_t *__restrict__ partial,
    JobSums *__restrict__ sums, Control *__restrict__ ctrl, uint32_t count,
    bf16d_result *__restrict__ results) {
    __shared__ uint32_t s_tmp[kWaves];
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
    const CompressJob job = jobs[j];
    const uint64_t first = dstart[j];
    const uint64_t ld = dt - first;

    uint32_t lens[kDescPerThread], descs[kDescPerThread];
    uint32_t mine = 0;
    unsigned long long c_sum = 0, r_sum = 0, pos_sum = 0, mant_sum = 0, nbm = 0, S = 0;
#pragma unroll
    for (uint32_t k = 0; k < kDescPerThread; ++k) {
        const uint64_t b = ld * kDescTile + kDescPerThread * tid + k;
        lens[k] = 0;
        descs[k] = 0;
        if (b >= job.nb) continue;
        const uint32_t d = desc[job.block0 + b];
        descs[k] = d;
#pragma unroll
        for (uint32_t w = 0; w < kWaves; ++w) S += partial[kWaves * (job.block0 + b) + w];
        const uint64_t left = job.n - b * kBlock;
        const uint32_t L = left < kBlock ? (uint32_t)left : kBlock;
        const uint32_t c = d & 0x3FFFu, r = (d >> 14) & 0x3FFFu, code = d >> 28;
        const uint32_t pb = code == kCodeBitmap ? (L + 7) / 8 : (c * code + 7) / 8;
        const uint32_t mb = (job.flags & kFlagOverwrite) ? 0u : (7 * c + 7) / 8;
        lens[k] = pb + mb + 2 * r;
        mine += lens[k];
        c_sum += c;
        r_sum += r;
        pos_sum += pb;
        mant_sum += mb;
        nbm += code == kCodeBitmap;
    }
    uint32_t total;
    uint32_t excl = block_exclusive_sum(mine, s_tmp, total);
    if (tid == 0) st_agent(&dstatus[dt], (ld == 0 ? kFlagPrefix : kFlagAggregate) | total);
    if (wave == 0) {
        const uint64_t e = (ld == 0) ? 0 : look_back(dstatus, dt, first);
        if (lane == 0) {
            if (ld != 0) st_agent(&dstatus[dt], kFlagPrefix | (e + total));
            s_excl = e;
        }
    }
    __syncthreads();
    // offsets, the descriptor table, and where each slot's record goes
    uint64_t off = s_excl + excl;
    const uint64_t cap = job.capacity;
#pragma unroll
    for (uint32_t k = 0; k < kDescPerThread; ++k) {
        const uint64_t b = ld * kDescTile + kDescPerThread * tid + k;
        if (b < job.nb) {
            offsets[job.block0 + b] = off;
            if (job.hdr + 4 * b + 4 <= cap)
                *reinterpret_cast<BF16D_GMEM uint32_t *>(job.payload + job.hdr + 4 * b) = descs[k];
            const uint64_t rel = job.hdr + 4 * job.nb + off;
            const uint32_t len = lens[k];
            PlaceEntry e;
            e.dst = job.payload + rel;
            e.len = (len > kSlot || rel >= cap) ? 0u
                                                 : (uint32_t)(cap - rel < len ? cap - rel : len);
            e.staged = len > slot_bytes ? kStaged : 0u;
            place[job.block0 + b] = e;
        }
        off += lens[k];
    }
    // the header totals of the job
    c_sum = block_sum(c_sum, s_tmp64);
    r_sum = block_sum(r_sum, s_tmp64);
    pos_sum = block_sum(pos_sum, s_tmp64);
    mant_sum = block_sum(mant_sum, s_tmp64);
    nbm = block_sum(nbm, s_tmp64);
    S = block_sum(S, s_tmp64);
    uint64_t dep = 0;
    if (tid == 0)   // exact mod 2^64, in any order
        dep = atomicAdd(&sums[j].csum, S) ^ atomicAdd(&sums[j].c, c_sum) ^
              atomicAdd(&sums[j].r, r_sum) ^ atomicAdd(&sums[j].pos, pos_sum) ^
              atomicAdd(&sums[j].mant, mant_sum) ^ atomicAdd(&sums[j].nbm, nbm);
    // the last workgroup to finish writes every job's header and result
    if (last_workgroup(&ctrl->scan_done, dep))
        for (uint32_t jj = tid; jj < count; jj += kThreads) finalize_job(jobs, sums, results, jj);
}

// ------------------------------------------------------------------- place ---
// Slot (or staged range) -> payload.  Each wave copies kPlaceTiles records:
// all their source words are requested before the first store, so enough
// bytes are in flight per wave.  Lane u of round m produces payload dword
// u + 64m of a record from source dwords i - 1 and i (the record's byte
// offset within a dword is fixed per record); the dwords a record shares
// with its neighbours, and anything past `capacity`, are written byte by
// byte or not at all.
//
// A staged record (one that did not fit its slot) waits at the payload
// buffer's tail, at an offset its slot holds.  It is copied down only if it
// lies wholly at or past the job's payload size P: then no record's final
// place overlaps it.  Otherwise the final records reach into the tail, and
// it is put on the re-encode list instead (encoded again, straight into its
// final place, after this kernel).
constexpr uint32_t kPlaceTiles = 4;
constexpr uint32_t kPlaceRounds = kSlot / 256;   // 64 lanes x 4 bytes per round

__global__ __launch_bounds__(kThreads) void place_kernel(const PlaceEntry *__restrict__ place,
                                                         const uint8_t *__restrict__ slots,
                                                         uint32_t slot_bytes,
                                                         const uint32_t *__restrict__ tile_job,
                                                         const JobSums *__restrict__ sums,
                                                         uint32_t *__restrict__ overflow,
                                                         Control *__restrict__ ctrl,
                                                         uint64_t tiles) {
    const uint32_t lane = threadIdx.x & 63;
    const uint64_t t0 = ((uint64_t)blockIdx.x * kWaves + (threadIdx.x >> 6)) * kPlaceTiles;
    if (t0 >= tiles) return;   // whole wave; the kernel has no barriers
    uint4 e = make_uint4(0, 0, 0, 0);
    uint64_t from = 0;   // lanes 0..3: where tile t0 + lane's record is read from
    if (lane < kPlaceTiles && t0 + lane < tiles) {
        const uint64_t t = t0 + lane;
        e = *reinterpret_cast<const uint4 *>(place + t);
        from = (uint64_t)(uintptr_t)(slots + t * slot_bytes);
        if (e.z != 0 && e.w == kStaged) {
            const ulonglong2 at = *reinterpret_cast<const ulonglong2 *>(slots + t * slot_bytes);
            if (at.x == 0) {   // never staged: already on the re-encode list
                e.z = 0;
            } else if (at.y >= sums[tile_job[t]].P) {
                from = at.x;
            } else {   // the final records reach into it: encode it again
                overflow[atomicAdd(&ctrl->overflow_count, 1u)] = (uint32_t)t;
                e.z = 0;
            }
        }
    }
    // a record of up to kSlot bytes at a byte offset of 1..3 spans one payload
    // dword more than its source: the extra round reads nothing
    uint32_t rec[kPlaceTiles][kPlaceRounds + 1];
#pragma unroll
    for (uint32_t k = 0; k < kPlaceTiles; ++k) {
        const uint32_t len = (uint32_t)__builtin_amdgcn_readlane((int)e.z, k);
        const uint64_t fk = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)from, k) |
                            (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(from >> 32), k)
                                << 32;
        const uint32_t *src = reinterpret_cast<const uint32_t *>((uintptr_t)fk);
#pragma unroll
        for (uint32_t m = 0; m < kPlaceRounds; ++m) {
            rec[k][m] = 0;
            if (256 * m < len && 4 * (lane + 64 * m) < len) rec[k][m] = src[lane + 64 * m];
        }
        rec[k][kPlaceRounds] = 0;
    }
#pragma unroll
    for (uint32_t k = 0; k < kPlaceTiles; ++k) {
        const uint32_t len = (uint32_t)__builtin_amdgcn_readlane((int)e.z, k);
        if (len == 0) continue;
        const uint64_t D = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)e.x, k) |
                           (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)e.y, k) << 32;
        const uint32_t sh = (uint32_t)(D & 3);
        BF16D_GMEM uint8_t *const a0 = reinterpret_cast<BF16D_GMEM uint8_t *>(D - sh);
        const uint32_t nout = (sh + len + 3) / 4;
        const uint32_t last_hi = ((sh + len - 1) & 3) + 1;   // valid bytes of the last dword
#pragma unroll
        for (uint32_t m = 0; m <= kPlaceRounds; ++m) {
            if (256 * m >= sh + len) continue;
            const uint32_t cur = rec[k][m];
            // lane 0 takes the previous round's last dword; read in uniform
            // control flow (see lane63)
            const uint32_t carry =
                m ? (uint32_t)__builtin_amdgcn_readlane((int)rec[k][m > 0 ? m - 1 : 0], 63) : 0u;
            const uint32_t prev = wave_shr1_fill(cur, carry);
            const uint32_t v = sh ? __builtin_amdgcn_alignbyte(cur, prev, 4 - sh) : cur;
            const uint32_t i = lane + 64 * m;
            if (i < nout) {
                const uint32_t lo = i == 0 ? sh : 0, hi = i == nout - 1 ? last_hi : 4;
                if (lo == 0 && hi == 4) {
                    *reinterpret_cast<BF16D_GMEM uint32_t *>(a0 + 4 * i) = v;
                } else {
                    for (uint32_t q = lo; q < hi; ++q) a0[4 * i + q] = (uint8_t)(v >> (8 * q));
                }
            }
        }
    }
}

// ---------------------------------------------------------------- reencode ---
// Tiles whose record exceeded a slot, encoded again straight into the
// payload now that their offsets are known.  The position and mantissa
// segments are built in LDS (<= 8192 bytes); the rare words, whole 16-bit
// words on byte boundaries, are stored directly.
// kOw: the instance for overwrite payloads (launched only when the call has
// one); each instance skips the other kind's tiles.
template <bool kOw>
__global__ __launch_bounds__(kThreads) void reencode_kernel(
    const CompressJob *__restrict__ jobs, const uint32_t *__restrict__ tile_job,
    const uint32_t *__restrict__ overflow, const uint64_t *__restrict__ offsets,
    const Control *__restrict__ ctrl) {
    __shared__ __attribute__((aligned(16))) uint16_t s_x[kBlock];
    __shared__ uint32_t s_rec[kPosMantMax / 4 + 4];
    __shared__ EncodeShared sh;
    const uint32_t tid = threadIdx.x;
    const uint32_t count = ctrl->overflow_count;
    init_gap_table(sh);   // ordered before use by the barriers in scan()
    for (uint32_t i = blockIdx.x; i < count; i += gridDim.x) {
        const uint64_t t = overflow[i];
        const CompressJob job = jobs[tile_job[t]];
        if (((job.flags & kFlagOverwrite) != 0) != kOw) continue;   // uniform
        const TileRef tr = tile_ref(job, t);
        uint4 o[kChunksPerThread], nw[kChunksPerThread];
        load_tile<false>(tr, o, nw);
        for (uint32_t u = tid; u < kPosMantMax / 4 + 4; u += kThreads) s_rec[u] = 0;
        TileFlags f;
        classify<kOw>(tr, o, nw, s_x, f);
        TileCode k;
        scan<kOw>(tr, f, sh, k);   // its barriers also order the clearing of s_rec
        or_fields<false, kOw>(s_rec, s_x, k);
        __syncthreads();

        BF16D_GMEM uint8_t *const pay = job.payload;
        const uint64_t cap = job.capacity;
        const uint64_t D = job.hdr + 4 * job.nb + offsets[t];
        const uint32_t pm = k.pb + k.mb;
        const uint32_t sh4 = (uint32_t)(D & 3);
        const uint64_t a0 = D - sh4;
        const uint32_t words = (sh4 + pm + 3) / 4;
        for (uint32_t u = tid; u < words; u += kThreads) {
            const uint32_t hi = s_rec[u];
            const uint32_t lo = u ? s_rec[u - 1] : 0u;
            const uint32_t v = sh4 ? ((hi << (8 * sh4)) | (lo >> (32 - 8 * sh4))) : hi;
            const uint64_t A = a0 + 4ull * u;
            if (A >= D && A + 4 <= D + pm && A + 4 <= cap) {
                *reinterpret_cast<BF16D_GMEM uint32_t *>(pay + A) = v;
            } else {
#pragma unroll
                for (uint32_t q = 0; q < 4; ++q) {
                    const uint64_t at = A + q;
                    if (at >= D && at < D + pm && at < cap) pay[at] = (uint8_t)(v >> (8 * q));
                }
            }
        }
        const uint64_t rare0 = D + pm;
        for (uint32_t bits = k.R; bits; bits &= bits - 1) {
            const uint32_t idx = __ffs(bits) - 1, ii = idx >> 3, s = idx & 7;
            const uint32_t q = tid + kThreads * ii;
            const uint32_t kk = ((uint32_t)(k.Kb >> (16 * ii)) & 0xFFFFu) +
                                __popc((k.R >> (8 * ii)) & ((1u << s) - 1));
            const uint32_t xs = s_x[8 * q + s];
            const uint64_t at = rare0 + 2 * kk;
            if (at + 2 <= cap) {
                if ((at & 1) == 0) {
                    *reinterpret_cast<BF16D_GMEM uint16_t *>(pay + at) = (uint16_t)xs;
                } else {
                    pay[at] = (uint8_t)xs;
                    pay[at + 1] = (uint8_t)(xs >> 8);
                }
            } else if (at < cap) {
                pay[at] = (uint8_t)xs;
            }
        }
        __syncthreads();   // s_x and s_rec are reused by the next tile
    }
}

hipError_t launch_compress(const Layout &l, uint8_t *ws, uint32_t count, uint64_t tiles,
                           uint64_t dtiles, bf16d_result *results, hipStream_t stream,
                           const bf16d_events *events, bool any_overwrite) {
    auto *ctrl = reinterpret_cast<Control *>(ws + l.control);
    auto *jobs = reinterpret_cast<const CompressJob *>(ws + l.jobs);
    auto *bstart = reinterpret_cast<const uint64_t *>(ws + l.block_start);
    auto *dstart = reinterpret_cast<const uint64_t *>(ws + l.dtile_start);
    auto *map = reinterpret_cast<uint32_t *>(ws + l.tile_job);
    auto *offsets = reinterpret_cast<uint64_t *>(ws + l.status);
    auto *partial = reinterpret_cast<uint64_t *>(ws + l.partial);
    auto *sums = reinterpret_cast<JobSums *>(ws + l.sums);
    auto *desc = reinterpret_cast<uint32_t *>(ws + l.desc);
    auto *dmap = reinterpret_cast<uint32_t *>(ws + l.dtile_job);
    auto *dstatus = reinterpret_cast<uint64_t *>(ws + l.dstatus);
    auto *slots = ws + l.slots;
    const uint32_t slot_bytes = l.slot_bytes;
    auto *overflow = reinterpret_cast<uint32_t *>(ws + l.overflow);
    auto *stage = reinterpret_cast<unsigned long long *>(ws + l.stage);
    auto *place = reinterpret_cast<PlaceEntry *>(ws + l.plan);

    SetupArgs sa{};
    sa.zero[0] = reinterpret_cast<uint32_t *>(ctrl);
    sa.zero_words[0] = sizeof(Control) / 4;
    sa.zero[1] = reinterpret_cast<uint32_t *>(sums);
    sa.zero_words[1] = sizeof(JobSums) / 4 * (uint64_t)count;
    sa.zero[2] = reinterpret_cast<uint32_t *>(stage);
    sa.zero_words[2] = 2 * (uint64_t)kStageWays * count;
    sa.start[0] = bstart;
    sa.map[0] = map;
    sa.tiles[0] = tiles;
    sa.start[1] = dstart;
    sa.map[1] = dmap;
    sa.status[1] = dstatus;
    sa.tiles[1] = dtiles;
    sa.count = count;
    launch_setup(sa, stream);
    if (tiles) {
        if (events && events->before && hipEventRecord(events->before, stream) != hipSuccess)
            return hipErrorInvalidValue;
        encode_kernel<<<(uint32_t)tiles, kThreads, 0, stream>>>(jobs, map, slots, slot_bytes,
                                                                stage, desc, partial, overflow,
                                                                ctrl);
        if (events && events->after && hipEventRecord(events->after, stream) != hipSuccess)
            return hipErrorInvalidValue;
        // its last workgroup also writes the headers and results
        record_offsets_kernel<<<(uint32_t)dtiles, kThreads, 0, stream>>>(
            jobs, dmap, dstart, desc, dstatus, offsets, place, slot_bytes, partial, sums, ctrl,
            count, results);
        const uint64_t per_block = (uint64_t)kWaves * kPlaceTiles;
        place_kernel<<<(uint32_t)((tiles + per_block - 1) / per_block), kThreads, 0, stream>>>(
            place, slots, slot_bytes, map, sums, overflow, ctrl, tiles);
        reencode_kernel<false><<<persistent_grid((const void *)reencode_kernel<false>, tiles),
                                 kThreads, 0, stream>>>(jobs, map, overflow, offsets, ctrl);
        if (any_overwrite)
            reencode_kernel<true><<<persistent_grid((const void *)reencode_kernel<true>, tiles),
                                    kThreads, 0, stream>>>(jobs, map, overflow, offsets, ctrl);
    } else {
        compress_finalize_kernel<<<(count + kThreads - 1) / kThreads, kThreads, 0, stream>>>(
            jobs, sums, count, results);
    }
    return hipGetLastError();
}

}  // namespace bf16d
