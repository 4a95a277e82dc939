// decompress.hip -- in-place BF16 delta decoder for gfx950.
//
// The receiver rebuilds the new weights by XOR-ing the decoded mask onto the
// old ones in HBM ("GPU-accelerated Weight Teleportation", sections "Delta
// update algebra" and "A strong baseline with Blackwell-native DE").  It
// then checks them against the trainer's checksum ("Every byte counts: ARCv3
// and the case for cross-region RL", section "Deep dive into ARCv3").
//
// Kernels of one batched call, in stream order:
//   desc_scan : validates every descriptor and builds the block offset table
//               (the exclusive sum of record sizes within each job).  It uses
//               the same decoupled look-back as the encoder, over tiles of
//               2048 descriptors.
//   prepare   : one thread per job; checks the header against the arguments
//               and against the descriptor sums.  A job that fails is
//               rejected before any weight is touched.
//   apply     : one workgroup per 8192-element block.  The block's old
//               weights are loaded into registers first, so HBM latency
//               overlaps the decode; occupancy (up to 6 workgroups per CU)
//               hides the rest.  The record is staged in LDS and
//               decoded into a dense 16 KiB XOR tile in LDS, checking that it
//               is canonical.  Then old ^ tile is formed, only the changed
//               16-byte chunks are written back, and the checksum terms of
//               the result are accumulated.
//   finalize  : one workgroup per job; reduces the checksum, compares it,
//               and writes the result.
//   rollback  : the apply kernel again, for the jobs that failed only.  XOR
//               is its own inverse, so this restores the old weights exactly.
#include "internal.hpp"

namespace bf16d {


__device__ __forceinline__ uint32_t block_length(uint64_t n, uint64_t b) {
    const uint64_t left = n - b * kBlock;
    return left < kBlock ? (uint32_t)left : kBlock;
}

// ---------------------------------------------------------------- desc_scan ---
__global__ __launch_bounds__(kThreads) void desc_scan_kernel(
    const DecompressJob *__restrict__ jobs, const uint32_t *__restrict__ dtile_job,
    uint64_t *__restrict__ dstatus, uint64_t *__restrict__ offsets,
    DecompressState *__restrict__ state, Control *__restrict__ ctrl) {
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
    const bool table_ok = job.payload_bytes >= kHeader + 4 * job.nb;

    uint32_t lens[kDescPerThread];
    uint32_t mine = 0, bad = table_ok ? 0u : 1u;
    unsigned long long c_sum = 0, r_sum = 0, pos_sum = 0, mant_sum = 0, nbm = 0;
#pragma unroll
    for (uint32_t k = 0; k < kDescPerThread; ++k) {
        const uint64_t d = ld * kDescTile + kDescPerThread * tid + k;
        lens[k] = 0;
        if (!table_ok || d >= job.nb) continue;
        const uint32_t desc =
            *reinterpret_cast<const uint32_t *>(job.payload + kHeader + 4 * d);
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
        bad |= (c > L) | (r > c);
        const uint32_t mb = (7 * c + 7) / 8;
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
    if (tid == 0) {
        DecompressState *st = &state[j];
        atomicAdd(&st->sum_c, c_sum);
        atomicAdd(&st->sum_r, r_sum);
        atomicAdd(&st->sum_pos, pos_sum);
        atomicAdd(&st->sum_mant, mant_sum);
        atomicAdd(&st->n_bitmap, nbm);
        if (any_bad) atomicOr(&st->desc_bad, 1u);
    }
}

// ------------------------------------------------------------------ prepare ---
__global__ void prepare_kernel(const DecompressJob *__restrict__ jobs,
                               DecompressState *__restrict__ state, uint32_t count) {
    const uint32_t j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= count) return;
    const DecompressJob job = jobs[j];
    DecompressState *st = &state[j];
    bool ok = job.payload_bytes >= kHeader;
    if (ok) {
        const uint32_t *h = reinterpret_cast<const uint32_t *>(job.payload);
        const uint64_t *h64 = reinterpret_cast<const uint64_t *>(job.payload);
        ok = h[0] == kMagicLo && h[1] == kMagicHi && h[2] == BF16D_FORMAT_VERSION &&
             h[3] == kBlock && h64[2] == job.n && job.payload_bytes >= kHeader + 4 * job.nb &&
             st->desc_bad == 0 && st->sum_c == h64[3] && st->sum_r == h64[4] &&
             st->sum_pos == h64[5] && st->sum_mant == h64[6] && 2 * st->sum_r == h64[7] &&
             kHeader + 4 * job.nb + st->sum_pos + st->sum_mant + 2 * st->sum_r ==
                 job.payload_bytes;
    }
    st->state = ok ? kStateReady : kStateRejected;
}

// -------------------------------------------------------------------- apply ---
// Records up to kStage bytes are staged in LDS; fields beyond are read from
// HBM (only dense blocks have larger records).
constexpr uint32_t kStage = 6144;
constexpr uint32_t kStageWords = kStage / 4;

// Bit reader over a record: bits [0, 8*kStage - 32) of the window come from
// LDS; later bits come from the payload in global memory.
struct RecordBits {
    const uint32_t *lds;        // staged dwords; window bit 0 = payload byte `a0`
    const uint8_t *payload;
    uint64_t a0;                // 4-aligned payload offset of the window
    uint64_t payload_bytes;
    uint32_t rb0;               // window bit of record bit 0

    __device__ __forceinline__ uint32_t get(uint32_t bitpos, uint32_t width) const {
        const uint32_t wb = rb0 + bitpos;
        const uint32_t d = wb >> 5, sh = wb & 31;
        uint64_t v;
        if (d + 1 < kStageWords) {
            v = (uint64_t)lds[d] | ((uint64_t)lds[d + 1] << 32);
        } else {
            v = 0;
            const uint64_t at = a0 + 4ull * d;
            for (uint32_t t = 0; t < 8; ++t)
                if (at + t < payload_bytes) v |= (uint64_t)payload[at + t] << (8 * t);
        }
        const uint64_t mask = (width >= 32) ? 0xFFFFFFFFull : ((1ull << width) - 1);
        return (uint32_t)((v >> sh) & mask);
    }
};

struct ApplyShared {
    uint32_t a[kWaves], b[kWaves], c[kWaves];
};

// Decode tile `tile` of job `j` and XOR it onto the weights.  s_x must be
// all zero on entry; it is all zero again on return.  kRollback: undo a
// previous pass (same decode, no checksum).
template <bool kRollback>
__device__ __forceinline__ void apply_tile(const DecompressJob &job, uint32_t j, uint64_t tile,
                                           DecompressState *__restrict__ state,
                                           const uint64_t *__restrict__ offsets,
                                           uint64_t *__restrict__ partial, uint16_t *s_x,
                                           uint32_t *s_raw, ApplyShared &sa) {
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t b = tile - job.block0;
    const uint64_t base = b * kBlock;
    const uint32_t L = block_length(job.n, b);

    // old weights first: their latency overlaps the decode
    uint4 o[kChunksPerThread];
#pragma unroll
    for (uint32_t i = 0; i < kChunksPerThread; ++i) {
        const uint32_t e0 = 8 * (tid + kThreads * i);
        o[i] = make_uint4(0, 0, 0, 0);
        if (e0 < L) o[i] = load_chunk(job.weights + base + e0, L - e0);
    }
    const uint32_t desc = *reinterpret_cast<const uint32_t *>(job.payload + kHeader + 4 * b);
    const uint32_t c = desc & 0x3FFFu, r = (desc >> 14) & 0x3FFFu, code = desc >> 28;
    const uint32_t pb = code == kCodeBitmap ? (L + 7) / 8 : (c * code + 7) / 8;
    const uint32_t mb = (7 * c + 7) / 8;
    const uint32_t len = pb + mb + 2 * r;
    const uint64_t D = kHeader + 4 * job.nb + offsets[tile];

    // stage the first kStage bytes of the record window
    RecordBits rb;
    rb.lds = s_raw;
    rb.payload = job.payload;
    rb.payload_bytes = job.payload_bytes;
    rb.rb0 = 8 * (uint32_t)(D & 3);
    rb.a0 = D & ~3ull;
    {
        const uint32_t nraw = (uint32_t)((D & 3) + len + 3) / 4 + 1;
        const uint32_t n_stage = nraw < kStageWords + 4 ? nraw : kStageWords + 4;
        for (uint32_t u = tid; u < n_stage; u += kThreads) {
            const uint64_t A = rb.a0 + 4ull * u;
            uint32_t v = 0;
            if (A + 4 <= job.payload_bytes) {
                v = *reinterpret_cast<const uint32_t *>(job.payload + A);
            } else {
                for (uint32_t t = 0; t < 4; ++t)
                    if (A + t < job.payload_bytes) v |= (uint32_t)job.payload[A + t] << (8 * t);
            }
            s_raw[u] = v;
        }
    }
    __syncthreads();   // record staged

    // ---- decode the record into s_x, checking that it is canonical ----
    const uint32_t mant0 = 8 * pb, rare0 = 8 * (pb + mb);
    uint32_t bad = 0;
    if (code == kCodeBitmap) {
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
        if (lane == 0) {
            sa.a[wave] = lane63(inc_pop);
            sa.b[wave] = lane63(inc_last);
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
                esc += rb.get(mant0 + 7 * jj, 7) == 0;
                ++jj;
            }
        }
        const uint32_t inc_esc = wave_incl_add(esc), wmax = lane63(wave_incl_max(maxg));
        __syncthreads();   // sa.a / sa.b reads done
        if (lane == 0) {
            sa.a[wave] = lane63(inc_esc);
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
            uint32_t x = rb.get(mant0 + 7 * jj, 7);
            if (x == 0) {
                if (e < r) {
                    x = rb.get(rare0 + 16 * e, 16);
                    bad |= (x & kExpSign) == 0;
                } else {
                    bad = 1;
                }
                ++e;
            }
            s_x[p] = (uint16_t)x;
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
            esc += rb.get(mant0 + 7 * jj, 7) == 0;
        }
        const uint32_t inc_g = wave_incl_add(sum_g1), inc_e = wave_incl_add(esc);
        const uint32_t wmax = lane63(wave_incl_max(maxg));
        if (lane == 0) {
            sa.a[wave] = lane63(inc_g);
            sa.b[wave] = lane63(inc_e);
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
            uint32_t x = rb.get(mant0 + 7 * jj, 7);
            if (x == 0) {
                if (e < r) {
                    x = rb.get(rare0 + 16 * e, 16);
                    bad |= (x & kExpSign) == 0;
                } else {
                    bad = 1;
                }
                ++e;
            }
            if (p < L) s_x[p] = (uint16_t)x; else bad = 1;
        }
        if (tid == 0 && 8 * pb > c * w)                  // position padding
            bad |= rb.get(c * w, 8 * pb - c * w) != 0;
    }
    if (tid == 0 && 8 * mb > 7 * c)                      // mantissa padding
        bad |= rb.get(mant0 + 7 * c, 8 * mb - 7 * c) != 0;
    bad = __syncthreads_or(bad);   // s_x complete

    // ---- new = old ^ tile; store only changed chunks; clear the tile ----
    uint64_t acc = 0;
    const uint64_t kg0 = ((base >> 2) + 1 + 2 * tid) * kGamma;
    constexpr uint64_t kRoundKg = (uint64_t)(2 * kThreads) * kGamma;
#pragma unroll
    for (uint32_t i = 0; i < kChunksPerThread; ++i) {
        const uint32_t q = tid + kThreads * i;
        const uint32_t e0 = 8 * q;
        const uint32_t valid = e0 < L ? (L - e0 < 8 ? L - e0 : 8) : 0;
        const uint4 t = reinterpret_cast<const uint4 *>(s_x)[q];
        const bool dirty = (t.x | t.y | t.z | t.w) != 0;
        uint4 nw = o[i];
        if (dirty) {
            reinterpret_cast<uint4 *>(s_x)[q] = make_uint4(0, 0, 0, 0);
            if (!bad) {
                nw = make_uint4(o[i].x ^ t.x, o[i].y ^ t.y, o[i].z ^ t.z, o[i].w ^ t.w);
                uint16_t *dstp = job.weights + base + e0;
                if (valid == 8) {
                    *reinterpret_cast<uint4 *>(dstp) = nw;
                } else {
                    for (uint32_t s = 0; s < valid; ++s) dstp[s] = (uint16_t)chunk_elem(nw, s);
                }
            }
        }
        if (!kRollback) {
            const uint64_t kg = kg0 + i * kRoundKg;
            if (valid > 0) acc += mix64(((uint64_t)nw.y << 32 | nw.x) ^ kg);
            if (valid > 4) acc += mix64(((uint64_t)nw.w << 32 | nw.z) ^ (kg + kGamma));
        }
    }
    if (!kRollback) {
        acc = wave_sum(acc);
        if (lane == 0) partial[kWaves * tile + wave] = acc;
        if (tid == 0 && bad) atomicOr(&state[j].block_bad, 1u);
    }
}

// The apply pass: one workgroup per tile of the jobs that passed the
// header and descriptor checks.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(6, 8)))
void apply_kernel(const DecompressJob *__restrict__ jobs, DecompressState *__restrict__ state,
                  const uint32_t *__restrict__ tile_job, const uint64_t *__restrict__ offsets,
                  uint64_t *__restrict__ partial) {
    __shared__ __attribute__((aligned(16))) uint16_t s_x[kBlock];   // dense XOR tile
    __shared__ uint32_t s_raw[kStageWords + 4];                       // staged record
    __shared__ ApplyShared sa;
    const uint64_t tile = blockIdx.x;
    const uint32_t j = tile_job[tile];
    if (state[j].state != kStateReady) return;
    for (uint32_t u = threadIdx.x; u < kBlock / 8; u += kThreads)
        reinterpret_cast<uint4 *>(s_x)[u] = make_uint4(0, 0, 0, 0);
    // (the barrier after staging orders this clearing before the decode)
    apply_tile<false>(jobs[j], j, tile, state, offsets, partial, s_x, s_raw, sa);
}

// The undo pass, for failed jobs only: a persistent grid that exits at once
// when nothing failed.
__global__ __launch_bounds__(kThreads) void rollback_kernel(
    const DecompressJob *__restrict__ jobs, DecompressState *__restrict__ state,
    const uint32_t *__restrict__ tile_job, const uint64_t *__restrict__ offsets,
    const Control *__restrict__ ctrl, uint64_t tiles) {
    __shared__ __attribute__((aligned(16))) uint16_t s_x[kBlock];
    __shared__ uint32_t s_raw[kStageWords + 4];
    __shared__ ApplyShared sa;
    if (ctrl->any_rollback == 0) return;
    for (uint32_t u = threadIdx.x; u < kBlock / 8; u += kThreads)
        reinterpret_cast<uint4 *>(s_x)[u] = make_uint4(0, 0, 0, 0);
    for (uint64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const uint32_t j = tile_job[tile];
        if (state[j].rollback == 0) continue;   // uniform across the workgroup
        apply_tile<true>(jobs[j], j, tile, state, offsets, nullptr, s_x, s_raw, sa);
        __syncthreads();   // LDS reused by the next tile
    }
}

// ----------------------------------------------------------------- finalize ---
__global__ __launch_bounds__(kThreads) void decompress_finalize_kernel(
    const DecompressJob *__restrict__ jobs, DecompressState *__restrict__ state,
    const uint64_t *__restrict__ partial, Control *__restrict__ ctrl,
    bf16d_result *__restrict__ results) {
    __shared__ unsigned long long s_tmp[kWaves];
    const uint32_t j = blockIdx.x;
    const DecompressJob job = jobs[j];
    DecompressState *st = &state[j];
    const bool ready = st->state == kStateReady;
    unsigned long long S = 0;
    if (ready)
        for (uint64_t b = threadIdx.x; b < job.nb; b += kThreads)
            for (uint32_t w = 0; w < kWaves; ++w) S += partial[kWaves * (job.block0 + b) + w];
    S = block_sum(S, s_tmp);
    if (threadIdx.x != 0) return;
    bf16d_result res;
    res.reserved = 0;
    res.payload_bytes = job.payload_bytes;
    if (!ready) {
        res.status = BF16D_EFORMAT;
        res.checksum = 0;
        res.n_changed = res.n_rare = res.n_bitmap_blocks = 0;
    } else {
        const uint64_t cs = mix64(S ^ job.n);
        res.status = st->block_bad ? BF16D_EFORMAT
                                   : (cs != job.checksum ? BF16D_ECHECKSUM : BF16D_OK);
        res.checksum = cs;
        res.n_changed = st->sum_c;
        res.n_rare = st->sum_r;
        res.n_bitmap_blocks = st->n_bitmap;
        if (res.status != BF16D_OK) {
            st->rollback = 1;
            atomicOr(&ctrl->any_rollback, 1u);
        }
    }
    results[j] = res;
}

hipError_t launch_decompress(const Layout &l, uint8_t *ws, uint32_t count, uint64_t tiles,
                             uint64_t dtiles, bf16d_result *results, hipStream_t stream,
                             const bf16d_events *events) {
    auto *ctrl = reinterpret_cast<Control *>(ws + l.control);
    auto *jobs = reinterpret_cast<const DecompressJob *>(ws + l.jobs);
    auto *bstart = reinterpret_cast<const uint64_t *>(ws + l.block_start);
    auto *dstart = reinterpret_cast<const uint64_t *>(ws + l.dtile_start);
    auto *map = reinterpret_cast<uint32_t *>(ws + l.tile_job);
    auto *offsets = reinterpret_cast<uint64_t *>(ws + l.status);
    auto *partial = reinterpret_cast<uint64_t *>(ws + l.partial);
    auto *dmap = reinterpret_cast<uint32_t *>(ws + l.dtile_job);
    auto *dstatus = reinterpret_cast<uint64_t *>(ws + l.dstatus);
    auto *state = reinterpret_cast<DecompressState *>(ws + l.state);

    launch_zero_words(reinterpret_cast<uint32_t *>(ctrl), sizeof(Control) / 4, stream);
    launch_zero_words(reinterpret_cast<uint32_t *>(state),
                      sizeof(DecompressState) / 4 * (uint64_t)count, stream);
    if (dtiles) {
        launch_map_tiles(dstart, count, dmap, dstatus, dtiles, stream);
        desc_scan_kernel<<<(uint32_t)dtiles, kThreads, 0, stream>>>(jobs, dmap, dstatus, offsets,
                                                                    state, ctrl);
    }
    prepare_kernel<<<(count + kThreads - 1) / kThreads, kThreads, 0, stream>>>(jobs, state,
                                                                               count);
    if (tiles) {
        launch_map_tiles(bstart, count, map, nullptr, tiles, stream);
        if (events && events->before && hipEventRecord(events->before, stream) != hipSuccess)
            return hipErrorInvalidValue;
        apply_kernel<<<(uint32_t)tiles, kThreads, 0, stream>>>(jobs, state, map, offsets, partial);
        if (events && events->after && hipEventRecord(events->after, stream) != hipSuccess)
            return hipErrorInvalidValue;
    }
    decompress_finalize_kernel<<<count, kThreads, 0, stream>>>(jobs, state, partial, ctrl,
                                                               results);
    if (tiles) {
        rollback_kernel<<<persistent_grid((const void *)rollback_kernel, tiles), kThreads, 0,
                          stream>>>(jobs, state, map, offsets, ctrl, tiles);
    }
    return hipGetLastError();
}

}  // namespace bf16d
