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
//               overlaps the decode.  The record is staged in LDS and
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

__device__ uint64_t look_back_d(uint64_t *status, uint64_t tile, uint64_t first) {
    const int lane = threadIdx.x & 63;
    uint64_t excl = 0;
    int64_t pred = (int64_t)tile - 1;
    for (;;) {
        const int64_t idx = pred - lane;
        uint64_t v = kFlagPrefix;
        if (idx >= (int64_t)first) {
            v = ld_acquire_agent(&status[idx]);
            while ((v >> 62) == 0) {
                __builtin_amdgcn_s_sleep(1);
                v = ld_acquire_agent(&status[idx]);
            }
        }
        const uint64_t pmask = __ballot((v >> 62) == 2);
        const int stop = pmask ? __ffsll((unsigned long long)pmask) - 1 : 63;
        const uint64_t mine = (lane <= stop) ? (v & kValueMask) : 0;
        excl += wave_sum(mine);
        if (pmask) return excl;
        pred -= 64;
    }
}

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
        const uint64_t e = (ld == 0) ? 0 : look_back_d(dstatus, dt, job.dtile0);
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
template <bool kRollback>
__global__ __launch_bounds__(kThreads) void apply_kernel(
    const DecompressJob *__restrict__ jobs, DecompressState *__restrict__ state,
    const uint32_t *__restrict__ tile_job, const uint64_t *__restrict__ offsets,
    uint64_t *__restrict__ partial, const Control *__restrict__ ctrl, uint64_t tiles) {
    __shared__ __attribute__((aligned(16))) uint16_t s_x[kBlock];   // dense XOR tile
    __shared__ uint32_t s_raw[kMaxRecord / 4 + 4];                    // staged record
    __shared__ uint32_t s_tmp32[kWaves];
    __shared__ int s_tmpi[kWaves];
    __shared__ unsigned long long s_tmp64[kWaves];

    if (kRollback && ctrl->any_rollback == 0) return;
    const uint32_t tid = threadIdx.x;

    for (uint64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const uint32_t j = tile_job[tile];
        if (kRollback ? state[j].rollback == 0 : state[j].state != kStateReady) continue;
        const DecompressJob job = jobs[j];
        const uint64_t b = tile - job.block0;
        const uint64_t base = b * kBlock;
        const uint32_t L = block_length(job.n, b);

        // old weights first: their latency overlaps the decode below
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
        const uint32_t sh = (uint32_t)(D & 3);
        const uint64_t a0 = D - sh;
        const uint32_t nraw = (sh + len + 3) / 4;
        for (uint32_t u = tid; u <= nraw; u += kThreads) {
            const uint64_t A = a0 + 4ull * u;
            uint32_t v = 0;
            if (A + 4 <= job.payload_bytes) {
                v = *reinterpret_cast<const uint32_t *>(job.payload + A);
            } else {
                for (uint32_t t = 0; t < 4; ++t)
                    if (A + t < job.payload_bytes) v |= (uint32_t)job.payload[A + t] << (8 * t);
            }
            s_raw[u] = v;
        }
        for (uint32_t u = tid; u < kBlock / 8; u += kThreads)
            reinterpret_cast<uint4 *>(s_x)[u] = make_uint4(0, 0, 0, 0);
        __syncthreads();

        // ---- decode the record into s_x, checking that it is canonical ----
        const uint32_t rb0 = 8 * sh;                      // record bit 0 within s_raw
        const uint32_t mant0 = rb0 + 8 * pb;              // first mantissa field
        const uint32_t rare0 = rb0 + 8 * (pb + mb);       // first rare word
        uint32_t bad = 0;
        if (code == kCodeBitmap) {
            // thread t owns bitmap bits [32t, 32t + 32) = elements 32t .. 32t+31
            const uint32_t lo = 32 * tid, seg_end = 8 * pb;
            uint32_t word = 0;
            if (lo < seg_end) {
                word = lds_get_bits(s_raw, rb0 + lo, 32);
                if (lo + 32 > seg_end) word &= (1u << (seg_end - lo)) - 1;
            }
            const uint32_t valid_mask =
                lo + 32 <= L ? 0xFFFFFFFFu : (lo >= L ? 0u : (1u << (L - lo)) - 1);
            bad |= (word & ~valid_mask) != 0;               // pad bits must be zero
            word &= valid_mask;
            uint32_t total;
            const uint32_t rank0 = block_exclusive_sum((uint32_t)__popc(word), s_tmp32, total);
            bad |= total != c;
            // the gap before each set bit -> the minimal gap-list width
            const int my_last = word ? (int)(lo + 31 - __clz(word)) : -1;
            int prev = block_exclusive_max(my_last, -1, s_tmpi);
            uint32_t maxg = 0, esc = 0;
            {
                uint32_t bits = word, jj = rank0;
                while (bits) {
                    const int p = (int)lo + __ffs(bits) - 1;
                    bits &= bits - 1;
                    const uint32_t g = (uint32_t)(p - prev - 1);
                    maxg = g > maxg ? g : maxg;
                    prev = p;
                    esc += lds_get_bits(s_raw, mant0 + 7 * jj, 7) == 0;
                    ++jj;
                }
            }
            maxg = block_max(maxg, s_tmp32);
            bad |= !(pb < (c * bit_length(maxg) + 7) / 8);
            uint32_t esc_total;
            uint32_t e = block_exclusive_sum(esc, s_tmp32, esc_total);
            bad |= esc_total != r;
            uint32_t bits = word, jj = rank0;
            while (bits) {
                const uint32_t p = lo + __ffs(bits) - 1;
                bits &= bits - 1;
                uint32_t x = lds_get_bits(s_raw, mant0 + 7 * jj, 7);
                if (x == 0) {
                    if (e < r) {
                        x = lds_get_bits(s_raw, rare0 + 16 * e, 16);
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
                const uint32_t g = w ? lds_get_bits(s_raw, rb0 + jj * w, w) : 0;
                sum_g1 += g + 1;
                maxg = g > maxg ? g : maxg;
                esc += lds_get_bits(s_raw, mant0 + 7 * jj, 7) == 0;
            }
            unsigned long long total;
            const unsigned long long ex = block_exclusive_sum(
                (unsigned long long)sum_g1 | ((unsigned long long)esc << 32), s_tmp64, total);
            const uint32_t total_g1 = (uint32_t)total, esc_total = (uint32_t)(total >> 32);
            bad |= (c > 0) && (total_g1 - 1 >= L);         // last position inside the block
            bad |= esc_total != r;
            maxg = block_max(maxg, s_tmp32);
            bad |= bit_length(maxg) != w;
            uint32_t run = (uint32_t)ex, e = (uint32_t)(ex >> 32);
            for (uint32_t jj = jb; jj < je; ++jj) {
                const uint32_t g = w ? lds_get_bits(s_raw, rb0 + jj * w, w) : 0;
                run += g + 1;
                const uint32_t p = run - 1;
                uint32_t x = lds_get_bits(s_raw, mant0 + 7 * jj, 7);
                if (x == 0) {
                    if (e < r) {
                        x = lds_get_bits(s_raw, rare0 + 16 * e, 16);
                        bad |= (x & kExpSign) == 0;
                    } else {
                        bad = 1;
                    }
                    ++e;
                }
                if (p < L) s_x[p] = (uint16_t)x; else bad = 1;
            }
            if (tid == 0 && 8 * pb > c * w)                  // position padding
                bad |= lds_get_bits(s_raw, rb0 + c * w, 8 * pb - c * w) != 0;
        }
        if (tid == 0 && 8 * mb > 7 * c)                      // mantissa padding
            bad |= lds_get_bits(s_raw, mant0 + 7 * c, 8 * mb - 7 * c) != 0;
        bad = __syncthreads_or(bad);

        // ---- new = old ^ tile; store only the chunks that changed ----
        unsigned long long acc = 0;
        if (!bad) {
#pragma unroll
            for (uint32_t i = 0; i < kChunksPerThread; ++i) {
                const uint32_t q = tid + kThreads * i;
                const uint32_t e0 = 8 * q;
                if (e0 >= L) continue;
                const uint32_t valid = L - e0 < 8 ? L - e0 : 8;
                const uint4 t = reinterpret_cast<const uint4 *>(s_x)[q];
                uint4 nw = o[i];
                if ((t.x | t.y | t.z | t.w) != 0) {
                    nw = make_uint4(o[i].x ^ t.x, o[i].y ^ t.y, o[i].z ^ t.z, o[i].w ^ t.w);
                    uint16_t *dstp = job.weights + base + e0;
                    if (valid == 8) {
                        *reinterpret_cast<uint4 *>(dstp) = nw;
                    } else {
                        for (uint32_t s = 0; s < valid; ++s) dstp[s] = (uint16_t)chunk_elem(nw, s);
                    }
                }
                if (!kRollback) acc += chunk_checksum(nw, base + e0, valid);
            }
        }
        if (!kRollback) {
            acc = block_sum(acc, s_tmp64);
            if (tid == 0) {
                partial[tile] = acc;
                if (bad) atomicOr(&state[j].block_bad, 1u);
            }
        }
        __syncthreads();   // LDS is reused by the next tile of this workgroup
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
        for (uint64_t b = threadIdx.x; b < job.nb; b += kThreads) S += partial[job.block0 + b];
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
                             uint64_t dtiles, bf16d_result *results, hipStream_t stream) {
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
        apply_kernel<false><<<(uint32_t)tiles, kThreads, 0, stream>>>(jobs, state, map, offsets,
                                                                      partial, ctrl, tiles);
    }
    decompress_finalize_kernel<<<count, kThreads, 0, stream>>>(jobs, state, partial, ctrl,
                                                               results);
    if (tiles) {
        const uint32_t grid = (uint32_t)(tiles < 2048 ? tiles : 2048);
        apply_kernel<true><<<grid, kThreads, 0, stream>>>(jobs, state, map, offsets, partial,
                                                          ctrl, tiles);
    }
    return hipGetLastError();
}

}  // namespace bf16d
