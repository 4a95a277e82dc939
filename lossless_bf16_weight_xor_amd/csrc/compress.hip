// compress.hip -- single-pass BF16 delta encoder for gfx950.
//
// One workgroup (256 threads = 4 waves of 64) encodes one 8192-element block
// of one job.  A batch of tensors is one grid: the tile-to-job map built by
// the setup kernel turns a tile index into (job, block).
//
// Per block, in one pass over HBM (old and new are each read once, the
// payload is written once):
//   1. 16-byte coalesced loads of old and new; x = old XOR new.  The XOR mask
//      of "GPU-accelerated Weight Teleportation", section "Delta update
//      algebra", lives only in registers and is never stored.
//   2. Classify each element: x == 0 is unchanged, (x & 0xFF80) == 0 is
//      mantissa-only, anything else is an exponent/sign change ("Every byte
//      counts: ARCv3 and the case for cross-region RL", section "Deep dive
//      into ARCv3").  The checksum terms of the new weights are accumulated
//      in the same pass.
//   3. Per-chunk counts, an LDS scan in element order, and compaction of the
//      changed positions into LDS.
//   4. Largest gap -> field width; the cheaper of gap list and bitmap.
//   5. Decoupled look-back (Merrill and Garland, "Single-pass Parallel
//      Prefix Scan with Decoupled Look-back", 2016) over the record sizes of
//      the job's blocks gives this record's byte offset.  The aggregate is
//      published before packing, so the look-back rarely waits.
//   6. The record (position | mantissa | rare segments) is built in LDS with
//      atomic ORs, one owner per field, so the bytes do not depend on
//      timing.  It is then stored with dword stores, plus byte stores at the
//      two ends it may share with neighbouring records.
// A finalize kernel then reduces the per-block statistics of each job into
// its header, its checksum and its result.
#include "internal.hpp"

namespace bf16d {

// Look-back by one wave: returns the exclusive prefix of tile `tile` over the
// tiles [first, tile) of its job.
__device__ uint64_t look_back(uint64_t *status, uint64_t tile, uint64_t first) {
    const int lane = threadIdx.x & 63;
    uint64_t excl = 0;
    int64_t pred = (int64_t)tile - 1;
    for (;;) {
        const int64_t idx = pred - lane;
        uint64_t v = kFlagPrefix;   // below the job's first tile: an empty inclusive prefix
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

__global__ __launch_bounds__(kThreads) void compress_kernel(
    const CompressJob *__restrict__ jobs, const uint32_t *__restrict__ tile_job,
    uint64_t *__restrict__ status, uint64_t *__restrict__ partial,
    uint32_t *__restrict__ desc_out, Control *__restrict__ ctrl) {
    __shared__ uint32_t s_pre[kChunks];                 // chunk counts, then prefixes
    __shared__ uint16_t s_pos[kBlock];                  // compacted changed positions
    __shared__ uint32_t s_rec[kMaxRecord / 4 + 4];      // record under construction
    __shared__ uint32_t s_tmp32[kWaves];
    __shared__ uint64_t s_tmp64[kWaves];
    __shared__ uint32_t s_tile;
    __shared__ uint64_t s_excl;

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63, wave = tid >> 6;

    // dynamic tile id: every smaller id belongs to a workgroup already running
    if (tid == 0)
        s_tile = __hip_atomic_fetch_add(&ctrl->ticket, 1u, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint64_t tile = s_tile;
    const CompressJob job = jobs[tile_job[tile]];
    const uint64_t b = tile - job.block0;
    const uint64_t base = b * kBlock;
    const uint64_t left = job.n - base;
    const uint32_t L = left < kBlock ? (uint32_t)left : kBlock;

    // 1-2: load, XOR, classify, checksum terms
    uint4 x[kChunksPerThread];
    uint32_t ch8[kChunksPerThread], rr8[kChunksPerThread];
    uint64_t acc = 0;
#pragma unroll
    for (uint32_t i = 0; i < kChunksPerThread; ++i) {
        const uint32_t q = tid + kThreads * i;
        const uint32_t e0 = 8 * q;
        uint4 o = make_uint4(0, 0, 0, 0), nw = make_uint4(0, 0, 0, 0);
        uint32_t valid = 0;
        if (e0 < L) {
            valid = L - e0 < 8 ? L - e0 : 8;
            o = load_chunk(job.src + base + e0, valid);
            nw = load_chunk(job.dst + base + e0, valid);
        }
        x[i] = make_uint4(o.x ^ nw.x, o.y ^ nw.y, o.z ^ nw.z, o.w ^ nw.w);
        acc += chunk_checksum(nw, base + e0, valid);
        uint32_t c8 = 0, r8 = 0;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const uint32_t xs = chunk_elem(x[i], s);
            c8 |= (xs != 0 ? 1u : 0u) << s;
            r8 |= ((xs & kExpSign) != 0 ? 1u : 0u) << s;
        }
        ch8[i] = c8;
        rr8[i] = r8;
        s_pre[q] = __popc(c8) | (__popc(r8) << 16);
    }
    __syncthreads();

    // 3: exclusive scan of (changed, rare) counts over chunks in element order
    uint32_t total;
    {
        uint32_t v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = s_pre[4 * tid + k];
        const uint32_t mine = v[0] + v[1] + v[2] + v[3];
        uint32_t excl = block_exclusive_sum(mine, s_tmp32, total);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            s_pre[4 * tid + k] = excl;
            excl += v[k];
        }
    }
    __syncthreads();
    const uint32_t c = total & 0xFFFFu;
    const uint32_t r = total >> 16;

    uint32_t pre[kChunksPerThread];
#pragma unroll
    for (uint32_t i = 0; i < kChunksPerThread; ++i) {
        const uint32_t q = tid + kThreads * i;
        pre[i] = s_pre[q];
        uint32_t bits = ch8[i], j = pre[i] & 0xFFFFu;
        while (bits) {
            s_pos[j++] = (uint16_t)(8 * q + __ffs(bits) - 1);
            bits &= bits - 1;
        }
    }
    __syncthreads();

    // 4: widest gap -> field width -> cheaper position encoding
    uint32_t maxgap = 0;
    for (uint32_t j = tid; j < c; j += kThreads) {
        const uint32_t g = j ? (uint32_t)s_pos[j] - s_pos[j - 1] - 1 : s_pos[0];
        maxgap = g > maxgap ? g : maxgap;
    }
    maxgap = block_max(maxgap, s_tmp32);
    const uint32_t w = bit_length(maxgap);
    const uint32_t delta_bytes = (c * w + 7) / 8;
    const uint32_t bitmap_bytes = (L + 7) / 8;
    const uint32_t code = bitmap_bytes < delta_bytes ? kCodeBitmap : w;
    const uint32_t pb = code == kCodeBitmap ? bitmap_bytes : delta_bytes;
    const uint32_t mb = (7 * c + 7) / 8;
    const uint32_t len = pb + mb + 2 * r;
    const uint32_t desc = c | (r << 14) | (code << 28);

    // 5a: publish this tile's aggregate (or, for a job's first tile, its prefix)
    if (tid == 0) st_agent(&status[tile], (b == 0 ? kFlagPrefix : kFlagAggregate) | len);

    // 6a: build the record in LDS
    const uint32_t rec_words = (len + 3) / 4 + 1;
    for (uint32_t u = tid; u < rec_words; u += kThreads) s_rec[u] = 0;
    __syncthreads();
    if (code == kCodeBitmap) {
#pragma unroll
        for (uint32_t i = 0; i < kChunksPerThread; ++i) {
            const uint32_t q = tid + kThreads * i;
            if (ch8[i]) atomicOr(&s_rec[q >> 2], ch8[i] << (8 * (q & 3)));
        }
    } else if (w > 0) {
        for (uint32_t j = tid; j < c; j += kThreads) {
            const uint32_t g = j ? (uint32_t)s_pos[j] - s_pos[j - 1] - 1 : s_pos[0];
            lds_or_bits(s_rec, j * w, g, w);
        }
    }
    const uint32_t mant_bit = 8 * pb, rare_bit = 8 * (pb + mb);
#pragma unroll
    for (uint32_t i = 0; i < kChunksPerThread; ++i) {
        uint32_t bits = ch8[i];
        uint32_t j = pre[i] & 0xFFFFu, k = pre[i] >> 16;
        while (bits) {
            const int s = __ffs(bits) - 1;
            bits &= bits - 1;
            const uint32_t xs = chunk_elem(x[i], s);
            if (xs & kExpSign) {
                lds_or_bits(s_rec, rare_bit + 16 * k, xs, 16);
                ++k;
            } else {
                lds_or_bits(s_rec, mant_bit + 7 * j, xs & kMant, 7);
            }
            ++j;
        }
    }

    // 5b: look back for the record's offset within the job's data region
    if (wave == 0) {
        const uint64_t excl = (b == 0) ? 0 : look_back(status, tile, job.block0);
        if (lane == 0) {
            if (b != 0) st_agent(&status[tile], kFlagPrefix | (excl + len));
            s_excl = excl;
        }
    }
    __syncthreads();

    // 6b: store descriptor and record, never at or beyond capacity
    uint8_t *const pay = job.payload;
    const uint64_t cap = job.capacity;
    if (tid == 0) {
        const uint64_t at = kHeader + 4 * b;
        if (at + 4 <= cap) *reinterpret_cast<uint32_t *>(pay + at) = desc;
        desc_out[tile] = desc;
    }
    const uint64_t D = kHeader + 4 * job.nb + s_excl;   // record start in the payload
    const uint32_t sh = (uint32_t)(D & 3);
    const uint64_t a0 = D - sh;
    const uint32_t words = (sh + len + 3) / 4;
    for (uint32_t u = tid; u < words; u += kThreads) {
        const uint32_t hi = s_rec[u];
        const uint32_t lo = u ? s_rec[u - 1] : 0u;
        const uint32_t v = sh ? ((hi << (8 * sh)) | (lo >> (32 - 8 * sh))) : hi;
        const uint64_t A = a0 + 4ull * u;
        if (A >= D && A + 4 <= D + len && A + 4 <= cap) {
            *reinterpret_cast<uint32_t *>(pay + A) = v;
        } else {
#pragma unroll
            for (uint32_t t = 0; t < 4; ++t) {
                const uint64_t at = A + t;
                if (at >= D && at < D + len && at < cap) pay[at] = (uint8_t)(v >> (8 * t));
            }
        }
    }

    // per-tile checksum partial sum (mod 2^64)
    acc = block_sum(acc, s_tmp64);
    if (tid == 0) partial[tile] = acc;
}

// One workgroup per job: header, checksum and result.
__global__ __launch_bounds__(kThreads) void compress_finalize_kernel(
    const CompressJob *__restrict__ jobs, const uint32_t *__restrict__ desc,
    const uint64_t *__restrict__ partial, bf16d_result *__restrict__ results) {
    __shared__ unsigned long long s_tmp[kWaves];
    const CompressJob job = jobs[blockIdx.x];
    unsigned long long S = 0, c = 0, r = 0, pos = 0, mant = 0, nbm = 0;
    for (uint64_t b = threadIdx.x; b < job.nb; b += kThreads) {
        const uint32_t d = desc[job.block0 + b];
        const uint64_t left = job.n - b * kBlock;
        const uint32_t L = left < kBlock ? (uint32_t)left : kBlock;
        const uint32_t cb = d & 0x3FFFu, rb = (d >> 14) & 0x3FFFu, code = d >> 28;
        S += partial[job.block0 + b];
        c += cb;
        r += rb;
        pos += code == kCodeBitmap ? (L + 7) / 8 : (cb * code + 7) / 8;
        mant += (7 * cb + 7) / 8;
        nbm += code == kCodeBitmap;
    }
    S = block_sum(S, s_tmp);
    c = block_sum(c, s_tmp);
    r = block_sum(r, s_tmp);
    pos = block_sum(pos, s_tmp);
    mant = block_sum(mant, s_tmp);
    nbm = block_sum(nbm, s_tmp);
    if (threadIdx.x != 0) return;
    const uint64_t rare = 2 * r;
    const uint64_t P = kHeader + 4 * job.nb + pos + mant + rare;
    const int status = P <= job.capacity ? BF16D_OK : BF16D_ECAPACITY;
    if (status == BF16D_OK) {
        uint32_t *h = reinterpret_cast<uint32_t *>(job.payload);
        uint64_t *h64 = reinterpret_cast<uint64_t *>(job.payload);
        h[0] = kMagicLo;
        h[1] = kMagicHi;
        h[2] = BF16D_FORMAT_VERSION;
        h[3] = kBlock;
        h64[2] = job.n;
        h64[3] = c;
        h64[4] = r;
        h64[5] = pos;
        h64[6] = mant;
        h64[7] = rare;
    }
    bf16d_result res;
    res.status = status;
    res.reserved = 0;
    res.payload_bytes = P;
    res.checksum = mix64(S ^ job.n);
    res.n_changed = c;
    res.n_rare = r;
    res.n_bitmap_blocks = nbm;
    results[blockIdx.x] = res;
}

hipError_t launch_compress(const Layout &l, uint8_t *ws, uint32_t count, uint64_t tiles,
                           bf16d_result *results, hipStream_t stream) {
    auto *ctrl = reinterpret_cast<Control *>(ws + l.control);
    auto *jobs = reinterpret_cast<const CompressJob *>(ws + l.jobs);
    auto *start = reinterpret_cast<const uint64_t *>(ws + l.block_start);
    auto *map = reinterpret_cast<uint32_t *>(ws + l.tile_job);
    auto *status = reinterpret_cast<uint64_t *>(ws + l.status);
    auto *partial = reinterpret_cast<uint64_t *>(ws + l.partial);
    auto *desc = reinterpret_cast<uint32_t *>(ws + l.desc);

    launch_zero_words(reinterpret_cast<uint32_t *>(ctrl), sizeof(Control) / 4, stream);
    if (tiles) {
        launch_map_tiles(start, count, map, status, tiles, stream);
        compress_kernel<<<(uint32_t)tiles, kThreads, 0, stream>>>(jobs, map, status, partial,
                                                                  desc, ctrl);
    }
    compress_finalize_kernel<<<count, kThreads, 0, stream>>>(jobs, desc, partial, results);
    return hipGetLastError();
}

}  // namespace bf16d
