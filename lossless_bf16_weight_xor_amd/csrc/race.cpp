// race.cpp -- the per-tensor codec race, on the host.
//
// "Every byte counts: ARCv3 and the case for cross-region RL", section "Deep
// dive into ARCv3": every tensor's structured output is also handed to
// several general-purpose compressors at once on the CPU, and the smallest
// result is kept.  Trainer hosts have idle cores while the GPUs train, so the
// extra CPU is spent where it is cheap.
//
// The codecs are reached through their public C APIs in the system's runtime
// libraries, opened with dlopen on first use: no headers are needed to build,
// and a host without one of them only loses that codec.  The prototypes below
// are those APIs' documented signatures (enums passed as int).
#include <dlfcn.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <memory>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

#include "bf16delta.h"

namespace {

constexpr uint64_t kFrameHeader = BF16D_RACE_FRAME_HEADER;
constexpr char kFrameMagic[8] = {'B', 'F', '1', '6', 'D', 'R', 'C', '1'};
constexpr uint64_t kLz4MaxInput = 0x7E000000ull;
constexpr uint32_t kMaxCandidates = 64;
constexpr uint32_t kMaxThreads = 1024;
constexpr uint32_t kCodecs = 7;

struct Codecs {
    // zstd
    size_t (*zstd_compress)(void *, size_t, const void *, size_t, int) = nullptr;
    size_t (*zstd_decompress)(void *, size_t, const void *, size_t) = nullptr;
    unsigned (*zstd_is_error)(size_t) = nullptr;
    // LZ4 and LZ4-HC (one library)
    int (*lz4_compress_fast)(const char *, char *, int, int, int) = nullptr;
    int (*lz4_compress_hc)(const char *, char *, int, int, int) = nullptr;
    int (*lz4_decompress_safe)(const char *, char *, int, int) = nullptr;
    // zlib
    int (*z_compress2)(unsigned char *, unsigned long *, const unsigned char *, unsigned long,
                       int) = nullptr;
    int (*z_uncompress)(unsigned char *, unsigned long *, const unsigned char *,
                        unsigned long) = nullptr;
    // Brotli
    int (*br_compress)(int, int, int, size_t, const uint8_t *, size_t *, uint8_t *) = nullptr;
    int (*br_decompress)(size_t, const uint8_t *, size_t *, uint8_t *) = nullptr;
    // xz
    int (*xz_encode)(uint32_t, int, const void *, const uint8_t *, size_t, uint8_t *, size_t *,
                     size_t) = nullptr;
    int (*xz_decode)(uint64_t *, uint32_t, const void *, const uint8_t *, size_t *, size_t,
                     uint8_t *, size_t *, size_t) = nullptr;

    bool have[kCodecs] = {true, false, false, false, false, false, false};
};

template <class F>
bool bind(void *h, const char *name, F &fn) {
    fn = h ? reinterpret_cast<F>(dlsym(h, name)) : nullptr;
    return fn != nullptr;
}

void *open_lib(const char *name) { return dlopen(name, RTLD_NOW | RTLD_LOCAL); }

const Codecs &codecs() {
    static Codecs c;
    static std::once_flag once;
    std::call_once(once, [] {
        void *h = open_lib("libzstd.so.1");
        c.have[BF16D_CODEC_ZSTD] = bind(h, "ZSTD_compress", c.zstd_compress) &&
                                   bind(h, "ZSTD_decompress", c.zstd_decompress) &&
                                   bind(h, "ZSTD_isError", c.zstd_is_error);
        h = open_lib("liblz4.so.1");
        const bool lz4_dec = bind(h, "LZ4_decompress_safe", c.lz4_decompress_safe);
        c.have[BF16D_CODEC_LZ4] = bind(h, "LZ4_compress_fast", c.lz4_compress_fast) && lz4_dec;
        c.have[BF16D_CODEC_LZ4HC] = bind(h, "LZ4_compress_HC", c.lz4_compress_hc) && lz4_dec;
        h = open_lib("libz.so.1");
        c.have[BF16D_CODEC_ZLIB] =
            bind(h, "compress2", c.z_compress2) && bind(h, "uncompress", c.z_uncompress);
        void *he = open_lib("libbrotlienc.so.1"), *hd = open_lib("libbrotlidec.so.1");
        c.have[BF16D_CODEC_BROTLI] = bind(he, "BrotliEncoderCompress", c.br_compress) &&
                                     bind(hd, "BrotliDecoderDecompress", c.br_decompress);
        h = open_lib("liblzma.so.5");
        c.have[BF16D_CODEC_XZ] = bind(h, "lzma_easy_buffer_encode", c.xz_encode) &&
                                 bind(h, "lzma_stream_buffer_decode", c.xz_decode);
    });
    return c;
}

bool level_ok(uint32_t codec, int32_t level) {
    switch (codec) {
        case BF16D_CODEC_STORED: return level == 0;
        case BF16D_CODEC_ZSTD: return level >= -5 && level <= 22;
        case BF16D_CODEC_LZ4: return level >= 1 && level <= 65537;
        case BF16D_CODEC_LZ4HC: return level >= 1 && level <= 12;
        case BF16D_CODEC_ZLIB: return level >= 1 && level <= 9;
        case BF16D_CODEC_BROTLI: return level >= 0 && level <= 11;
        case BF16D_CODEC_XZ: return level >= 0 && level <= 6;
        default: return false;
    }
}

// Compress in[0, n) into out[0, cap).  Returns the body size, or 0 when the
// codec fails or its output does not fit (then the candidate loses).
uint64_t encode(const Codecs &c, uint32_t codec, int32_t level, const uint8_t *in, uint64_t n,
                uint8_t *out, uint64_t cap) {
    switch (codec) {
        case BF16D_CODEC_ZSTD: {
            const size_t r = c.zstd_compress(out, cap, in, n, level);
            return c.zstd_is_error(r) ? 0 : r;
        }
        case BF16D_CODEC_LZ4:
        case BF16D_CODEC_LZ4HC: {
            if (n >= kLz4MaxInput) return 0;
            const int dcap = int(std::min<uint64_t>(cap, 0x7FFFFFFFull));
            const int r = codec == BF16D_CODEC_LZ4
                              ? c.lz4_compress_fast(reinterpret_cast<const char *>(in),
                                                    reinterpret_cast<char *>(out), int(n), dcap,
                                                    level)
                              : c.lz4_compress_hc(reinterpret_cast<const char *>(in),
                                                  reinterpret_cast<char *>(out), int(n), dcap,
                                                  level);
            return r > 0 ? uint64_t(r) : 0;
        }
        case BF16D_CODEC_ZLIB: {
            unsigned long len = cap;
            return c.z_compress2(out, &len, in, n, level) == 0 ? len : 0;
        }
        case BF16D_CODEC_BROTLI: {
            size_t len = cap;
            return c.br_compress(level, 22, 0, n, in, &len, out) == 1 ? len : 0;
        }
        case BF16D_CODEC_XZ: {
            size_t pos = 0;
            return c.xz_encode(uint32_t(level), 1, nullptr, in, n, out, &pos, cap) == 0 ? pos : 0;
        }
        default: return 0;
    }
}

// Decode a body of `n` bytes into exactly `raw` bytes at out.
bool decode(const Codecs &c, uint32_t codec, const uint8_t *in, uint64_t n, uint8_t *out,
            uint64_t raw) {
    switch (codec) {
        case BF16D_CODEC_STORED:
            if (n != raw) return false;
            if (n) std::memcpy(out, in, n);
            return true;
        case BF16D_CODEC_ZSTD: {
            const size_t r = c.zstd_decompress(out, raw, in, n);
            return !c.zstd_is_error(r) && r == raw;
        }
        case BF16D_CODEC_LZ4:
        case BF16D_CODEC_LZ4HC: {
            if (raw >= kLz4MaxInput || n > 0x7FFFFFFFull) return false;
            const int r = c.lz4_decompress_safe(reinterpret_cast<const char *>(in),
                                                reinterpret_cast<char *>(out), int(n), int(raw));
            return r >= 0 && uint64_t(r) == raw;
        }
        case BF16D_CODEC_ZLIB: {
            unsigned long len = raw;
            return c.z_uncompress(out, &len, in, n) == 0 && len == raw;
        }
        case BF16D_CODEC_BROTLI: {
            size_t len = raw;
            return c.br_decompress(n, in, &len, out) == 1 && len == raw;
        }
        case BF16D_CODEC_XZ: {
            uint64_t memlimit = ~uint64_t(0);
            size_t in_pos = 0, out_pos = 0;
            return c.xz_decode(&memlimit, 0, nullptr, in, &in_pos, n, out, &out_pos, raw) == 0 &&
                   in_pos == n && out_pos == raw;
        }
        default: return false;
    }
}

// Hash of the raw bytes, so that a body a codec decodes without complaint but
// to other bytes is still caught: mix64(S ^ n), S the sum mod 2^64 of
// mix64(W_k ^ (k + 1) * 0x9E3779B97F4A7C15) over the little-endian 64-bit
// words W_k of the bytes (the last one zero-padded), mix64 the SplitMix64
// finaliser (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", 2014).
uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

uint64_t raw_hash(const uint8_t *p, uint64_t n) {
    constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
    uint64_t S = 0, k = 0;
    for (; 8 * k + 8 <= n; ++k) {
        uint64_t w;
        std::memcpy(&w, p + 8 * k, 8);
        S += mix64(w ^ ((k + 1) * kGamma));
    }
    if (8 * k < n) {
        uint64_t w = 0;
        std::memcpy(&w, p + 8 * k, n - 8 * k);
        S += mix64(w ^ ((k + 1) * kGamma));
    }
    return mix64(S ^ n);
}

void put_header(uint8_t *f, uint32_t codec, int32_t level, uint64_t raw, uint64_t hash) {
    std::memcpy(f, kFrameMagic, 8);
    std::memcpy(f + 8, &codec, 4);
    std::memcpy(f + 12, &level, 4);
    std::memcpy(f + 16, &raw, 8);
    std::memcpy(f + 24, &hash, 8);
}

// Runs task(i) for i in [0, n) on up to `threads` threads (the caller's
// thread is one of them).
template <class Task>
void run_parallel(uint32_t threads, size_t n, Task task) {
    if (threads == 0) threads = std::max(1u, std::thread::hardware_concurrency());
    threads = uint32_t(std::min<size_t>(std::min<uint32_t>(threads, kMaxThreads), n));
    std::atomic<size_t> next{0};
    auto worker = [&] {
        for (size_t i; (i = next.fetch_add(1)) < n;) task(i);
    };
    std::vector<std::thread> pool;
    for (uint32_t t = 1; t < threads; ++t) {
        try {
            pool.emplace_back(worker);
        } catch (...) {
            break;  // fewer threads: the remaining ones take all the work
        }
    }
    worker();
    for (auto &th : pool) th.join();
}

struct Best {
    std::mutex m;
    uint64_t body = 0;      // body bytes of the best frame so far
    uint32_t rank = 0;      // 0: stored; k + 1: candidate k
};

}  // namespace

extern "C" {

int bf16d_codec_available(uint32_t codec) {
    return codec < kCodecs && codecs().have[codec] ? 1 : 0;
}

uint64_t bf16d_race_bound(uint64_t bytes) { return kFrameHeader + bytes; }

int bf16d_race_compress(bf16d_race_job *jobs, uint32_t count, const bf16d_codec *candidates,
                        uint32_t n_candidates, uint32_t threads) {
    if (!jobs || (n_candidates && !candidates) || n_candidates > kMaxCandidates ||
        threads > kMaxThreads)
        return BF16D_EINVAL;
    const Codecs &c = codecs();
    for (uint32_t k = 0; k < n_candidates; ++k) {
        const bf16d_codec &cd = candidates[k];
        if (cd.codec >= kCodecs || !level_ok(cd.codec, cd.level) || !c.have[cd.codec])
            return BF16D_EINVAL;
    }
    for (uint32_t j = 0; j < count; ++j) {
        const bf16d_race_job &J = jobs[j];
        if ((J.in_bytes && !J.in) || !J.out || J.out_capacity < bf16d_race_bound(J.in_bytes))
            return BF16D_EINVAL;
    }
    std::vector<Best> best(count);
    std::vector<uint64_t> hash(count);
    for (uint32_t j = 0; j < count; ++j) best[j].body = jobs[j].in_bytes;
    // every (job, candidate) pair, largest inputs first
    std::vector<uint32_t> order(count);
    for (uint32_t j = 0; j < count; ++j) order[j] = j;
    std::stable_sort(order.begin(), order.end(), [&](uint32_t a, uint32_t b) {
        return jobs[a].in_bytes > jobs[b].in_bytes;
    });
    // task i < count hashes job order[i]; the rest race (job, candidate) pairs
    const size_t tasks = size_t(count) * (n_candidates + 1);
    run_parallel(threads, tasks, [&](size_t i) {
        if (i < count) {
            hash[order[i]] = raw_hash(jobs[order[i]].in, jobs[order[i]].in_bytes);
            return;
        }
        i -= count;
        const uint32_t j = order[i / n_candidates], k = uint32_t(i % n_candidates);
        const bf16d_race_job &J = jobs[j];
        if (J.in_bytes == 0) return;
        std::unique_ptr<uint8_t[]> scratch(new (std::nothrow) uint8_t[J.in_bytes]);
        if (!scratch) return;  // no memory for this candidate: it loses
        // only a body smaller than the raw input can win
        const uint64_t body = encode(c, candidates[k].codec, candidates[k].level, J.in,
                                     J.in_bytes, scratch.get(), J.in_bytes);
        if (body == 0) return;
        Best &b = best[j];
        std::lock_guard<std::mutex> lock(b.m);
        if (body < b.body || (body == b.body && b.rank != 0 && k + 1 < b.rank)) {
            std::memcpy(J.out + kFrameHeader, scratch.get(), body);
            b.body = body;
            b.rank = k + 1;
        }
    });
    for (uint32_t j = 0; j < count; ++j) {
        bf16d_race_job &J = jobs[j];
        const Best &b = best[j];
        const uint32_t codec = b.rank ? candidates[b.rank - 1].codec : BF16D_CODEC_STORED;
        const int32_t level = b.rank ? candidates[b.rank - 1].level : 0;
        if (!b.rank && J.in_bytes) std::memcpy(J.out + kFrameHeader, J.in, J.in_bytes);
        put_header(J.out, codec, level, J.in_bytes, hash[j]);
        J.out_bytes = kFrameHeader + b.body;
        J.codec = codec;
        J.level = level;
        J.status = BF16D_OK;
    }
    return BF16D_OK;
}

int bf16d_race_frame_info(const uint8_t *frame, uint64_t frame_bytes, uint64_t *raw_bytes,
                          uint32_t *codec, int32_t *level) {
    if (!frame || frame_bytes < kFrameHeader || std::memcmp(frame, kFrameMagic, 8) != 0)
        return BF16D_EFORMAT;
    uint32_t cd;
    int32_t lv;
    uint64_t raw;
    std::memcpy(&cd, frame + 8, 4);
    std::memcpy(&lv, frame + 12, 4);
    std::memcpy(&raw, frame + 16, 8);
    if (cd >= kCodecs || !level_ok(cd, lv)) return BF16D_EFORMAT;
    if (raw_bytes) *raw_bytes = raw;
    if (codec) *codec = cd;
    if (level) *level = lv;
    return BF16D_OK;
}

int bf16d_race_decompress(bf16d_race_job *jobs, uint32_t count, uint32_t threads) {
    if (!jobs || threads > kMaxThreads) return BF16D_EINVAL;
    for (uint32_t j = 0; j < count; ++j)
        if ((jobs[j].in_bytes && !jobs[j].in) || (jobs[j].out_capacity && !jobs[j].out))
            return BF16D_EINVAL;
    const Codecs &c = codecs();
    run_parallel(threads, count, [&](size_t j) {
        bf16d_race_job &J = jobs[j];
        J.out_bytes = 0;
        uint64_t raw = 0;
        uint32_t codec = 0;
        int32_t level = 0;
        if (bf16d_race_frame_info(J.in, J.in_bytes, &raw, &codec, &level) != BF16D_OK) {
            J.status = BF16D_EFORMAT;
            return;
        }
        J.codec = codec;
        J.level = level;
        if (!c.have[codec]) {
            J.status = BF16D_ECODEC;
        } else if (J.out_capacity < raw) {
            J.status = BF16D_ECAPACITY;
        } else if (uint8_t none = 0; !decode(c, codec, J.in + kFrameHeader,
                                             J.in_bytes - kFrameHeader, raw ? J.out : &none,
                                             raw)) {
            J.status = BF16D_EFORMAT;
        } else if (uint64_t want; std::memcpy(&want, J.in + 24, 8), raw_hash(J.out, raw) != want) {
            J.status = BF16D_EFORMAT;   // decoded, but not to the bytes that were framed
        } else {
            J.out_bytes = raw;
            J.status = BF16D_OK;
        }
    });
    return BF16D_OK;
}

}  // extern "C"
