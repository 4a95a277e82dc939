// probe.hip -- measurement aids, not steps of the method.
//
// Both take the blocks in the main kernels' order: each XCD (workgroup index
// mod 8) a contiguous range of blocks.
//
// probe_read_kernel: the encoder's whole-block access pattern with nothing
// else: one workgroup of 256 threads per 8192-element block, four 16-byte
// loads per thread from each array, all in flight together.  Its time is the
// read ceiling of that pattern on the device, against which the encoder
// (both checkpoints, read with the encoder's non-temporal loads) and the
// apply pass (one, read with its plain loads) are compared.
//
// probe_write_kernel: the apply pass's writes alone: each 16-byte chunk a
// bitmap marks is written, in the same block order, and nothing is read.
// Beside the read probe it shows how the in-place traffic splits into reads
// of every weight and writes of the changed chunks.
//
// probe_inplace_kernel: the apply pass's traffic with nothing else: the same
// whole-block reads of one array, and each 16-byte chunk that a bitmap marks
// written back, unchanged, in place.  Given the chunks a delta changes, its
// time is the cost of an in-place apply's traffic (reads of every weight plus
// writes of the changed chunks) through the simplest kernel: a reference
// point for the apply pass, not a strict lower bound, since the order and
// timing of the writes change their cost.  The published HBM peak stays the
// roofline of both.
#include "internal.hpp"
#include "bf16delta_probe.h"

namespace bf16d {

// Plain pointers in the signature (an address-space qualifier there would
// give the kernel a different name in the host and device passes); they are
// made global inside.
template <bool kTwo>
__global__ __launch_bounds__(kThreads) void probe_read_kernel(const uint16_t *__restrict__ pa,
                                                              const uint16_t *__restrict__ pb,
                                                              uint64_t *__restrict__ sink,
                                                              uint64_t key) {
    auto *a = (BF16D_GMEM const uint16_t *)pa;
    auto *b = (BF16D_GMEM const uint16_t *)pb;
    const uint64_t base = xcd_tile(blockIdx.x, gridDim.x) * kBlock;
    uint4 x[kChunksPerThread], y[kChunksPerThread];
#pragma unroll
    for (uint32_t i = 0; i < kChunksPerThread; ++i) {
        const uint64_t e0 = base + 8 * (threadIdx.x + kThreads * i);
        if constexpr (kTwo) {   // the encoder's loads: non-temporal
            x[i] = load_stream16(a + e0);
            y[i] = load_stream16(b + e0);
        } else {                // the apply pass's loads: plain
            x[i] = *reinterpret_cast<BF16D_GMEM const uint4 *>(a + e0);
            y[i] = make_uint4(0, 0, 0, 0);
        }
    }
    uint64_t acc = 0;
#pragma unroll
    for (uint32_t i = 0; i < kChunksPerThread; ++i)
        acc += ((uint64_t)(x[i].x ^ y[i].x) << 32 | (x[i].y ^ y[i].y)) +
               ((uint64_t)(x[i].z ^ y[i].z) << 32 | (x[i].w ^ y[i].w));
    // keeps the loads: the store happens only if the fold hits the caller's key
    if (acc == key) sink[0] = acc;
}

// dirty: bit (c & 31) of word c >> 5 marks chunk c (elements 8c .. 8c + 7).
__global__ __launch_bounds__(kThreads) void probe_inplace_kernel(uint16_t *__restrict__ pw,
                                                                 const uint32_t *__restrict__ pd,
                                                                 uint64_t *__restrict__ sink,
                                                                 uint64_t key) {
    auto *w = (BF16D_GMEM uint16_t *)pw;
    auto *dirty = (BF16D_GMEM const uint32_t *)pd;
    const uint64_t base = xcd_tile(blockIdx.x, gridDim.x) * kBlock;
    const uint64_t word0 = base / 8 / 32;   // the block's 1024 chunk bits: 32 words
    uint4 x[kChunksPerThread];
    uint32_t m[kChunksPerThread];
#pragma unroll
    for (uint32_t i = 0; i < kChunksPerThread; ++i) {
        const uint32_t q = threadIdx.x + kThreads * i;
        x[i] = *reinterpret_cast<BF16D_GMEM const uint4 *>(w + base + 8 * q);
        m[i] = dirty[word0 + (q >> 5)];
    }
    uint64_t acc = 0;
#pragma unroll
    for (uint32_t i = 0; i < kChunksPerThread; ++i) {
        const uint32_t q = threadIdx.x + kThreads * i;
        acc += ((uint64_t)x[i].x << 32 | x[i].y) + ((uint64_t)x[i].z << 32 | x[i].w);
        if ((m[i] >> (q & 31)) & 1u) {
            uint4 v = x[i];
            // the value is opaque here, so the store of what was just loaded
            // from the same place is not removed as redundant
            asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
            *reinterpret_cast<BF16D_GMEM uint4 *>(w + base + 8 * q) = v;
        }
    }
    if (acc == key) sink[0] = acc;
}

int probe_inplace(uint16_t *w, uint64_t n, const uint32_t *dirty, uint64_t *sink, uint64_t key,
                  hipStream_t stream) {
    const uint64_t blocks = n / kBlock;
    if (!w || !dirty || !sink || ((uintptr_t)w & 15) || ((uintptr_t)dirty & 3) ||
        ((uintptr_t)sink & 7) || blocks > 0x7FFFFFFFull)
        return BF16D_EINVAL;
    if (blocks == 0) return BF16D_OK;
    probe_inplace_kernel<<<(uint32_t)blocks, kThreads, 0, stream>>>(w, dirty, sink, key);
    return hipGetLastError() == hipSuccess ? BF16D_OK : BF16D_EHIP;
}

// dirty as in probe_inplace_kernel; each marked chunk of w is overwritten
// (with a pattern derived from the bitmap), nothing is read from w.
__global__ __launch_bounds__(kThreads) void probe_write_kernel(uint16_t *__restrict__ pw,
                                                               const uint32_t *__restrict__ pd) {
    auto *w = (BF16D_GMEM uint16_t *)pw;
    auto *dirty = (BF16D_GMEM const uint32_t *)pd;
    const uint64_t base = xcd_tile(blockIdx.x, gridDim.x) * kBlock;
    const uint64_t word0 = base / 8 / 32;
#pragma unroll
    for (uint32_t i = 0; i < kChunksPerThread; ++i) {
        const uint32_t q = threadIdx.x + kThreads * i;
        const uint32_t m = dirty[word0 + (q >> 5)];
        if ((m >> (q & 31)) & 1u)
            *reinterpret_cast<BF16D_GMEM uint4 *>(w + base + 8 * q) = make_uint4(m, q, m ^ q, ~m);
    }
}

int probe_write(uint16_t *w, uint64_t n, const uint32_t *dirty, hipStream_t stream) {
    const uint64_t blocks = n / kBlock;
    if (!w || !dirty || ((uintptr_t)w & 15) || ((uintptr_t)dirty & 3) || blocks > 0x7FFFFFFFull)
        return BF16D_EINVAL;
    if (blocks == 0) return BF16D_OK;
    probe_write_kernel<<<(uint32_t)blocks, kThreads, 0, stream>>>(w, dirty);
    return hipGetLastError() == hipSuccess ? BF16D_OK : BF16D_EHIP;
}

int probe_read(const uint16_t *a, const uint16_t *b, uint64_t n, uint64_t *sink, uint64_t key,
               hipStream_t stream) {
    const uint64_t blocks = n / kBlock;
    if (!a || !sink || ((uintptr_t)a & 15) || ((uintptr_t)b & 15) || ((uintptr_t)sink & 7) ||
        blocks > 0x7FFFFFFFull)
        return BF16D_EINVAL;
    if (blocks == 0) return BF16D_OK;
    if (b)
        probe_read_kernel<true><<<(uint32_t)blocks, kThreads, 0, stream>>>(a, b, sink, key);
    else
        probe_read_kernel<false><<<(uint32_t)blocks, kThreads, 0, stream>>>(a, b, sink, key);
    return hipGetLastError() == hipSuccess ? BF16D_OK : BF16D_EHIP;
}

}  // namespace bf16d

extern "C" int bf16d_probe_read(const uint16_t *a, const uint16_t *b, uint64_t n, uint64_t *sink,
                                uint64_t key, hipStream_t stream) {
    return bf16d::probe_read(a, b, n, sink, key, stream);
}

extern "C" int bf16d_probe_inplace(uint16_t *w, uint64_t n, const uint32_t *dirty, uint64_t *sink,
                                   uint64_t key, hipStream_t stream) {
    return bf16d::probe_inplace(w, n, dirty, sink, key, stream);
}

extern "C" int bf16d_probe_write(uint16_t *w, uint64_t n, const uint32_t *dirty,
                                 hipStream_t stream) {
    return bf16d::probe_write(w, n, dirty, stream);
}
