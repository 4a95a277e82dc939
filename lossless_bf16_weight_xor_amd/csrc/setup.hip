// setup.hip -- the kernel that prepares a batched call: the tile -> job maps
// (the "plan" that lets one launch cover every tensor of a checkpoint, as the
// single-launch XOR apply of "GPU-accelerated Weight Teleportation", section
// "A strong baseline with Blackwell-native DE", reads a CPU-prepared plan),
// and zero fills of look-back words and per-job state.
#include "internal.hpp"

namespace bf16d {

// The zero fills and tile maps of one call, in one launch: map[m][t] = j
// with start[m][j] <= t < start[m][j + 1] (a binary search of the job start
// table), and status[m][t] cleared alongside when given.
__global__ void setup_kernel(SetupArgs a) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    const uint64_t i0 = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x;
#pragma unroll
    for (int z = 0; z < 3; ++z)
        for (uint64_t i = i0; i < a.zero_words[z]; i += stride) a.zero[z][i] = 0;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        for (uint64_t t = i0; t < a.tiles[m]; t += stride) {
            uint32_t lo = 0, hi = a.count;   // invariant: start[lo] <= t < start[hi]
            while (hi - lo > 1) {
                const uint32_t mid = (lo + hi) >> 1;
                if (a.start[m][mid] <= t) lo = mid; else hi = mid;
            }
            a.map[m][t] = lo;
            if (a.status[m]) a.status[m][t] = 0;
        }
    }
}

static uint32_t grid_for(uint64_t items) {
    const uint64_t g = (items + kThreads - 1) / kThreads;
    return (uint32_t)(g < 4096 ? (g ? g : 1) : 4096);
}

uint32_t persistent_grid(const void *kernel, uint64_t tiles, size_t dynamic_lds) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, dynamic_lds) !=
            hipSuccess ||
        cus <= 0 || per_cu <= 0) {
        cus = 256;
        per_cu = 2;
    }
    const uint64_t g = (uint64_t)cus * (uint64_t)per_cu;
    return (uint32_t)(tiles < g ? (tiles ? tiles : 1) : g);
}

void launch_setup(const SetupArgs &a, hipStream_t stream) {
    uint64_t items = 0;
    for (int z = 0; z < 3; ++z) items = a.zero_words[z] > items ? a.zero_words[z] : items;
    for (int m = 0; m < 2; ++m) items = a.tiles[m] > items ? a.tiles[m] : items;
    setup_kernel<<<grid_for(items), kThreads, 0, stream>>>(a);
}

}  // namespace bf16d
