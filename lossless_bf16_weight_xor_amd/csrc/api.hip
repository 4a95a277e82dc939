// api.hip -- host side of the libbf16delta C ABI (see include/bf16delta.h).
//
// Validates arguments, computes the workspace layout, copies the job table
// (the CPU-prepared "plan") into the workspace, and enqueues the kernels.
// Nothing here allocates device memory or keeps state between calls.
#include <algorithm>
#include <cstring>
#include <mutex>
#include <vector>

#include "internal.hpp"

using namespace bf16d;

namespace {

constexpr uint64_t kMaxTiles = 1ull << 24;   // grid limit: tiles * 256 threads < 2^32
constexpr uint64_t kMaxSize = UINT64_MAX >> 2;   // element counts and byte sizes: at most 2^62

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

uint64_t blocks_of(uint64_t n) { return (n + kBlock - 1) / kBlock; }

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
    bool written;
};

// A written range may overlap no other range; read ranges may overlap each other.
bool ranges_disjoint(std::vector<Range> &v) {
    v.erase(std::remove_if(v.begin(), v.end(), [](const Range &r) { return r.hi <= r.lo; }),
            v.end());
    std::sort(v.begin(), v.end(), [](const Range &a, const Range &b) { return a.lo < b.lo; });
    // sweep: compare each range with the furthest-reaching earlier written range
    // and the furthest-reaching earlier range of any kind
    uintptr_t reach_any = 0, reach_written = 0;
    for (const Range &r : v) {
        if (r.lo < reach_written) return false;
        if (r.written && r.lo < reach_any) return false;
        reach_any = std::max(reach_any, r.hi);
        if (r.written) reach_written = std::max(reach_written, r.hi);
    }
    return true;
}

int upload(void *ws, const std::vector<uint8_t> &host, size_t at, hipStream_t stream) {
    if (host.empty()) return BF16D_OK;
    // Pageable source: the runtime stages it before returning, so `host` may be freed.
    hipError_t e = hipMemcpyAsync(static_cast<uint8_t *>(ws) + at, host.data(), host.size(),
                                  hipMemcpyHostToDevice, stream);
    return e == hipSuccess ? BF16D_OK : BF16D_EHIP;
}

}  // namespace

namespace bf16d {

// a remap's segments: block-aligned, in order, back to back from 0, covering n
bool remap_valid(const bf16d_remap &m, uint64_t n) {
    if (!m.segments) return false;
    uint64_t at = 0;
    for (uint32_t k = 0; k < m.count; ++k) {
        const bf16d_segment &g = m.segments[k];
        if (g.first != at || g.first % kBlock != 0 || g.count == 0 || !g.dst ||
            !aligned16(g.dst) || g.count > kMaxSize - at)
            return false;
        if (k + 1 < m.count && g.count % kBlock != 0) return false;
        at += g.count;
    }
    return at == n;
}

int decompress_prep(const bf16d_decompress_job *jobs, uint32_t count, DecompressPrep &p,
                    const bf16d_remap *remaps, bool mapped) {
    p.bstart.assign(size_t(count) + 1, 0);
    p.dstart.assign(size_t(count) + 1, 0);
    for (uint32_t j = 0; j < count; ++j) {
        const bf16d_decompress_job &J = jobs[j];
        if (mapped) {
            // checked against the prepared plan by the caller
        } else if (remaps && remaps[j].count > 0) {
            if (J.weights || !remap_valid(remaps[j], J.n)) return BF16D_EINVAL;
        } else if (J.n > 0 && (!J.weights || !aligned16(J.weights))) {
            return BF16D_EINVAL;
        }
        // an empty payload may be NULL; it is then rejected on the device as too short
        if ((J.payload_bytes > 0 && !J.payload) || !aligned16(J.payload)) return BF16D_EINVAL;
        // sizes beyond 2^62 cannot describe real buffers, and would wrap the
        // address arithmetic of the overlap checks
        if (J.n > kMaxSize || J.payload_bytes > kMaxSize) return BF16D_EINVAL;
        const uint64_t nb = blocks_of(J.n);
        p.bstart[j + 1] = p.bstart[j] + nb;
        p.dstart[j + 1] = p.dstart[j] + (nb + kDescTile - 1) / kDescTile;
    }
    p.tiles = p.bstart[count];
    p.dtiles = p.dstart[count];
    return p.tiles >= kMaxTiles ? BF16D_EINVAL : BF16D_OK;
}

size_t decompress_table_bytes(const Layout &l, uint32_t count) {
    return l.dtile_start + 8 * (size_t(count) + 1) - l.jobs;
}

void decompress_table(const bf16d_decompress_job *jobs, uint32_t count, const DecompressPrep &p,
                      const Layout &l, uint8_t *out, bool verify_first) {
    auto *dj = reinterpret_cast<DecompressJob *>(out);
    for (uint32_t j = 0; j < count; ++j) {
        dj[j].weights = (BF16D_GMEM uint16_t *)jobs[j].weights;
        dj[j].n = jobs[j].n;
        dj[j].payload = (BF16D_GMEM const uint8_t *)jobs[j].payload;
        dj[j].payload_bytes = jobs[j].payload_bytes;
        dj[j].checksum = jobs[j].checksum;
        dj[j].block0 = p.bstart[j];
        dj[j].nb = p.bstart[j + 1] - p.bstart[j];
        dj[j].dtile0 = p.dstart[j];
        dj[j].segs = nullptr;
        dj[j].nsegs = 0;
        dj[j].version = nullptr;
        dj[j].verify_first = verify_first ? 1u : 0u;
        dj[j].undo = nullptr;
    }
    std::memcpy(out + (l.block_start - l.jobs), p.bstart.data(), 8 * p.bstart.size());
    std::memcpy(out + (l.dtile_start - l.jobs), p.dstart.data(), 8 * p.dstart.size());
}

}  // namespace bf16d

namespace {

// The batched decompress, optionally remapped and with the receiver's version
// words: checks, job table (and the remap segments after the layout), upload,
// launch.
int decompress_call(const bf16d_decompress_job *jobs, const bf16d_remap *remaps,
                    uint64_t *versions, uint32_t count, void *workspace, size_t workspace_bytes,
                    bf16d_result *results, hipStream_t stream, const bf16d_events *events,
                    bool verify_first = false) {
    if (!jobs || count == 0 || !results || !workspace || !aligned16(workspace))
        return BF16D_EINVAL;
    if (versions && (reinterpret_cast<uintptr_t>(versions) & 7u) != 0) return BF16D_EINVAL;
    DecompressPrep prep;
    int rc = decompress_prep(jobs, count, prep, remaps);
    if (rc != BF16D_OK) return rc;
    const Layout l = make_layout(prep.tiles, prep.dtiles, count, false);
    size_t nsegs = 0;
    if (remaps)
        for (uint32_t j = 0; j < count; ++j) nsegs += remaps[j].count;
    const size_t seg_at = align_up(l.total, 256);
    const size_t need = nsegs ? seg_at + sizeof(RemapSegment) * nsegs : l.total;
    if (workspace_bytes < need) return BF16D_EINVAL;
    // room for an undo area (one byte per payload byte) lets overwrite
    // payloads be written in place in one pass; without it they are verified
    // first and written after
    const size_t undo_at = align_up(need, 256);
    size_t undo_bytes = 0;
    for (uint32_t j = 0; j < count; ++j) undo_bytes += align_up(jobs[j].payload_bytes, 16);
    const bool with_undo = !verify_first && workspace_bytes >= undo_at &&
                           workspace_bytes - undo_at >= undo_bytes;
    const size_t used = with_undo ? undo_at + undo_bytes : need;
    std::vector<Range> ranges;
    ranges.reserve(2 * size_t(count) + nsegs + 3);
    for (uint32_t j = 0; j < count; ++j) {
        const bf16d_decompress_job &J = jobs[j];
        if (remaps && remaps[j].count > 0) {
            for (uint32_t k = 0; k < remaps[j].count; ++k) {
                const bf16d_segment &g = remaps[j].segments[k];
                ranges.push_back({reinterpret_cast<uintptr_t>(g.dst),
                                  reinterpret_cast<uintptr_t>(g.dst) + 2 * g.count, true});
            }
        } else {
            ranges.push_back({reinterpret_cast<uintptr_t>(J.weights),
                              reinterpret_cast<uintptr_t>(J.weights) + 2 * J.n, true});
        }
        ranges.push_back({reinterpret_cast<uintptr_t>(J.payload),
                          reinterpret_cast<uintptr_t>(J.payload) + J.payload_bytes, false});
    }
    ranges.push_back({reinterpret_cast<uintptr_t>(workspace),
                      reinterpret_cast<uintptr_t>(workspace) + used, true});
    ranges.push_back({reinterpret_cast<uintptr_t>(results),
                      reinterpret_cast<uintptr_t>(results + count), true});
    if (versions)
        ranges.push_back({reinterpret_cast<uintptr_t>(versions),
                          reinterpret_cast<uintptr_t>(versions + count), true});
    if (!ranges_disjoint(ranges)) return BF16D_EINVAL;

    std::vector<uint8_t> host(decompress_table_bytes(l, count), 0);
    decompress_table(jobs, count, prep, l, host.data(), verify_first);
    if (with_undo) {
        auto *dj = reinterpret_cast<DecompressJob *>(host.data());
        size_t at = undo_at;
        for (uint32_t j = 0; j < count; ++j) {
            dj[j].undo = (BF16D_GMEM uint8_t *)(static_cast<uint8_t *>(workspace) + at);
            at += align_up(jobs[j].payload_bytes, 16);
        }
    }
    if (versions) {
        auto *dj = reinterpret_cast<DecompressJob *>(host.data());
        for (uint32_t j = 0; j < count; ++j) dj[j].version = (BF16D_GMEM uint64_t *)(versions + j);
    }
    std::vector<uint8_t> segs(sizeof(RemapSegment) * nsegs, 0);
    if (nsegs) {
        auto *dj = reinterpret_cast<DecompressJob *>(host.data());
        auto *ds = reinterpret_cast<RemapSegment *>(segs.data());
        auto *dev = (BF16D_GMEM const RemapSegment *)(static_cast<uint8_t *>(workspace) + seg_at);
        size_t at = 0;
        for (uint32_t j = 0; j < count; ++j) {
            if (remaps[j].count == 0) continue;
            dj[j].segs = dev + at;
            dj[j].nsegs = remaps[j].count;
            for (uint32_t k = 0; k < remaps[j].count; ++k, ++at) {
                const bf16d_segment &g = remaps[j].segments[k];
                ds[at].first = g.first;
                ds[at].count = g.count;
                ds[at].dst = (BF16D_GMEM uint16_t *)g.dst;
                ds[at].pad = 0;
            }
        }
        rc = upload(workspace, segs, seg_at, stream);
        if (rc != BF16D_OK) return rc;
    }
    rc = upload(workspace, host, l.jobs, stream);
    if (rc != BF16D_OK) return rc;
    return launch_decompress(l, static_cast<uint8_t *>(workspace), count, prep.tiles, prep.dtiles,
                             results, stream, events, nullptr, verify_first) == hipSuccess
               ? BF16D_OK
               : BF16D_EHIP;
}

}  // namespace

// ---- prepared remaps -------------------------------------------------------------
// The host plan of bf16d_remap_prepare, in caller memory: a header, each job's
// (weights, n) as prepared, and the sorted physical ranges the jobs write.
namespace {

constexpr uint64_t kPlanMagic = 0x504D5244363146ull;   // "F16DRMP"

struct PlanHeader {
    uint64_t magic;
    uint32_t count, pad;
    uint64_t nranges;   // sorted, pairwise disjoint written ranges
    uint64_t tiles;     // blocks of the batch: entries of the block map
};
struct PlanJob {
    uint64_t weights, n;
};
struct PlanRange {
    uint64_t lo, hi;
};

size_t plan_bytes(uint32_t count, uint64_t ranges) {
    return sizeof(PlanHeader) + sizeof(PlanJob) * size_t(count) + sizeof(PlanRange) * ranges;
}

// does [lo, hi) overlap one of the sorted, disjoint ranges r[0, m)?
bool overlaps_sorted(const PlanRange *r, uint64_t m, uint64_t lo, uint64_t hi) {
    if (hi <= lo) return false;
    uint64_t a = 0, b = m;   // first range with r.hi > lo
    while (a < b) {
        const uint64_t mid = (a + b) / 2;
        if (r[mid].hi <= lo) a = mid + 1; else b = mid;
    }
    return a < m && r[a].lo < hi;
}

}  // namespace

extern "C" {

size_t bf16d_remap_plan_bytes(uint32_t count, uint64_t total_segments) {
    return plan_bytes(count, total_segments + count);
}

size_t bf16d_remap_map_bytes(uint64_t total_n, uint32_t count) {
    return 8 * (size_t)(blocks_of(total_n) + count);
}

int bf16d_remap_prepare(const bf16d_decompress_job *jobs, const bf16d_remap *remaps,
                        uint32_t count, void *plan, size_t plan_size, uint64_t *block_map,
                        size_t map_bytes, hipStream_t stream) {
    if (!jobs || count == 0 || !plan || !block_map ||
        (reinterpret_cast<uintptr_t>(block_map) & 7u) != 0)
        return BF16D_EINVAL;
    // the layout: block-aligned segments in order, or plain weights
    std::vector<Range> ranges;
    uint64_t tiles = 0;
    for (uint32_t j = 0; j < count; ++j) {
        const bf16d_decompress_job &J = jobs[j];
        if (J.n > kMaxSize) return BF16D_EINVAL;
        if (remaps && remaps[j].count > 0) {
            if (J.weights || !remap_valid(remaps[j], J.n)) return BF16D_EINVAL;
            for (uint32_t k = 0; k < remaps[j].count; ++k) {
                const bf16d_segment &g = remaps[j].segments[k];
                ranges.push_back({reinterpret_cast<uintptr_t>(g.dst),
                                  reinterpret_cast<uintptr_t>(g.dst) + 2 * g.count, true});
            }
        } else {
            if (J.n > 0 && (!J.weights || !aligned16(J.weights))) return BF16D_EINVAL;
            ranges.push_back({reinterpret_cast<uintptr_t>(J.weights),
                              reinterpret_cast<uintptr_t>(J.weights) + 2 * J.n, true});
        }
        tiles += blocks_of(J.n);
    }
    if (tiles >= kMaxTiles || map_bytes < 8 * tiles) return BF16D_EINVAL;
    ranges.push_back({reinterpret_cast<uintptr_t>(block_map),
                      reinterpret_cast<uintptr_t>(block_map) + 8 * tiles, true});
    if (!ranges_disjoint(ranges)) return BF16D_EINVAL;   // sorts them, drops empty ones
    // the plan keeps the weights' ranges, not the map's
    ranges.erase(std::remove_if(ranges.begin(), ranges.end(),
                                [&](const Range &r) {
                                    return r.lo == reinterpret_cast<uintptr_t>(block_map);
                                }),
                 ranges.end());
    if (plan_size < plan_bytes(count, ranges.size())) return BF16D_EINVAL;

    // the block map: each block's first weight
    std::vector<uint64_t> map(tiles);
    uint64_t t = 0;
    for (uint32_t j = 0; j < count; ++j) {
        const bf16d_decompress_job &J = jobs[j];
        const uint64_t nb = blocks_of(J.n);
        if (remaps && remaps[j].count > 0) {
            uint32_t k = 0;
            for (uint64_t b = 0; b < nb; ++b) {
                const uint64_t e = b * kBlock;
                while (remaps[j].segments[k].first + remaps[j].segments[k].count <= e) ++k;
                const bf16d_segment &g = remaps[j].segments[k];
                map[t++] = reinterpret_cast<uintptr_t>(g.dst + (e - g.first));
            }
        } else {
            for (uint64_t b = 0; b < nb; ++b)
                map[t++] = reinterpret_cast<uintptr_t>(J.weights + b * kBlock);
        }
    }
    if (tiles && hipMemcpyAsync(block_map, map.data(), 8 * tiles, hipMemcpyHostToDevice,
                                stream) != hipSuccess)
        return BF16D_EHIP;

    auto *h = static_cast<PlanHeader *>(plan);
    h->magic = kPlanMagic;
    h->count = count;
    h->pad = 0;
    h->nranges = ranges.size();
    h->tiles = tiles;
    auto *pj = reinterpret_cast<PlanJob *>(h + 1);
    for (uint32_t j = 0; j < count; ++j)
        pj[j] = {reinterpret_cast<uintptr_t>(jobs[j].weights), jobs[j].n};
    auto *pr = reinterpret_cast<PlanRange *>(pj + count);
    for (size_t i = 0; i < ranges.size(); ++i) pr[i] = {ranges[i].lo, ranges[i].hi};
    return BF16D_OK;
}

int bf16d_decompress_remapped_prepared(const bf16d_decompress_job *jobs, uint32_t count,
                                       const void *plan, const uint64_t *block_map,
                                       void *workspace, size_t workspace_bytes,
                                       bf16d_result *results, hipStream_t stream) {
    if (!jobs || count == 0 || !plan || !block_map || !results || !workspace ||
        !aligned16(workspace))
        return BF16D_EINVAL;
    const auto *h = static_cast<const PlanHeader *>(plan);
    if (h->magic != kPlanMagic || h->count != count) return BF16D_EINVAL;
    const auto *pj = reinterpret_cast<const PlanJob *>(h + 1);
    const auto *pr = reinterpret_cast<const PlanRange *>(pj + count);
    // the jobs the plan was made for: same tensors, in the same order
    for (uint32_t j = 0; j < count; ++j)
        if (pj[j].weights != reinterpret_cast<uintptr_t>(jobs[j].weights) ||
            pj[j].n != jobs[j].n)
            return BF16D_EINVAL;
    DecompressPrep prep;
    int rc = decompress_prep(jobs, count, prep, nullptr, true);
    if (rc != BF16D_OK) return rc;
    if (prep.tiles != h->tiles) return BF16D_EINVAL;
    const Layout l = make_layout(prep.tiles, prep.dtiles, count, false);
    if (workspace_bytes < l.total) return BF16D_EINVAL;
    // this call's buffers against each other, and against the prepared
    // physical ranges (sorted: a binary search each)
    std::vector<Range> mine;
    mine.reserve(size_t(count) + 3);
    for (uint32_t j = 0; j < count; ++j)
        mine.push_back({reinterpret_cast<uintptr_t>(jobs[j].payload),
                        reinterpret_cast<uintptr_t>(jobs[j].payload) + jobs[j].payload_bytes,
                        false});
    mine.push_back({reinterpret_cast<uintptr_t>(workspace),
                    reinterpret_cast<uintptr_t>(workspace) + l.total, true});
    mine.push_back({reinterpret_cast<uintptr_t>(results),
                    reinterpret_cast<uintptr_t>(results + count), true});
    mine.push_back({reinterpret_cast<uintptr_t>(block_map),
                    reinterpret_cast<uintptr_t>(block_map) + 8 * prep.tiles, false});
    for (const Range &r : mine)
        if (overlaps_sorted(pr, h->nranges, r.lo, r.hi)) return BF16D_EINVAL;
    if (!ranges_disjoint(mine)) return BF16D_EINVAL;

    std::vector<uint8_t> host(decompress_table_bytes(l, count), 0);
    decompress_table(jobs, count, prep, l, host.data());
    rc = upload(workspace, host, l.jobs, stream);
    if (rc != BF16D_OK) return rc;
    return launch_decompress(l, static_cast<uint8_t *>(workspace), count, prep.tiles,
                             prep.dtiles, results, stream, nullptr, block_map) == hipSuccess
               ? BF16D_OK
               : BF16D_EHIP;
}

uint64_t bf16d_max_payload_bytes(uint64_t n) {
    const uint64_t full = n / kBlock, tail = n % kBlock;
    uint64_t total = kHeader + 4 * blocks_of(n) + full * (uint64_t)kMaxRecord;
    if (tail) total += (tail + 7) / 8 + (7 * tail + 7) / 8 + 2 * tail;
    return total;
}

size_t bf16d_compress_workspace_bytes(uint64_t total_n, uint32_t count, uint32_t slot_bytes) {
    if (slot_bytes < kMinSlot || slot_bytes > kSlot || slot_bytes % 16 != 0) return 0;
    const uint64_t tiles = blocks_of(total_n) + count;
    const uint64_t dtiles = (tiles + kDescTile - 1) / kDescTile + count;
    return make_layout(tiles, dtiles, count, true, slot_bytes).total;
}

size_t bf16d_workspace_bytes(uint64_t total_n, uint32_t count) {
    const uint64_t tiles = blocks_of(total_n) + count;
    const uint64_t dtiles = (tiles + kDescTile - 1) / kDescTile + count;
    const size_t c = make_layout(tiles, dtiles, count, true).total;
    // decompress; the streamed form keeps a decompress layout per compute
    // lane (at most two), then every group's job table (at most 1024 bytes per
    // job with alignment)
    const size_t d = 2 * make_layout(tiles, dtiles, count, false).total + 512 +
                     1024 * size_t(count);
    return c > d ? c : d;
}

}  // extern "C"

namespace {

// The batched compress; bindings (may be NULL) make version-2 payloads.
int compress_call(const bf16d_compress_job *jobs, const bf16d_binding *bindings, uint32_t count,
                  void *workspace, size_t workspace_bytes, bf16d_result *results,
                  hipStream_t stream, const bf16d_events *events) {
    if (!jobs || count == 0 || !results || !workspace || !aligned16(workspace))
        return BF16D_EINVAL;
    if (bindings)
        for (uint32_t j = 0; j < count; ++j)
            if ((bindings[j].flags & ~BF16D_BIND_OVERWRITE) != 0 || bindings[j].reserved != 0)
                return BF16D_EINVAL;
    std::vector<uint64_t> start(size_t(count) + 1, 0), dstart(size_t(count) + 1, 0);
    std::vector<Range> ranges;
    ranges.reserve(3 * size_t(count) + 2);
    for (uint32_t j = 0; j < count; ++j) {
        const bf16d_compress_job &J = jobs[j];
        if (J.n > 0 && (!J.src || !J.dst || !aligned16(J.src) || !aligned16(J.dst)))
            return BF16D_EINVAL;
        if (J.capacity > 0 && (!J.payload || !aligned16(J.payload))) return BF16D_EINVAL;
        // records may be staged anywhere below `capacity`: it must describe
        // a real buffer (and not wrap the overlap checks' address arithmetic)
        if (J.n > kMaxSize || J.capacity > kMaxSize) return BF16D_EINVAL;
        start[j + 1] = start[j] + blocks_of(J.n);
        dstart[j + 1] = dstart[j] + (blocks_of(J.n) + kDescTile - 1) / kDescTile;
        ranges.push_back({reinterpret_cast<uintptr_t>(J.src),
                          reinterpret_cast<uintptr_t>(J.src) + 2 * J.n, false});
        ranges.push_back({reinterpret_cast<uintptr_t>(J.dst),
                          reinterpret_cast<uintptr_t>(J.dst) + 2 * J.n, false});
        ranges.push_back({reinterpret_cast<uintptr_t>(J.payload),
                          reinterpret_cast<uintptr_t>(J.payload) + J.capacity, true});
    }
    const uint64_t tiles = start[count], dtiles = dstart[count];
    if (tiles >= kMaxTiles) return BF16D_EINVAL;
    // the largest record slot the workspace holds: kSlot, or less
    uint32_t slot = kSlot;
    Layout l = make_layout(tiles, dtiles, count, true, slot);
    if (workspace_bytes < l.total) {
        const Layout l0 = make_layout(tiles, dtiles, count, true, 0);
        if (tiles == 0 || workspace_bytes < l0.total) return BF16D_EINVAL;
        const uint64_t per = (workspace_bytes - l0.total) / tiles / 16 * 16;
        slot = (uint32_t)(per < kSlot ? per : kSlot);
        // the slot region's alignment may cost up to 255 bytes: step down
        while (slot >= kMinSlot &&
               workspace_bytes < (l = make_layout(tiles, dtiles, count, true, slot)).total)
            slot -= 16;
        if (slot < kMinSlot) return BF16D_EINVAL;
    }
    ranges.push_back({reinterpret_cast<uintptr_t>(workspace),
                      reinterpret_cast<uintptr_t>(workspace) + l.total, true});
    ranges.push_back({reinterpret_cast<uintptr_t>(results),
                      reinterpret_cast<uintptr_t>(results + count), true});
    if (!ranges_disjoint(ranges)) return BF16D_EINVAL;

    // job table, block starts and scan-tile starts, laid out as in the workspace
    std::vector<uint8_t> host(l.dtile_start + 8 * (size_t(count) + 1) - l.jobs, 0);
    auto *dj = reinterpret_cast<CompressJob *>(host.data());
    for (uint32_t j = 0; j < count; ++j) {
        dj[j].src = (BF16D_GMEM const uint16_t *)jobs[j].src;
        dj[j].dst = (BF16D_GMEM const uint16_t *)jobs[j].dst;
        dj[j].n = jobs[j].n;
        dj[j].payload = (BF16D_GMEM uint8_t *)jobs[j].payload;
        dj[j].capacity = jobs[j].capacity;
        dj[j].block0 = start[j];
        dj[j].nb = start[j + 1] - start[j];
        dj[j].hdr = bindings ? kHeaderBound : kHeader;
        dj[j].flags = bindings ? bindings[j].flags : 0;
        dj[j].base_version = bindings ? bindings[j].base_version : 0;
        dj[j].target_version = bindings ? bindings[j].target_version : 0;
    }
    std::memcpy(host.data() + (l.block_start - l.jobs), start.data(), 8 * start.size());
    std::memcpy(host.data() + (l.dtile_start - l.jobs), dstart.data(), 8 * dstart.size());
    int rc = upload(workspace, host, l.jobs, stream);
    if (rc != BF16D_OK) return rc;
    bool any_overwrite = false;
    for (uint32_t j = 0; bindings && j < count; ++j)
        any_overwrite |= (bindings[j].flags & BF16D_BIND_OVERWRITE) != 0;
    return launch_compress(l, static_cast<uint8_t *>(workspace), count, tiles, dtiles, results,
                           stream, events, any_overwrite) == hipSuccess
               ? BF16D_OK
               : BF16D_EHIP;
}

}  // namespace

extern "C" {

int bf16d_compress(const bf16d_compress_job *jobs, uint32_t count, void *workspace,
                   size_t workspace_bytes, bf16d_result *results, hipStream_t stream) {
    return compress_call(jobs, nullptr, count, workspace, workspace_bytes, results, stream,
                         nullptr);
}

int bf16d_compress_ex(const bf16d_compress_job *jobs, uint32_t count, void *workspace,
                      size_t workspace_bytes, bf16d_result *results, hipStream_t stream,
                      const bf16d_events *events) {
    return compress_call(jobs, nullptr, count, workspace, workspace_bytes, results, stream,
                         events);
}

int bf16d_compress_bound(const bf16d_compress_job *jobs, const bf16d_binding *bindings,
                         uint32_t count, void *workspace, size_t workspace_bytes,
                         bf16d_result *results, hipStream_t stream) {
    if (!bindings) return BF16D_EINVAL;
    return compress_call(jobs, bindings, count, workspace, workspace_bytes, results, stream,
                         nullptr);
}

int bf16d_decompress_bound(const bf16d_decompress_job *jobs, uint64_t *versions, uint32_t count,
                           void *workspace, size_t workspace_bytes, bf16d_result *results,
                           hipStream_t stream) {
    return decompress_call(jobs, nullptr, versions, count, workspace, workspace_bytes, results,
                           stream, nullptr);
}

int bf16d_decompress_verified(const bf16d_decompress_job *jobs, uint32_t count,
                              void *workspace, size_t workspace_bytes, bf16d_result *results,
                              hipStream_t stream, const bf16d_events *events) {
    return decompress_call(jobs, nullptr, nullptr, count, workspace, workspace_bytes, results,
                           stream, events, true);
}

int bf16d_decompress(const bf16d_decompress_job *jobs, uint32_t count, void *workspace,
                     size_t workspace_bytes, bf16d_result *results, hipStream_t stream) {
    return bf16d_decompress_ex(jobs, count, workspace, workspace_bytes, results, stream, nullptr);
}

int bf16d_decompress_ex(const bf16d_decompress_job *jobs, uint32_t count, void *workspace,
                        size_t workspace_bytes, bf16d_result *results, hipStream_t stream,
                        const bf16d_events *events) {
    return decompress_call(jobs, nullptr, nullptr, count, workspace, workspace_bytes, results,
                           stream, events);
}

}  // extern "C"

// ---- allocation-free decompress ------------------------------------------------
// The library's own scratch for bf16d_decompress_noalloc: one array per GPU
// (each device that loads the library's code holds its own copy until the
// process ends).  In host code `scratch` names a host-side stand-in, not
// device memory: its device address is taken once per device with
// hipGetSymbolAddress and only that address is passed to kernels.
static __device__ __align__(256) uint8_t scratch[BF16D_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void *g_scratch[kMaxDevices];   // device address of `scratch` per device, once taken

// The scratch of the current device (which must be `stream`'s device), taken
// on the first call made on that device.
int current_scratch(hipStream_t stream, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BF16D_EHIP;
    if (stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return BF16D_EHIP;
        if (sdev != dev) return BF16D_EINVAL;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BF16D_EHIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return BF16D_OK;
}

}  // namespace

extern "C" {

int bf16d_decompress_noalloc(const bf16d_decompress_job *jobs, uint32_t count,
                             bf16d_result *results, hipStream_t stream) {
    if (!jobs || count == 0 || !results) return BF16D_EINVAL;
    // the size check first: a batch the scratch cannot hold touches nothing
    DecompressPrep prep;
    const int rc = decompress_prep(jobs, count, prep, nullptr);
    if (rc != BF16D_OK) return rc;
    if (make_layout(prep.tiles, prep.dtiles, count, false).total > BF16D_NOALLOC_SCRATCH_BYTES)
        return BF16D_EINVAL;
    void *ws = nullptr;
    const int sc = current_scratch(stream, &ws);
    if (sc != BF16D_OK) return sc;
    return decompress_call(jobs, nullptr, nullptr, count, ws, BF16D_NOALLOC_SCRATCH_BYTES,
                           results, stream, nullptr);
}

size_t bf16d_workspace_bytes_remapped(uint64_t total_n, uint32_t count, uint64_t total_segments) {
    return bf16d_workspace_bytes(total_n, count) + 256 + sizeof(RemapSegment) * total_segments;
}

int bf16d_decompress_remapped(const bf16d_decompress_job *jobs, const bf16d_remap *remaps,
                              uint32_t count, void *workspace, size_t workspace_bytes,
                              bf16d_result *results, hipStream_t stream) {
    return decompress_call(jobs, remaps, nullptr, count, workspace, workspace_bytes, results,
                           stream, nullptr);
}

int bf16d_delta_compress(const uint16_t *src, const uint16_t *dst, uint64_t n, uint8_t *payload,
                         uint64_t capacity, void *workspace, size_t workspace_bytes,
                         bf16d_result *result, hipStream_t stream) {
    const bf16d_compress_job job = {src, dst, n, payload, capacity};
    return bf16d_compress(&job, 1, workspace, workspace_bytes, result, stream);
}

int bf16d_delta_decompress(uint16_t *src_inout, uint64_t n, const uint8_t *payload,
                           uint64_t payload_bytes, uint64_t checksum, void *workspace,
                           size_t workspace_bytes, bf16d_result *result, hipStream_t stream) {
    const bf16d_decompress_job job = {src_inout, n, payload, payload_bytes, checksum};
    return bf16d_decompress(&job, 1, workspace, workspace_bytes, result, stream);
}

const char *bf16d_status_string(int status) {
    switch (status) {
        case BF16D_OK: return "OK";
        case BF16D_EINVAL: return "EINVAL: invalid arguments";
        case BF16D_ECAPACITY: return "ECAPACITY: payload capacity too small";
        case BF16D_EFORMAT: return "EFORMAT: malformed or mismatched payload";
        case BF16D_ECHECKSUM: return "ECHECKSUM: rebuilt weights fail the checksum";
        case BF16D_EHIP: return "EHIP: HIP runtime error";
        case BF16D_ECODEC: return "ECODEC: codec library not available";
        case BF16D_EVERSION: return "EVERSION: the weights are not the payload's base version";
        default: return "unknown status";
    }
}

int bf16d_format_version(void) { return BF16D_FORMAT_VERSION; }

}  // extern "C"
