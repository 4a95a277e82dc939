// streamed.hip -- the streamed receiver: host-resident payloads applied in
// place group by group through a ring of device slots.
//
// The double-buffered pipeline of "GPU-accelerated Weight Teleportation",
// sections "Overlapping DE and SM" and "Assembling the weight teleporter",
// on MI355X: the DMA engines copy group g's payloads into slot g % S on the
// copy stream while the CUs apply earlier groups from the other slots on the
// compute stream.  Events order each copy after the apply that last read its
// slot, and each apply after its copy.  With S = 2 a copy waits for the apply
// just before it, and every cross-stream wait (tens of microseconds) lands
// on the copies' critical path; a third slot gives the copies a whole group
// of slack.  Each transfer also has a fixed cost of its own (about 10 us,
// 18 us with the event after it); the groups' copies alternate over the
// caller's copy streams, so one engine's set-up overlaps another's
// transfer.  Everything is validated before any work is enqueued.
//
// Each group's apply is a whole batched decompress call (six launches: the
// set-up, descriptor scan and plan before the apply kernel, the checksum sum
// and fix-up after it).  On one compute stream those short kernels add up
// to a third of the apply time and keep the copies waiting for slots.  With
// several compute lanes (the caller's stream plus `lanes` more), group g runs
// on lane g % (1 + lanes) with a workspace region of its own, so one group's
// short kernels overlap another group's apply.
#include <algorithm>
#include <cstdint>
#include <vector>

#include "internal.hpp"

using namespace bf16d;

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
uint64_t align16(uint64_t v) { return (v + 15) & ~uint64_t(15); }

struct Span {
    uintptr_t lo, hi;
};

// The device ranges written by the call (weights, the slots, workspace,
// results) may not overlap.
bool spans_disjoint(std::vector<Span> v) {
    v.erase(std::remove_if(v.begin(), v.end(), [](const Span &s) { return s.hi <= s.lo; }),
            v.end());
    std::sort(v.begin(), v.end(), [](const Span &a, const Span &b) { return a.lo < b.lo; });
    for (size_t i = 1; i < v.size(); ++i)
        if (v[i].lo < v[i - 1].hi) return false;
    return true;
}

constexpr uint32_t kMaxSlots = 64;
constexpr uint32_t kMaxCopyStreams = 8;
constexpr uint32_t kMaxLanes = 1;   // extra compute lanes beside the caller's stream

struct Events {
    hipEvent_t start = nullptr, tables = nullptr;
    std::vector<hipEvent_t> copied, applied, done;
    bool ok = true;
    Events(uint32_t slots, uint32_t lanes)
        : copied(slots, nullptr), applied(slots, nullptr), done(lanes, nullptr) {
        ok = hipEventCreateWithFlags(&start, hipEventDisableTiming) == hipSuccess &&
             hipEventCreateWithFlags(&tables, hipEventDisableTiming) == hipSuccess;
        for (uint32_t s = 0; s < slots && ok; ++s)
            ok = hipEventCreateWithFlags(&copied[s], hipEventDisableTiming) == hipSuccess &&
                 hipEventCreateWithFlags(&applied[s], hipEventDisableTiming) == hipSuccess;
        for (uint32_t l = 0; l < lanes && ok; ++l)
            ok = hipEventCreateWithFlags(&done[l], hipEventDisableTiming) == hipSuccess;
    }
    ~Events() {
        // an event still pending in a stream is released once it completes
        if (start) (void)hipEventDestroy(start);
        if (tables) (void)hipEventDestroy(tables);
        for (size_t s = 0; s < copied.size(); ++s) {
            if (copied[s]) (void)hipEventDestroy(copied[s]);
            if (applied[s]) (void)hipEventDestroy(applied[s]);
        }
        for (hipEvent_t e : done)
            if (e) (void)hipEventDestroy(e);
    }
};

}  // namespace

extern "C" int bf16d_decompress_streamed(const bf16d_stream_job *jobs, uint32_t count,
                                         const uint32_t *group_end, uint32_t groups,
                                         void *staging, size_t slot_bytes, uint32_t slots,
                                         void *workspace, size_t workspace_bytes,
                                         bf16d_result *results, hipStream_t compute,
                                         const hipStream_t *copy, uint32_t copy_streams,
                                         const hipStream_t *lanes, uint32_t n_lanes) {
    if (!jobs || count == 0 || !group_end || groups == 0 || groups > count || !staging ||
        !aligned16(staging) || slot_bytes == 0 || slot_bytes % 16 != 0 || slots < 2 ||
        slots > kMaxSlots || slot_bytes > SIZE_MAX / slots || !workspace ||
        !aligned16(workspace) || !results || !copy || copy_streams == 0 ||
        copy_streams > kMaxCopyStreams || n_lanes > kMaxLanes || (n_lanes > 0 && !lanes))
        return BF16D_EINVAL;
    const uint32_t n_run = 1 + n_lanes;   // compute lanes: the caller's stream first
    auto lane_stream = [&](uint32_t g) { return g % n_run == 0 ? compute : lanes[g % n_run - 1]; };
    // groups partition [0, count) in order; each group's payloads fit a slot.
    // Each group's decompress jobs point into its slot.
    std::vector<bf16d_decompress_job> dj(count);
    std::vector<uint64_t> offset(count, 0);
    std::vector<Span> spans;
    spans.reserve(size_t(count) + 4);
    uint32_t first = 0;
    for (uint32_t g = 0; g < groups; ++g) {
        const uint32_t end = group_end[g];
        if (end <= first || end > count || (g + 1 == groups && end != count)) return BF16D_EINVAL;
        uint8_t *slot = static_cast<uint8_t *>(staging) + (g % slots) * slot_bytes;
        uint64_t packed = 0;
        for (uint32_t j = first; j < end; ++j) {
            const bf16d_stream_job &J = jobs[j];
            if (J.payload_bytes > 0 && !J.payload) return BF16D_EINVAL;
            if (J.payload_bytes > slot_bytes) return BF16D_EINVAL;
            offset[j] = packed;
            packed += align16(J.payload_bytes);
            dj[j] = {J.weights, J.n, slot + offset[j], J.payload_bytes, J.checksum};
            spans.push_back({reinterpret_cast<uintptr_t>(J.weights),
                             reinterpret_cast<uintptr_t>(J.weights) + 2 * J.n});
        }
        if (packed > slot_bytes) return BF16D_EINVAL;
        first = end;
    }
    // every group's job table, laid out as its decompress call expects, all
    // uploaded at once after the largest group's workspace layout
    std::vector<DecompressPrep> prep(groups);
    std::vector<Layout> lay(groups);
    std::vector<size_t> table_at(groups);
    size_t base = 0, tables = 0;
    first = 0;
    for (uint32_t g = 0; g < groups; ++g) {
        const uint32_t end = group_end[g], cnt = end - first;
        if (decompress_prep(dj.data() + first, cnt, prep[g]) != BF16D_OK) return BF16D_EINVAL;
        lay[g] = make_layout(prep[g].tiles, prep[g].dtiles, cnt, false);
        base = std::max(base, lay[g].total);
        table_at[g] = tables;
        tables += align_up(decompress_table_bytes(lay[g], cnt), 256);
        first = end;
    }
    // lane l's call layout at l * base; the job tables after all of them
    base = align_up(base, 256);
    const size_t lanes_bytes = base * n_run;
    const size_t need = lanes_bytes + tables;
    if (workspace_bytes < need) return BF16D_EINVAL;
    spans.push_back({reinterpret_cast<uintptr_t>(staging),
                     reinterpret_cast<uintptr_t>(staging) + slots * slot_bytes});
    spans.push_back({reinterpret_cast<uintptr_t>(workspace),
                     reinterpret_cast<uintptr_t>(workspace) + need});
    spans.push_back({reinterpret_cast<uintptr_t>(results),
                     reinterpret_cast<uintptr_t>(results + count)});
    if (!spans_disjoint(spans)) return BF16D_EINVAL;
    std::vector<uint8_t> host(tables, 0);
    first = 0;
    for (uint32_t g = 0; g < groups; ++g) {
        const uint32_t end = group_end[g];
        decompress_table(dj.data() + first, end - first, prep[g], lay[g], host.data() + table_at[g]);
        // the kernels of group g read their job table from its place after the
        // lanes' layouts; offsets are relative to the group's lane region
        const size_t jobs_at = lanes_bytes + table_at[g] - (g % n_run) * base;
        lay[g].block_start = jobs_at + (lay[g].block_start - lay[g].jobs);
        lay[g].dtile_start = jobs_at + (lay[g].dtile_start - lay[g].jobs);
        lay[g].jobs = jobs_at;
        first = end;
    }

    Events ev(slots, n_run);
    if (!ev.ok) return BF16D_EHIP;
    auto fail = [](hipError_t e) { return e != hipSuccess; };
    auto *ws = static_cast<uint8_t *>(workspace);
    // the copies start after the caller's earlier work on the compute stream;
    // the job tables go up meanwhile (one upload; the source is pageable, so
    // the runtime stages it before returning), and the other lanes start
    // after them
    if (fail(hipEventRecord(ev.start, compute))) return BF16D_EHIP;
    for (uint32_t c = 0; c < copy_streams; ++c)
        if (fail(hipStreamWaitEvent(copy[c], ev.start, 0))) return BF16D_EHIP;
    if (fail(hipMemcpyAsync(ws + lanes_bytes, host.data(), host.size(), hipMemcpyHostToDevice,
                            compute)) ||
        fail(hipEventRecord(ev.tables, compute)))
        return BF16D_EHIP;
    for (uint32_t l = 0; l < n_lanes; ++l)
        if (fail(hipStreamWaitEvent(lanes[l], ev.tables, 0))) return BF16D_EHIP;
    first = 0;
    for (uint32_t g = 0; g < groups; ++g) {
        const uint32_t end = group_end[g], s = g % slots;
        hipStream_t cs = copy[g % copy_streams];
        uint8_t *slot = static_cast<uint8_t *>(staging) + s * slot_bytes;
        // the slot is free once the apply of group g - slots has read it
        if (g >= slots && fail(hipStreamWaitEvent(cs, ev.applied[s], 0))) return BF16D_EHIP;
        // one copy per run of payloads that lie in host memory exactly as
        // they are packed in the slot (the padding between them then comes
        // along; nothing reads it)
        for (uint32_t j = first; j < end;) {
            if (jobs[j].payload_bytes == 0) {
                ++j;
                continue;
            }
            uint32_t k = j + 1;
            while (k < end && jobs[k].payload_bytes > 0 &&
                   jobs[k].payload == jobs[j].payload + (offset[k] - offset[j]))
                ++k;
            const uint64_t bytes = offset[k - 1] - offset[j] + jobs[k - 1].payload_bytes;
            if (fail(hipMemcpyAsync(slot + offset[j], jobs[j].payload, bytes,
                                    hipMemcpyHostToDevice, cs)))
                return BF16D_EHIP;
            j = k;
        }
        hipStream_t ls = lane_stream(g);
        if (fail(hipEventRecord(ev.copied[s], cs)) ||
            fail(hipStreamWaitEvent(ls, ev.copied[s], 0)) ||
            fail(launch_decompress(lay[g], ws + (g % n_run) * base, end - first, prep[g].tiles,
                                   prep[g].dtiles, results + first, ls, nullptr)) ||
            fail(hipEventRecord(ev.applied[s], ls)))
            return BF16D_EHIP;
        first = end;
    }
    // the caller's stream completes only after every lane
    for (uint32_t l = 0; l < n_lanes; ++l)
        if (fail(hipEventRecord(ev.done[l], lanes[l])) ||
            fail(hipStreamWaitEvent(compute, ev.done[l], 0)))
            return BF16D_EHIP;
    return BF16D_OK;
}
