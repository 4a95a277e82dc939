"""Lossless delta compression of BF16 checkpoints on AMD MI355X (gfx950).

Python binding of libbf16delta (include/bf16delta.h).  It only marshals
arguments: torch tensors supply device memory and streams, and every step of
compression and decompression runs in the library's HIP kernels.  There is no
CPU fallback; tensors must live on a HIP device.  The one host step is the
codec race over finished payloads (race_compress / race_decompress), which the
pages run on the CPU by design; it too runs in the library.

The call shapes follow "Every byte counts: ARCv3 and the case for
cross-region RL", section "Using ARCv3":

    payload, checksum = delta_compress(src, dst)
    restored = delta_decompress(src, payload, checksum)   # src is rebuilt in place

The wire format is this project's own "bf16delta_v1", not ARCv3's.
"""
from __future__ import annotations

import ctypes
from typing import Sequence

import torch

from . import _native
from ._native import (OK, EINVAL, ECAPACITY, EFORMAT, ECHECKSUM, EHIP, EVERSION, BLOCK_ELEMS,
                      HEADER_BYTES, CompressJob, DecompressJob, RESULT_BYTES)

FORMAT = "bf16delta_v1"
BOUND_EXTRA_BYTES = 32   # a version-2 header is 32 bytes longer
_ALIGN = 256   # payload slots inside an arena start on this boundary

__all__ = ["delta_compress", "delta_decompress", "compress_batch", "decompress_batch",
           "CompressBatch", "DecompressBatch", "StreamedDecompress", "RemappedBatch",
           "decompress_remapped", "race_compress", "race_decompress", "codec_available",
           "RaceFrame", "DEFAULT_RACE", "FormatError", "ChecksumError",
           "CapacityError", "max_payload_bytes", "workspace_bytes", "FORMAT"]


class FormatError(ValueError):
    """The payload is malformed or does not match the tensor (weights end old)."""


class ChecksumError(RuntimeError):
    """The rebuilt weights fail the checksum (weights end old)."""


class CapacityError(RuntimeError):
    """A payload buffer is too small."""


def max_payload_bytes(n: int) -> int:
    return int(_native.lib().bf16d_max_payload_bytes(n))


def workspace_bytes(total_n: int, count: int) -> int:
    return int(_native.lib().bf16d_workspace_bytes(total_n, count))


def _check_format(compression_format: str) -> None:
    if compression_format != FORMAT:
        raise ValueError(f"unsupported compression_format {compression_format!r}: this "
                         f"library reads and writes {FORMAT!r} only")


def _weights_ptr(t: torch.Tensor, what: str) -> int:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{what} must be a tensor on a HIP device (got "
                        f"{getattr(t, 'device', type(t))}); there is no CPU path")
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{what} must hold 16-bit patterns (bfloat16), got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if t.numel() and t.data_ptr() % 16:
        raise ValueError(f"{what} must be 16-byte aligned")
    return t.data_ptr() if t.numel() else 0


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check_rc(rc: int, what: str) -> None:
    if rc != OK:
        raise RuntimeError(f"{what} failed: {_native.status_string(rc)}")


def _events(events):
    """(before, after) timing-enabled torch.cuda.Event pair -> bf16d_events*, or None."""
    if events is None:
        return None
    before, after = events
    for e in (before, after):
        if e.cuda_event == 0:       # torch creates the HIP event on first use
            e.record()
    return ctypes.byref(_native.Events(before.cuda_event, after.cuda_event))


def _results(buf: torch.Tensor, count: int) -> list[dict]:
    host = buf[: count * RESULT_BYTES].cpu().numpy().tobytes()
    out = []
    for j in range(count):
        r = _native.Result.from_buffer_copy(host, j * RESULT_BYTES)
        out.append({k: int(getattr(r, k)) for k, _ in _native.Result._fields_ if k != "reserved"})
    return out


class CompressBatch:
    """A prepared batched compress call over fixed (src, dst) pairs.

    It owns one payload arena (a slot of `capacity[j]` bytes per job), the
    workspace, and a device result buffer.  `run()` enqueues one batched call
    on the current stream.  `results()` waits for it and returns one dict
    per job."""

    def __init__(self, pairs: Sequence[tuple[torch.Tensor, torch.Tensor]],
                 capacities: Sequence[int] | None = None, bindings=None,
                 slot_bytes: int | None = None):
        """bindings: None (version-1 payloads), or per job (base_version,
        target_version, overwrite) for version-2 payloads (bf16d_compress_bound).
        slot_bytes: None for the full workspace (a 2 KiB record slot per block,
        12.5 % of the weights), or a smaller slot (a multiple of 16, 16 to
        2048; 256 makes the workspace about 1.9 % of the weights), records
        that do not fit being staged in the payload buffer's spare room
        (bf16d_compress_workspace_bytes)."""
        if not pairs:
            raise ValueError("empty batch")
        self.device = pairs[0][0].device
        self.count = len(pairs)
        self.n = [p[0].numel() for p in pairs]
        self.bindings = None
        if bindings is not None:
            if len(bindings) != self.count:
                raise ValueError("one binding per job")
            self.bindings = (_native.Binding * self.count)(
                *[_native.Binding(int(b) & 0xFFFFFFFFFFFFFFFF, int(t) & 0xFFFFFFFFFFFFFFFF,
                                  _native.BIND_OVERWRITE if ow else 0, 0)
                  for b, t, ow in bindings])
        if capacities is None:
            extra = BOUND_EXTRA_BYTES if bindings is not None else 0
            capacities = [max_payload_bytes(n) + extra for n in self.n]
        self.capacity = [int(c) for c in capacities]
        self.offset = []
        at = 0
        for cap in self.capacity:
            self.offset.append(at)
            at += (cap + _ALIGN - 1) // _ALIGN * _ALIGN
        self.arena = torch.empty(max(at, _ALIGN), dtype=torch.uint8, device=self.device)
        if slot_bytes is None:
            self.ws_bytes = workspace_bytes(sum(self.n), self.count)
        else:
            self.ws_bytes = int(_native.lib().bf16d_compress_workspace_bytes(
                sum(self.n), self.count, int(slot_bytes)))
            if self.ws_bytes == 0:
                raise ValueError("slot_bytes must be a multiple of 16 from 16 to 2048")
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.result_buf = torch.empty(self.count * RESULT_BYTES, dtype=torch.uint8,
                                      device=self.device)
        self.jobs = (CompressJob * self.count)()
        base = self.arena.data_ptr()
        self.pairs = list(pairs)   # keep the tensors alive
        for j, (src, dst) in enumerate(pairs):
            if src.shape != dst.shape:
                raise ValueError(f"job {j}: src and dst differ in shape")
            if src.device != self.device or dst.device != self.device:
                raise ValueError("all tensors of a batch must be on one device")
            self.jobs[j] = CompressJob(_weights_ptr(src, "src"), _weights_ptr(dst, "dst"),
                                       src.numel(), base + self.offset[j], self.capacity[j])

    def run(self, events=None) -> None:
        """Enqueue the call.  `events`: optional (before, after) torch.cuda.Event
        pair, recorded around the encode kernel."""
        if self.bindings is not None:
            if events is not None:
                raise ValueError("kernel events are not offered for bound payloads")
            rc = _native.lib().bf16d_compress_bound(self.jobs, self.bindings, self.count,
                                                    self.workspace.data_ptr(), self.ws_bytes,
                                                    self.result_buf.data_ptr(),
                                                    _stream(self.device))
            _check_rc(rc, "bf16d_compress_bound")
            return
        ev = _events(events)
        rc = _native.lib().bf16d_compress_ex(self.jobs, self.count, self.workspace.data_ptr(),
                                             self.ws_bytes, self.result_buf.data_ptr(),
                                             _stream(self.device), ev)
        _check_rc(rc, "bf16d_compress")

    def results(self) -> list[dict]:
        return _results(self.result_buf, self.count)

    def payload(self, j: int, nbytes: int) -> torch.Tensor:
        return self.arena[self.offset[j]: self.offset[j] + nbytes]


class DecompressBatch:
    """A prepared batched in-place decompress call over fixed (weights, payload,
    checksum) triples.  `run()` enqueues it on the current stream."""

    def __init__(self, items: Sequence[tuple[torch.Tensor, torch.Tensor, int]],
                 versions: torch.Tensor | None = None, verify_first: bool = False,
                 workspace_bytes_override: int | None = None):
        """versions: None, or the receiver's version words, an int64 tensor of
        len(items) on the weights' device, checked against version-2 payloads
        and advanced in place (bf16d_decompress_bound).
        verify_first: check every job before writing it, so that a failing
        payload never touches its weights (bf16d_decompress_verified; not
        with version words).
        workspace_bytes_override: a workspace of this size instead of
        bf16d_workspace_bytes (which leaves room for the undo area of
        overwrite payloads; a smaller one verifies them first instead)."""
        if verify_first and versions is not None:
            raise ValueError("verify_first is not offered with version words")
        self.verify_first = verify_first
        if not items:
            raise ValueError("empty batch")
        self.device = items[0][0].device
        self.count = len(items)
        self.items = list(items)
        self.versions = versions
        if versions is not None:
            if (versions.device != self.device or versions.dtype not in (torch.int64,
                                                                         torch.uint64)
                    or versions.numel() != self.count or not versions.is_contiguous()):
                raise TypeError("versions must be a contiguous 64-bit tensor with one word "
                                "per job on the weights' device")
        n_total = sum(w.numel() for w, _, _ in items)
        self.ws_bytes = workspace_bytes(n_total, self.count) if workspace_bytes_override is None \
            else int(workspace_bytes_override)
        self.workspace = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8,
                                     device=self.device)
        self.result_buf = torch.empty(self.count * RESULT_BYTES, dtype=torch.uint8,
                                      device=self.device)
        self.jobs = (DecompressJob * self.count)()
        for j, (w, payload, checksum) in enumerate(items):
            self._set(j, w, payload, checksum)

    def _set(self, j, w, payload, checksum):
        if payload.dtype != torch.uint8 or payload.device != self.device or \
                not payload.is_contiguous():
            raise TypeError("payload must be a contiguous uint8 tensor on the weights' device")
        if payload.data_ptr() % 16:
            raise ValueError("payload must be 16-byte aligned")
        self.jobs[j] = DecompressJob(_weights_ptr(w, "weights"), w.numel(), payload.data_ptr(),
                                     payload.numel(), int(checksum) & 0xFFFFFFFFFFFFFFFF)

    def set_checksum(self, j: int, checksum: int) -> None:
        self.jobs[j].checksum = int(checksum) & 0xFFFFFFFFFFFFFFFF

    def run(self, events=None) -> None:
        """Enqueue the call.  `events`: optional (before, after) torch.cuda.Event
        pair, recorded around the apply kernel."""
        if self.versions is not None:
            if events is not None:
                raise ValueError("kernel events are not offered with version words")
            rc = _native.lib().bf16d_decompress_bound(self.jobs, self.versions.data_ptr(),
                                                      self.count, self.workspace.data_ptr(),
                                                      self.ws_bytes, self.result_buf.data_ptr(),
                                                      _stream(self.device))
            _check_rc(rc, "bf16d_decompress_bound")
            return
        ev = _events(events)
        fn = _native.lib().bf16d_decompress_verified if self.verify_first else \
            _native.lib().bf16d_decompress_ex
        rc = fn(self.jobs, self.count, self.workspace.data_ptr(), self.ws_bytes,
                self.result_buf.data_ptr(), _stream(self.device), ev)
        _check_rc(rc, "bf16d_decompress")

    def results(self) -> list[dict]:
        return _results(self.result_buf, self.count)


# The streamed receiver's copy and compute-lane streams, created once per
# device and shared by every StreamedDecompress: HIP spreads streams over a
# few hardware queues (4 by default), and streams that share a queue run one
# after the other, so each receiver creating streams of its own would soon
# put its copies and its applies on one queue.
_side_streams: dict = {}


def _streams(device: torch.device, kind: str, count: int) -> list:
    key = (device.index, kind)
    have = _side_streams.setdefault(key, [])
    while len(have) < count:
        have.append(torch.cuda.Stream(device=device))
    return have[:count]


class StreamedDecompress:
    """A prepared streamed receiver (bf16d_decompress_streamed): payloads in
    pinned host memory, applied in place group by group through a ring of
    device slots, the copies on streams of their own.  The copy and lane
    streams are shared by every receiver on a device, so calls of different
    receivers must not overlap in time.

    items  : (weights device tensor, payload host uint8 tensor, checksum);
             pin the payloads (torch's pin_memory) for the copies to overlap.
    groups : number of jobs in each group, in order (for a model, a layer).
    slots  : device slots in the ring (2 to 64); with 3 the copies do not
             wait on the apply just before them, and with 5 (the default)
             they almost never wait (7B-shaped checkpoint, one layer per
             group: 1.04x the plain copy of the payloads, against 1.05x with
             4 slots and 1.11x with 3).
    copy_streams : streams the groups' copies alternate over (1 to 8); with
             2 each transfer's fixed cost hides behind the other's transfer.
             More than 2 beside two lanes exceeds HIP's 4 hardware queues by
             default, and streams that share a queue serialise (3 measured
             1.5x slower).
    lanes  : compute streams the groups' applies alternate over (1 or 2):
             the current stream, and with 2 one more, so that a group's
             short kernels overlap the previous group's apply.
    The device slots are sized for the largest group."""

    def __init__(self, items: Sequence[tuple[torch.Tensor, torch.Tensor, int]],
                 groups: Sequence[int], slots: int = 5, copy_streams: int = 2, lanes: int = 2):
        if not items or not groups or sum(groups) != len(items) or min(groups) <= 0:
            raise ValueError("groups must be positive and cover every item")
        if not 2 <= slots <= 64:
            raise ValueError("slots must be between 2 and 64")
        if not 1 <= copy_streams <= 8:
            raise ValueError("copy_streams must be between 1 and 8")
        if lanes not in (1, 2):
            raise ValueError("lanes must be 1 or 2")
        self.slots = slots
        self.device = items[0][0].device
        self.count = len(items)
        self.items = list(items)   # keep the tensors alive
        self.jobs = (_native.StreamJob * self.count)()
        pad16 = lambda b: (b + 15) // 16 * 16
        for j, (w, p, cs) in enumerate(items):
            if p.device.type != "cpu" or p.dtype != torch.uint8 or not p.is_contiguous():
                raise TypeError("payloads must be contiguous uint8 tensors in host memory")
            self.jobs[j] = _native.StreamJob(_weights_ptr(w, "weights"), w.numel(),
                                             p.data_ptr() if p.numel() else None, p.numel(),
                                             int(cs) & 0xFFFFFFFFFFFFFFFF)
        ends, at, slot = [], 0, 16
        for g in groups:
            slot = max(slot, sum(pad16(self.items[j][1].numel()) for j in range(at, at + g)))
            at += g
            ends.append(at)
        self.groups = len(ends)
        self.group_end = (ctypes.c_uint32 * self.groups)(*ends)
        self.slot_bytes = pad16(slot)
        self.staging = torch.empty(slots * self.slot_bytes, dtype=torch.uint8,
                                   device=self.device)
        self.ws_bytes = workspace_bytes(sum(w.numel() for w, _, _ in items), self.count)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.result_buf = torch.empty(self.count * RESULT_BYTES, dtype=torch.uint8,
                                      device=self.device)
        self.copy_streams = _streams(self.device, "copy", copy_streams)
        self._copy = (ctypes.c_void_p * copy_streams)(*[c.cuda_stream for c in self.copy_streams])
        self.lane_streams = _streams(self.device, "lane", lanes - 1)
        self._lanes = (ctypes.c_void_p * max(1, lanes - 1))(
            *[c.cuda_stream for c in self.lane_streams])

    @staticmethod
    def pin_packed(payloads: Sequence[torch.Tensor]) -> list[torch.Tensor]:
        """Copies of `payloads` packed into one pinned host buffer, each at the
        next 16-byte boundary: the layout in which a group's payloads are
        copied to the device with one transfer."""
        pad16 = lambda b: (b + 15) // 16 * 16
        total = sum(pad16(p.numel()) for p in payloads)
        flat = torch.empty(max(total, 16), dtype=torch.uint8).pin_memory()
        out, at = [], 0
        for p in payloads:
            view = flat[at:at + p.numel()]
            view.copy_(p.reshape(-1).view(torch.uint8))
            out.append(view)
            at += pad16(p.numel())
        return out

    def run(self) -> None:
        """Enqueue the call on the current stream (copies on self.copy_streams)."""
        rc = _native.lib().bf16d_decompress_streamed(
            self.jobs, self.count, self.group_end, self.groups, self.staging.data_ptr(),
            self.slot_bytes, self.slots, self.workspace.data_ptr(), self.ws_bytes,
            self.result_buf.data_ptr(), _stream(self.device), self._copy, len(self.copy_streams),
            self._lanes if self.lane_streams else None, len(self.lane_streams))
        _check_rc(rc, "bf16d_decompress_streamed")

    def results(self) -> list[dict]:
        return _results(self.result_buf, self.count)


class RemappedBatch:
    """A prepared remapped decompress (bf16d_decompress_remapped): payloads
    made from logical tensors, applied in place onto reordered physical
    layouts in one batched call.

    items: (target, payload, checksum) per tensor.  target is either a weights
    tensor (no remap) or (n, segments) with segments a list of (first, view):
    logical elements [first, first + view.numel()) of the n-element tensor
    live in `view` (a contiguous 16-bit device view, `first` a multiple of
    8192).
    prepared: True (the default) checks and uploads the layout once
    (bf16d_remap_prepare) and makes every run() a prepared call
    (bf16d_decompress_remapped_prepared); False passes the segments at every
    call (bf16d_decompress_remapped)."""

    def __init__(self, items, prepared: bool = True):
        if not items:
            raise ValueError("empty batch")
        self.count = len(items)
        self.items = list(items)   # keep the tensors alive
        self.jobs = (DecompressJob * self.count)()
        self.remaps = (_native.Remap * self.count)()
        self._keep = []
        total_n, total_segs, device = 0, 0, None
        for j, (target, payload, checksum) in enumerate(items):
            if payload.dtype != torch.uint8 or payload.device.type != "cuda" or \
                    not payload.is_contiguous():
                raise TypeError("payload must be a contiguous uint8 device tensor")
            device = payload.device
            if isinstance(target, torch.Tensor):
                n, wptr = target.numel(), _weights_ptr(target, "weights")
                self.remaps[j] = _native.Remap(None, 0)
            else:
                n, segs = target
                arr = (_native.Segment * len(segs))()
                for k, (first, view) in enumerate(segs):
                    arr[k] = _native.Segment(first, view.numel(), _weights_ptr(view, "segment"))
                self._keep.append(arr)
                self.remaps[j] = _native.Remap(arr, len(segs))
                wptr, total_segs = None, total_segs + len(segs)
            self.jobs[j] = DecompressJob(wptr, n, payload.data_ptr() if payload.numel() else None,
                                         payload.numel(), int(checksum) & 0xFFFFFFFFFFFFFFFF)
            total_n += n
        self.device = device
        self.ws_bytes = int(_native.lib().bf16d_workspace_bytes_remapped(total_n, self.count,
                                                                         total_segs))
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.result_buf = torch.empty(self.count * RESULT_BYTES, dtype=torch.uint8,
                                      device=device)
        self.prepared = prepared
        if prepared:
            L = _native.lib()
            self.plan = ctypes.create_string_buffer(
                int(L.bf16d_remap_plan_bytes(self.count, total_segs)))
            map_bytes = int(L.bf16d_remap_map_bytes(total_n, self.count))
            self.block_map = torch.empty(map_bytes // 8, dtype=torch.int64, device=device)
            rc = L.bf16d_remap_prepare(self.jobs, self.remaps, self.count, self.plan,
                                       len(self.plan), self.block_map.data_ptr(), map_bytes,
                                       _stream(device))
            _check_rc(rc, "bf16d_remap_prepare")

    def run(self) -> None:
        if self.prepared:
            rc = _native.lib().bf16d_decompress_remapped_prepared(
                self.jobs, self.count, self.plan, self.block_map.data_ptr(),
                self.workspace.data_ptr(), self.ws_bytes, self.result_buf.data_ptr(),
                _stream(self.device))
            _check_rc(rc, "bf16d_decompress_remapped_prepared")
            return
        rc = _native.lib().bf16d_decompress_remapped(
            self.jobs, self.remaps, self.count, self.workspace.data_ptr(), self.ws_bytes,
            self.result_buf.data_ptr(), _stream(self.device))
        _check_rc(rc, "bf16d_decompress_remapped")

    def results(self) -> list[dict]:
        return _results(self.result_buf, self.count)


def decompress_remapped(items, prepared: bool = True) -> list[dict]:
    """One remapped decompress call (see RemappedBatch); returns the per-job
    result dicts."""
    batch = RemappedBatch(items, prepared)
    batch.run()
    return batch.results()


# Below this many bytes of worst-case payload a batch gets worst-case
# capacities up front, so that it never runs twice; above it, a first guess
# (1/16 of the weights plus the framing) keeps the arena small, and only the
# jobs that report a larger size are compressed again.
_UPFRONT_LIMIT = 256 << 20


def _first_capacity(n: int) -> int:
    """A first guess at the payload size: framing plus 1/16 of the weights
    (the payload of a delta changing up to about 6 % of the elements)."""
    nb = -(-n // BLOCK_ELEMS)
    return min(max_payload_bytes(n), HEADER_BYTES + 4 * nb + (2 * n) // 16 + 4096)


def compress_batch(pairs: Sequence[tuple[torch.Tensor, torch.Tensor]], bindings=None):
    """Compress several (src, dst) pairs in one batched call.  bindings: None,
    or per pair (base_version, target_version, overwrite) for version-2
    payloads.

    Capacities: the worst case (bf16d_max_payload_bytes) when the whole batch's
    worst case is below 256 MiB, so small batches always finish in one call;
    otherwise a first guess of 1/16 of the weights, and the jobs that report
    ECAPACITY (with their exact size) are compressed again in a second batch
    of their own.

    Returns a list of (payload uint8 tensor, checksum int, stats dict).  The
    payloads are views into one or two device arenas."""
    extra = BOUND_EXTRA_BYTES if bindings is not None else 0
    worst = [max_payload_bytes(s.numel()) + extra for s, _ in pairs]
    if sum(worst) <= _UPFRONT_LIMIT:
        caps = worst
    else:
        caps = [_first_capacity(s.numel()) + extra for s, _ in pairs]
    batch = CompressBatch(pairs, caps, bindings)
    batch.run()
    res = batch.results()
    where = [(batch, j) for j in range(len(pairs))]
    short = [j for j, r in enumerate(res) if r["status"] == ECAPACITY]
    if short:
        again = CompressBatch([pairs[j] for j in short], [res[j]["payload_bytes"] for j in short],
                              None if bindings is None else [bindings[j] for j in short])
        again.run()
        for k, (j, r) in enumerate(zip(short, again.results())):
            res[j] = r
            where[j] = (again, k)
    out = []
    for j, r in enumerate(res):
        if r["status"] != OK:
            raise RuntimeError(f"job {j}: {_native.status_string(r['status'])}")
        b, k = where[j]
        out.append((b.payload(k, r["payload_bytes"]), r["checksum"], r))
    return out


def decompress_batch(items: Sequence[tuple[torch.Tensor, torch.Tensor, int]],
                     versions: torch.Tensor | None = None,
                     verify_first: bool = False) -> list[dict]:
    """Apply several payloads in place in one batched call, optionally with the
    receiver's version words or verified first (see DecompressBatch).
    Returns the per-job result dicts, without raising on per-job failures."""
    batch = DecompressBatch(items, versions, verify_first)
    batch.run()
    return batch.results()


def delta_compress(src: torch.Tensor, dst: torch.Tensor, compression_format: str = FORMAT):
    """(compressed_diff, checksum) of the update src -> dst.  Both are bf16
    tensors of one shape on a HIP device; the payload is a uint8 device tensor."""
    _check_format(compression_format)
    payload, checksum, _ = compress_batch([(src, dst)])[0]
    return payload.clone(), checksum


def delta_decompress(src: torch.Tensor, compressed_diff: torch.Tensor, checksum: int,
                     compression_format: str = FORMAT) -> torch.Tensor:
    """Rebuild the new weights in place in `src` and return it.  Raises
    FormatError or ChecksumError (with `src` holding the old weights exactly)
    if the payload does not apply."""
    _check_format(compression_format)
    r = decompress_batch([(src, compressed_diff, checksum)])[0]
    if r["status"] == EFORMAT:
        raise FormatError("payload rejected (malformed or not for this tensor); weights unchanged")
    if r["status"] == ECHECKSUM:
        raise ChecksumError("rebuilt weights fail the checksum; weights restored to the old values")
    if r["status"] != OK:
        raise RuntimeError(_native.status_string(r["status"]))
    return src


# ------------------------------------------------------------- codec race ---
# The one host step of the path: "Every byte counts: ARCv3 and the case for
# cross-region RL", section "Deep dive into ARCv3", races general-purpose
# codecs over each tensor's output on the CPU and keeps the smallest.  The race
# itself runs in the library (bf16d_race_compress / bf16d_race_decompress);
# this only marshals host buffers.

# candidates raced when the caller names none: fast and strong settings of the
# common families, about 4 minutes of one core per GB of payload; xz and the
# highest levels are left to callers with more idle cores
DEFAULT_RACE = (("lz4", 1), ("zstd", 1), ("zstd", 3), ("zstd", 9), ("zlib", 6), ("brotli", 5))


class RaceFrame(tuple):
    """(frame uint8 host tensor, codec name, level) of one raced payload."""
    __slots__ = ()

    def __new__(cls, frame, codec, level):
        return super().__new__(cls, (frame, codec, level))

    frame = property(lambda self: self[0])
    codec = property(lambda self: self[1])
    level = property(lambda self: self[2])


_CODEC_NAMES = {v: k for k, v in _native.CODECS.items()}


def codec_available(name: str) -> bool:
    """Whether this host has the runtime library of codec `name`."""
    return bool(_native.lib().bf16d_codec_available(_native.CODECS[name]))


def _host_u8(buf, what: str) -> torch.Tensor:
    if not isinstance(buf, torch.Tensor):
        buf = torch.from_numpy(buf) if hasattr(buf, "__array_interface__") else buf
    if (not isinstance(buf, torch.Tensor) or buf.device.type != "cpu"
            or buf.dtype != torch.uint8 or not buf.is_contiguous()):
        raise TypeError(f"{what} must be a contiguous uint8 buffer in host memory")
    return buf.reshape(-1)


def _ptr(t: torch.Tensor):
    return t.data_ptr() if t.numel() else None


def race_compress(payloads, candidates=DEFAULT_RACE, threads: int = 0) -> list[RaceFrame]:
    """Race `candidates` ((codec name, level) pairs) over every host payload on
    `threads` CPU threads (0: all) and return each payload's smallest frame."""
    ins = [_host_u8(p, "payload") for p in payloads]
    cands = (_native.Codec * max(len(candidates), 1))()
    for k, (name, level) in enumerate(candidates):
        if name not in _native.CODECS:
            raise ValueError(f"unknown codec {name!r}")
        cands[k] = _native.Codec(_native.CODECS[name], level)
    lib = _native.lib()
    outs = [torch.empty(int(lib.bf16d_race_bound(t.numel())), dtype=torch.uint8) for t in ins]
    jobs = (_native.RaceJob * max(len(ins), 1))()
    for j, (t, o) in enumerate(zip(ins, outs)):
        jobs[j] = _native.RaceJob(_ptr(t), t.numel(), o.data_ptr(), o.numel(), 0, 0, 0, 0, 0)
    rc = lib.bf16d_race_compress(jobs, len(ins), cands, len(candidates), threads)
    if rc != OK:
        raise ValueError(f"bf16d_race_compress: {_native.status_string(rc)} (an unknown or "
                         f"unavailable codec, or a level out of range)")
    return [RaceFrame(o[:jobs[j].out_bytes], _CODEC_NAMES[jobs[j].codec], jobs[j].level)
            for j, o in enumerate(outs)]


def race_decompress(frames, threads: int = 0, pin: bool = False) -> list[torch.Tensor]:
    """Decode race frames back into payloads (uint8 host tensors).  With
    pin=True the payloads are packed into one pinned buffer at 16-byte
    boundaries, the layout StreamedDecompress copies in one transfer per
    group.  Raises FormatError for a malformed frame."""
    ins = [_host_u8(f[0] if isinstance(f, RaceFrame) else f, "frame") for f in frames]
    lib = _native.lib()
    raw = []
    for t in ins:
        n = ctypes.c_uint64(0)
        if lib.bf16d_race_frame_info(_ptr(t), t.numel(), ctypes.byref(n), None, None) != OK:
            raise FormatError("not a race frame")
        raw.append(n.value)
    pad16 = lambda b: (b + 15) // 16 * 16
    if pin:
        flat = torch.empty(max(sum(pad16(b) for b in raw), 16), dtype=torch.uint8,
                           pin_memory=True)
        at = [0]
        for b in raw[:-1]:
            at.append(at[-1] + pad16(b))
        outs = [flat[a:a + b] for a, b in zip(at, raw)]
    else:
        outs = [torch.empty(b, dtype=torch.uint8) for b in raw]
    jobs = (_native.RaceJob * max(len(ins), 1))()
    for j, (t, o) in enumerate(zip(ins, outs)):
        jobs[j] = _native.RaceJob(_ptr(t), t.numel(), _ptr(o), o.numel(), 0, 0, 0, 0, 0)
    rc = lib.bf16d_race_decompress(jobs, len(ins), threads)
    _check_rc(rc, "bf16d_race_decompress")
    for j in range(len(ins)):
        if jobs[j].status != OK:
            err = FormatError if jobs[j].status == EFORMAT else RuntimeError
            raise err(f"frame {j}: {_native.status_string(jobs[j].status)}")
    return outs
