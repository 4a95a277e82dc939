"""Benchmark of the BF16 delta hot path on one MI355X.

Workload: a 7B-shaped BF16 checkpoint pair: 32 layers, hidden 4096, FFN
11008, vocab 32000, 291 tensors and 6.74e9 elements per checkpoint.  Both
checkpoints sit in HBM.  2% of each tensor's elements change, with a
95/4.5/0.5 mantissa/exponent/sign mix.  In 2-D tensors the changes are
clustered: 70% fall in 10% of the rows.

One step is the whole hot path over the checkpoint:
  - one batched compress of all 291 tensors (old, new -> payloads +
    checksums);
  - one batched, checksum-verified, in-place decompress of those payloads
    into a receiver copy of the weights.
The receiver copy alternates between old and new.  A payload depends only on
the XOR mask, so the same payload takes new back to old, verified against
old's checksum.

Reported:
  value     : GB/s of BF16 weights through the round trip, 2*n / step time
  compress  : GB/s of weights, and % of HBM peak on algorithmic bytes (4n + P)
  decompress: GB/s of weights, and % of HBM peak on algorithmic bytes (2n + P + 2c)
  roofline  : the encode kernel (the dominant kernel of a step) against 8 TB/s,
              timed with events recorded around it on its stream
  roofline_decompress : the apply kernel the same way, and on its effective
              bytes: 2n + P + every 32-byte sector that holds a change (the
              device writes sectors, not the changed elements alone); and its
              fraction of the in-place floor probe timed in the same rounds
  decompress_verify_first : the two-pass decompress that checks every job
              before writing it (weights untouched on failure), against the
              single in-place pass
  compress_small_workspace : the same compress with 256-byte record slots
              (workspace about 1.9 % of the weights instead of 12.9 %)
  change_rate_sweep : compress and decompress of one 1 GiB tensor at 0.085,
              1, 3 and 5 % uniform changes, each kernel timed after a cache
              flush, with their main kernels' fractions of 8 TB/s, of the read
              ceiling and of the in-place floor, and a compress timed right
              after a decompress; the bitmap / gap-list histogram per rate
  achievable: the read ceiling of the encoder's access pattern (a probe
              kernel that only reads, with the kernels' own loads), over old
              and new and over old alone, and each main kernel's fraction of
              it; the apply pass's changed-chunk writes alone; and the
              in-place floor (a probe that reads old and writes back,
              unchanged, the 16-byte chunks the delta changes: a reference
              point for that traffic, not a strict bound), timed in the same
              rounds as the apply kernel over the receiver's own buffer
  remapped_decompress : the same decompress onto a layout with each layer's
              gate and up projections paired in groups of 64 rows
  bound_overwrite : the same pair as version-2 overwrite payloads (absolute
              values, written in place with an undo log)
  codec_race : the host race of general-purpose codecs over every payload,
              and the payload % of the weights after it
  streamed_receiver : the same decompress with the payloads in pinned host
              memory, copied in layer by layer while earlier layers are
              applied, through a ring of five device slots with the copies
              on two streams and the applies on two compute lanes (and with
              three slots and one lane, and two slots on one stream, for
              comparison);
              PCIe-inclusive, context, not `value`
  cpu_baseline : the CPU oracle on a bounded sample of the same workload, on
              one core, and beside it on up to 16 host threads

Only one GPU is used; --gpus above 1 is refused.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "compress / decompress GB/s of BF16 weights (% of HBM peak); payload % of orig"
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "encode_kernel_7b_traffic.txt")
KERNEL_SOURCES = ("lossless_bf16_weight_xor_amd/csrc/compress.hip",
                  "lossless_bf16_weight_xor_amd/csrc/internal.hpp")
APPLY_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "apply_kernel_7b_traffic.txt")
APPLY_SOURCES = ("lossless_bf16_weight_xor_amd/csrc/decompress.hip",
                 "lossless_bf16_weight_xor_amd/csrc/internal.hpp")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def ensure_built():
    from lossless_bf16_weight_xor_amd import _native
    if not os.path.exists(_native.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()


def generate(workload: str, device, limit=None):
    from lossless_bf16_weight_xor_amd import synth
    if workload == "7b":
        it = synth.config2(device, limit=limit)
        desc = ("7B-shaped BF16 checkpoint pair (32 layers, hidden 4096, FFN 11008, vocab 32000, "
                "291 tensors), both resident; 2% of elements changed per tensor, 95/4.5/0.5 "
                "mantissa/exponent/sign, 70% of changes in 10% of rows")
    elif workload == "70b-half":
        it = synth.config5(device, limit=limit)
        desc = ("one-GPU share of a 70B-shaped model: 40 of 80 layers (hidden 8192, FFN 28672, "
                "GQA 64q/8kv, head_dim 128, 360 tensors); 1% uniform changes, 95/4.5/0.5")
    elif workload.startswith("c3-") and workload[3:] in synth.C3_RATES:
        rate = workload[3:]
        src, dst = synth.config3(device, rate)
        it = [("tensor", src, dst)]
        desc = (f"one 1-D BF16 tensor of 536,870,912 elements (1 GiB), {float(rate) * 100:g}% "
                "uniform changes, 95/4.5/0.5")
    else:
        raise SystemExit(f"unknown workload {workload}")
    names, pairs = [], []
    for name, src, dst in it:
        names.append(name)
        pairs.append((src.reshape(-1), dst.reshape(-1)))
    return names, pairs, desc


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(elements: int, profile=TRAFFIC_PROFILE, sources=KERNEL_SOURCES):
    """HBM bytes per launch of a kernel (the encoder by default) from its
    committed counter summary, or None if there is none, it was taken on
    another workload (element count), or the kernel sources changed since."""
    if not os.path.exists(profile):
        return None
    fields = {}
    with open(profile) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != kernel_source_hash(sources):
        return None
    if fields.get("elements_per_call") != str(elements):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def layer_groups(names, layers_per_group=1):
    """Sizes of the groups of consecutive tensors: each transformer layer is a
    unit, and so is every tensor outside the layers; a group holds
    `layers_per_group` units."""
    keys = [".".join(n.split(".")[:2]) if n.startswith("layers.") else n for n in names]
    units = []
    for i, k in enumerate(keys):
        if i and k == keys[i - 1]:
            units[-1] += 1
        else:
            units.append(1)
    return [sum(units[i:i + layers_per_group]) for i in range(0, len(units), layers_per_group)]


def streamed(bd, names, pairs, payloads, cs_new, cs_old, steps, td, layers_per_group, slots,
             copies, lanes):
    """The streamed receiver: payloads in pinned host memory, applied layer by
    layer through a ring of `slots` device slots while the next layers'
    payloads are copied in.  Reported next to the device-resident numbers,
    never as `value`."""
    dev = pairs[0][0].device
    host = bd.StreamedDecompress.pin_packed([p.cpu() for p in payloads])
    groups = layer_groups(names, layers_per_group)
    recv = [s.clone() for s, _ in pairs]
    sd = bd.StreamedDecompress(list(zip(recv, host, cs_new)), groups, slots=slots,
                               copy_streams=copies, lanes=lanes)
    # the host-to-device copy of every payload byte on its own
    P = sum(h.numel() for h in host)
    flat = torch.empty(P, dtype=torch.uint8).pin_memory()
    at = 0
    for h in host:
        flat[at:at + h.numel()].copy_(h)
        at += h.numel()
    dbuf = torch.empty(P, dtype=torch.uint8, device=dev)
    t_h2d, t_str = [], []
    direction = 0
    warm = 4   # the first calls map the pinned buffer and are slower
    for i in range(steps + warm):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record()
        dbuf.copy_(flat, non_blocking=True)
        e[1].record()
        cs = cs_new if direction == 0 else cs_old
        for j in range(len(cs)):
            sd.jobs[j].checksum = cs[j]
        e[2].record()
        sd.run()
        e[3].record()
        torch.cuda.synchronize()
        assert all(r["status"] == bd.OK for r in sd.results()), "streamed decompress failed"
        direction ^= 1
        if i >= warm:
            t_h2d.append(e[0].elapsed_time(e[1]) / 1e3)
            t_str.append(e[2].elapsed_time(e[3]) / 1e3)
    for w, (s, d) in zip(recv, pairs):
        ref = d if direction == 1 else s
        assert torch.equal(w.view(torch.int16), ref.view(torch.int16)), "streamed not bit-exact"
    n = sum(s.numel() for s, _ in pairs)
    ts, th = float(np.median(t_str)), float(np.median(t_h2d))
    slot = sd.slot_bytes
    del recv, sd, dbuf
    return {"layers_per_group": layers_per_group, "groups": len(groups), "slots": slots,
            "copy_streams": copies, "lanes": lanes,
            "slot_bytes": slot,
            "ms": round(1e3 * ts, 4),
            "gbps_weights_pcie_inclusive": round(2 * n / ts / 1e9, 2),
            "h2d_payload_ms": round(1e3 * th, 4), "h2d_gbps": round(P / th / 1e9, 2),
            "device_resident_decompress_ms": round(1e3 * td, 4),
            "overlap": round((th + td) / ts, 3)}


def codec_race(bd, payloads, threads):
    """The host codec race over every payload (trainer side), then the race
    decode into one pinned buffer (receiver side), on `threads` CPU threads.
    The pages give 0.19% of the BF16 weight size as the average payload of
    real RL deltas; this workload's changes are synthetic, so that figure is
    context only."""
    host = [p.cpu() for p in payloads]
    raw = sum(h.numel() for h in host)
    t0 = time.perf_counter()
    frames = bd.race_compress(host, bd.DEFAULT_RACE, threads=threads)
    t_race = time.perf_counter() - t0
    t0 = time.perf_counter()
    back = bd.race_decompress(frames, threads=threads, pin=True)
    t_dec = time.perf_counter() - t0
    assert all(torch.equal(a, b) for a, b in zip(back, host)), "race round trip not exact"
    raced = sum(f.frame.numel() for f in frames)
    winners = {}
    for f in frames:
        key = f"{f.codec}-{f.level}" if f.codec != "stored" else "stored"
        winners[key] = winners.get(key, 0) + 1
    return {"candidates": [f"{c}-{l}" for c, l in bd.DEFAULT_RACE], "threads": threads,
            "structured_bytes": raw, "raced_bytes": raced,
            "raced_over_structured": round(raced / raw, 4),
            "race_s": round(t_race, 3), "race_mb_per_s": round(raw / t_race / 1e6, 1),
            "decode_s": round(t_dec, 3), "decode_mb_per_s": round(raw / t_dec / 1e6, 1),
            "winners": winners}


def small_workspace(bd, pairs, comp, res, steps, slot_bytes=256):
    """The same batched compress with 256-byte record slots instead of 2 KiB
    (the workspace about 1.9 % of the weights instead of 12.9 %), records
    that do not fit staged in the payload arena's spare room; timed in turns
    with the full-workspace call, same capacities, payloads compared."""
    caps = comp.capacity
    small = bd.CompressBatch(pairs, caps, slot_bytes=slot_bytes)
    t_full, t_small = [], []
    for i in range(steps + 1):
        for b, ts in ((comp, t_full), (small, t_small)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            b.run()
            e1.record()
            torch.cuda.synchronize()
            if i:
                ts.append(e0.elapsed_time(e1) / 1e3)
    sres = small.results()
    same = all(a["status"] == b["status"] == bd.OK and a["payload_bytes"] == b["payload_bytes"]
               and torch.equal(comp.payload(j, a["payload_bytes"]),
                               small.payload(j, b["payload_bytes"]))
               for j, (a, b) in enumerate(zip(res, sres)))
    assert same, "small-workspace payloads differ from the full-workspace ones"
    w_bytes = 2 * sum(s.numel() for s, _ in pairs)
    tf, tsm = float(np.median(t_full)), float(np.median(t_small))
    out = {"slot_bytes": slot_bytes, "workspace_bytes": small.ws_bytes,
           "workspace_pct_of_weights": round(100 * small.ws_bytes / w_bytes, 3),
           "full_workspace_pct_of_weights": round(100 * comp.ws_bytes / w_bytes, 3),
           "ms": round(1e3 * tsm, 4), "full_workspace_ms": round(1e3 * tf, 4),
           "time_ratio": round(tsm / tf, 4), "payloads_identical": same}
    del small
    return out


def verify_first(bd, pairs, payloads, cs_new, cs_old, steps):
    """The verify-first decompress (bf16d_decompress_verified: a checking pass
    with no stores, then a pass that writes the verified jobs' changed
    chunks) timed in turns with the single in-place pass on a receiver of its
    own; both receivers end bit-exact."""
    recv_a = [s.clone() for s, _ in pairs]
    recv_b = [s.clone() for s, _ in pairs]
    fused = bd.DecompressBatch([(w, p, c) for w, p, c in zip(recv_a, payloads, cs_new)])
    vf = bd.DecompressBatch([(w, p, c) for w, p, c in zip(recv_b, payloads, cs_new)],
                            verify_first=True)
    tf, tv, tk, direction = [], [], [], 0
    for i in range(steps + 1):
        cs = cs_new if direction == 0 else cs_old
        for j in range(len(cs)):
            fused.jobs[j].checksum = cs[j]
            vf.jobs[j].checksum = cs[j]
        e = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        e[0].record()
        fused.run()
        e[1].record()
        e[2].record()
        vf.run(events=(e[3], e[4]))
        e[5].record()
        torch.cuda.synchronize()
        assert all(r["status"] == bd.OK for r in fused.results()), "in-place decompress failed"
        assert all(r["status"] == bd.OK for r in vf.results()), "verified decompress failed"
        direction ^= 1
        if i:
            tf.append(e[0].elapsed_time(e[1]) / 1e3)
            tv.append(e[2].elapsed_time(e[5]) / 1e3)
            tk.append(e[3].elapsed_time(e[4]) / 1e3)
    for wa, wb, (s, d) in zip(recv_a, recv_b, pairs):
        want = d if direction == 1 else s
        assert torch.equal(wa.view(torch.int16), want.view(torch.int16)), "in-place not exact"
        assert torch.equal(wb.view(torch.int16), want.view(torch.int16)), "verified not exact"
    t_f, t_v, t_k = (float(np.median(x)) for x in (tf, tv, tk))
    del recv_a, recv_b, fused, vf
    return {"ms": round(1e3 * t_v, 4), "check_pass_ms": round(1e3 * t_k, 4),
            "in_place_ms_same_rounds": round(1e3 * t_f, 4), "ratio_to_in_place": round(t_v / t_f, 4)}


def remapped(bd, names, shapes, pairs, payloads, cs_new, cs_old, steps):
    """The same batched decompress with every layer's gate and up projections
    paired in groups of 64 rows in one fused buffer (the physical layout of a
    fused MoE/MLP kernel), applied through block-aligned segments prepared
    once (bf16d_remap_prepare; each call then reads the block map)."""
    G = 64
    items, fused, checks = [], [], []
    by_name = {n: j for j, n in enumerate(names)}
    done = set()
    for j, name in enumerate(names):
        if j in done:
            continue
        if name.endswith("gate_proj") and name[:-9] + "up_proj" in by_name:
            k = by_name[name[:-9] + "up_proj"]
            gate, up = pairs[j][0], pairs[k][0]
            R, C = shapes[j]
            g2, u2 = gate.view(R, C), up.view(R, C)
            f = torch.empty((2 * R, C), dtype=gate.dtype, device=gate.device)
            for g in range(R // G):
                f[2 * G * g: 2 * G * g + G] = g2[G * g: G * (g + 1)]
                f[2 * G * g + G: 2 * G * (g + 1)] = u2[G * g: G * (g + 1)]
            flat = f.reshape(-1)
            for jj, which in ((j, 0), (k, 1)):
                segs = [(G * g * C, flat[(2 * G * g + which * G) * C:(2 * G * g + which * G + G) * C])
                        for g in range(R // G)]
                items.append(((R * C, segs), payloads[jj], cs_new[jj]))
                checks.append(jj)
            fused.append((f, j, k, R, C))
            done.update((j, k))
        else:
            w = pairs[j][0].clone()
            items.append((w, payloads[j], cs_new[j]))
            checks.append(j)
            done.add(j)
    batch = bd.RemappedBatch(items, prepared=True)
    # the plain decompress of the same payloads onto the logical layout, timed
    # in turns with the remapped one
    plain_recv = [s.clone() for s, _ in pairs]
    plain = bd.DecompressBatch([(w, p, c) for w, p, c in zip(plain_recv, payloads, cs_new)])
    ts, tp, direction = [], [], 0
    for i in range(steps + 1):
        for q, jj in enumerate(checks):
            batch.jobs[q].checksum = (cs_new if direction == 0 else cs_old)[jj]
        for j in range(len(cs_new)):
            plain.jobs[j].checksum = (cs_new if direction == 0 else cs_old)[j]
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record()
        batch.run()
        e[1].record()
        e[2].record()
        plain.run()
        e[3].record()
        torch.cuda.synchronize()
        assert all(r["status"] == bd.OK for r in batch.results()), "remapped decompress failed"
        assert all(r["status"] == bd.OK for r in plain.results()), "plain decompress failed"
        direction ^= 1
        if i:
            ts.append(e[0].elapsed_time(e[1]) / 1e3)
            tp.append(e[2].elapsed_time(e[3]) / 1e3)
    # after an even number of calls the weights are old again: check one pair
    f, j, k, R, C = fused[0]
    src = pairs[j][0] if direction == 0 else pairs[j][1]
    assert torch.equal(f[:G].reshape(-1).view(torch.int16), src[:G * C].view(torch.int16))
    n = sum(s.numel() for s, _ in pairs)
    t, t_plain = float(np.median(ts)), float(np.median(tp))
    n_fused = len(fused)
    del batch, fused, items, plain, plain_recv
    return {"gate_up_pairs_fused": n_fused, "rows_per_group": G, "ms": round(1e3 * t, 4),
            "gbps_weights": round(2 * n / t / 1e9, 2),
            "plain_ms_same_rounds": round(1e3 * t_plain, 4),
            "ratio_to_plain": round(t / t_plain, 4)}


def bound_overwrite(bd, pairs, steps):
    """Version-2 payloads of the same checkpoint pair in overwrite form (each
    change carries its new value; with the workspace bf16d_workspace_bytes
    sizes, the apply writes in place and keeps the replaced values in an undo
    area), bound from version 1 to 2, applied with the receiver's version
    words.  Reports the payload size and whole-call times beside the XOR
    path's."""
    n = sum(s.numel() for s, _ in pairs)
    binds = [(1, 2, True)] * len(pairs)
    caps = [bd._first_capacity(s.numel()) + bd.BOUND_EXTRA_BYTES for s, _ in pairs]
    comp = bd.CompressBatch(pairs, caps, binds)
    comp.run()
    res = comp.results()
    if any(r["status"] != bd.OK for r in res):
        comp = bd.CompressBatch(pairs, [r["payload_bytes"] for r in res], binds)
        comp.run()
        res = comp.results()
    assert all(r["status"] == bd.OK for r in res), "overwrite compress failed"
    P = sum(r["payload_bytes"] for r in res)
    recv = [s.clone() for s, _ in pairs]
    ver = torch.ones(len(pairs), dtype=torch.int64, device=pairs[0][0].device)
    items = [(w, comp.payload(j, r["payload_bytes"]), r["checksum"])
             for j, (w, r) in enumerate(zip(recv, res))]
    dec = bd.DecompressBatch(items, ver)
    t_c, t_d = [], []
    for i in range(steps + 1):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record()
        comp.run()
        e[1].record()
        for w, (s, _) in zip(recv, pairs):
            w.copy_(s)
        ver.fill_(1)
        e[2].record()
        dec.run()
        e[3].record()
        torch.cuda.synchronize()
        assert all(r["status"] == bd.OK for r in dec.results()), "overwrite decompress failed"
        assert ver.cpu().tolist() == [2] * len(pairs), "version words not committed"
        if i:
            t_c.append(e[0].elapsed_time(e[1]) / 1e3)
            t_d.append(e[2].elapsed_time(e[3]) / 1e3)
    for w, (_, d) in zip(recv, pairs):
        assert torch.equal(w.view(torch.int16), d.view(torch.int16)), "overwrite not bit-exact"
    tc, td = float(np.median(t_c)), float(np.median(t_d))
    del recv, dec, comp
    return {"payload_bytes": P, "payload_pct_of_orig": round(100 * P / (2 * n), 4),
            "compress_ms": round(1e3 * tc, 4), "compress_gbps_weights": round(2 * n / tc / 1e9, 2),
            "decompress_ms": round(1e3 * td, 4),
            "decompress_gbps_weights": round(2 * n / td / 1e9, 2)}


def dirty_chunks(pairs, n, dev):
    """One bit per 16-byte chunk of the first n elements of the workload's
    tensors laid end to end (bit c & 31 of int32 word c >> 5 for chunk c): set
    where old and new differ in any of the chunk's 8 elements."""
    nchunks = n // 8192 * 1024
    bits = torch.zeros(nchunks, dtype=torch.bool, device=dev)
    at = 0
    for src, dst in pairs:
        m = src.numel()
        if at >= nchunks * 8:
            break
        d = src.reshape(-1).view(torch.int16) != dst.reshape(-1).view(torch.int16)
        lead, tail = at % 8, -(at + m) % 8
        z = lambda k: torch.zeros(k, dtype=torch.bool, device=dev)
        c = torch.cat([z(lead), d, z(tail)]).view(-1, 8).any(1)
        c0 = at // 8
        k = min(c.numel(), nchunks - c0)
        bits[c0:c0 + k] |= c[:k]
        at += m
    w8 = torch.tensor([1, 2, 4, 8, 16, 32, 64, 128], dtype=torch.uint8, device=dev)
    packed = (bits.view(-1, 8).to(torch.uint8) * w8).sum(1, dtype=torch.uint8)
    chunk_pct = 100 * bits.float().mean().item()
    line_pct = 100 * bits.view(-1, 8).any(1).float().mean().item()
    return packed.view(torch.int32), chunk_pct, line_pct


def read_ceiling(a, b, steps, dirty=None):
    """The read ceiling of the encoder's access pattern (bf16d_probe_read: one
    workgroup per 8192-element block, 16-byte loads, nothing else) over the
    two flat arrays a and b, as the encoder reads old and new, and over a
    alone, as the apply pass reads old.  Their contents do not matter; the
    caller allocates them before anything is timed.  With the workload's changed-chunk
    bitmap, also the apply pass's writes alone (bf16d_probe_write into b: the
    changed 16-byte chunks, no reads)."""
    from lossless_bf16_weight_xor_amd import probe
    sink = torch.empty(1, dtype=torch.int64, device=a.device)
    full = a.numel() // 8192 * 8192
    out = {}
    for key, arrays in (("read2", (a, b)), ("read1", (a, None))):
        probe.probe_read(*arrays, sink=sink)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(steps):
            probe.probe_read(*arrays, sink=sink)
        ev[1].record()
        torch.cuda.synchronize()
        t = ev[0].elapsed_time(ev[1]) / 1e3 / steps
        nbytes = (2 if arrays[1] is not None else 1) * 2 * full
        out[key] = {"bytes": nbytes, "ms": round(1e3 * t, 4), "gbps": round(nbytes / t / 1e9, 2),
                    "pct_of_peak": round(100 * nbytes / t / 1e9 / HBM_PEAK_GBPS, 2)}
    if dirty is not None:
        probe.probe_write(b, dirty)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(steps):
            probe.probe_write(b, dirty)
        ev[1].record()
        torch.cuda.synchronize()
        out["write_changed_chunks_only"] = {
            "ms": round(ev[0].elapsed_time(ev[1]) / steps, 4),
            "note": "the apply pass's writes alone (no reads); with read1 it splits the "
                    "in-place floor into its two parts"}
    return out


def flat_receiver(tensors, dev):
    """Copies of `tensors` laid end to end in one buffer, as views (None and
    plain clones if some tensor's size is not a multiple of 8 elements, which
    would leave a view off a 16-byte boundary)."""
    if any(t.numel() % 8 for t in tensors):
        return None, [t.clone() for t in tensors]
    buf = torch.empty(sum(t.numel() for t in tensors), dtype=torch.int16, device=dev)
    views, at = [], 0
    for t in tensors:
        v = buf[at:at + t.numel()]
        v.copy_(t.reshape(-1).view(torch.int16))
        views.append(v.view(t.dtype))
        at += t.numel()
    return buf, views


def apply_against_floor(decompress_once, check, rbuf, dirty, rounds):
    """apply_kernel and the in-place floor probe, timed in the same rounds
    over the same memory.  Each round is one verified decompress of the
    workload (its apply kernel between HIP events), then bf16d_probe_inplace
    over the receiver's buffer: every whole block read, and every 16-byte
    chunk that the delta changes written back unchanged, with nothing
    decoded."""
    from lossless_bf16_weight_xor_amd import probe
    n = dirty.numel() // 32 * 8192
    sink = torch.empty(1, dtype=torch.int64, device=rbuf.device)
    ta, tp = [], []
    for i in range(rounds + 1):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        decompress_once((e[0], e[1]))
        torch.cuda.synchronize()
        check()
        e[2].record()
        probe.probe_inplace(rbuf[:n], dirty, sink=sink)
        e[3].record()
        torch.cuda.synchronize()
        if i >= 1:
            ta.append(e[0].elapsed_time(e[1]))
            tp.append(e[2].elapsed_time(e[3]))
    return {"ms": round(float(np.median(tp)), 4), "elements": n, "rounds": rounds,
            "apply_kernel_same_rounds_ms": round(float(np.median(ta)), 4)}


def dirty_write_units(pairs):
    """(32-byte sectors, 128-byte lines) that hold at least one changed
    element, counted per tensor from its start (tensors start on 256-byte
    boundaries, so these are the device's sectors and lines)."""
    sectors = lines = 0
    for src, dst in pairs:
        d = src.reshape(-1).view(torch.int16) != dst.reshape(-1).view(torch.int16)
        m = d.numel()
        pad = (-m) % 64
        if pad:
            d = torch.cat([d, torch.zeros(pad, dtype=torch.bool, device=d.device)])
        sectors += int(d.view(-1, 16).any(1).sum().item())
        lines += int(d.view(-1, 64).any(1).sum().item())
    return sectors, lines


def change_rate_sweep(bd, dev, steps, with_floor=True):
    """Compress and verified in-place decompress of one 1 GiB tensor
    (536,870,912 elements, uniform changes, 95/4.5/0.5) at each change rate
    of the sweep: whole calls and their main kernels, with events on the
    call's stream.  Each rate's payload is the same bytes over all the calls
    (checked), and the receiver ends bit-exact.

    A kernel that writes leaves dirty lines in the caches, and their
    write-back lands in whatever runs next; on a 1 GiB call that is a
    sizeable share.  With `with_floor` (the probe library), every timed
    kernel starts after an untimed read of 1 GiB of other memory, so each is
    charged its own traffic only, and every round also times the in-place
    floor probe over the receiver (its reads plus the changed chunks written
    back unchanged) and the read ceiling over old and new
    (bf16d_probe_read).  Every round also times a compress right after the
    decompress, as the main step runs them."""
    from lossless_bf16_weight_xor_amd import synth
    if with_floor:
        from lossless_bf16_weight_xor_amd import probe
    out = []
    for rate in synth.C3_RATES:
        src, dst = synth.config3(dev, rate)
        n = src.numel()
        comp = bd.CompressBatch([(src, dst)], [bd._first_capacity(n)])
        comp.run()
        r = comp.results()[0]
        assert r["status"] == bd.OK, f"sweep {rate}: compress {r['status']}"
        P, c = r["payload_bytes"], r["n_changed"]
        payload = comp.payload(0, P)
        ref = payload.clone()
        rev = bd.CompressBatch([(dst, src)], [P])
        rev.run()
        cs_old, cs_new = rev.results()[0]["checksum"], r["checksum"]
        del rev
        recv = src.clone()
        dec = bd.DecompressBatch([(recv, payload, cs_new)])
        sink = torch.empty(1, dtype=torch.int64, device=dev)
        dirty = flush_buf = None
        if with_floor:
            dirty = dirty_chunks([(src, dst)], n, dev)[0]
            flush_buf = torch.empty(1 << 29, dtype=torch.int16, device=dev)

        def flush():
            if flush_buf is not None:
                probe.probe_read(flush_buf, None, sink=sink)

        t = {k: [] for k in ("call_c", "enc", "call_d", "app", "call_c2", "enc2", "floor",
                             "read2")}
        direction = 0
        for i in range(steps + 2):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(16)]
            flush()
            e[0].record()
            comp.run(events=(e[1], e[2]))
            e[3].record()
            flush()
            dec.jobs[0].checksum = cs_new if direction == 0 else cs_old
            e[4].record()
            dec.run(events=(e[5], e[6]))
            e[7].record()
            # the main step's order: a compress right after a decompress
            e[8].record()
            comp.run(events=(e[9], e[10]))
            e[11].record()
            torch.cuda.synchronize()
            assert dec.results()[0]["status"] == bd.OK, f"sweep {rate}: decompress"
            direction ^= 1
            if with_floor:
                flush()
                e[12].record()
                probe.probe_inplace(recv, dirty, sink=sink)
                e[13].record()
                flush()
                e[14].record()
                probe.probe_read(src, dst, sink=sink)
                e[15].record()
                torch.cuda.synchronize()
            if i >= 2:
                for k, (x, y) in (("call_c", (0, 3)), ("enc", (1, 2)), ("call_d", (4, 7)),
                                  ("app", (5, 6)), ("call_c2", (8, 11)), ("enc2", (9, 10))):
                    t[k].append(e[x].elapsed_time(e[y]) / 1e3)
                if with_floor:
                    t["floor"].append(e[12].elapsed_time(e[13]) / 1e3)
                    t["read2"].append(e[14].elapsed_time(e[15]) / 1e3)
        assert torch.equal(payload, ref), f"sweep {rate}: payload changed between calls"
        want = dst if direction == 1 else src
        assert torch.equal(recv.view(torch.int16), want.view(torch.int16)), f"sweep {rate}"
        sectors, lines = dirty_write_units([(src, dst)])
        ca, da = 4 * n + P, 2 * n + P + 2 * c
        m = {k: float(np.median(v)) for k, v in t.items() if v}
        out.append({
            "rate": rate, "elements": n, "payload_pct_of_orig": round(100 * P / (2 * n), 4),
            # the per-block position encoding chosen: bitmaps, the rest gap lists
            "blocks": (n + 8191) // 8192, "bitmap_blocks": r["n_bitmap_blocks"],
            "caches_flushed_before_each_kernel": with_floor,
            "compress_ms": round(1e3 * m["call_c"], 4),
            "compress_hbm_pct": round(100 * ca / m["call_c"] / 1e9 / HBM_PEAK_GBPS, 2),
            "encode_kernel_ms": round(1e3 * m["enc"], 4),
            "encode_kernel_frac": round(ca / m["enc"] / 1e9 / HBM_PEAK_GBPS, 4),
            "compress_after_decompress_ms": round(1e3 * m["call_c2"], 4),
            "compress_after_decompress_hbm_pct": round(
                100 * ca / m["call_c2"] / 1e9 / HBM_PEAK_GBPS, 2),
            "encode_kernel_after_decompress_ms": round(1e3 * m["enc2"], 4),
            "decompress_ms": round(1e3 * m["call_d"], 4),
            "decompress_hbm_pct": round(100 * da / m["call_d"] / 1e9 / HBM_PEAK_GBPS, 2),
            "apply_kernel_ms": round(1e3 * m["app"], 4),
            "apply_kernel_frac": round(da / m["app"] / 1e9 / HBM_PEAK_GBPS, 4),
            "dirty_sectors_pct": round(100 * sectors / (n / 16), 3),
            "dirty_lines_pct": round(100 * lines / (n / 64), 3)})
        if with_floor:
            out[-1]["inplace_floor_ms"] = round(1e3 * m["floor"], 4)
            out[-1]["apply_kernel_frac_of_inplace_floor"] = round(m["floor"] / m["app"], 4)
            out[-1]["read2_ms"] = round(1e3 * m["read2"], 4)
            out[-1]["encode_kernel_frac_of_read2"] = round(m["read2"] / m["enc"], 4)
        log(f"sweep {rate}: compress {out[-1]['compress_ms']} ms "
            f"({out[-1]['compress_hbm_pct']}%; {out[-1]['compress_after_decompress_ms']} ms "
            f"right after a decompress), decompress {out[-1]['decompress_ms']} ms "
            f"({out[-1]['decompress_hbm_pct']}%)"
            + (f"; encode_kernel {out[-1]['encode_kernel_frac_of_read2']} of the read ceiling, "
               f"apply_kernel {out[-1]['apply_kernel_frac_of_inplace_floor']} of the in-place "
               f"floor" if with_floor else ""))
        del comp, dec, recv, payload, ref, src, dst, dirty, flush_buf
        torch.cuda.empty_cache()
    return out


def cpu_baseline(pairs, gpu_payloads, budget_s: float):
    """The CPU oracle, single-threaded, timed on a bounded sample of the
    workload's tensors, walking from the last tensor back.  Each oracle
    payload is also compared byte for byte with the GPU's.  Beside it
    (`parallel`), the same oracle on up to 16 host threads over the sample's
    first ~2 GB."""
    import oracle
    from lossless_bf16_weight_xor_amd import synth
    t_c = t_d = 0.0
    n_done = 0
    names = []
    mismatches = 0
    # one core, as the oracle's single thread would use anyway; restored after
    saved = os.sched_getaffinity(0)
    core = min(saved)
    os.sched_setaffinity(0, {core})
    try:
        for j in range(len(pairs) - 1, -1, -1):
            src, dst = pairs[j]
            a = synth.bits(src).cpu().numpy().astype(np.uint16)
            b = synth.bits(dst).cpu().numpy().astype(np.uint16)
            t0 = time.perf_counter()
            payload, cs, _ = oracle.compress(a, b)
            t1 = time.perf_counter()
            w = a.copy()
            st = oracle.decompress_inplace(w, payload, cs)
            t2 = time.perf_counter()
            assert st == oracle.OK and np.array_equal(w, b)
            got = gpu_payloads[j]
            if got is not None and not (got.size == payload.size and np.array_equal(got, payload)):
                mismatches += 1
            t_c += t1 - t0
            t_d += t2 - t1
            n_done += a.size
            names.append(j)
            if t_c + t_d > budget_s:
                break
    finally:
        os.sched_setaffinity(0, saved)
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    # the same oracle over the host's cores (at most 16, the share of one GPU):
    # a thread per tensor, the oracle's C calls running without the
    # interpreter lock, on the sample's first ~2 GB of weights
    threads = max(1, min(16, len(saved)))
    arrays, nbytes = [], 0
    for j in names:
        if nbytes >= 2e9:
            break
        src, dst = pairs[j]
        arrays.append((synth.bits(src).cpu().numpy().astype(np.uint16),
                       synth.bits(dst).cpu().numpy().astype(np.uint16)))
        nbytes += 2 * src.numel()

    def one(ab):
        a, b = ab
        payload, cs, _ = oracle.compress(a, b)
        w = a.copy()
        assert oracle.decompress_inplace(w, payload, cs) == oracle.OK and np.array_equal(w, b)

    from concurrent.futures import ThreadPoolExecutor
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as pool:
        list(pool.map(one, arrays))
    t_par = time.perf_counter() - t0
    parallel = {"value": round(nbytes / t_par / 1e9, 4), "unit": "GB/s", "threads": threads,
                "sample": f"{len(arrays)} tensors ({nbytes / 1e9:.3f} GB of BF16 weights), "
                          "compress + decompress, one tensor per thread"}
    del arrays
    return {
        "value": round(2 * n_done / (t_c + t_d) / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{len(names)} of {len(pairs)} tensors ({2 * n_done / 1e9:.3f} GB of BF16 "
                  f"weights), compress + decompress, single-threaded C oracle pinned to one core",
        "compress_gbps": round(2 * n_done / t_c / 1e9, 4),
        "decompress_gbps": round(2 * n_done / t_d / 1e9, 4),
        "payload_mismatches_vs_gpu": mismatches,
        "cpu_model": cpu_model,
        "cores_available": len(saved),
        "parallel": parallel,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="7b",
                    choices=["7b", "70b-half"] + ["c3-" + r for r in ("0.00085", "0.01", "0.03",
                                                                      "0.05")],
                    help="7b (the default), the 70B half-model share, or one 1 GiB tensor at a "
                         "change rate (c3-<rate>)")
    ap.add_argument("--limit", type=int, default=None, help="first N tensors only (debug)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of CPU oracle work for the baseline (0 disables)")
    ap.add_argument("--no-streamed", action="store_true",
                    help="skip the streamed receiver (payloads in pinned host memory)")
    ap.add_argument("--no-remapped", action="store_true",
                    help="skip the remapped apply (gate/up paired in groups of 64 rows)")
    ap.add_argument("--no-bound", action="store_true",
                    help="skip the version-2 overwrite payloads")
    ap.add_argument("--no-race", action="store_true",
                    help="skip the host codec race over the payloads")
    ap.add_argument("--race-threads", type=int, default=16,
                    help="CPU threads of the codec race (capped at the host's cores)")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the read-ceiling probe (bf16d_probe_read)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the change-rate sweep (one 1 GiB tensor at 0.085/1/3/5 %%)")
    ap.add_argument("--with-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--main-only", action="store_true",
                    help="the main step and its probes only (profiling): none of the other "
                         "measurements, so every compress and decompress kernel launched is "
                         "one of the main workload's")
    args = ap.parse_args()
    if args.main_only:
        args.no_streamed = args.no_remapped = args.no_bound = args.no_race = True
        args.no_sweep = True
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the delta path is "
                          "per-GPU (each rank would compress and apply the tensors it holds)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    ensure_built()
    import lossless_bf16_weight_xor_amd as bd

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    names, pairs, desc = generate(args.workload, dev, args.limit)
    torch.cuda.synchronize()
    n_total = sum(s.numel() for s, _ in pairs)
    log(f"generated {len(pairs)} tensors, {n_total} elements in {time.time() - t0:.1f}s")
    # the read probes' two flat arrays, held from here to the end, so that the
    # ceilings do not follow the other measurements' allocations and frees
    probe_arrays = None
    if not args.no_probe:
        n_probe = min(n_total, 8_000_000_000)
        probe_arrays = (torch.empty(n_probe, dtype=torch.int16, device=dev),
                        torch.empty(n_probe, dtype=torch.int16, device=dev))

    # payload capacity: framing + 1/16 of the weights, exact size on overflow
    caps = [bd._first_capacity(s.numel()) for s, _ in pairs]
    comp = bd.CompressBatch(pairs, caps)
    comp.run()
    res = comp.results()
    if any(r["status"] != bd.OK for r in res):
        caps = [r["payload_bytes"] for r in res]
        comp = bd.CompressBatch(pairs, caps)
        comp.run()
        res = comp.results()
    assert all(r["status"] == bd.OK for r in res), "compress failed"
    cs_new = [r["checksum"] for r in res]
    payload_total = sum(r["payload_bytes"] for r in res)
    n_changed = sum(r["n_changed"] for r in res)
    n_rare = sum(r["n_rare"] for r in res)
    n_bitmap = sum(r["n_bitmap_blocks"] for r in res)
    payloads = [comp.payload(j, r["payload_bytes"]) for j, r in enumerate(res)]

    # checksums of old: compress the reverse direction (same payload bytes)
    rev = bd.CompressBatch([(d, s) for s, d in pairs], caps)
    rev.run()
    rres = rev.results()
    cs_old = [r["checksum"] for r in rres]
    same = all(torch.equal(rev.payload(j, r["payload_bytes"]), payloads[j])
               for j, r in enumerate(rres))
    assert same, "reverse payload differs"
    del rev

    # the receiver: the old tensors laid end to end in one buffer, so the
    # in-place floor probe can later run over the memory the apply pass writes
    rbuf, receiver = flat_receiver([s for s, _ in pairs], dev)
    dec = bd.DecompressBatch([(w, p, c) for w, p, c in zip(receiver, payloads, cs_new)])
    torch.cuda.synchronize()
    log(f"payload {payload_total} B ({100 * payload_total / (2 * n_total):.3f}% of orig), "
        f"changed {n_changed}, rare {n_rare}, bitmap blocks {n_bitmap}")

    direction = [0]   # 0: receiver holds old, 1: it holds new

    def set_checksums():
        cs = cs_new if direction[0] == 0 else cs_old
        for j in range(len(cs)):
            dec.jobs[j].checksum = cs[j]

    def step(ev=None):
        set_checksums()
        if ev: ev[0].record()
        comp.run(events=(ev[1], ev[2]) if ev else None)
        if ev: ev[3].record()
        dec.run(events=(ev[4], ev[5]) if ev else None)
        if ev: ev[6].record()
        direction[0] ^= 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.warmup:
        assert all(r["status"] == bd.OK for r in dec.results()), "warm-up decompress failed"

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    for e in evs:                      # create the HIP events outside the timed region
        for x in e:
            x.record()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    dres = dec.results()
    assert all(r["status"] == bd.OK for r in dres), "decompress failed in the timed region"
    assert all(r["status"] == bd.OK for r in comp.results()), "compress failed in the timed region"
    def check_receiver():
        expect_new = direction[0] == 1
        for w, (s, d) in zip(receiver, pairs):
            ref = d if expect_new else s
            assert torch.equal(w.view(torch.int16), ref.view(torch.int16)), "receiver not bit-exact"

    check_receiver()

    def durations(a, b):
        return [evs[i][a].elapsed_time(evs[i][b]) / 1e3 for i in range(args.steps)]

    def avg(a, b):
        return float(np.mean(durations(a, b)))

    tc, td = avg(0, 3), avg(3, 6)            # whole calls
    t_enc, t_app = avg(1, 2), avg(4, 5)      # their main kernels
    ms_per_step = 1e3 * elapsed / args.steps
    w_bytes = 2 * n_total
    comp_alg = 4 * n_total + payload_total
    dec_alg = 2 * n_total + payload_total + 2 * n_changed
    value = w_bytes / (elapsed / args.steps) / 1e9

    # the decompress's write traffic at the device's granularity: every
    # 32-byte sector (and 128-byte line) holding a change is written
    dirty_sectors, dirty_lines = dirty_write_units(pairs)
    dec_eff = 2 * n_total + payload_total + 32 * dirty_sectors

    # the changed 16-byte chunks (for the probes), then the apply kernel and
    # the in-place floor in the same rounds over the receiver's memory
    dirty = floor = None
    if not args.no_probe:
        dirty, chunk_pct, line_pct = dirty_chunks(pairs, n_total // 8192 * 8192, dev)
        if rbuf is not None:
            def decompress_once(events):
                set_checksums()
                dec.run(events=events)
                direction[0] ^= 1

            def check_statuses():
                assert all(r["status"] == bd.OK for r in dec.results()), "decompress failed"

            floor = apply_against_floor(decompress_once, check_statuses, rbuf, dirty, 6)
            floor["dirty_chunks_pct"] = round(chunk_pct, 3)
            floor["dirty_lines_pct"] = round(line_pct, 3)
            check_receiver()
            log(f"in-place floor over the receiver: {floor['ms']} ms, apply kernel in the same "
                f"rounds {floor['apply_kernel_same_rounds_ms']} ms "
                f"({floor['dirty_lines_pct']}% of 128-byte lines written)")

    ceiling = None
    if probe_arrays is not None:
        ceiling = read_ceiling(*probe_arrays, max(3, args.steps // 2),
                               dirty if n_total <= 8_000_000_000 else None)
        del dirty
        ceiling["encode_kernel_frac_of_read2"] = round(comp_alg / t_enc / 1e9 /
                                                       ceiling["read2"]["gbps"], 4)
        ceiling["apply_kernel_frac_of_read1"] = round(dec_alg / t_app / 1e9 /
                                                      ceiling["read1"]["gbps"], 4)
        log(f"read ceiling: {ceiling['read2']['gbps']} GB/s over two arrays, "
            f"{ceiling['read1']['gbps']} GB/s over one")
        # (the probe covers whole 8192-element blocks of the receiver's buffer:
        # all but the last few thousand elements of the workload)
        if floor is not None and floor["elements"] >= 0.999 * n_total:
            ceiling["inplace_floor"] = floor
            ceiling["apply_kernel_frac_of_inplace_floor"] = round(
                floor["ms"] / floor["apply_kernel_same_rounds_ms"], 4)

    if args.with_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    small_ws = None
    if not args.main_only:
        small_ws = small_workspace(bd, pairs, comp, res, 5)
        log(f"compress with 256-byte slots: workspace {small_ws['workspace_pct_of_weights']}% "
            f"of the weights, {small_ws['ms']} ms ({small_ws['time_ratio']}x the full workspace)")

    vf_info = None
    # (two more receivers would not fit beside the 70B share)
    if args.workload != "70b-half" and not args.main_only:
        vf_info = verify_first(bd, pairs, payloads, cs_new, cs_old, 4)
        vf_info["hbm_pct"] = round(100 * dec_alg / (vf_info["ms"] / 1e3) / 1e9 / HBM_PEAK_GBPS, 2)
        log(f"verify-first decompress: {vf_info['ms']} ms ({vf_info['ratio_to_in_place']}x the "
            f"in-place pass)")

    remap_info = None
    if not args.no_remapped and args.workload in ("7b", "70b-half"):
        from lossless_bf16_weight_xor_amd import synth
        specs = synth.seven_b_specs() if args.workload == "7b" else synth.config5_specs()
        remap_info = remapped(bd, names, [sp.shape for sp in specs], pairs, payloads, cs_new,
                              cs_old, 4)
        # the same payloads and changes: the algorithmic bytes of the plain decompress
        remap_info["hbm_pct"] = round(100 * dec_alg / (remap_info["ms"] / 1e3) / 1e9 /
                                      HBM_PEAK_GBPS, 2)

    bound_info = None
    if not args.no_bound:
        bound_info = bound_overwrite(bd, pairs, 3)
        # algorithmic bytes with the overwrite payload: 4n + P to compress,
        # 2n + P + 2c to decompress (the same changes)
        P_ow = bound_info["payload_bytes"]
        bound_info["compress_hbm_pct"] = round(
            100 * (4 * n_total + P_ow) / (bound_info["compress_ms"] / 1e3) / 1e9 / HBM_PEAK_GBPS, 2)
        bound_info["decompress_hbm_pct"] = round(
            100 * (2 * n_total + P_ow + 2 * n_changed) / (bound_info["decompress_ms"] / 1e3) / 1e9
            / HBM_PEAK_GBPS, 2)

    race_info = None
    if not args.no_race:
        race_info = codec_race(bd, payloads, max(1, min(args.race_threads, os.cpu_count() or 1)))
        race_info["payload_pct_after_race"] = round(100 * race_info["raced_bytes"] / w_bytes, 4)
        log(f"codec race: {race_info['raced_bytes']} B "
            f"({race_info['payload_pct_after_race']}% of orig) in {race_info['race_s']} s")

    stream_info = None
    if not args.no_streamed:
        # Right after a large free (in this process or a recent one: the GPU test
        # suite's 140 GB test, for one) the streamed copies stop overlapping the
        # applies for some seconds to a minute, outside the library; measured
        # here after the other measurements, for that reason.  A line above 1.35x
        # the plain copy of its payloads (fresh: 1.13-1.19x; in that state:
        # 1.6-2.7x) is measured again after 15 s, at most twice; every attempt
        # is reported.
        stream_info = []
        for lpg, slots, copies, lanes in ((1, 5, 2, 2), (1, 3, 2, 1), (1, 2, 1, 1)):
            tries = []
            for attempt in range(3):
                r = streamed(bd, names, pairs, payloads, cs_new, cs_old, 5, td, lpg, slots, copies,
                             lanes)
                tries.append(r["ms"])
                if r["ms"] <= 1.35 * r["h2d_payload_ms"] or attempt == 2:
                    break
                log(f"streamed {lpg} layer(s)/group: {r['ms']} ms, over 1.35x the plain copy; "
                    "measuring again in 15 s")
                time.sleep(15)
            r["attempts_ms"] = tries
            stream_info.append(r)

    # after the streamed receiver: the sweep frees its buffers, and a large
    # free slows the streamed receiver's copies for some seconds
    sweep = None
    if not args.no_sweep and args.workload == "7b":
        sweep = change_rate_sweep(bd, dev, 5, with_floor=not args.no_probe)

    # the probe arrays go last: a large free slows the streamed copies for a while
    del probe_arrays
    torch.cuda.empty_cache()

    gpu_payloads = [None] * len(pairs)
    cpu = None
    if args.cpu_budget > 0:
        for j in range(len(pairs) - 1, max(-1, len(pairs) - 40), -1):
            gpu_payloads[j] = payloads[j].cpu().numpy()
        cpu = cpu_baseline(pairs, gpu_payloads, args.cpu_budget)

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16",
        "data": "synthetic",
        "config": {"workload": desc, "tensors": len(pairs), "elements": n_total,
                   "weights_bytes": w_bytes, "parallelism": "single GPU"},
        "compress": {"gbps_weights": round(w_bytes / tc / 1e9, 2),
                     # device memory beside the inputs: the call's workspace
                     # and the payload arena (first-guess capacities)
                     "workspace_bytes": comp.ws_bytes,
                     "workspace_pct_of_weights": round(100 * comp.ws_bytes / w_bytes, 3),
                     "arena_bytes": comp.arena.numel(),
                     "arena_pct_of_weights": round(100 * comp.arena.numel() / w_bytes, 3),
                     "hbm_pct": round(100 * comp_alg / tc / 1e9 / HBM_PEAK_GBPS, 2),
                     "ms": round(1e3 * tc, 4),
                     "ms_median": round(1e3 * float(np.median(durations(0, 3))), 4),
                     "ms_min": round(1e3 * min(durations(0, 3)), 4),
                     "encode_kernel_ms": round(1e3 * t_enc, 4),
                     "algorithmic_bytes": comp_alg},
        "decompress": {"gbps_weights": round(w_bytes / td / 1e9, 2),
                       "workspace_bytes": dec.ws_bytes,
                       "hbm_pct": round(100 * dec_alg / td / 1e9 / HBM_PEAK_GBPS, 2),
                       "ms": round(1e3 * td, 4),
                       "ms_median": round(1e3 * float(np.median(durations(3, 6))), 4),
                       "ms_min": round(1e3 * min(durations(3, 6)), 4),
                       "apply_kernel_ms": round(1e3 * t_app, 4),
                       "algorithmic_bytes": dec_alg},
        "payload_pct_of_orig": round(100 * payload_total / w_bytes, 4),
        "payload_bytes": payload_total,
        "n_changed": n_changed, "n_rare": n_rare, "bitmap_blocks": n_bitmap,
        "roofline": {"bound": "hbm", "kernel": "encode_kernel",
                     "achieved": round(comp_alg / t_enc / 1e9, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(comp_alg / t_enc / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(n_total)},
        "roofline_decompress": {"bound": "hbm", "kernel": "apply_kernel",
                                "achieved": round(dec_alg / t_app / 1e9, 2),
                                "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                "frac": round(dec_alg / t_app / 1e9 / HBM_PEAK_GBPS, 4),
                                "traffic": measured_traffic(n_total, APPLY_TRAFFIC_PROFILE,
                                                            APPLY_SOURCES),
                                # 2n + P + every 32-byte sector holding a change:
                                # the writes at the granularity the device moves
                                "effective_bytes": dec_eff,
                                "effective_achieved": round(dec_eff / t_app / 1e9, 2),
                                "effective_frac": round(dec_eff / t_app / 1e9 / HBM_PEAK_GBPS, 4),
                                "dirty_sectors_pct": round(100 * dirty_sectors * 16 / n_total, 3),
                                "dirty_lines_pct": round(100 * dirty_lines * 64 / n_total, 3),
                                "target_pct": 60.0,
                                "target_met": bool(100 * dec_alg / td / 1e9 / HBM_PEAK_GBPS
                                                   >= 60.0),
                                # the kernel against the in-place floor probe (the same
                                # reads and changed-chunk writes, nothing else), timed in
                                # the same rounds over the same buffer
                                "inplace_floor_ms": floor["ms"] if floor else None,
                                "frac_of_inplace_floor": (
                                    round(floor["ms"] / floor["apply_kernel_same_rounds_ms"], 4)
                                    if floor else None)},
        "change_rate_sweep": sweep,
        "compress_small_workspace": small_ws,
        "decompress_verify_first": vf_info,
        "achievable": ceiling,
        "streamed_receiver": stream_info,
        "remapped_decompress": remap_info,
        "bound_overwrite": bound_info,
        "codec_race": race_info,
        "cpu_baseline": cpu,
        "env": {"torch": torch.__version__, "hip": torch.version.hip,
                "device": torch.cuda.get_device_name(dev),
                "checksums_sha256": hashlib.sha256(
                    np.array(cs_new, dtype=np.uint64).tobytes()).hexdigest()},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
