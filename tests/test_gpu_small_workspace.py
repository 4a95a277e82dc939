"""Compress with small record slots (bf16d_compress_workspace_bytes) against
the oracle (MI355X).

With slots smaller than a block's record, the record is staged at the tail
of the job's payload buffer and copied down once the offsets are known, or,
when the final payload reaches into the staged range, encoded a second time
from the weights.  The payload bytes must not depend on which of the three
ways a record took: every case is compared with the oracle byte for byte,
with room for every staged record, for some, and for none.
"""
import numpy as np
import pytest
import torch

import oracle
import lossless_bf16_weight_xor_amd as bd
from lossless_bf16_weight_xor_amd import synth
from tests.gpu_util import assert_same_bytes, log, oracle_of, pair, payload_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

SPECS = [((3 * 8192 + 77,), "0.02"), ((8192,), "0.2"), ((5 * 8192 + 3,), "0.6"),
         ((2 * 8192,), "1.0"), ((70001,), "0.001"), ((1,), "1.0"), ((0,), "0"),
         ((513, 129), "0.13"), ((64, 8192), "0.05"), ((4096, 64), "0.3")]


def _pairs(seed0):
    out = []
    for i, (shape, rate) in enumerate(SPECS):
        if shape == (0,):
            s = torch.empty(0, dtype=torch.bfloat16, device=DEV)
            out.append((s, s.clone()))
        else:
            s, d = pair(shape, rate, synth.MIX_ADVERSARIAL, seed0 + i, DEV)
            out.append((s.reshape(-1), d.reshape(-1)))
    return out


def _run(pairs, caps, slot, bindings=None):
    b = bd.CompressBatch(pairs, caps, bindings, slot_bytes=slot)
    b.arena.fill_(0xA5)
    b.run()
    return b, b.results()


@pytest.mark.parametrize("slot", [16, 64, 256, 1024])
@pytest.mark.parametrize("room", ["plenty", "exact", "some"])
def test_small_slots_give_the_oracle_payloads(slot, room):
    """plenty: worst-case capacities, every staged record is copied down;
    exact: capacity = payload size, no staged record survives (all encoded
    again); some: capacity = payload + 1/4 of it, some survive."""
    log(f"case small slots slot={slot} room={room}")
    pairs = _pairs(4000)
    refs = [oracle_of(s, d) for s, d in pairs]
    P = [len(r[0]) for r in refs]
    if room == "plenty":
        caps = [bd.max_payload_bytes(s.numel()) for s, _ in pairs]
    elif room == "exact":
        caps = P
    else:
        caps = [p + p // 4 for p in P]
    b, res = _run(pairs, caps, slot)
    for j, ((s, d), r, (ref, cs, _)) in enumerate(zip(pairs, res, refs)):
        assert r["status"] == bd.OK, (j, r["status"])
        assert r["checksum"] == cs and r["payload_bytes"] == P[j], j
        assert_same_bytes(payload_np(b.payload(j, P[j])), ref, f"slot {slot} {room} job {j}")
        # nothing is written past the capacity
        tail = b.arena[b.offset[j] + caps[j]: b.offset[j] + (caps[j] + 255) // 256 * 256]
        assert bool((tail == 0xA5).all()), f"job {j}: wrote past the capacity"


def test_small_slots_report_the_exact_size_when_the_capacity_is_short():
    log("case small slots, capacity too small")
    pairs = _pairs(4100)
    refs = [oracle_of(s, d) for s, d in pairs]
    P = [len(r[0]) for r in refs]
    caps = [max(0, p // 2) for p in P]
    b, res = _run(pairs, caps, 64)
    for j, r in enumerate(res):
        assert r["status"] == (bd.ECAPACITY if caps[j] < P[j] else bd.OK), j
        assert r["payload_bytes"] == P[j], j
        tail = b.arena[b.offset[j] + caps[j]: b.offset[j] + (caps[j] + 255) // 256 * 256]
        assert bool((tail == 0xA5).all()), f"job {j}: wrote past the capacity"


@pytest.mark.parametrize("overwrite", [False, True])
def test_small_slots_with_bound_payloads(overwrite):
    log(f"case small slots, version-2 payloads overwrite={overwrite}")
    pairs = [p for p in _pairs(4200) if p[0].numel() > 0]
    binds = [(10 + j, 11 + j, overwrite) for j in range(len(pairs))]
    caps = [bd.max_payload_bytes(s.numel()) + bd.BOUND_EXTRA_BYTES for s, _ in pairs]
    b, res = _run(pairs, caps, 32, binds)
    for j, ((s, d), r) in enumerate(zip(pairs, res)):
        from tests.gpu_util import to_u16
        want, cs, _ = oracle.compress_v2(to_u16(s), to_u16(d), 10 + j, 11 + j, overwrite)
        assert r["status"] == bd.OK and r["checksum"] == cs, j
        assert_same_bytes(payload_np(b.payload(j, r["payload_bytes"])), want, f"job {j}")


def test_small_slots_on_the_7b_shaped_checkpoint():
    """All 291 tensors with 256-byte slots (the workspace about 1.9 % of the
    weights) and the first-guess capacities: payloads identical to those of
    the full workspace, and the full workspace's to the oracle's on a sample
    (every tensor is compared in the full-size test)."""
    log("case 7B-shaped checkpoint with 256-byte slots")
    pairs = [(s.reshape(-1), d.reshape(-1)) for _, s, d in synth.config2(DEV)]
    caps = [bd._first_capacity(s.numel()) for s, _ in pairs]
    full = bd.CompressBatch(pairs, caps)
    full.run()
    fres = full.results()
    small = bd.CompressBatch(pairs, caps, slot_bytes=256)
    small.run()
    sres = small.results()
    n = sum(s.numel() for s, _ in pairs)
    assert small.ws_bytes <= 0.02 * 2 * n, small.ws_bytes / (2 * n)
    for j, (a, b) in enumerate(zip(fres, sres)):
        assert a["status"] == b["status"] == bd.OK, j
        assert a["checksum"] == b["checksum"] and a["payload_bytes"] == b["payload_bytes"], j
        assert torch.equal(full.payload(j, a["payload_bytes"]),
                           small.payload(j, b["payload_bytes"])), j
    for j in (0, 1, 5, 100, 290):
        ref, cs, _ = oracle_of(*pairs[j])
        assert_same_bytes(payload_np(small.payload(j, sres[j]["payload_bytes"])), ref, f"{j}")
