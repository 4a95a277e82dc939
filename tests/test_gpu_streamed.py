"""GPU tests of the streamed receiver (bf16d_decompress_streamed): host-resident
payloads applied in place group by group through a ring of device slots.

The payloads come from the GPU compressor, whose bytes the other parity tests
pin to the oracle; here the streamed apply must rebuild every tensor bit for
bit, and each failure must end exactly as the oracle's decoder ends it.
"""
import numpy as np
import pytest
import torch

import lossless_bf16_weight_xor_amd as bd
import oracle
from lossless_bf16_weight_xor_amd import synth
from tests.gpu_util import log, to_u16

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

SHAPES = [(3 * 8192 + 77,), (8192,), (4096, 64), (1,), (0,), (70001,), (2 * 8192,),
          (513, 129), (8191,), (5 * 8192 + 3,), (12345,), (64, 64)]


def _make(seed0=500):
    pairs = [synth.make_pair(shape, "0.03", synth.MIX_ADVERSARIAL, seed0 + i, DEV)
             for i, shape in enumerate(SHAPES)]
    pairs = [(s.reshape(-1), d.reshape(-1)) for s, d in pairs]
    out = bd.compress_batch(pairs)
    payloads = [p.cpu().pin_memory() for p, _, _ in out]
    checksums = [cs for _, cs, _ in out]
    return pairs, payloads, checksums


def _run(pairs, payloads, checksums, groups, slots=3, copy_streams=2, lanes=2):
    recv = [s.clone() for s, _ in pairs]
    sd = bd.StreamedDecompress(list(zip(recv, payloads, checksums)), groups, slots=slots,
                               copy_streams=copy_streams, lanes=lanes)
    sd.run()
    return recv, sd.results()


@pytest.mark.parametrize("lanes", [1, 2])
@pytest.mark.parametrize("slots,copies", [(2, 1), (3, 2), (5, 3)])
@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("groups", [[3, 1, 4, 4], [1] * 12, [12], [5, 7]])
def test_streamed_apply_rebuilds_every_tensor(groups, packed, slots, copies, lanes):
    """packed: all payloads in one pinned buffer at 16-byte boundaries, so each
    group goes over in one transfer; otherwise one pinned tensor each.  With
    two lanes, consecutive groups are applied on two compute streams."""
    log(f"case streamed groups={groups} packed={packed} slots={slots} copies={copies} "
        f"lanes={lanes}")
    pairs, payloads, checksums = _make()
    if packed:
        payloads = bd.StreamedDecompress.pin_packed(payloads)
    recv, res = _run(pairs, payloads, checksums, groups, slots, copies, lanes)
    assert [r["status"] for r in res] == [bd.OK] * len(pairs)
    for j, (w, (_, d)) in enumerate(zip(recv, pairs)):
        assert torch.equal(w.view(torch.int16), d.view(torch.int16)), f"tensor {j}"


def test_streamed_failures_match_the_oracle():
    log("case streamed failures")
    pairs, payloads, checksums = _make(seed0=900)
    payloads = [p.clone().pin_memory() for p in payloads]
    checksums = list(checksums)
    checksums[2] ^= 1                                  # wrong checksum
    payloads[5][-1] ^= 0x40                            # last record byte of a dense tensor
    payloads[9][70] ^= 0x01                            # a descriptor byte
    recv, res = _run(pairs, payloads, checksums, [4, 4, 4])
    for j, ((s, d), r) in enumerate(zip(pairs, res)):
        w = to_u16(s).copy()
        want = oracle.decompress_inplace(w, payloads[j].numpy(), checksums[j])
        assert r["status"] == want, f"tensor {j}: {r['status']} vs oracle {want}"
        assert np.array_equal(to_u16(recv[j]), w), f"tensor {j}: final weights"
    assert res[2]["status"] == bd.ECHECKSUM
    assert {res[5]["status"], res[9]["status"]} <= {bd.EFORMAT, bd.ECHECKSUM}
    assert all(res[j]["status"] == bd.OK for j in (0, 1, 3, 4, 6, 7, 8, 10, 11))


@pytest.mark.parametrize("lanes", [1, 2])
@pytest.mark.parametrize("slots,copies", [(2, 1), (2, 2), (3, 2), (3, 4)])
def test_streamed_many_groups_reuse_the_slots_in_turn(slots, copies, lanes):
    """40 one-tensor groups: each slot is refilled 40 / slots times, so every
    copy waits for the apply `slots` groups back, on whichever copy stream
    its group falls to, and that apply ran on whichever lane its group fell
    to."""
    log(f"case streamed 40 groups slots={slots} copies={copies} lanes={lanes}")
    pairs = [synth.make_pair((8192 * (1 + i % 3) + i,), "0.05", synth.MIX_DEFAULT, 1300 + i, DEV)
             for i in range(40)]
    out = bd.compress_batch(pairs)
    payloads = [p.cpu().pin_memory() for p, _, _ in out]
    recv, res = _run(pairs, payloads, [cs for _, cs, _ in out], [1] * 40, slots, copies, lanes)
    assert all(r["status"] == bd.OK for r in res)
    for w, (_, d) in zip(recv, pairs):
        assert torch.equal(w.view(torch.int16), d.view(torch.int16))


def test_raced_payloads_stream_into_the_receiver():
    """The whole trip: GPU compress, the host codec race on the trainer side,
    race decode into one pinned buffer on the receiver side, then the
    streamed apply.  Every tensor must come out bit for bit."""
    log("case raced payloads -> streamed receiver")
    pairs, payloads, checksums = _make(seed0=1700)
    frames = bd.race_compress([p.cpu() for p in payloads], bd.DEFAULT_RACE, threads=8)
    assert sum(f.frame.numel() for f in frames) <= sum(32 + p.numel() for p in payloads)
    raw = bd.race_decompress(frames, threads=8, pin=True)
    for q, p in zip(raw, payloads):
        assert torch.equal(q, p.cpu())
    recv, res = _run(pairs, raw, checksums, [4, 4, 4])
    assert [r["status"] for r in res] == [bd.OK] * len(pairs)
    for w, (_, d) in zip(recv, pairs):
        assert torch.equal(w.view(torch.int16), d.view(torch.int16))


def test_streamed_groups_mix_xor_and_overwrite_payloads():
    """Version-1 XOR payloads and version-2 overwrite payloads in the same
    groups: each group's commit pass writes its verified overwrite jobs."""
    log("case streamed mixed versions")
    shapes = [(3 * 8192 + 77,), (8192,), (70001,), (2 * 8192,), (12345,), (4096, 64)]
    pairs = [tuple(t.reshape(-1) for t in synth.make_pair(sh, r, synth.MIX_ADVERSARIAL,
                                                          2100 + i, DEV))
             for i, (sh, r) in enumerate(zip(shapes, ["0.03", "0.6", "0.02", "1.0", "0.1",
                                                      "0.3"]))]
    payloads, checksums = [], []
    for j, (s, d) in enumerate(pairs):
        binds = [(0, 1, True)] if j % 2 else None
        p, cs, _ = bd.compress_batch([(s, d)], binds)[0]
        payloads.append(p.cpu().pin_memory())
        checksums.append(cs)
    checksums[5] ^= 1                       # an overwrite job that must stay untouched
    recv, res = _run(pairs, payloads, checksums, [2, 3, 1])
    assert [r["status"] for r in res] == [bd.OK] * 5 + [bd.ECHECKSUM]
    for j, (w, (s, d)) in enumerate(zip(recv, pairs)):
        ref = s if j == 5 else d
        assert torch.equal(w.view(torch.int16), ref.view(torch.int16)), f"tensor {j}"
