"""GPU parity of version-2 payloads (bf16d_compress_bound /
bf16d_decompress_bound) against the CPU oracle.

Version 2 binds a payload to the version it was made against and the one it
produces, and its overwrite records carry absolute values (the NeMo
Delta-Compressed Refit summary; "GPU-accelerated Weight Teleportation",
section "Eval, fault tolerance, and resuming from trained checkpoints").
Each case checks:
- payload bytes and checksum identical to the oracle's;
- the apply rebuilds the new weights and moves the version word, as the
  oracle does;
- an overwrite payload rebuilds the new weights from any partial write;
- every failure ends with the oracle's status, weights and version word.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import lossless_bf16_weight_xor_amd as bd
from lossless_bf16_weight_xor_amd import synth
from tests.gpu_util import assert_same_bytes, log, payload_np, to_device, to_u16

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

# shapes and rates chosen to reach every decode path: the register fast path
# (<= 1024 changes per block), the general gap list, bitmaps, records larger
# than a compress slot (re-encoded), short last blocks and empty tensors
CASES = [((3 * 8192 + 77,), "0.05", 1), ((8192,), "0.2", 2), ((5 * 8192 + 3,), "0.6", 3),
         ((2 * 8192,), "1.0", 4), ((70001,), "0.001", 5), ((1,), "1.0", 6), ((0,), "0", 7),
         ((513, 129), "0.13", 8), ((8191,), "0.3", 9), ((64, 8192), "0.02", 10)]


def _pair(shape, rate, seed):
    return synth.make_pair(shape, rate, synth.MIX_ADVERSARIAL, seed, DEV, "uniform")


def _versions(vals):
    return torch.tensor([v & 0x7FFFFFFFFFFFFFFF for v in vals], dtype=torch.int64, device=DEV)


@pytest.mark.parametrize("overwrite", [False, True])
def test_bound_payloads_match_the_oracle(overwrite):
    pairs = [tuple(t.reshape(-1) for t in _pair(*c)) for c in CASES]
    binds = [(100 + j, 200 + j, overwrite) for j in range(len(pairs))]
    out = bd.compress_batch(pairs, binds)
    for j, ((s, d), (p, cs, st)) in enumerate(zip(pairs, out)):
        log(f"case bound compress overwrite={overwrite} job {j} n={s.numel()}")
        want, want_cs, want_st = oracle.compress_v2(to_u16(s), to_u16(d), 100 + j, 200 + j,
                                                    overwrite=overwrite)
        assert cs == want_cs, f"job {j}: checksum"
        assert_same_bytes(payload_np(p), want, f"job {j}")
        assert st["n_changed"] == want_st["n_changed"] and st["n_rare"] == want_st["n_rare"]
    # apply from the base version: new weights, target version
    recv = [s.clone() for s, _ in pairs]
    ver = _versions([100 + j for j in range(len(pairs))])
    res = bd.decompress_batch([(w, p, cs) for w, (p, cs, _) in zip(recv, out)], ver)
    assert [r["status"] for r in res] == [bd.OK] * len(pairs)
    assert ver.cpu().tolist() == [200 + j for j in range(len(pairs))]
    for j, (w, (_, d)) in enumerate(zip(recv, pairs)):
        assert torch.equal(w.view(torch.int16), d.view(torch.int16)), f"job {j}"
    # once more: the versions now differ from the bases, so nothing moves
    res = bd.decompress_batch([(w, p, cs) for w, (p, cs, _) in zip(recv, out)], ver)
    assert [r["status"] for r in res] == [bd.EVERSION] * len(pairs)
    assert ver.cpu().tolist() == [200 + j for j in range(len(pairs))]
    for w, (_, d) in zip(recv, pairs):
        assert torch.equal(w.view(torch.int16), d.view(torch.int16))


@pytest.mark.parametrize("rate", ["0.1", "0.2", "0.3", "0.6", "0.9"])
def test_overwrite_over_many_seeds(rate):
    """Dense overwrite blocks, whose records outgrow the staged window: each
    must apply exactly as the oracle does, for several draws."""
    pairs = [tuple(t.reshape(-1) for t in _pair((2 * 8192 + 7 * k,), rate, 300 + k))
             for k in range(6)]
    out = bd.compress_batch(pairs, [(3, 4, True)] * len(pairs))
    recv = [s.clone() for s, _ in pairs]
    log(f"case overwrite rate {rate}")
    ver = _versions([3] * len(pairs))
    res = bd.decompress_batch([(w, p, cs) for w, (p, cs, _) in zip(recv, out)], ver)
    for j, ((s, d), (p, cs, _), r) in enumerate(zip(pairs, out, res)):
        want, want_cs, _ = oracle.compress_v2(to_u16(s), to_u16(d), 3, 4, overwrite=True)
        assert_same_bytes(payload_np(p), want, f"rate {rate} job {j}")
        assert r["status"] == bd.OK, f"rate {rate} job {j}: {r['status']}"
        assert torch.equal(recv[j].view(torch.int16), d.view(torch.int16)), f"job {j}"
    assert ver.cpu().tolist() == [4] * len(pairs)


def test_overwrite_rebuilds_from_any_partial_write():
    pairs = [tuple(t.reshape(-1) for t in _pair(*c)) for c in CASES if c[0] != (0,)]
    out = bd.compress_batch(pairs, [(0, 1, True)] * len(pairs))
    gen = torch.Generator(device="cpu").manual_seed(5)
    for trial in range(3):
        log(f"case overwrite partial write trial {trial}")
        recv = []
        for s, d in pairs:
            take = (torch.rand(s.numel(), generator=gen) < 0.5).to(DEV)
            recv.append(torch.where(take, d, s))        # some changes already written
        ver = _versions([0] * len(pairs))
        res = bd.decompress_batch([(w, p, cs) for w, (p, cs, _) in zip(recv, out)], ver)
        assert all(r["status"] == bd.OK for r in res)
        assert ver.cpu().tolist() == [1] * len(pairs)
        for w, (_, d) in zip(recv, pairs):
            assert torch.equal(w.view(torch.int16), d.view(torch.int16))


def test_failures_match_the_oracle_in_one_mixed_batch():
    """Version-1, bound XOR and overwrite payloads in one call, some of them
    broken: every job must end exactly as the oracle's decoder ends it."""
    log("case mixed batch with failures")
    shapes = [((3 * 8192 + 5,), "0.05"), ((8192,), "0.3"), ((2 * 8192 + 1,), "0.6"),
              ((70001,), "0.02"), ((4096,), "1.0"), ((9000,), "0.1")]
    pairs = [tuple(t.reshape(-1) for t in _pair(sh, r, 40 + i)) for i, (sh, r) in
             enumerate(shapes)]
    kinds = ["v1", "xor", "ow", "ow", "xor", "ow"]
    payloads, checksums = [], []
    for (s, d), k in zip(pairs, kinds):
        if k == "v1":
            p, cs, _ = bd.compress_batch([(s, d)])[0]
        else:
            p, cs, _ = bd.compress_batch([(s, d)], [(7, 8, k == "ow")])[0]
        payloads.append(p.clone())
        checksums.append(cs)
    checksums[1] ^= 1                       # bound XOR, wrong checksum: rolled back
    checksums[2] ^= 1                       # overwrite, wrong checksum: never written
    payloads[3][-1] ^= 0x10                 # overwrite, corrupt value: checksum fails
    recv = [s.clone() for s, _ in pairs]
    # job 3 starts half written, job 4's receiver holds another version
    s3, d3 = pairs[3]
    half = torch.arange(s3.numel(), device=DEV) % 2 == 0
    recv[3] = torch.where(half, d3, s3)
    start = [to_u16(w).copy() for w in recv]
    vers0 = [7, 7, 7, 7, 6, 7]
    ver = _versions(vers0)
    res = bd.decompress_batch([(w, p, cs) for w, p, cs in zip(recv, payloads, checksums)], ver)
    got_ver = ver.cpu().tolist()
    for j in range(len(pairs)):
        w = start[j].copy()
        want, want_ver = oracle.decompress_v2_inplace(w, payload_np(payloads[j]), checksums[j],
                                                      vers0[j])
        assert res[j]["status"] == want, f"job {j}: {res[j]['status']} vs oracle {want}"
        assert got_ver[j] == want_ver, f"job {j}: version"
        assert np.array_equal(to_u16(recv[j]), w), f"job {j}: weights"
    assert [r["status"] for r in res] == [bd.OK, bd.ECHECKSUM, bd.ECHECKSUM, bd.ECHECKSUM,
                                          bd.EVERSION, bd.OK]


def test_worked_examples_v2_byte_for_byte(golden_dir):
    with open(os.path.join(golden_dir, "worked_examples_v2.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        log(f"case golden v2 {case['name']}")
        n = case["n"]
        old = np.full(n, int(case["old"]["fill"], 16), dtype=np.uint16)
        new = old.copy()
        for i, v in case["new_changes"].items():
            new[int(i)] = int(v, 16)
        if n == 0:
            src = torch.empty(0, dtype=torch.bfloat16, device=DEV)
            dst = src.clone()
        else:
            src, dst = to_device(old, DEV), to_device(new, DEV)
        p, cs, _ = bd.compress_batch([(src, dst)],
                                     [(case["base"], case["target"], bool(case["flags"] & 1))])[0]
        b = payload_np(p)
        assert len(b) == case["payload_bytes"], case["name"]
        assert bytes(b[96 + 4 * (-(-n // 8192)):]).hex().upper() == case["data_hex"].upper()


def test_plain_decompress_reads_bound_payloads_without_the_binding():
    log("case plain decompress of v2 payloads")
    pairs = [tuple(t.reshape(-1) for t in _pair((3 * 8192 + 9,), "0.05", 60 + k))
             for k in range(2)]
    out = bd.compress_batch(pairs, [(1, 2, False), (1, 2, True)])
    recv = [s.clone() for s, _ in pairs]
    res = bd.decompress_batch([(w, p, cs) for w, (p, cs, _) in zip(recv, out)])
    assert [r["status"] for r in res] == [bd.OK, bd.OK]
    for w, (_, d) in zip(recv, pairs):
        assert torch.equal(w.view(torch.int16), d.view(torch.int16))


def _smallest_workspace(items, versions):
    """The smallest workspace the call accepts (no room for an undo area):
    found by bisection on the host-side size check, which refuses a short
    workspace before enqueueing anything."""
    lo, hi = 0, bd.workspace_bytes(sum(w.numel() for w, _, _ in items), len(items))
    while hi - lo > 256:
        mid = (lo + hi) // 2 // 256 * 256
        batch = bd.DecompressBatch(items, versions, workspace_bytes_override=mid)
        try:
            batch.run()
            hi = mid
        except RuntimeError:
            lo = mid
        torch.cuda.synchronize()
    return hi


@pytest.mark.parametrize("room", ["undo", "none"])
def test_overwrite_in_place_and_verified_first_end_alike(room):
    """Overwrite payloads are written in place with an undo log when the
    workspace has room for it, and verified first otherwise.  Either way:
    the oracle's statuses, the new weights on OK, and the weights exactly as
    they were (partly written or not) on a failure."""
    log(f"case overwrite room={room}")
    shapes = [((3 * 8192 + 5,), "0.05"), ((8192,), "0.3"), ((2 * 8192 + 1,), "0.6"),
              ((70001,), "0.02"), ((4096,), "1.0")]
    pairs = [tuple(t.reshape(-1) for t in _pair(sh, r, 70 + i)) for i, (sh, r) in
             enumerate(shapes)]
    out = bd.compress_batch(pairs, [(7, 8, True)] * len(pairs))
    payloads = [p.clone() for p, _, _ in out]
    checksums = [cs for _, cs, _ in out]
    checksums[1] ^= 1                       # wrong checksum
    payloads[3][-1] ^= 0x10                 # a corrupt value: the checksum fails
    recv = [s.clone() for s, _ in pairs]
    s4, d4 = pairs[4]
    recv[4] = torch.where(torch.arange(s4.numel(), device=DEV) % 3 == 0, d4, s4)  # partly written
    start = [to_u16(w).copy() for w in recv]
    ver = _versions([7] * len(pairs))
    items = [(w, p, cs) for w, p, cs in zip(recv, payloads, checksums)]
    override = None if room == "undo" else _smallest_workspace(items, ver)
    ver = _versions([7] * len(pairs))
    res = bd.DecompressBatch(items, ver, workspace_bytes_override=override)
    res.run()
    res = res.results()
    got_ver = ver.cpu().tolist()
    for j in range(len(pairs)):
        w = start[j].copy()
        want, want_ver = oracle.decompress_v2_inplace(w, payload_np(payloads[j]), checksums[j], 7)
        assert res[j]["status"] == want, f"job {j}: {res[j]['status']} vs oracle {want}"
        assert got_ver[j] == want_ver, f"job {j}: version"
        assert np.array_equal(to_u16(recv[j]), w), f"job {j}: weights"
    assert [r["status"] for r in res] == [bd.OK, bd.ECHECKSUM, bd.OK, bd.ECHECKSUM, bd.OK]
