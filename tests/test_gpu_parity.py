"""GPU parity of libbf16delta against the CPU oracle (MI355X, gfx950).

Every case runs the HIP path through the C ABI (via the Python binding) and
the oracle on the same bytes.  It then checks four things:
- the payload and checksum are byte-identical;
- in-place decompression rebuilds dst bit for bit;
- a second compression gives the same bytes, which catches races in the
  look-back and the LDS packing;
- the failure statuses and the final weights match the oracle's.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from lossless_bf16_weight_xor_amd import (ECHECKSUM, EFORMAT, OK, ChecksumError,
                                          CompressBatch, FormatError, compress_batch,
                                          decompress_batch, delta_compress,
                                          delta_decompress, synth)
from tests import payload_view as pv
from tests.gpu_util import assert_same_bytes, log, oracle_of, pair, payload_np, to_device, to_u16

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _check_pair(src, dst, what):
    log(f"case {what}: n={src.numel()}")
    payload, cs = delta_compress(src, dst)
    ref_payload, ref_cs, stats = oracle_of(src, dst)
    assert cs == ref_cs, f"{what}: checksum"
    assert_same_bytes(payload_np(payload), ref_payload, what)
    payload2, cs2 = delta_compress(src, dst)
    assert cs2 == cs and torch.equal(payload2, payload), f"{what}: not deterministic"
    w = src.clone()
    delta_decompress(w, payload, cs)
    assert torch.equal(w.view(torch.int16), dst.view(torch.int16)), f"{what}: round trip"
    return payload, cs, stats


def test_worked_examples_byte_for_byte(golden_dir):
    with open(os.path.join(golden_dir, "worked_examples.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
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
        payload, cs = delta_compress(src, dst)
        p = payload_np(payload)
        assert len(p) == case["payload_bytes"], case["name"]
        assert bytes(p[pv.data_offset(n):]).hex().upper() == case["data_hex"].upper()
        assert [int(d) for d in pv.descriptors(p, n)] == [int(d, 16) for d in case["descriptors"]]
        assert cs == oracle.checksum(new)


def test_config1_single_tensor():
    src, dst = synth.config1(DEV)
    _, _, stats = _check_pair(src, dst, "config1")
    assert stats["n_changed"] == 20972


@pytest.mark.parametrize("n", [1, 2, 3, 5, 63, 64, 65, 127, 8191, 8192, 8193, 3 * 8192 + 5,
                               70001])
def test_odd_lengths_and_ragged_tails(n):
    src, dst = pair((n,), "0.05", synth.MIX_ADVERSARIAL, 1000 + n, DEV)
    _check_pair(src, dst, f"ragged n={n}")


@pytest.mark.parametrize("rate", ["0", "0.00085", "0.01", "0.14", "0.2", "0.3", "0.6", "1"])
def test_change_rates_span_both_position_encodings(rate):
    src, dst = pair((9 * 8192 + 333,), rate, synth.MIX_DEFAULT, 77, DEV)
    _check_pair(src, dst, f"rate={rate}")


def _two_block_pair(p0, c1, r1):
    """Block 0: one mantissa change at p0 (or none); block 1: c1 changes 8 apart,
    the first r1 of them also flipping an exponent bit."""
    n = 2 * 8192
    old = np.full(n, 0x3F80, dtype=np.uint16)
    new = old.copy()
    if p0 is not None:
        new[p0] ^= 0x0001
    pos = 8192 + 8 * np.arange(c1)
    new[pos] ^= 0x0001
    new[pos[:r1]] ^= 0x0100
    return old, new


# Block 1's record is 2046..2048 bytes (the largest that goes through the
# 2 KiB slot) and block 0's record (0..3 bytes) puts it at every byte offset
# within a dword: the copy then spans one dword more than the slot.
@pytest.mark.parametrize("p0", [None, 0, 1, 300])
@pytest.mark.parametrize("c1,r1", [(1000, 399), (1003, 396), (1000, 398)])
def test_largest_slot_records_at_every_byte_offset(p0, c1, r1):
    old, new = _two_block_pair(p0, c1, r1)
    payload, _, _ = oracle.compress(old, new)
    lens = [pv.record_bytes(int(d), pv.block_len(old.size, b))
            for b, d in enumerate(pv.descriptors(payload, old.size))]
    assert lens[1] in (2046, 2047, 2048), lens
    assert (pv.data_offset(old.size) + lens[0]) % 4 == {None: 0, 0: 1, 1: 2, 300: 3}[p0]
    _check_pair(to_device(old, DEV), to_device(new, DEV), f"p0={p0} c1={c1} r1={r1}")


def test_all_rare_changes():
    n = 5 * 8192 + 1
    src, _ = pair((n,), "0", synth.MIX_DEFAULT, 5, DEV)
    dst = (src.view(torch.int16) ^ torch.tensor(-32768, dtype=torch.int16, device=DEV)).view(
        torch.bfloat16)
    _, _, stats = _check_pair(src, dst, "all sign flips")
    assert stats["n_rare"] == n


def test_page_api_example_on_gpu():
    """The pages' own example ("Using ARCv3"), moved to the GPU.  About 22%
    of elements change, so every block is a bitmap."""
    src, dst = synth.page_example(seed=0)
    src, dst = src.to(DEV), dst.to(DEV)
    payload, cs, stats = _check_pair(src, dst, "page example")
    assert stats["n_bitmap_blocks"] == 128
    restored = src.clone()
    restored = delta_decompress(restored, payload, cs)
    assert torch.equal(restored.view(torch.uint8), dst.view(torch.uint8))


@pytest.mark.parametrize("case", synth.C4_CASES)
def test_config4_adversarial_full_size(case):
    """The 64 MiB adversarial and edge cases at full size."""
    src, dst = synth.config4(DEV, case)
    _check_pair(src, dst, f"config4 {case}")


def test_batched_call_matches_per_tensor_oracle():
    """One batched call over mixed sizes and densities, including an empty
    tensor, matches the oracle per job."""
    specs = [((0,), "0.02"), ((1,), "1"), ((4096, 3),  "0.02"), ((8192,), "0.2"),
             ((3, 8192 + 1), "0.05"), ((1024, 1024), "0.02"), ((7,), "0"), ((100000,), "0.6")]
    pairs = []
    for i, (shape, rate) in enumerate(specs):
        if shape == (0,):
            s = torch.empty(0, dtype=torch.bfloat16, device=DEV)
            pairs.append((s, s.clone()))
        else:
            pairs.append(pair(shape, rate, synth.MIX_ADVERSARIAL, 300 + i, DEV))
    out = compress_batch(pairs)
    for j, ((src, dst), (payload, cs, _)) in enumerate(zip(pairs, out)):
        ref_payload, ref_cs, _ = oracle_of(src, dst)
        assert cs == ref_cs, j
        assert_same_bytes(payload_np(payload), ref_payload, f"batch job {j}")
    ws = [s.clone() for s, _ in pairs]
    res = decompress_batch([(w, p, cs) for w, (p, cs, _) in zip(ws, out)])
    for j, (w, (_, dst), r) in enumerate(zip(ws, pairs, res)):
        assert r["status"] == OK, j
        assert torch.equal(w.view(torch.int16), dst.view(torch.int16)), j


def test_thousands_of_tiny_jobs_in_one_call():
    """3000 tensors of 0..300 elements (every tenth one empty) in one call:
    the per-job passes of the descriptor scan and checksum sum run many
    rounds over a workgroup's threads, and most tiles are ragged."""
    log("case 3000 tiny jobs")
    rng = np.random.default_rng(77)
    sizes = rng.integers(1, 301, size=3000)
    sizes[::10] = 0
    rates = ["0", "0.02", "0.2", "1"]
    pairs = []
    for j, n in enumerate(sizes):
        if n == 0:
            s = torch.empty(0, dtype=torch.bfloat16, device=DEV)
            pairs.append((s, s.clone()))
        else:
            s, d = pair((int(n),), rates[j % 4], synth.MIX_ADVERSARIAL, 7000 + j, "cpu")
            pairs.append((s.to(DEV), d.to(DEV)))
    out = compress_batch(pairs)
    for j, ((src, dst), (payload, cs, _)) in enumerate(zip(pairs, out)):
        ref_payload, ref_cs, _ = oracle_of(src, dst)
        assert cs == ref_cs, j
        assert_same_bytes(payload_np(payload), ref_payload, f"tiny job {j}")
    ws = [s.clone() for s, _ in pairs]
    res = decompress_batch([(w, p, cs) for w, (p, cs, _) in zip(ws, out)])
    for j, (w, (_, dst), r) in enumerate(zip(ws, pairs, res)):
        assert r["status"] == OK, j
        assert torch.equal(w.view(torch.int16), dst.view(torch.int16)), j


def test_compress_batch_compresses_again_only_the_dense_jobs():
    """A batch whose worst case passes 256 MiB starts from a first guess of
    1/16 of the weights; the dense job that does not fit is compressed again
    on its own (its payload lands in a second arena), the sparse ones are
    not, and every payload is the oracle's."""
    log("case first-guess capacities with one dense job")
    pairs = [pair((32 * 2 ** 20,), "0.01", synth.MIX_DEFAULT, 41, DEV),
             pair((64 * 2 ** 20,), "0.3", synth.MIX_DEFAULT, 42, DEV),
             pair((8192 * 3 + 5,), "0.02", synth.MIX_DEFAULT, 43, DEV)]
    out = compress_batch(pairs)
    arenas = [p.untyped_storage().data_ptr() for p, _, _ in out]
    assert arenas[0] == arenas[2] != arenas[1]
    for j, ((src, dst), (payload, cs, _)) in enumerate(zip(pairs, out)):
        ref_payload, ref_cs, _ = oracle_of(src, dst)
        assert cs == ref_cs, j
        assert_same_bytes(payload_np(payload), ref_payload, f"job {j}")


def test_capacity_too_small_reports_the_exact_size():
    src, dst = pair((5 * 8192,), "0.3", synth.MIX_DEFAULT, 9, DEV)
    ref_payload, _, _ = oracle_of(src, dst)
    guard = 4096
    for cap in (0, 64, len(ref_payload) // 2, len(ref_payload) - 1):
        batch = CompressBatch([(src, dst)], [cap + guard])
        batch.capacity[0] = cap
        batch.jobs[0].capacity = cap
        batch.arena.fill_(0xA5)
        batch.run()
        r = batch.results()[0]
        assert r["status"] == 2 and r["payload_bytes"] == len(ref_payload), cap
        tail = batch.arena[cap: cap + guard].cpu().numpy()
        assert (tail == 0xA5).all(), f"capacity {cap}: wrote past the capacity"


# ---------------------------------------------------- failure injection ---

@pytest.fixture(scope="module")
def injected():
    src, dst = pair((4 * 8192 + 123,), "0.05", synth.MIX_ADVERSARIAL, 21, DEV)
    payload, cs = delta_compress(src, dst)
    return src, dst, payload_np(payload), cs


def _gpu_apply(src, payload_bytes: np.ndarray, cs, verify_first=False):
    w = src.clone()
    p = torch.from_numpy(payload_bytes.copy()).to(DEV) if payload_bytes.size else \
        torch.zeros(16, dtype=torch.uint8, device=DEV)[:0]
    r = decompress_batch([(w, p, cs)], verify_first=verify_first)[0]
    return r["status"], w


def _oracle_apply(src, payload_bytes, cs):
    w = to_u16(src).copy()
    return oracle.decompress_inplace(w, payload_bytes, cs), w


def _same_outcome(src, p, cs, what, verify_first=False):
    st_g, w_g = _gpu_apply(src, p, cs, verify_first)
    st_o, w_o = _oracle_apply(src, p, cs)
    assert st_g == st_o, f"{what}: status gpu {st_g} oracle {st_o}"
    assert np.array_equal(to_u16(w_g), w_o), f"{what}: weights differ from the oracle's"
    return st_g


def test_wrong_checksum_rolls_back(injected):
    src, dst, p, cs = injected
    assert _same_outcome(src, p, cs ^ 1, "wrong checksum") == ECHECKSUM
    with pytest.raises(ChecksumError):
        w = src.clone()
        delta_decompress(w, torch.from_numpy(p).to(DEV), cs ^ 1)
    assert torch.equal(w.view(torch.int16), src.view(torch.int16))


def test_wrong_baseline_rolls_back(injected):
    src, dst, p, cs = injected
    bad = src.clone()
    bad.view(torch.int16)[5] ^= 1
    assert _same_outcome(bad, p, cs, "wrong baseline") == ECHECKSUM


@pytest.mark.parametrize("offset", [0, 8, 12, 16, 24, 32, 40, 48, 56, 64, 65, 66])
def test_corrupt_header_or_table(injected, offset):
    src, dst, p, cs = injected
    q = p.copy()
    q[offset] ^= 0x01
    assert _same_outcome(src, q, cs, f"header byte {offset}") == EFORMAT


@pytest.mark.parametrize("cut", [1, 7, 63, 200])
def test_truncated(injected, cut):
    src, dst, p, cs = injected
    assert _same_outcome(src, p[:-cut], cs, f"truncated {cut}") == EFORMAT


def test_short_payloads(injected):
    src, dst, p, cs = injected
    for k in (0, 10, 63, 64, 70):
        assert _same_outcome(src, p[:k], cs, f"short {k}") == EFORMAT


def test_every_record_byte_and_bit_of_block0(injected):
    """Flip each bit of the first 96 record bytes.  The GPU must give the same
    status and the same final weights as the oracle every time."""
    src, dst, p, cs = injected
    start = pv.data_offset(src.numel())
    for byte in range(start, min(start + 96, p.size)):
        for bit in range(8):
            q = p.copy()
            q[byte] ^= np.uint8(1 << bit)
            st = _same_outcome(src, q, cs, f"byte {byte} bit {bit}")
            assert st in (EFORMAT, ECHECKSUM)


def test_non_canonical_blocks_match_the_oracle():
    import struct
    a = np.zeros(16, np.uint16)
    b = a.copy()
    b[2] = 0x0001
    src, dst = to_device(a, DEV), to_device(b, DEV)
    payload, cs = delta_compress(src, dst)
    p = payload_np(payload)
    q = p.copy()
    q[64:68] = np.frombuffer(struct.pack("<I", 1 | (3 << 28)), np.uint8)   # non-minimal width
    assert _same_outcome(src, q, cs, "width 3 for gap 2") == EFORMAT
    hdr = bytearray(bytes(p[:64]))
    hdr[40:48] = struct.pack("<Q", 2)
    q = np.frombuffer(bytes(hdr) + struct.pack("<I", 1 | (15 << 28)) + bytes([0x04, 0x00, 0x01]),
                      np.uint8)
    assert _same_outcome(src, q, cs, "bitmap where gap list is smaller") == EFORMAT
    a2 = np.zeros(16, np.uint16)
    b2 = a2.copy()
    b2[3] = 0x8000
    src2, dst2 = to_device(a2, DEV), to_device(b2, DEV)
    payload2, cs2 = delta_compress(src2, dst2)
    q = payload_np(payload2).copy()
    q[pv.data_offset(16) + 2] = 0x05
    q[pv.data_offset(16) + 3] = 0x00
    assert _same_outcome(src2, q, cs2, "rare word without exponent/sign bits") == EFORMAT


def test_failure_in_one_job_leaves_the_others_applied():
    pairs = [pair((3 * 8192 + 9,), "0.02", synth.MIX_DEFAULT, 60 + i, DEV) for i in range(3)]
    out = compress_batch(pairs)
    ws = [s.clone() for s, _ in pairs]
    items = [(w, p, cs) for w, (p, cs, _) in zip(ws, out)]
    items[1] = (ws[1], out[1][0], out[1][1] ^ 0xFF)
    res = decompress_batch(items)
    assert [r["status"] for r in res] == [OK, ECHECKSUM, OK]
    assert torch.equal(ws[0].view(torch.int16), pairs[0][1].view(torch.int16))
    assert torch.equal(ws[1].view(torch.int16), pairs[1][0].view(torch.int16))
    assert torch.equal(ws[2].view(torch.int16), pairs[2][1].view(torch.int16))


def test_payload_applies_in_both_directions():
    """The payload depends only on the mask: applied to new with old's
    checksum it gives old."""
    src, dst = pair((6 * 8192 + 1,), "0.02", synth.MIX_DEFAULT, 88, DEV)
    payload, cs_new = delta_compress(src, dst)
    back, cs_old = delta_compress(dst, src)
    assert torch.equal(back, payload)
    w = dst.clone()
    delta_decompress(w, payload, cs_old)
    assert torch.equal(w.view(torch.int16), src.view(torch.int16))


# ------------------------------------------------- verify-first decompress ---

def test_verified_decompress_failures_match_the_oracle(injected):
    """bf16d_decompress_verified: the same statuses and final weights as the
    oracle for a wrong checksum, a wrong baseline, header and table
    corruption, truncation and flipped record bits."""
    src, dst, p, cs = injected
    log("case verify-first failures")
    assert _same_outcome(src, p, cs, "good", True) == OK
    assert _same_outcome(src, p, cs ^ 1, "wrong checksum", True) == ECHECKSUM
    bad = src.clone()
    bad.view(torch.int16)[5] ^= 1
    assert _same_outcome(bad, p, cs, "wrong baseline", True) == ECHECKSUM
    for offset in (0, 8, 24, 64, 66):
        q = p.copy()
        q[offset] ^= 0x01
        assert _same_outcome(src, q, cs, f"header byte {offset}", True) == EFORMAT
    assert _same_outcome(src, p[:-7], cs, "truncated", True) == EFORMAT
    start = pv.data_offset(src.numel())
    for byte in range(start, min(start + 48, p.size)):
        for bit in (0, 3, 6):
            q = p.copy()
            q[byte] ^= np.uint8(1 << bit)
            assert _same_outcome(src, q, cs, f"byte {byte} bit {bit}", True) in (EFORMAT,
                                                                                 ECHECKSUM)


@pytest.mark.parametrize("rate", ["0.02", "0.3", "1"])
def test_verified_decompress_batch_rebuilds_and_refuses(rate):
    """A batch of ragged tensors (gap lists, bitmaps, short last blocks), the
    second job with a wrong checksum: the others are rebuilt bit for bit and
    the failing one is left exactly as it was."""
    log(f"case verify-first batch rate={rate}")
    pairs = [pair((n,), rate, synth.MIX_ADVERSARIAL, 8100 + k, DEV)
             for k, n in enumerate((3 * 8192 + 77, 8192, 70001, 1, 5 * 8192))]
    out = compress_batch(pairs)
    ws = [s.clone() for s, _ in pairs]
    items = [(w, p, cs) for w, (p, cs, _) in zip(ws, out)]
    items[1] = (ws[1], out[1][0], out[1][1] ^ 0x77)
    res = decompress_batch(items, verify_first=True)
    assert [r["status"] for r in res] == [OK, ECHECKSUM, OK, OK, OK]
    for j, (w, (s, d)) in enumerate(zip(ws, pairs)):
        want = s if j == 1 else d
        assert torch.equal(w.view(torch.int16), want.view(torch.int16)), j
