"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: one batched compress over every tensor of a checkpoint
(`CompressBatch` with the same first payload capacities), then one batched
in-place decompress (`DecompressBatch`).

- 1 GiB tensor at four change rates: every payload byte and checksum is
  compared with the oracle's.
- 7B-shaped checkpoint (291 tensors, 6.7e9 elements): every tensor is compared
  with the oracle, byte for byte.
- 70B-shaped half model (360 tensors, 3.4e10 elements): every tensor is
  compared with the oracle, byte for byte.  Every tensor is also checked by
  properties that hold at any size: the exact class counts the generator
  planted, the round trip, a payload that depends only on the XOR mask
  (compressing new -> old gives the same bytes), and the same payloads from
  a compress with 256-byte record slots.
- The 7B-shaped checkpoint is also rebuilt by the verify-first call.

The oracle is single-threaded; the checkpoints' tensors are compared on a
pool of host threads (the oracle's C calls run without the interpreter lock),
each tensor copied to the host just before its turn so that only a bounded
number of tensors is held in host memory at once.
"""
import os
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import lossless_bf16_weight_xor_amd as bd
import oracle
from lossless_bf16_weight_xor_amd import synth
from tests.gpu_util import assert_same_bytes, log, to_u16

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _compress_like_bench(pairs):
    caps = [bd._first_capacity(s.numel()) for s, _ in pairs]
    comp = bd.CompressBatch(pairs, caps)
    comp.run()
    res = comp.results()
    if any(r["status"] != bd.OK for r in res):
        assert all(r["status"] in (bd.OK, bd.ECAPACITY) for r in res)
        caps = [r["payload_bytes"] for r in res]
        comp = bd.CompressBatch(pairs, caps)
        comp.run()
        res = comp.results()
    assert all(r["status"] == bd.OK for r in res), "compress failed"
    return comp, res


def _check_against_oracle(src, dst, payload, result, what):
    a, b = to_u16(src), to_u16(dst)
    ref_payload, ref_cs, stats = oracle.compress(a, b)
    assert result["checksum"] == ref_cs, f"{what}: checksum"
    assert result["n_changed"] == stats["n_changed"] and result["n_rare"] == stats["n_rare"]
    assert_same_bytes(payload.cpu().numpy(), ref_payload, what)


def _check_all_against_oracle(pairs, comp, res, names, threads=None, in_flight=None):
    """_check_against_oracle over every tensor, on a thread pool.  The host
    copies are made on this thread, in order, at most `in_flight` tensors
    ahead of the comparisons."""
    threads = threads or max(1, min(16, os.cpu_count() or 1))
    in_flight = in_flight or 2 * threads
    gate = threading.Semaphore(in_flight)
    done = [0]
    lock = threading.Lock()

    def work(a, b, got, r, what):
        try:
            ref_payload, ref_cs, stats = oracle.compress(a, b)
            assert r["checksum"] == ref_cs, f"{what}: checksum"
            assert r["n_changed"] == stats["n_changed"] and r["n_rare"] == stats["n_rare"], what
            assert_same_bytes(got, ref_payload, what)
            with lock:
                done[0] += 1
                if done[0] % 60 == 0:
                    log(f"  oracle agrees on {done[0]} tensors")
        finally:
            gate.release()

    futures = []
    with ThreadPoolExecutor(threads) as pool:
        for j, ((s, d), r) in enumerate(zip(pairs, res)):
            gate.acquire()
            got = comp.payload(j, r["payload_bytes"]).cpu().numpy()
            futures.append(pool.submit(work, to_u16(s), to_u16(d), got, r, names[j]))
        for f in futures:
            f.result()
    return done[0]


def _apply_in_place_and_compare(pairs, comp, res):
    """Batched decompress into src (in place), then src must equal dst."""
    items = [(s, comp.payload(j, r["payload_bytes"]), r["checksum"])
             for j, ((s, _), r) in enumerate(zip(pairs, res))]
    dec = bd.DecompressBatch(items)
    dec.run()
    dres = dec.results()
    assert all(r["status"] == bd.OK for r in dres), "decompress failed"
    for j, (s, d) in enumerate(pairs):
        assert torch.equal(s.view(torch.int16), d.view(torch.int16)), f"tensor {j}: round trip"


@pytest.mark.parametrize("rate", synth.C3_RATES)
def test_config3_one_gib_tensor_every_byte(rate):
    log(f"case 1 GiB tensor rate={rate}")
    src, dst = synth.config3(DEV, rate)
    pairs = [(src, dst)]
    comp, res = _compress_like_bench(pairs)
    k = synth.exact_count(rate, src.numel())
    assert res[0]["n_changed"] == k
    _check_against_oracle(src, dst, comp.payload(0, res[0]["payload_bytes"]), res[0],
                          f"1 GiB rate {rate}")
    _apply_in_place_and_compare(pairs, comp, res)


def test_config2_7b_checkpoint_every_tensor():
    log("case 7B-shaped checkpoint, all 291 tensors")
    pairs = [(s.reshape(-1), d.reshape(-1)) for _, s, d in synth.config2(DEV)]
    comp, res = _compress_like_bench(pairs)
    specs = synth.seven_b_specs()
    for j, ((s, d), r) in enumerate(zip(pairs, res)):
        k = synth.exact_count("0.02", s.numel())
        _, n_exp, n_sign = synth.class_counts(k)
        assert r["n_changed"] == k and r["n_rare"] == n_exp + n_sign, specs[j].name
    assert _check_all_against_oracle(pairs, comp, res, [sp.name for sp in specs]) == 291
    log("  oracle agrees on all 291 tensors")
    # the verify-first call on copies of the old weights: the same new weights
    copies = [s.clone() for s, _ in pairs]
    vdec = bd.DecompressBatch([(c, comp.payload(j, r["payload_bytes"]), r["checksum"])
                               for j, (c, r) in enumerate(zip(copies, res))], verify_first=True)
    vdec.run()
    assert all(r["status"] == bd.OK for r in vdec.results()), "verified decompress failed"
    for j, (c, (_, d)) in enumerate(zip(copies, pairs)):
        assert torch.equal(c.view(torch.int16), d.view(torch.int16)), specs[j].name
    del copies, vdec
    log("  verify-first decompress bit-exact")
    _apply_in_place_and_compare(pairs, comp, res)


def test_config5_70b_half_model_every_tensor():
    log("case 70B-shaped half model, 360 tensors")
    specs = synth.config5_specs()
    pairs = [(s.reshape(-1), d.reshape(-1)) for _, s, d in synth.config5(DEV)]
    assert len(pairs) == len(specs) == 360
    comp, res = _compress_like_bench(pairs)
    log("  compressed")
    assert _check_all_against_oracle(pairs, comp, res, [sp.name for sp in specs]) == 360
    log("  oracle agrees on all 360 tensors")
    for j, ((s, _), r) in enumerate(zip(pairs, res)):
        k = synth.exact_count("0.01", s.numel())
        _, n_exp, n_sign = synth.class_counts(k)
        assert r["n_changed"] == k and r["n_rare"] == n_exp + n_sign, specs[j].name
    # the payload depends only on the mask: new -> old gives the same bytes
    rev = bd.CompressBatch([(d, s) for s, d in pairs], [r["payload_bytes"] for r in res])
    rev.run()
    rres = rev.results()
    for j, r in enumerate(rres):
        assert r["status"] == bd.OK and r["payload_bytes"] == res[j]["payload_bytes"]
        assert torch.equal(rev.payload(j, r["payload_bytes"]),
                           comp.payload(j, res[j]["payload_bytes"])), specs[j].name
    del rev
    log("  reverse payloads identical")
    # 256-byte record slots (a workspace under 2 % of the weights), the same
    # first-guess capacities: the same payload bytes
    small = bd.CompressBatch(pairs, [bd._first_capacity(s.numel()) for s, _ in pairs],
                             slot_bytes=256)
    assert small.ws_bytes <= 0.02 * 2 * sum(s.numel() for s, _ in pairs)
    small.run()
    for j, r in enumerate(small.results()):
        assert r["status"] == bd.OK and r["payload_bytes"] == res[j]["payload_bytes"], j
        assert r["checksum"] == res[j]["checksum"], specs[j].name
        assert torch.equal(small.payload(j, r["payload_bytes"]),
                           comp.payload(j, res[j]["payload_bytes"])), specs[j].name
    del small
    log("  256-byte slots give the same payloads")
    _apply_in_place_and_compare(pairs, comp, res)
    log("  round trip bit-exact")


def test_tensor_beyond_four_billion_elements():
    """One tensor of 2^32 + 12345 elements with every element changed and a
    third of them rare: its payload passes 4 GiB, so block indices, record
    offsets and the payload arena all need 64 bits.  The head and the tail
    blocks are compared with the oracle run on those blocks alone (a block's
    record depends only on its own elements); the whole tensor by the round
    trip and by the payload depending only on the mask."""
    n = (1 << 32) + 12345
    log(f"case tensor of {n} elements, all changed")
    src, dst = synth.huge_pair(n, 77, DEV)
    pairs = [(src, dst)]
    comp, res = _compress_like_bench(pairs)
    r = res[0]
    assert r["n_changed"] == n
    # rare: i % 3 == 0, plus i % 97 == 0 among the others
    assert r["n_rare"] == -(-n // 3) + (-(-n // 97) - -(-n // 291))
    P = r["payload_bytes"]
    assert P > (1 << 32), P
    payload = comp.payload(0, P)
    nb = -(-n // 8192)
    desc = payload[64:64 + 4 * nb].cpu().numpy().view("<u4").astype(np.int64)
    c, rr, code = desc & 0x3FFF, (desc >> 14) & 0x3FFF, desc >> 28
    L = np.full(nb, 8192, np.int64)
    L[-1] = n - 8192 * (nb - 1)
    pb = np.where(code == 15, (L + 7) // 8, (c * np.where(code == 15, 0, code) + 7) // 8)
    lens = pb + (7 * c + 7) // 8 + 2 * rr
    starts = 64 + 4 * nb + np.concatenate([[0], np.cumsum(lens)[:-1]])
    assert starts[-1] + lens[-1] == P
    for name, b0, b1 in (("head", 0, 3), ("tail", nb - 3, nb)):
        lo, hi = 8192 * b0, min(n, 8192 * b1)
        ref, ref_cs, _ = oracle.compress(to_u16(src[lo:hi]), to_u16(dst[lo:hi]))
        k = b1 - b0
        assert np.array_equal(desc[b0:b1], ref[64:64 + 4 * k].view("<u4").astype(np.int64)), name
        got = payload[int(starts[b0]):int(starts[b1 - 1] + lens[b1 - 1])].cpu().numpy()
        assert_same_bytes(got, ref[64 + 4 * k:], f"{name} records")
    log("  head and tail blocks agree with the oracle")
    rev = bd.CompressBatch([(dst, src)], [P])
    rev.run()
    rres = rev.results()
    assert rres[0]["status"] == bd.OK and rres[0]["payload_bytes"] == P
    assert torch.equal(rev.payload(0, P), payload)
    del rev
    log("  reverse payload identical")
    _apply_in_place_and_compare(pairs, comp, res)
    log("  round trip bit-exact")
