"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: one batched compress over every tensor of a checkpoint
(`CompressBatch` with the same first payload capacities), then one batched
in-place decompress (`DecompressBatch`).

- 1 GiB tensor at four change rates: every payload byte and checksum is
  compared with the oracle's.
- 7B-shaped checkpoint (291 tensors, 6.7e9 elements): every tensor is compared
  with the oracle, byte for byte.
- 70B-shaped half model (360 tensors, 3.4e10 elements): the oracle checks the
  tensors of the first and the last layer byte for byte.  Every tensor is
  checked by properties that hold at any size: the exact class counts the
  generator planted, the round trip, and a payload that depends only on the
  XOR mask (compressing new -> old gives the same bytes).
"""
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
        _check_against_oracle(s, d, comp.payload(j, r["payload_bytes"]), r, specs[j].name)
        k = synth.exact_count("0.02", s.numel())
        _, n_exp, n_sign = synth.class_counts(k)
        assert r["n_changed"] == k and r["n_rare"] == n_exp + n_sign, specs[j].name
        if j % 50 == 0:
            log(f"  oracle agrees up to tensor {j}")
    _apply_in_place_and_compare(pairs, comp, res)


def test_config5_70b_half_model_sampled_and_properties():
    log("case 70B-shaped half model, 360 tensors")
    specs = synth.config5_specs()
    pairs = [(s.reshape(-1), d.reshape(-1)) for _, s, d in synth.config5(DEV)]
    assert len(pairs) == len(specs) == 360
    comp, res = _compress_like_bench(pairs)
    log("  compressed")
    per_layer = len(specs) // 40
    sampled = set(range(per_layer)) | set(range(len(specs) - per_layer, len(specs)))
    for j in sorted(sampled):
        s, d = pairs[j]
        _check_against_oracle(s, d, comp.payload(j, res[j]["payload_bytes"]), res[j],
                              specs[j].name)
    log(f"  oracle agrees on {len(sampled)} sampled tensors")
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
    _apply_in_place_and_compare(pairs, comp, res)
    log("  round trip bit-exact")
