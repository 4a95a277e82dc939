"""The decoder's canonical-record and bounds rules on the GPU, against the
oracle (MI355X).

The same hand-built payloads as the CPU pins (`tests/decoder_rule_cases.py`),
each breaking one rule, go through the batched decompress.  The GPU must give
the oracle's status (EFORMAT) and final weights (old), and must not write
outside the tensor: the weights are a view at the start of a larger buffer
whose tail holds a guard pattern, so a position past the tensor would land
in the guard, inside the same allocation.  Descriptor-table errors must be
reported before the binding of a version-2 payload is looked at.
"""
import numpy as np
import pytest
import torch

import oracle
import lossless_bf16_weight_xor_amd as bd
from tests import decoder_rule_cases as rules
from tests.gpu_util import log, to_u16

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
GUARD = 16384
CASES = rules.all_cases()
TABLE_CASES = rules.descriptor_table_cases()


def _guarded(old: np.ndarray):
    buf = np.concatenate([old, np.full(GUARD, 0xA5A5, np.uint16)])
    t = torch.from_numpy(buf.view(np.int16).copy()).to(DEV)
    return t, t[:old.size]


@pytest.mark.parametrize("case", CASES, ids=[c.name for c in CASES])
def test_rule_breaking_payload_matches_the_oracle(case):
    log(f"case decoder rule: {case.name} n={case.old.size}")
    cs = oracle.checksum(case.new)
    buf, w = _guarded(case.old)
    p = torch.from_numpy(case.payload.copy()).to(DEV)
    r = bd.decompress_batch([(w, p, cs)])[0]
    ref = case.old.copy()
    st_o = oracle.decompress_inplace(ref, case.payload, cs)
    assert st_o == oracle.EFORMAT
    assert r["status"] == st_o, f"status gpu {r['status']} oracle {st_o}"
    got = to_u16(buf)
    assert np.array_equal(got[:case.old.size], ref), "weights differ from the oracle's"
    assert (got[case.old.size:] == 0xA5A5).all(), "wrote past the tensor"


@pytest.mark.parametrize("case", TABLE_CASES, ids=[c.name for c in TABLE_CASES])
def test_descriptor_table_errors_come_before_the_binding(case):
    log(f"case descriptor table: {case.name}")
    cs = oracle.checksum(case.new)
    for held in (rules.OTHER_VERSION, rules.BASE_VERSION):
        buf, w = _guarded(case.old)
        p = torch.from_numpy(case.payload.copy()).to(DEV)
        ver = torch.tensor([held], dtype=torch.int64, device=DEV)
        r = bd.decompress_batch([(w, p, cs)], ver)[0]
        ref = case.old.copy()
        st_o, ver_o = oracle.decompress_v2_inplace(ref, case.payload, cs, held)
        assert (st_o, ver_o) == (oracle.EFORMAT, held)
        assert r["status"] == st_o, f"held {held}: status gpu {r['status']} oracle {st_o}"
        assert int(ver.item()) == ver_o
        got = to_u16(buf)
        assert np.array_equal(got[:case.old.size], ref)
        assert (got[case.old.size:] == 0xA5A5).all()


def test_all_rule_cases_in_one_batch():
    """Every case in one batched call beside a good job: each fails on its
    own, and the good job is applied."""
    log("case all decoder-rule payloads in one batch")
    good_old = np.full(3 * 8192 + 5, 0x3F80, np.uint16)
    good_new = good_old.copy()
    good_new[::37] ^= 0x0005
    gp, gcs, _ = oracle.compress(good_old, good_new)
    items, bufs = [], []
    for case in CASES:
        buf, w = _guarded(case.old)
        bufs.append(buf)
        items.append((w, torch.from_numpy(case.payload.copy()).to(DEV),
                      oracle.checksum(case.new)))
    gbuf, gw = _guarded(good_old)
    items.insert(len(items) // 2, (gw, torch.from_numpy(gp).to(DEV), gcs))
    res = bd.decompress_batch(items)
    k = len(CASES) // 2
    assert res[k]["status"] == bd.OK
    assert np.array_equal(to_u16(gbuf)[:good_old.size], good_new)
    for j, (case, buf) in enumerate(zip(CASES, bufs)):
        r = res[j if j < k else j + 1]
        assert r["status"] == bd.EFORMAT, case.name
        got = to_u16(buf)
        assert np.array_equal(got[:case.old.size], case.old), case.name
        assert (got[case.old.size:] == 0xA5A5).all(), case.name
