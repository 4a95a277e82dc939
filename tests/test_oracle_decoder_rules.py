"""The oracle decoder's canonical-record and bounds rules, one pin each (CPU).

Every rule is exercised by a payload built by hand from the format definition
(`tests/decoder_rule_cases.py`): the payload describes the pair's change but
breaks exactly that rule.  The oracle must answer EFORMAT and leave the
weights old; a decoder without the rule would instead rebuild `new` (OK) or
write past the tensor, which the guard words after it would show.

Why the rules matter: they make the payload a function of the change mask, so
that "identical to the oracle" is well defined, and the bounds rule is what
keeps a malformed record from writing outside the tensor.  The receiver may
never leave an update placed wrongly or half-applied (NeMo-DCR summary,
"Results and significance").
"""
import numpy as np
import pytest

import oracle
from lossless_bf16_weight_xor_amd import synth
from tests import decoder_rule_cases as rules
from tests import payload_build as pb
from tests import payload_view as pv

GUARD = 16384
CASES = rules.all_cases()


def _guarded_apply(old, payload, cs):
    """Apply to a view of the first n elements of a larger buffer whose tail
    is a guard pattern; returns (status, weights, guard intact)."""
    buf = np.concatenate([old, np.full(GUARD, 0xA5A5, np.uint16)])
    w = buf[:old.size]
    st = oracle.decompress_inplace(w, payload, cs)
    return st, buf[:old.size].copy(), bool((buf[old.size:] == 0xA5A5).all())


@pytest.mark.parametrize("case", CASES, ids=[c.name for c in CASES])
def test_rule_breaking_payload_is_rejected_and_weights_end_old(case):
    st, w, guard_ok = _guarded_apply(case.old, case.payload, oracle.checksum(case.new))
    assert guard_ok, "wrote past the tensor"
    assert st == oracle.EFORMAT, oracle.STATUS_NAMES.get(st, st)
    assert np.array_equal(w, case.old)


@pytest.mark.parametrize("case", CASES, ids=[c.name for c in CASES])
def test_the_same_change_encoded_canonically_applies(case):
    """Control: the pair's own payload rebuilds `new`, so each rejection above
    is the broken rule's doing and not the checksum's."""
    payload, cs, _ = oracle.compress(case.old, case.new)
    assert cs == oracle.checksum(case.new)
    nb = -(-case.old.size // pb.BLOCK)
    own = pb.payload(case.old.size, [pb.block_of(case.old, case.new, b) for b in range(nb)])
    assert np.array_equal(payload, own)
    st, w, guard_ok = _guarded_apply(case.old, payload, cs)
    assert guard_ok and st == oracle.OK and np.array_equal(w, case.new)


def test_the_independent_record_checker_rejects_every_case():
    for case in CASES:
        n = case.old.size
        descs = pv.descriptors(case.payload, n)
        off = pv.data_offset(n)
        bad = 0
        for b, d in enumerate(descs):
            L = pv.block_len(n, b)
            ln = sum(pb.segment_sizes(int(d), L))
            bad += pb.check_record(bytes(case.payload[off:off + ln]), int(d), L) is None
            off += ln
        assert bad == 1, case.name


@pytest.mark.parametrize("seed,rate,shape", [(1, "0.02", (3 * 8192 + 17,)),
                                             (2, "0.25", (2 * 8192 + 5,)),
                                             (3, "0.6", (8192 + 1,)),
                                             (4, "0.00085", (4 * 8192,))])
def test_independent_encoder_writes_the_oracle_bytes(seed, rate, shape):
    """The test-side encoder, written from the format definition, produces the
    oracle's payload byte for byte (gap lists, bitmaps, ragged tails)."""
    src, dst = synth.make_pair(shape, rate, synth.MIX_ADVERSARIAL, 500 + seed, "cpu")
    a = synth.bits(src).numpy().astype(np.uint16)
    b = synth.bits(dst).numpy().astype(np.uint16)
    payload, _, _ = oracle.compress(a, b)
    nb = -(-a.size // pb.BLOCK)
    assert np.array_equal(payload, pb.payload(a.size, [pb.block_of(a, b, k) for k in range(nb)]))


TABLE_CASES = rules.descriptor_table_cases()


@pytest.mark.parametrize("case", TABLE_CASES, ids=[c.name for c in TABLE_CASES])
def test_descriptor_table_is_checked_before_the_binding(case):
    """A malformed descriptor table is EFORMAT even for a receiver holding
    another version, with weights and version word untouched; only a
    well-formed payload can report EVERSION."""
    w = case.old.copy()
    st, ver = oracle.decompress_v2_inplace(w, case.payload, oracle.checksum(case.new),
                                           rules.OTHER_VERSION)
    assert st == oracle.EFORMAT, oracle.STATUS_NAMES.get(st, st)
    assert ver == rules.OTHER_VERSION and np.array_equal(w, case.old)
    # from the base version the same bytes are still refused
    w = case.old.copy()
    st, ver = oracle.decompress_v2_inplace(w, case.payload, oracle.checksum(case.new),
                                           rules.BASE_VERSION)
    assert st == oracle.EFORMAT and ver == rules.BASE_VERSION and np.array_equal(w, case.old)


def test_a_well_formed_bound_payload_reports_the_version():
    """Control for the cases above: the canonical bound payload of the same
    change gives EVERSION to the other version and OK from the base."""
    case = TABLE_CASES[0]
    p, cs, _ = oracle.compress_v2(case.old, case.new, rules.BASE_VERSION, rules.TARGET_VERSION)
    assert np.array_equal(p, pb.payload(16, [pb.block_of(case.old, case.new, 0)],
                                        (rules.BASE_VERSION, rules.TARGET_VERSION)))
    w = case.old.copy()
    assert oracle.decompress_v2_inplace(w, p, cs, rules.OTHER_VERSION) == \
        (oracle.EVERSION, rules.OTHER_VERSION)
    assert oracle.decompress_v2_inplace(w, p, cs, rules.BASE_VERSION) == \
        (oracle.OK, rules.TARGET_VERSION)
    assert np.array_equal(w, case.new)
