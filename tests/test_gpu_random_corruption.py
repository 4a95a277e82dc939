"""Random corruptions of valid payloads, applied on the GPU in one batched call
and by the oracle one by one: every job must end with the oracle's status and
the oracle's weights (new on OK; old, untouched or rolled back, otherwise).

Each payload gets one to three random byte flips anywhere in its bytes
(header, binding block, descriptor table or records), or, for some jobs, a
wrong checksum or no flip at all.  The dedicated tests pin each decoder rule
one at a time; this one applies many combinations of them in a single launch,
where the jobs share the descriptor scan, the plan and the apply grid.

Modes: version-1 XOR payloads through bf16d_decompress and through the
verify-first call; version-2 payloads (overwrite and XOR mixed, overwrite
ones applied in place with the undo log) without and with the receiver's
version words."""
import numpy as np
import pytest
import torch

import lossless_bf16_weight_xor_amd as bd
import oracle
from lossless_bf16_weight_xor_amd import synth
from tests.gpu_util import log, to_u16

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

SPECS = [((8192,), "0.02"), ((3 * 8192 + 5,), "0.05"), ((4096,), "0.3"), ((700,), "1.0"),
         ((2 * 8192,), "0.6"), ((64, 1000), "0.01"), ((8191,), "0.15"), ((16384 + 1,), "0.00085"),
         ((5000,), "0.25"), ((12345,), "0.03")]
BASE, TARGET = 5, 6


def _corrupt(payload: np.ndarray, rng: np.random.Generator):
    q = payload.copy()
    for _ in range(int(rng.integers(1, 4))):
        at = int(rng.integers(0, q.size))
        q[at] ^= np.uint8(1 << int(rng.integers(0, 8)))
    return q


@pytest.mark.parametrize("mode", ["v1", "v1-verify-first", "v2", "v2-versions"])
@pytest.mark.parametrize("seed", [1, 2])
def test_random_corruptions_match_the_oracle(seed, mode):
    rng = np.random.default_rng(1000 + 10 * seed + len(mode))
    pairs = []
    for j, (shape, rate) in enumerate(SPECS * 6):
        s, d = synth.make_pair(shape, rate, synth.MIX_ADVERSARIAL, 7000 + 100 * seed + j, DEV)
        pairs.append((s.reshape(-1), d.reshape(-1)))
    v2 = mode.startswith("v2")
    bindings = [(BASE, TARGET, j % 2 == 0) for j in range(len(pairs))] if v2 else None
    out = bd.compress_batch(pairs, bindings)
    cases = []
    for j, ((s, d), (p, cs, _)) in enumerate(zip(pairs, out)):
        payload = p.cpu().numpy()
        kind = j % 6
        if kind == 0:
            q, c = payload, cs                      # intact
        elif kind == 1:
            q, c = payload, cs ^ (1 << int(rng.integers(0, 64)))   # wrong checksum
        else:
            q, c = _corrupt(payload, rng), cs     # flipped bytes
        cases.append((s, d, q, c))
    log(f"case random corruptions seed={seed} mode={mode}: {len(cases)} jobs in one call")
    recv = [s.clone() for s, _, _, _ in cases]
    dev_payloads = [torch.from_numpy(q.copy()).to(DEV) for _, _, q, _ in cases]
    items = [(w, p, c) for w, p, (_, _, _, c) in zip(recv, dev_payloads, cases)]
    versions = None
    if mode == "v2-versions":
        # every receiver at the base version, but a few at another one
        words = [BASE if j % 11 else BASE + 7 for j in range(len(cases))]
        versions = torch.tensor(words, dtype=torch.int64, device=DEV)
        batch = bd.DecompressBatch(items, versions=versions)
    else:
        batch = bd.DecompressBatch(items, verify_first=(mode == "v1-verify-first"))
    batch.run()
    res = batch.results()
    got_words = versions.cpu().tolist() if versions is not None else None
    statuses = []
    for j, ((s, d, q, c), w, r) in enumerate(zip(cases, recv, res)):
        ref = to_u16(s).copy()
        if v2:
            word = None if versions is None else (BASE if j % 11 else BASE + 7)
            st, word_after = oracle.decompress_v2_inplace(ref, q, c, word)
            if versions is not None:
                assert got_words[j] == word_after, f"job {j}: version word"
        else:
            st = oracle.decompress_inplace(ref, q, c)
        assert r["status"] == st, f"job {j}: gpu {r['status']} oracle {st}"
        assert np.array_equal(to_u16(w), ref), f"job {j}: weights differ from the oracle's"
        statuses.append(st)
    # the mix covers every outcome
    assert {bd.OK, bd.ECHECKSUM, bd.EFORMAT} <= set(statuses), sorted(set(statuses))
    if mode == "v2-versions":
        assert bd.EVERSION in statuses
