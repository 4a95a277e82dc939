"""The allocation-free decompress (bf16d_decompress_noalloc) against the
workspace form (bf16d_decompress), through the C ABI (MI355X).

Both calls run the same kernels; the allocation-free one keeps its workspace in
the library's static per-GPU scratch.  Each case applies the same payloads
to two copies of the old weights, one per entry point, and requires equal
per-job results and bit-identical weights.  Two calls in a row, the second
one smaller, show that what the first call leaves in the scratch does not
leak into the second.  Failures (a wrong checksum, a corrupt record, a
malformed header) must end as in the workspace form.
"""
import ctypes

import numpy as np
import pytest
import torch

import lossless_bf16_weight_xor_amd as bd
from lossless_bf16_weight_xor_amd import _native, synth
from tests.gpu_util import log, to_u16

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _job_array(items):
    jobs = (_native.DecompressJob * len(items))()
    for j, (w, p, cs) in enumerate(items):
        jobs[j] = _native.DecompressJob(w.data_ptr() if w.numel() else 0, w.numel(),
                                        p.data_ptr() if p.numel() else 0, p.numel(),
                                        int(cs) & 0xFFFFFFFFFFFFFFFF)
    return jobs


def _noalloc(items):
    res = torch.empty(len(items) * _native.RESULT_BYTES, dtype=torch.uint8, device=DEV)
    rc = _native.lib().bf16d_decompress_noalloc(
        _job_array(items), len(items), res.data_ptr(),
        torch.cuda.current_stream(DEV).cuda_stream)
    return rc, res


def _results(res, count):
    return bd._results(res, count)


def _workspace_form(items):
    count = len(items)
    n_total = sum(w.numel() for w, _, _ in items)
    ws_bytes = _native.lib().bf16d_workspace_bytes(n_total, count)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    res = torch.empty(count * _native.RESULT_BYTES, dtype=torch.uint8, device=DEV)
    rc = _native.lib().bf16d_decompress(_job_array(items), count, ws.data_ptr(), ws_bytes,
                                        res.data_ptr(), torch.cuda.current_stream(DEV).cuda_stream)
    assert rc == bd.OK
    return _results(res, count)


def _batch(specs, seed0, bindings=None):
    """(old, new, payload, checksum) per spec (shape, rate); the payloads come
    from the batched compress (version-2 ones with `bindings`)."""
    pairs = [synth.make_pair(sh, rate, synth.MIX_ADVERSARIAL, seed0 + j, DEV)
             for j, (sh, rate) in enumerate(specs)]
    pairs = [(s.reshape(-1), d.reshape(-1)) for s, d in pairs]
    out = bd.compress_batch(pairs, bindings)
    return [(s, d, p.clone(), cs) for (s, d), (p, cs, _) in zip(pairs, out)]


def _compare(cases, what):
    """Apply every case through both entry points; break some jobs first."""
    items_a, items_b = [], []
    for k, (s, d, p, cs) in enumerate(cases):
        if k % 5 == 1:
            cs ^= 0x5A                         # wrong checksum: rolled back
        if k % 5 == 3 and p.numel() > 200:
            p = p.clone()
            p[-1] ^= 0x01                      # a corrupt last record byte
        if k % 7 == 6:
            p = p.clone()
            p[0] ^= 0x01                       # bad magic: nothing touched
        items_a.append((s.clone(), p, cs))
        items_b.append((s.clone(), p, cs))
    log(f"case {what}: {len(cases)} jobs, {sum(c[0].numel() for c in cases)} elements")
    rc, res = _noalloc(items_a)
    assert rc == bd.OK, _native.status_string(rc)
    got = _results(res, len(items_a))
    want = _workspace_form(items_b)
    assert got == want, what
    statuses = [r["status"] for r in got]
    for j, ((wa, _, _), (wb, _, _), (s, d, _, _)) in enumerate(zip(items_a, items_b, cases)):
        assert torch.equal(wa.view(torch.int16), wb.view(torch.int16)), f"{what} job {j}"
        want_w = d if statuses[j] == bd.OK else s
        assert torch.equal(wa.view(torch.int16), want_w.view(torch.int16)), f"{what} job {j}"
    return statuses


def test_two_calls_in_a_row_match_the_workspace_form():
    big = [((4096, 4096), "0.02"), ((11008, 4096), "0.02"), ((4096,), "0.02"),
           ((3 * 8192 + 77,), "0.3"), ((8192,), "0.6"), ((0,), "0"), ((70001,), "1.0"),
           ((2048, 4096), "0.00085"), ((1,), "1.0"), ((5 * 8192 + 5,), "0.05")] * 2
    st1 = _compare(_batch(big, 900), "first call")
    assert {bd.OK, bd.ECHECKSUM, bd.EFORMAT} <= set(st1)
    small = [((8192 + 13,), "0.05"), ((3,), "1.0"), ((1000, 37), "0.2")]
    st2 = _compare(_batch(small, 950), "second call, smaller")
    assert st2[0] == bd.OK and st2[1] == bd.ECHECKSUM


def test_overwrite_payloads_match_the_workspace_form():
    """Version-2 payloads, overwrite and XOR mixed, with the same failures:
    both forms have room for the undo area (the scratch, and the workspace
    bf16d_workspace_bytes sizes), so overwrite jobs are written in place and
    the failing ones restored, with equal results and weights."""
    specs = [((1024, 1024), "0.02"), ((3 * 8192 + 5,), "0.05"), ((4096,), "0.3"),
             ((2 * 8192,), "0.02"), ((777,), "1.0"), ((8192,), "0.01"), ((5000,), "0.1")]
    bindings = [(7, 8, j % 2 == 0) for j in range(len(specs))]
    st = _compare(_batch(specs, 970, bindings), "version-2 payloads")
    assert {bd.OK, bd.ECHECKSUM} <= set(st)


def test_a_batch_larger_than_the_scratch_is_refused_untouched():
    """400,000 empty tensors need more than the 64 MiB scratch for their
    per-job tables: EINVAL, nothing enqueued; a call after it still works."""
    log("case batch larger than the scratch")
    hdr, cs, _ = bd.compress_batch([(torch.empty(0, dtype=torch.bfloat16, device=DEV),) * 2])[0]
    hdr = hdr.clone()
    count = 400_000
    jobs = (_native.DecompressJob * count)()
    for j in range(count):
        jobs[j] = _native.DecompressJob(0, 0, hdr.data_ptr(), hdr.numel(), cs)
    res = torch.full((count * _native.RESULT_BYTES,), 0xEE, dtype=torch.uint8, device=DEV)
    rc = _native.lib().bf16d_decompress_noalloc(jobs, count, res.data_ptr(),
                                                torch.cuda.current_stream(DEV).cuda_stream)
    torch.cuda.synchronize()
    assert rc == bd.EINVAL
    assert bool((res == 0xEE).all()), "results written by a refused call"
    # 4,000 of them fit, and apply (empty tensors: OK)
    rc, res = _noalloc([(torch.empty(0, dtype=torch.bfloat16, device=DEV), hdr, cs)] * 4000)
    assert rc == bd.OK
    assert all(r["status"] == bd.OK for r in _results(res, 4000))
    _compare(_batch([((8192 * 2 + 1,), "0.02")], 970), "after a refused call")


def test_a_whole_7b_shaped_checkpoint_in_one_call():
    """All 291 tensors of the 7B-shaped checkpoint (822,593 blocks) fit the
    scratch in one call, and the result equals the workspace form's."""
    specs = synth.seven_b_specs()
    assert sum(-(-int(np.prod(sp.shape)) // 8192) for sp in specs) == 822_593
    log("case 7B-shaped checkpoint in one allocation-free call")
    pairs = [(s.reshape(-1), d.reshape(-1)) for _, s, d in synth.config2(DEV)]
    out = bd.compress_batch(pairs)
    items_a = [(s.clone(), p, cs) for (s, _), (p, cs, _) in zip(pairs, out)]
    rc, res = _noalloc(items_a)
    assert rc == bd.OK, _native.status_string(rc)
    got = _results(res, len(items_a))
    assert all(r["status"] == bd.OK for r in got)
    for (w, _, _), (_, d) in zip(items_a, pairs):
        assert torch.equal(w.view(torch.int16), d.view(torch.int16))
    del items_a
    items_b = [(s.clone(), p, cs) for (s, _), (p, cs, _) in zip(pairs, out)]
    assert _workspace_form(items_b) == got
