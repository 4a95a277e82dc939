"""GPU parity of the remapped apply (bf16d_decompress_remapped): payloads made
from logical tensors land on a reordered physical layout.

The layout of "GPU-accelerated Weight Teleportation", section "Working with
low-precision RL": gate and up projections paired in groups of 64 rows in one
fused buffer.  The expected physical buffer is built on the CPU by pairing the
logical new weights the same way; the payloads themselves are pinned to the
oracle by the other parity tests, and every job's status here must match the
oracle's decoder run on the logical tensors.
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
G = 64   # rows per group


def _paired(gate, up):
    """[2R, C] with rows gate[64g:64g+64], up[64g:64g+64] for each group g."""
    R, C = gate.shape
    out = torch.empty((2 * R, C), dtype=gate.dtype, device=gate.device)
    for g in range(R // G):
        out[2 * G * g: 2 * G * g + G] = gate[G * g: G * (g + 1)]
        out[2 * G * g + G: 2 * G * (g + 1)] = up[G * g: G * (g + 1)]
    return out


def _segments(fused, which, R, C):
    """(first, view) segments of gate (which=0) or up (which=1) in `fused`."""
    flat = fused.reshape(-1)
    return [(G * g * C, flat[(2 * G * g + which * G) * C: (2 * G * g + which * G + G) * C])
            for g in range(R // G)]


@pytest.mark.parametrize("prepared", [True, False])
@pytest.mark.parametrize("R,C", [(512, 128), (256, 4096)])
def test_gate_up_paired_in_groups_of_64(R, C, prepared):
    log(f"case remapped gate/up R={R} C={C} prepared={prepared}")
    (g0, g1) = synth.make_pair((R, C), "0.03", synth.MIX_DEFAULT, 2000 + R, DEV)
    (u0, u1) = synth.make_pair((R, C), "0.03", synth.MIX_DEFAULT, 3000 + R, DEV)
    # an identity job and a ragged two-segment job in the same call
    (x0, x1) = synth.make_pair((70001,), "0.05", synth.MIX_ADVERSARIAL, 4000 + R, DEV)
    (y0, y1) = synth.make_pair((3 * 8192 + 77,), "0.05", synth.MIX_ADVERSARIAL, 5000 + R, DEV)
    out = bd.compress_batch([(g0.reshape(-1), g1.reshape(-1)), (u0.reshape(-1), u1.reshape(-1)),
                             (x0, x1), (y0, y1)])
    fused = _paired(g0, u0)
    want = _paired(g1, u1)
    xw = x0.clone()
    ya = torch.empty(2 * 8192, dtype=torch.bfloat16, device=DEV).copy_(y0[:2 * 8192])
    yb = torch.empty(8192 + 77, dtype=torch.bfloat16, device=DEV).copy_(y0[2 * 8192:])
    items = [((R * C, _segments(fused, 0, R, C)), out[0][0], out[0][1]),
             ((R * C, _segments(fused, 1, R, C)), out[1][0], out[1][1]),
             (xw, out[2][0], out[2][1]),
             ((y0.numel(), [(0, ya), (2 * 8192, yb)]), out[3][0], out[3][1])]
    res = bd.decompress_remapped(items, prepared)
    assert [r["status"] for r in res] == [bd.OK] * 4
    assert torch.equal(fused.view(torch.int16), want.view(torch.int16))
    assert torch.equal(xw.view(torch.int16), x1.view(torch.int16))
    assert torch.equal(torch.cat([ya, yb]).view(torch.int16), y1.view(torch.int16))


@pytest.mark.parametrize("prepared", [True, False])
def test_remapped_failure_leaves_the_physical_layout_old(prepared):
    log(f"case remapped failure prepared={prepared}")
    R, C = 256, 128
    (g0, g1) = synth.make_pair((R, C), "0.03", synth.MIX_DEFAULT, 6000, DEV)
    (u0, u1) = synth.make_pair((R, C), "0.03", synth.MIX_DEFAULT, 6001, DEV)
    out = bd.compress_batch([(g0.reshape(-1), g1.reshape(-1)), (u0.reshape(-1), u1.reshape(-1))])
    fused = _paired(g0, u0)
    old = fused.clone()
    bad_payload = out[1][0].clone()
    bad_payload[-1] ^= 0x20
    items = [((R * C, _segments(fused, 0, R, C)), out[0][0], out[0][1] ^ 1),   # wrong checksum
             ((R * C, _segments(fused, 1, R, C)), bad_payload, out[1][1])]     # bad record
    res = bd.decompress_remapped(items, prepared)
    for j, (src, payload, cs) in enumerate([(g0, out[0][0], out[0][1] ^ 1),
                                             (u0, bad_payload, out[1][1])]):
        w = to_u16(src).copy()
        assert res[j]["status"] == oracle.decompress_inplace(w, payload.cpu().numpy(), cs)
        assert res[j]["status"] != bd.OK
    assert torch.equal(fused.view(torch.int16), old.view(torch.int16))


@pytest.mark.parametrize("prepared", [True, False])
@pytest.mark.parametrize("overwrite", [False, True])
def test_remapped_apply_of_version_2_payloads(overwrite, prepared):
    """Bound payloads through the remapped call (the binding is not checked
    there).  Overwrite records land at their remapped positions: the prepared
    call verifies them first and writes them after; the plain remapped call,
    whose workspace has room for an undo area, writes them in place and
    restores the kept values of a job that fails."""
    log(f"case remapped version-2 overwrite={overwrite} prepared={prepared}")
    R, C = 512, 128
    (g0, g1) = synth.make_pair((R, C), "0.3", synth.MIX_ADVERSARIAL, 6100, DEV)
    (u0, u1) = synth.make_pair((R, C), "0.03", synth.MIX_ADVERSARIAL, 6101, DEV)
    out = bd.compress_batch([(g0.reshape(-1), g1.reshape(-1)), (u0.reshape(-1), u1.reshape(-1))],
                            [(1, 2, overwrite), (1, 2, overwrite)])
    fused = _paired(g0, u0)
    want = _paired(g1, u1)
    items = [((R * C, _segments(fused, 0, R, C)), out[0][0], out[0][1]),
             ((R * C, _segments(fused, 1, R, C)), out[1][0], out[1][1])]
    res = bd.decompress_remapped(items, prepared=prepared)
    assert [r["status"] for r in res] == [bd.OK, bd.OK]
    assert torch.equal(fused.view(torch.int16), want.view(torch.int16))
    # a wrong checksum leaves the fused layout as it was (untouched, or
    # written and then restored)
    before = fused.clone()
    items[0] = (items[0][0], out[0][0], out[0][1] ^ 1)
    res = bd.decompress_remapped(items[:1], prepared=prepared)
    assert res[0]["status"] == bd.ECHECKSUM
    assert torch.equal(fused.view(torch.int16), before.view(torch.int16))


def test_remapped_sparse_overwrite_payloads_in_place_and_restored():
    """Sparse overwrite payloads through the plain remapped call, whose
    workspace (bf16d_workspace_bytes_remapped) leaves room for the undo area:
    they are written in place at their remapped positions.  A job given a
    wrong checksum ends with its physical layout as it was (the kept values
    written back), the other job rebuilt; the same batch then applies."""
    log("case remapped sparse overwrite, undo path")
    R, C = 1024, 256
    (g0, g1) = synth.make_pair((R, C), "0.02", synth.MIX_DEFAULT, 6300, DEV)
    (u0, u1) = synth.make_pair((R, C), "0.02", synth.MIX_DEFAULT, 6301, DEV)
    out = bd.compress_batch([(g0.reshape(-1), g1.reshape(-1)), (u0.reshape(-1), u1.reshape(-1))],
                            [(3, 4, True), (3, 4, True)])
    n = R * C
    payload_total = out[0][0].numel() + out[1][0].numel()
    ws = bd._native.lib().bf16d_workspace_bytes_remapped(2 * n, 2, 2 * (R // 64))
    assert payload_total < ws // 2   # room for the undo area beside the call's layout
    fused = _paired(g0, u0)
    old = fused.clone()
    items = [((n, _segments(fused, 0, R, C)), out[0][0], out[0][1] ^ 1),
             ((n, _segments(fused, 1, R, C)), out[1][0], out[1][1])]
    res = bd.decompress_remapped(items, prepared=False)
    assert [r["status"] for r in res] == [bd.ECHECKSUM, bd.OK]
    want = _paired(g0, u1)   # job 0 restored, job 1 rebuilt
    assert torch.equal(fused.view(torch.int16), want.view(torch.int16))
    fused.copy_(old)
    items[0] = (items[0][0], out[0][0], out[0][1])
    res = bd.decompress_remapped(items, prepared=False)
    assert [r["status"] for r in res] == [bd.OK, bd.OK]
    assert torch.equal(fused.view(torch.int16), _paired(g1, u1).view(torch.int16))


def test_a_prepared_layout_serves_many_steps():
    """One prepare, then steps that alternate the direction (old -> new -> old
    ...) with the same payloads and the other checksum; every step checked.
    A job table that differs from the prepared one is refused."""
    log("case prepared remap over many steps")
    R, C = 1024, 256
    (g0, g1) = synth.make_pair((R, C), "0.02", synth.MIX_DEFAULT, 6200, DEV)
    (u0, u1) = synth.make_pair((R, C), "0.02", synth.MIX_DEFAULT, 6201, DEV)
    (x0, x1) = synth.make_pair((3 * 8192 + 5,), "0.02", synth.MIX_DEFAULT, 6202, DEV)
    pairs = [(g0.reshape(-1), g1.reshape(-1)), (u0.reshape(-1), u1.reshape(-1)), (x0, x1)]
    fwd = bd.compress_batch(pairs)
    back = bd.compress_batch([(d, s) for s, d in pairs])
    fused, xw = _paired(g0, u0), x0.clone()
    items = [((R * C, _segments(fused, 0, R, C)), fwd[0][0], fwd[0][1]),
             ((R * C, _segments(fused, 1, R, C)), fwd[1][0], fwd[1][1]),
             (xw, fwd[2][0], fwd[2][1])]
    batch = bd.RemappedBatch(items, prepared=True)
    want = [(_paired(g0, u0), x0), (_paired(g1, u1), x1)]
    for step in range(6):
        direction = (step + 1) % 2           # after this step: 1 = new, 0 = old
        for j in range(3):
            batch.jobs[j].checksum = (fwd if direction else back)[j][1]
        batch.run()
        assert [r["status"] for r in batch.results()] == [bd.OK] * 3, step
        wf, wx = want[direction]
        assert torch.equal(fused.view(torch.int16), wf.view(torch.int16)), step
        assert torch.equal(xw.view(torch.int16), wx.view(torch.int16)), step
    # another tensor in place of the prepared one: refused, nothing enqueued
    other = x0.clone()
    saved = batch.jobs[2].weights
    batch.jobs[2].weights = other.data_ptr()
    with pytest.raises(RuntimeError):
        batch.run()
    batch.jobs[2].weights = saved
    # a payload that lies inside the prepared weights: refused
    saved_p = batch.jobs[0].payload
    batch.jobs[0].payload = fused.data_ptr() + 4096
    with pytest.raises(RuntimeError):
        batch.run()
    batch.jobs[0].payload = saved_p
    # the refused calls enqueued nothing: the weights are still old
    for j in range(3):
        batch.jobs[j].checksum = fwd[j][1]
    batch.run()
    assert [r["status"] for r in batch.results()] == [bd.OK] * 3
    assert torch.equal(fused.view(torch.int16), want[1][0].view(torch.int16))
    assert torch.equal(xw.view(torch.int16), want[1][1].view(torch.int16))
