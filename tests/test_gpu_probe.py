"""The read-ceiling, in-place floor and write-only probes (measurement aids):
argument checks, that they run over whole blocks, that the in-place probe
leaves its array as it was, and that the write probe writes exactly the
marked chunks.  They compute nothing the method uses, so there is no
oracle value to compare; the checks are that they accept what they document
and refuse the rest."""
import pytest
import torch

import lossless_bf16_weight_xor_amd as bd
from lossless_bf16_weight_xor_amd import _native, probe

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_probe_runs_over_one_and_two_arrays():
    dev = torch.device("cuda:0")
    a = torch.randint(-32768, 32767, (3 * 8192 + 5,), dtype=torch.int16, device=dev)
    b = torch.randint(-32768, 32767, a.shape, dtype=torch.int16, device=dev)
    sink = torch.zeros(1, dtype=torch.int64, device=dev)
    probe.probe_read(a, b, sink=sink)
    probe.probe_read(a, None, sink=sink)
    probe.probe_read(a[:100], None, sink=sink)   # no whole block: nothing launched
    torch.cuda.synchronize()


def test_probe_refuses_bad_arguments():
    dev = torch.device("cuda:0")
    a = torch.zeros(8192 * 2, dtype=torch.int16, device=dev)
    sink = torch.zeros(1, dtype=torch.int64, device=dev)
    L = _native.probe_lib()
    s = torch.cuda.current_stream().cuda_stream
    assert L.bf16d_probe_read(0, 0, 8192, sink.data_ptr(), 1, s) == bd.EINVAL
    assert L.bf16d_probe_read(a.data_ptr(), 0, 8192, 0, 1, s) == bd.EINVAL
    assert L.bf16d_probe_read(a.data_ptr() + 2, 0, 8192, sink.data_ptr(), 1, s) == bd.EINVAL
    assert L.bf16d_probe_read(a.data_ptr(), a.data_ptr() + 8, 8192, sink.data_ptr(), 1,
                              s) == bd.EINVAL
    assert L.bf16d_probe_read(a.data_ptr(), 0, 0, sink.data_ptr(), 1, s) == bd.OK
    with pytest.raises(ValueError):
        probe.probe_read(a, a[:8192], sink=sink)   # b shorter than a
    torch.cuda.synchronize()


def test_inplace_probe_leaves_the_array_as_it_was():
    """The in-place floor probe writes marked chunks back unchanged: after two
    runs (some blocks fully marked, one partly, one not at all) every element
    is what it was, and the sink is untouched (its key is not hit)."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(5)
    w = torch.randint(-32768, 32767, (3 * 8192 + 5,), dtype=torch.int16, device=dev,
                      generator=g)
    before = w.clone()
    dirty = torch.zeros(3 * 32, dtype=torch.int32, device=dev)
    dirty[:32] = torch.randint(-2**31, 2**31 - 1, (32,), dtype=torch.int32, device=dev,
                               generator=g)
    dirty[32:64] = -1   # every chunk of the second block
    sink = torch.full((1,), 7, dtype=torch.int64, device=dev)
    probe.probe_inplace(w, dirty, sink=sink)
    probe.probe_inplace(w, dirty, sink=sink)
    probe.probe_inplace(w[:100], dirty, sink=sink)   # no whole block: nothing launched
    torch.cuda.synchronize()
    assert torch.equal(w, before)
    assert sink.item() == 7


def test_inplace_probe_refuses_bad_arguments():
    dev = torch.device("cuda:0")
    w = torch.zeros(8192 * 2, dtype=torch.int16, device=dev)
    dirty = torch.zeros(64, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int64, device=dev)
    L = _native.probe_lib()
    s = torch.cuda.current_stream().cuda_stream
    pw, pd, ps = w.data_ptr(), dirty.data_ptr(), sink.data_ptr()
    assert L.bf16d_probe_inplace(0, 8192, pd, ps, 1, s) == bd.EINVAL
    assert L.bf16d_probe_inplace(pw, 8192, 0, ps, 1, s) == bd.EINVAL
    assert L.bf16d_probe_inplace(pw, 8192, pd, 0, 1, s) == bd.EINVAL
    assert L.bf16d_probe_inplace(pw + 2, 8192, pd, ps, 1, s) == bd.EINVAL
    assert L.bf16d_probe_inplace(pw, 8192, pd + 2, ps, 1, s) == bd.EINVAL
    assert L.bf16d_probe_inplace(pw, 8192, pd, ps + 4, 1, s) == bd.EINVAL
    assert L.bf16d_probe_inplace(pw, 0, pd, ps, 1, s) == bd.OK
    with pytest.raises(ValueError):
        probe.probe_inplace(w, dirty[:63], sink=sink)   # fewer than 32 words per block
    with pytest.raises(ValueError):
        probe.probe_inplace(w, dirty.view(torch.int16), sink=sink)
    torch.cuda.synchronize()


def test_write_probe_writes_exactly_the_marked_chunks():
    """The write-only probe touches the marked 16-byte chunks of whole blocks
    and nothing else."""
    n = 3 * 8192 + 100
    w = torch.zeros(n, dtype=torch.int16, device=DEV)
    dirty = torch.zeros(32 * 3, dtype=torch.int32, device=DEV)
    marked = [0, 5, 31, 32, 1023, 1024 + 7, 2 * 1024 + 1000]
    for c in marked:
        dirty[c >> 5] |= 1 << (c & 31)
    probe.probe_write(w, dirty)
    torch.cuda.synchronize()
    got = (w.view(-1)[:3 * 8192].view(-1, 8) != 0).any(1).nonzero().flatten().tolist()
    assert got == marked
    assert int((w[3 * 8192:] != 0).sum()) == 0     # the partial last block is not a whole block
    L = _native.probe_lib()
    s = torch.cuda.current_stream().cuda_stream
    assert L.bf16d_probe_write(w.data_ptr() + 2, n, dirty.data_ptr(), s) == bd.EINVAL
    assert L.bf16d_probe_write(w.data_ptr(), n, 0, s) == bd.EINVAL
