"""The read-ceiling probe (a measurement aid): argument checks and that it
runs over whole blocks.  It computes nothing the method uses, so there is no
oracle value to compare; the checks are that it accepts what it documents
and refuses the rest."""
import pytest
import torch

import lossless_bf16_weight_xor_amd as bd
from lossless_bf16_weight_xor_amd import _native

pytestmark = pytest.mark.gpu


def test_probe_runs_over_one_and_two_arrays():
    dev = torch.device("cuda:0")
    a = torch.randint(-32768, 32767, (3 * 8192 + 5,), dtype=torch.int16, device=dev)
    b = torch.randint(-32768, 32767, a.shape, dtype=torch.int16, device=dev)
    sink = torch.zeros(1, dtype=torch.int64, device=dev)
    bd.probe_read(a, b, sink=sink)
    bd.probe_read(a, None, sink=sink)
    bd.probe_read(a[:100], None, sink=sink)   # no whole block: nothing launched
    torch.cuda.synchronize()


def test_probe_refuses_bad_arguments():
    dev = torch.device("cuda:0")
    a = torch.zeros(8192 * 2, dtype=torch.int16, device=dev)
    sink = torch.zeros(1, dtype=torch.int64, device=dev)
    L = _native.lib()
    s = torch.cuda.current_stream().cuda_stream
    assert L.bf16d_probe_read(0, 0, 8192, sink.data_ptr(), 1, s) == bd.EINVAL
    assert L.bf16d_probe_read(a.data_ptr(), 0, 8192, 0, 1, s) == bd.EINVAL
    assert L.bf16d_probe_read(a.data_ptr() + 2, 0, 8192, sink.data_ptr(), 1, s) == bd.EINVAL
    assert L.bf16d_probe_read(a.data_ptr(), a.data_ptr() + 8, 8192, sink.data_ptr(), 1,
                              s) == bd.EINVAL
    assert L.bf16d_probe_read(a.data_ptr(), 0, 0, sink.data_ptr(), 1, s) == bd.OK
    with pytest.raises(ValueError):
        bd.probe_read(a, a[:8192], sink=sink)   # b shorter than a
    torch.cuda.synchronize()
