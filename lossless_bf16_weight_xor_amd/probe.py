"""Python side of the benchmark's measurement aids (bf16delta_probe.h,
libbf16delta_probe.so): the read ceiling of the encoder's access pattern and
the in-place floor of the apply pass's traffic.  They are not steps of the
method and are not part of the product library.  Argument marshalling only.
"""
from __future__ import annotations

import torch

from . import _native
from . import _check_rc, _stream, _weights_ptr
from ._native import BLOCK_ELEMS

_PROBE_KEY = 0x9E3779B97F4A7C15   # the probe stores only if its fold equals this


def probe_read(a: torch.Tensor, b: torch.Tensor | None = None,
               sink: torch.Tensor | None = None) -> None:
    """Measurement aid: read a (and b) with the encoder's access pattern and
    nothing else, enqueued on the current stream (`bf16d_probe_read`)."""
    pa = _weights_ptr(a, "a")
    pb = 0
    if b is not None:
        pb = _weights_ptr(b, "b")
        if b.device != a.device or b.numel() < a.numel():
            raise ValueError("b must be on a's device and hold at least as many elements")
    if sink is None:
        sink = torch.empty(1, dtype=torch.int64, device=a.device)
    if sink.device != a.device or sink.dtype != torch.int64 or sink.numel() < 1:
        raise ValueError("sink must be an int64 tensor on a's device")
    _check_rc(_native.probe_lib().bf16d_probe_read(pa, pb, a.numel(), sink.data_ptr(), _PROBE_KEY,
                                             _stream(a.device)), "bf16d_probe_read")


def probe_inplace(w: torch.Tensor, dirty: torch.Tensor, sink: torch.Tensor | None = None) -> None:
    """Measurement aid: read w with the apply pass's access pattern and write
    back, unchanged, each 16-byte chunk that `dirty` marks (one bit per chunk,
    int32 words, `bf16d_probe_inplace`), enqueued on the current stream."""
    pw = _weights_ptr(w, "w")
    if (dirty.device != w.device or dirty.dtype != torch.int32 or not dirty.is_contiguous()
            or dirty.numel() < 32 * (w.numel() // BLOCK_ELEMS)):
        raise ValueError("dirty must be a contiguous int32 tensor on w's device with 32 words "
                         "per 8192-element block")
    if sink is None:
        sink = torch.empty(1, dtype=torch.int64, device=w.device)
    if sink.device != w.device or sink.dtype != torch.int64 or sink.numel() < 1:
        raise ValueError("sink must be an int64 tensor on w's device")
    _check_rc(_native.probe_lib().bf16d_probe_inplace(pw, w.numel(), dirty.data_ptr(), sink.data_ptr(),
                                                _PROBE_KEY, _stream(w.device)),
              "bf16d_probe_inplace")


def probe_write(w: torch.Tensor, dirty: torch.Tensor) -> None:
    """Measurement aid: write (a pattern) each 16-byte chunk of w that `dirty`
    marks, read nothing (`bf16d_probe_write`); w is a scratch array."""
    pw = _weights_ptr(w, "w")
    if (dirty.device != w.device or dirty.dtype != torch.int32 or not dirty.is_contiguous()
            or dirty.numel() < 32 * (w.numel() // BLOCK_ELEMS)):
        raise ValueError("dirty must be a contiguous int32 tensor on w's device with 32 words "
                         "per 8192-element block")
    _check_rc(_native.probe_lib().bf16d_probe_write(pw, w.numel(), dirty.data_ptr(),
                                                    _stream(w.device)), "bf16d_probe_write")
