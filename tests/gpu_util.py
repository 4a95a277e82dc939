"""Helpers shared by the GPU tests (no method arithmetic here)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from lossless_bf16_weight_xor_amd import synth


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).reshape(-1).cpu().numpy().view(np.uint16)


def to_device(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(a.astype(np.uint16).view(np.int16).copy()).to(device).view(
        torch.bfloat16)


def payload_np(p: torch.Tensor) -> np.ndarray:
    return p.cpu().numpy()


def oracle_of(src: torch.Tensor, dst: torch.Tensor):
    return oracle.compress(to_u16(src), to_u16(dst))


def assert_same_bytes(got: np.ndarray, want: np.ndarray, what: str) -> None:
    if got.shape != want.shape or not np.array_equal(got, want):
        n = min(got.size, want.size)
        diff = np.flatnonzero(got[:n] != want[:n])
        first = int(diff[0]) if diff.size else n
        raise AssertionError(f"{what}: payload differs (len {got.size} vs {want.size}, "
                             f"first differing byte {first})")


def pair(shape, rate, mix, seed, device, layout="uniform"):
    return synth.make_pair(shape, rate, mix, seed, device, layout)
