"""Test-side reader of the bf16delta_v1 header and descriptor table.

It parses only the framing: the 64-byte header and the per-block descriptors.
It never decodes records.  The tests use it to check the encoder's bytes
against values worked out independently.  It is written from the format
definition and shares nothing with either implementation.
"""
from __future__ import annotations

import struct

import numpy as np

BLOCK = 8192
HEADER = 64


def header(payload) -> dict:
    b = bytes(np.asarray(payload, dtype=np.uint8)[:HEADER])
    magic = b[:8]
    version, block_elems = struct.unpack_from("<II", b, 8)
    n, n_changed, n_rare, pos_bytes, mant_bytes, rare_bytes = struct.unpack_from("<6Q", b, 16)
    return dict(magic=magic, version=version, block_elems=block_elems, n=n,
                n_changed=n_changed, n_rare=n_rare, pos_bytes=pos_bytes,
                mant_bytes=mant_bytes, rare_bytes=rare_bytes)


def descriptors(payload, n: int) -> np.ndarray:
    nb = -(-n // BLOCK)
    raw = np.asarray(payload, dtype=np.uint8)[HEADER:HEADER + 4 * nb]
    return raw.view("<u4").astype(np.int64)


def split(desc):
    """descriptor -> (c, r, code)"""
    return desc & 0x3FFF, (desc >> 14) & 0x3FFF, desc >> 28


def block_len(n: int, b: int) -> int:
    return min(BLOCK, n - b * BLOCK)


def record_bytes(desc: int, L: int) -> int:
    c, r, code = split(int(desc))
    pos = -(-L // 8) if code == 15 else -(-(c * code) // 8)
    return pos + -(-(7 * c) // 8) + 2 * r


def data_offset(n: int) -> int:
    return HEADER + 4 * (-(-n // BLOCK))
