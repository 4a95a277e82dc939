"""Test-side reader of the bf16delta header and descriptor table.

It parses the framing: the 64-byte header, the 32-byte binding block of a
version-2 payload, and the per-block descriptors; `overwrite_record` reads an
overwrite record's positions and values.  The tests use it to check the encoder's bytes
against values worked out independently.  It is written from the format
definition and shares nothing with either implementation.
"""
from __future__ import annotations

import struct

import numpy as np

BLOCK = 8192
HEADER = 64
HEADER_V2 = 96


def header(payload) -> dict:
    b = bytes(np.asarray(payload, dtype=np.uint8)[:HEADER])
    magic = b[:8]
    version, block_elems = struct.unpack_from("<II", b, 8)
    n, n_changed, n_rare, pos_bytes, mant_bytes, rare_bytes = struct.unpack_from("<6Q", b, 16)
    return dict(magic=magic, version=version, block_elems=block_elems, n=n,
                n_changed=n_changed, n_rare=n_rare, pos_bytes=pos_bytes,
                mant_bytes=mant_bytes, rare_bytes=rare_bytes)


def header_bytes(payload) -> int:
    return HEADER_V2 if header(payload)["version"] == 2 else HEADER


def binding(payload) -> dict:
    """The version-2 binding block."""
    b = bytes(np.asarray(payload, dtype=np.uint8)[HEADER:HEADER_V2])
    base, target, flags, res0, res1 = struct.unpack("<QQIIQ", b)
    return dict(base=base, target=target, flags=flags, reserved=(res0, res1))


def descriptors(payload, n: int) -> np.ndarray:
    nb = -(-n // BLOCK)
    h = header_bytes(payload)
    raw = np.asarray(payload, dtype=np.uint8)[h:h + 4 * nb]
    return raw.view("<u4").astype(np.int64)


def split(desc):
    """descriptor -> (c, r, code)"""
    return desc & 0x3FFF, (desc >> 14) & 0x3FFF, desc >> 28


def block_len(n: int, b: int) -> int:
    return min(BLOCK, n - b * BLOCK)


def position_bytes(desc: int, L: int) -> int:
    c, _, code = split(int(desc))
    return -(-L // 8) if code == 15 else -(-(c * code) // 8)


def record_bytes(desc: int, L: int, overwrite: bool = False) -> int:
    c, r, code = split(int(desc))
    mant = 0 if overwrite else -(-(7 * c) // 8)
    return position_bytes(desc, L) + mant + 2 * r


def data_offset(n: int, header_size: int = HEADER) -> int:
    return header_size + 4 * (-(-n // BLOCK))


def _bits(buf: bytes, at: int, width: int) -> int:
    v = 0
    for t in range(width):
        k = at + t
        v |= ((buf[k // 8] >> (k % 8)) & 1) << t
    return v


def overwrite_record(rec: bytes, desc: int, L: int):
    """(positions, values) of an overwrite record, read bit by bit."""
    c, _, code = split(int(desc))
    if code == 15:
        pos = [j for j in range(L) if _bits(rec, j, 1)]
    else:
        pos, p = [], -1
        for j in range(c):
            p += _bits(rec, j * code, code) + 1
            pos.append(p)
    pb = position_bytes(desc, L)
    vals = [rec[pb + 2 * j] | (rec[pb + 2 * j + 1] << 8) for j in range(c)]
    return pos, vals
