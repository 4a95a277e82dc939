"""Test-side writer and checker of bf16delta_v1 records.

Written from the format definition, not from either implementation, so that
tests can hand-build payloads that break exactly one rule of the format and
work out, independently of the oracle, what a decoder must make of a record.

Format facts used here ("Every byte counts: ARCv3 and the case for
cross-region RL", section "Deep dive into ARCv3" and its block-encoding
figure, with the project's own framing):
- a block of L elements has c changes at positions p_0 < ... < p_{c-1}, r of
  them touching the exponent or sign (XOR & 0xFF80 != 0);
- the position segment is either c gap fields of w bits (g_0 = p_0,
  g_j = p_j - p_{j-1} - 1, w the bit length of the largest gap) or one bit per
  element; the bitmap is used only when it is strictly smaller in bytes;
- the mantissa segment holds c 7-bit fields, the mantissa XOR, or 0 for an
  exponent/sign change (the escape into the rare segment);
- the rare segment holds r little-endian u16 words, the whole XOR;
- fields are packed LSB-first and each segment is zero-padded to a byte;
- descriptor = c | r << 14 | code << 28 (code = w, or 15 for a bitmap);
- header: magic, version 1, block size, n, and the five totals.
"""
from __future__ import annotations

import struct

import numpy as np

BLOCK = 8192
MAGIC = b"BF16DXOR"
BITMAP = 15


def pack(fields) -> bytes:
    """(value, width) pairs, LSB-first, zero-padded to a whole byte."""
    bits = []
    for v, w in fields:
        bits.extend((v >> t) & 1 for t in range(w))
    out = bytearray((len(bits) + 7) // 8)
    for k, b in enumerate(bits):
        out[k // 8] |= b << (k % 8)
    return bytes(out)


def gaps_of(positions) -> list[int]:
    out, prev = [], -1
    for p in positions:
        out.append(p - prev - 1)
        prev = p
    return out


def record(positions, xors, L, mode=None, width=None):
    """(descriptor, record bytes) of one block.  `mode` "delta" or "bitmap"
    and `width` override the canonical choice, to build non-canonical
    records on purpose."""
    c = len(positions)
    gaps = gaps_of(positions)
    wmin = max(gaps).bit_length() if c else 0
    if mode is None:
        mode = "bitmap" if (L + 7) // 8 < (c * wmin + 7) // 8 else "delta"
    if mode == "bitmap":
        code = BITMAP
        on = set(positions)
        pos_seg = pack([(1 if j in on else 0, 1) for j in range(L)])
    else:
        code = wmin if width is None else width
        pos_seg = pack([(g, code) for g in gaps])
    mant = pack([((x & 0x7F) if (x & 0xFF80) == 0 else 0, 7) for x in xors])
    rare_words = [x for x in xors if x & 0xFF80]
    rare = b"".join(struct.pack("<H", x) for x in rare_words)
    desc = c | len(rare_words) << 14 | code << 28
    return desc, pos_seg + mant + rare


def segment_sizes(desc: int, L: int):
    c, r, code = desc & 0x3FFF, (desc >> 14) & 0x3FFF, desc >> 28
    pb = (L + 7) // 8 if code == BITMAP else (c * code + 7) // 8
    return pb, (7 * c + 7) // 8, 2 * r


def payload(n: int, blocks, binding=None) -> np.ndarray:
    """A version-1 payload from per-block (descriptor, record bytes).  The
    header totals are the sums the descriptors imply, so a payload built
    from one bad record has a consistent header and table.  With `binding`
    = (base_version, target_version), a version-2 XOR payload: the 32-byte
    binding block (base, target, flags 0, zero words) follows the header."""
    nb = -(-n // BLOCK)
    assert len(blocks) == nb
    tot = [0, 0, 0, 0, 0]
    for b, (desc, rec) in enumerate(blocks):
        L = min(BLOCK, n - b * BLOCK)
        pb, mb, rb = segment_sizes(desc, L)
        assert len(rec) == pb + mb + rb, (b, len(rec), pb, mb, rb)
        tot[0] += desc & 0x3FFF
        tot[1] += (desc >> 14) & 0x3FFF
        tot[2] += pb
        tot[3] += mb
        tot[4] += rb
    head = MAGIC + struct.pack("<II", 1 if binding is None else 2, BLOCK) + \
        struct.pack("<6Q", n, *tot)
    if binding is not None:
        head += struct.pack("<QQIIQ", binding[0], binding[1], 0, 0, 0)
    table = b"".join(struct.pack("<I", d) for d, _ in blocks)
    body = b"".join(rec for _, rec in blocks)
    return np.frombuffer(head + table + body, np.uint8).copy()


def empty_block():
    return 0, b""


def block_of(old: np.ndarray, new: np.ndarray, b: int, **kw):
    """The canonical record of block b of a pair (or with the overrides of
    `record`)."""
    lo = b * BLOCK
    x = old[lo:lo + BLOCK] ^ new[lo:lo + BLOCK]
    pos = [int(i) for i in np.flatnonzero(x)]
    return record(pos, [int(x[i]) for i in pos], len(x), **kw)


def _bits(buf: bytes) -> int:
    """The byte string as one LSB-first integer: stream bit k is bit k."""
    return int.from_bytes(bytes(buf), "little")


def _field(big: int, at: int, width: int) -> int:
    return (big >> at) & ((1 << width) - 1)


def check_record(rec: bytes, desc: int, L: int):
    """Decode one record with every rule of the format: returns
    (positions, xor words) if it is canonical, else None."""
    c, r, code = desc & 0x3FFF, (desc >> 14) & 0x3FFF, desc >> 28
    if code == 14 or c > L or r > c:
        return None
    pb, mb, rb = segment_sizes(desc, L)
    if len(rec) != pb + mb + rb:
        return None
    seg = _bits(rec[:pb])
    if code == BITMAP:
        if c == 0:
            return None
        pos = [j for j in range(L) if _field(seg, j, 1)]
        if len(pos) != c or seg >> L:       # pad bits must be zero
            return None
        w = max(gaps_of(pos)).bit_length()
        if not (pb < (c * w + 7) // 8):      # a bitmap only when strictly smaller
            return None
    else:
        if c == 0 and code != 0:
            return None
        if pb > (L + 7) // 8:                # a gap list only when no larger
            return None
        gaps = [_field(seg, j * code, code) for j in range(c)]
        if c and max(gaps).bit_length() != code:
            return None
        pos, p = [], -1
        for g in gaps:
            p += g + 1
            pos.append(p)
        if pos and pos[-1] >= L:
            return None
        if seg >> (c * code):               # pad bits must be zero
            return None
    mant = _bits(rec[pb:pb + mb])
    rare = rec[pb + mb:]
    xs, e = [], 0
    for j in range(c):
        f = _field(mant, 7 * j, 7)
        if f:
            xs.append(f)
            continue
        if e >= r:
            return None
        x = rare[2 * e] | rare[2 * e + 1] << 8
        if (x & 0xFF80) == 0:
            return None
        xs.append(x)
        e += 1
    if e != r or mant >> (7 * c):
        return None
    return pos, xs
