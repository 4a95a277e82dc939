"""Hand-built payloads that each break one rule of the decoder.

Every case is a (old, new) pair and a payload built with `payload_build`
from the format definition.  The payload describes the pair's change except
for one deliberately broken rule, and the caller passes the checksum of
`new`.  A decoder that enforces the rule must answer EFORMAT and leave the
weights old; one that skips it would rebuild `new` (status OK), or write
outside the tensor, so every case tells the two apart.

The rules (the format's canonical-record and bounds rules, which make the
payload a function of the change mask; the receiver must never leave an
update half-applied, NeMo-DCR summary, "Results and significance"):
- a gap list is used only when it is no larger than the bitmap;
- a bitmap's pad bits (past the block's last element) are zero;
- a bitmap has exactly c bits set;
- gap-list positions stay inside the block (full blocks and the short last
  block of a tensor; sparse and dense blocks);
- the number of zero mantissa fields (escapes) is exactly r.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from tests import payload_build as pb

BLOCK = pb.BLOCK
BASE = 0x3F80        # 1.0: any base works, the rules are about the mask


@dataclass
class Case:
    name: str
    old: np.ndarray
    new: np.ndarray
    payload: np.ndarray
    at_descriptor: bool    # caught by the descriptor check (nothing touched)


def _pair(n, changes):
    old = np.full(n, BASE, np.uint16)
    new = old.copy()
    for p, x in changes.items():
        if p < n:
            new[p] ^= x
    return old, new


def _blocks(old, new, **override):
    """Canonical records of every block, with block b replaced by
    override[f"b{b}"] = (desc, record)."""
    nb = -(-old.size // BLOCK)
    return [override.get(f"b{b}", pb.block_of(old, new, b)) for b in range(nb)]


def gap_list_where_bitmap_is_smaller():
    out = []
    # 16 elements, changes at 0..7 and 10: gaps 0 x8 then 2 -> w = 2, 18 bits
    # = 3 bytes against a 2-byte bitmap, so the bitmap is canonical
    pos = list(range(8)) + [10]
    old, new = _pair(16, {p: 1 for p in pos})
    assert pb.block_of(old, new, 0)[0] >> 28 == pb.BITMAP
    rec = pb.record(pos, [1] * len(pos), 16, mode="delta")
    out.append(Case("gap list where the bitmap is smaller (16 elements)", old, new,
                    pb.payload(16, [rec]), True))
    # a whole block with about 25 % changes
    rng = np.random.default_rng(5)
    pos = sorted(int(p) for p in rng.choice(BLOCK, 2100, replace=False))
    xs = [int(v) for v in rng.integers(1, 128, len(pos))]
    old, new = _pair(BLOCK, dict(zip(pos, xs)))
    assert pb.block_of(old, new, 0)[0] >> 28 == pb.BITMAP
    rec = pb.record(pos, xs, BLOCK, mode="delta")
    out.append(Case("gap list where the bitmap is smaller (whole block)", old, new,
                    pb.payload(BLOCK, [rec]), True))
    return out


def _set_bit(rec: bytes, k: int, v: int) -> bytes:
    b = bytearray(rec)
    if v:
        b[k // 8] |= 1 << (k % 8)
    else:
        b[k // 8] &= ~(1 << (k % 8)) & 0xFF
    return bytes(b)


def bitmap_pad_bits():
    out = []
    pos = list(range(8)) + [10]
    # a 13-element tensor: the bitmap has 3 pad bits (13, 14, 15)
    old, new = _pair(13, {p: 1 for p in pos})
    desc, rec = pb.block_of(old, new, 0)
    assert desc >> 28 == pb.BITMAP and len(rec) == 2 + 8
    for k in (13, 15):
        out.append(Case(f"bitmap pad bit {k} set (13 elements)", old, new,
                        pb.payload(13, [(desc, _set_bit(rec, k, 1))]), False))
    # the short bitmap block after a whole block that is applied first and
    # must be rolled back
    n = BLOCK + 13
    ch = {p: 1 for p in range(0, BLOCK, 97)}
    ch.update({BLOCK + p: 1 for p in pos})
    old, new = _pair(n, ch)
    desc, rec = pb.block_of(old, new, 1)
    assert desc >> 28 == pb.BITMAP
    out.append(Case("bitmap pad bit set in the last block", old, new,
                    pb.payload(n, _blocks(old, new, b1=(desc, _set_bit(rec, 14, 1)))), False))
    return out


def bitmap_popcount():
    out = []
    pos = list(range(8)) + [10]
    old, new = _pair(16, {p: 1 for p in pos})
    desc, rec = pb.block_of(old, new, 0)
    assert desc >> 28 == pb.BITMAP
    # one bit more than c past the last change (the first c positions are the
    # true ones), one more before it, and one less
    for what, k, v in (("extra bit after the last change", 12, 1),
                       ("extra bit among the changes", 9, 1),
                       ("missing bit", 10, 0)):
        out.append(Case(f"bitmap popcount != c: {what}", old, new,
                        pb.payload(16, [(desc, _set_bit(rec, k, v))]), False))
    # a whole block
    rng = np.random.default_rng(6)
    pos = sorted(int(p) for p in rng.choice(BLOCK - 64, 2100, replace=False))
    old, new = _pair(BLOCK, {p: 0x0002 for p in pos})
    desc, rec = pb.block_of(old, new, 0)
    assert desc >> 28 == pb.BITMAP
    out.append(Case("bitmap popcount != c: extra bit (whole block)", old, new,
                    pb.payload(BLOCK, [(desc, _set_bit(rec, BLOCK - 3, 1))]), False))
    return out


def gap_positions_past_the_block():
    out = []
    # block 0 of two lists a position 4 past its end, i.e. element 4 of block
    # 1, which is where `new` has that change
    n = 2 * BLOCK
    old, new = _pair(n, {8190: 1, BLOCK + 4: 1})
    rec = pb.record([8190, BLOCK + 4], [1, 1], BLOCK)
    assert rec[0] >> 28 == 13
    out.append(Case("gap list past a whole block (sparse)", old, new,
                    pb.payload(n, [rec, pb.empty_block()]), False))
    # a dense gap list (more than 1024 changes): 1,100 gaps of 7
    pos = [8 * j + 7 for j in range(1100)]
    old, new = _pair(n, {p: 1 for p in pos})
    rec = pb.record(pos, [1] * len(pos), BLOCK)
    assert rec[0] >> 28 == 3
    out.append(Case("gap list past a whole block (dense)", old, new,
                    pb.payload(n, [rec, pb.empty_block()]), False))
    # the short last block of a tensor: positions past the tensor's end
    n = BLOCK + 100
    old, new = _pair(n, {BLOCK + 50: 1})
    rec = pb.record([50, 111], [1, 1], 100)
    assert rec[0] >> 28 == 6
    out.append(Case("gap list past the end of the tensor (sparse)", old, new,
                    pb.payload(n, [pb.empty_block(), rec]), False))
    n = BLOCK + 5000
    pos = [5 * j + 4 for j in range(1100)]
    old, new = _pair(n, {BLOCK + p: 1 for p in pos})
    rec = pb.record(pos, [1] * len(pos), 5000)
    assert rec[0] >> 28 == 3 and pos[-1] >= 5000
    out.append(Case("gap list past the end of the tensor (dense)", old, new,
                    pb.payload(n, [pb.empty_block(), rec]), False))
    return out


def escape_count():
    out = []
    old, new = _pair(16, {3: 0x0001})
    # r = 1, but no field escapes; the rare word is there
    desc = 1 | 1 << 14 | 2 << 28
    rec = pb.pack([(3, 2)]) + pb.pack([(1, 7)]) + b"\x00\x80"
    out.append(Case("escapes < r", old, new, pb.payload(16, [(desc, rec)]), False))
    # r = 2, one escape
    old, new = _pair(16, {3: 0x8000, 5: 0x0001})
    desc = 2 | 2 << 14 | 2 << 28
    rec = pb.pack([(3, 2), (1, 2)]) + pb.pack([(0, 7), (1, 7)]) + b"\x00\x80\x00\x80"
    out.append(Case("escapes < r (one rare word unused)", old, new,
                    pb.payload(16, [(desc, rec)]), False))
    # r = 0, one escape
    desc = 2 | 0 << 14 | 2 << 28
    rec = pb.pack([(3, 2), (1, 2)]) + pb.pack([(0, 7), (1, 7)])
    out.append(Case("escapes > r", old, new, pb.payload(16, [(desc, rec)]), False))
    # a dense gap list (general decoder) whose last rare word is unused
    pos = list(range(0, 2 * 1100, 2))
    xs = [0x8000 if j % 10 == 0 else 0x0003 for j in range(len(pos))]
    old, new = _pair(BLOCK, dict(zip(pos, xs)))
    desc, rec = pb.block_of(old, new, 0)
    r = (desc >> 14) & 0x3FFF
    desc2 = (desc & ~(0x3FFF << 14)) | (r + 1) << 14
    out.append(Case("escapes < r (dense gap list)", old, new,
                    pb.payload(BLOCK, [(desc2, rec + b"\x00\x80")]), False))
    return out


@dataclass
class TableCase:
    """A descriptor that breaks a rule of the descriptor table, in a
    version-2 payload bound to base BASE_VERSION.  The table is checked
    before the binding, so a receiver holding another version must still get
    EFORMAT (not EVERSION) with weights and version word untouched.  Each of
    these descriptors would also fail a later block-level rule, which gives
    the same weights; the order of the two answers is what tells them apart."""
    name: str
    old: np.ndarray
    new: np.ndarray
    payload: np.ndarray


BASE_VERSION, TARGET_VERSION, OTHER_VERSION = 5, 6, 4


def descriptor_table_cases():
    out = []
    old, new = _pair(16, {3: 0x0001})
    bind = (BASE_VERSION, TARGET_VERSION)
    # code 14 (no meaning) read as a 14-bit gap list: 2 position bytes
    out.append(TableCase("code 14", old, new, pb.payload(
        16, [(1 | 14 << 28, pb.pack([(3, 14)]) + pb.pack([(1, 7)]))], bind)))
    # c = 17 > L = 16, gap list of width 0
    out.append(TableCase("c > L", old, new, pb.payload(
        16, [(17, pb.pack([(1, 7)] * 17))], bind)))
    # r = 2 > c = 1
    out.append(TableCase("r > c", old, new, pb.payload(
        16, [(1 | 2 << 14 | 2 << 28, pb.pack([(3, 2)]) + pb.pack([(0, 7)]) + b"\x00\x80" * 2)],
        bind)))
    # a bitmap with no change
    out.append(TableCase("bitmap with c = 0", old, new, pb.payload(
        16, [(15 << 28, b"\x00\x00")], bind)))
    # no change but a non-zero width
    out.append(TableCase("c = 0 with width 3", old, new, pb.payload(16, [(3 << 28, b"")], bind)))
    # a gap list larger than the bitmap (also a block-level rule's concern)
    pos = list(range(8)) + [10]
    old2, new2 = _pair(16, {p: 1 for p in pos})
    out.append(TableCase("gap list larger than the bitmap", old2, new2, pb.payload(
        16, [pb.record(pos, [1] * len(pos), 16, mode="delta")], bind)))
    return out


def all_cases():
    return (gap_list_where_bitmap_is_smaller() + bitmap_pad_bits() + bitmap_popcount() +
            gap_positions_past_the_block() + escape_count())
