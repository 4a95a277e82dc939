"""TEST INFRASTRUCTURE ONLY: ctypes access to the plain CPU oracle.

The oracle (``bf16delta_oracle.c``) is the slow, single-threaded, obviously
correct CPU encoder/decoder of the bf16delta_v1 format.  Only the test suite,
the smoke check and the benchmark's CPU-baseline leg may import this module;
the GPU library and its Python binding never do, and share no code with it.

The method it implements: the delta of two BF16 checkpoints is their XOR
("GPU-accelerated Weight Teleportation", section "Delta update algebra"); each
changed element is classified as mantissa-only or exponent/sign change, the
unchanged ones are dropped and the two kinds are packed into separate streams,
checked on the receiver by a checksum ("Every byte counts: ARCv3 and the case
for cross-region RL", section "Deep dive into ARCv3" and its block-encoding
figure).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libbf16delta_oracle.so")

OK, EINVAL, ECAPACITY, EFORMAT, ECHECKSUM, EVERSION = 0, 1, 2, 3, 4, 7
STATUS_NAMES = {OK: "OK", EINVAL: "EINVAL", ECAPACITY: "ECAPACITY",
                EFORMAT: "EFORMAT", ECHECKSUM: "ECHECKSUM", EVERSION: "EVERSION"}
FLAG_OVERWRITE = 1
HEADER_V2_BYTES = 96


class _RefResult(ctypes.Structure):
    _fields_ = [("payload_bytes", ctypes.c_uint64),
                ("checksum", ctypes.c_uint64),
                ("n_changed", ctypes.c_uint64),
                ("n_rare", ctypes.c_uint64),
                ("n_bitmap_blocks", ctypes.c_uint64)]


def build(force: bool = False) -> str:
    """Compile the oracle with the C compiler (make) if needed."""
    if force or not os.path.exists(_LIB_PATH):
        subprocess.run(["make", "-B", "-C", _HERE], check=True,
                       stdout=subprocess.DEVNULL)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, p = ctypes.c_uint64, ctypes.c_void_p
        lib.bf16d_ref_mix64.argtypes = [u64]
        lib.bf16d_ref_mix64.restype = u64
        lib.bf16d_ref_checksum.argtypes = [p, u64]
        lib.bf16d_ref_checksum.restype = u64
        lib.bf16d_ref_max_payload_bytes.argtypes = [u64]
        lib.bf16d_ref_max_payload_bytes.restype = u64
        lib.bf16d_ref_compress.argtypes = [p, p, u64, p, u64, ctypes.POINTER(_RefResult)]
        lib.bf16d_ref_compress.restype = ctypes.c_int
        lib.bf16d_ref_decompress.argtypes = [p, u64, p, u64, u64]
        lib.bf16d_ref_decompress.restype = ctypes.c_int
        lib.bf16d_ref_compress_v2.argtypes = [p, p, u64, u64, u64, ctypes.c_uint32, p, u64,
                                              ctypes.POINTER(_RefResult)]
        lib.bf16d_ref_compress_v2.restype = ctypes.c_int
        lib.bf16d_ref_decompress_v2.argtypes = [p, u64, p, u64, u64, p]
        lib.bf16d_ref_decompress_v2.restype = ctypes.c_int
        _lib = lib
    return _lib


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected uint16 bit patterns, got {a.dtype}")
    return a.reshape(-1)


def mix64(z: int) -> int:
    return int(_load().bf16d_ref_mix64(z & 0xFFFFFFFFFFFFFFFF))


def checksum(w) -> int:
    w = _u16(w)
    return int(_load().bf16d_ref_checksum(w.ctypes.data, w.size))


def max_payload_bytes(n: int) -> int:
    return int(_load().bf16d_ref_max_payload_bytes(n))


def compress_raw(src, dst, capacity: int | None = None):
    """Returns (status, payload ndarray[uint8] of `capacity` bytes, stats dict)."""
    src, dst = _u16(src), _u16(dst)
    if src.size != dst.size:
        raise ValueError("src and dst differ in length")
    n = src.size
    if capacity is None:
        capacity = max_payload_bytes(n)
    buf = np.zeros(max(capacity, 1), dtype=np.uint8)
    res = _RefResult()
    st = _load().bf16d_ref_compress(src.ctypes.data, dst.ctypes.data, n,
                                    buf.ctypes.data, capacity, ctypes.byref(res))
    stats = {k: int(getattr(res, k)) for k, _ in _RefResult._fields_}
    return int(st), buf[:capacity], stats


def compress(src, dst):
    """Encode src -> dst; returns (payload bytes as ndarray[uint8], checksum, stats)."""
    st, buf, stats = compress_raw(src, dst)
    if st != OK:
        raise RuntimeError(f"oracle compress failed: {STATUS_NAMES.get(st, st)}")
    return buf[:stats["payload_bytes"]].copy(), stats["checksum"], stats


def decompress_inplace(weights: np.ndarray, payload, checksum_value: int) -> int:
    """Apply payload onto `weights` (uint16, modified in place); returns the status."""
    if weights.dtype != np.uint16 or not weights.flags["C_CONTIGUOUS"]:
        raise TypeError("weights must be a C-contiguous uint16 array")
    pay = np.ascontiguousarray(payload, dtype=np.uint8).reshape(-1)
    ptr = pay.ctypes.data if pay.size else None
    return int(_load().bf16d_ref_decompress(weights.ctypes.data, weights.size,
                                            ptr, pay.size,
                                            checksum_value & 0xFFFFFFFFFFFFFFFF))


# ------------------------------------------------------------- version 2 ---

def compress_v2_raw(src, dst, base_version: int, target_version: int, flags: int = 0,
                    capacity: int | None = None):
    """Version-2 encode (binding, and with flags & FLAG_OVERWRITE absolute
    values); returns (status, payload ndarray of `capacity` bytes, stats)."""
    src, dst = _u16(src), _u16(dst)
    if src.size != dst.size:
        raise ValueError("src and dst differ in length")
    n = src.size
    if capacity is None:
        capacity = max_payload_bytes(n) + 32
    buf = np.zeros(max(capacity, 1), dtype=np.uint8)
    res = _RefResult()
    st = _load().bf16d_ref_compress_v2(src.ctypes.data, dst.ctypes.data, n,
                                       base_version & 0xFFFFFFFFFFFFFFFF,
                                       target_version & 0xFFFFFFFFFFFFFFFF, flags,
                                       buf.ctypes.data, capacity, ctypes.byref(res))
    stats = {k: int(getattr(res, k)) for k, _ in _RefResult._fields_}
    return int(st), buf[:capacity], stats


def compress_v2(src, dst, base_version: int, target_version: int, overwrite: bool = False):
    """Returns (payload ndarray[uint8], checksum, stats) of a version-2 payload."""
    st, buf, stats = compress_v2_raw(src, dst, base_version, target_version,
                                     FLAG_OVERWRITE if overwrite else 0)
    if st != OK:
        raise RuntimeError(f"oracle compress_v2 failed: {STATUS_NAMES.get(st, st)}")
    return buf[:stats["payload_bytes"]].copy(), stats["checksum"], stats


def decompress_v2_inplace(weights: np.ndarray, payload, checksum_value: int,
                          version: int | None):
    """Apply a version-1 or -2 payload with the receiver's version word
    (None: no word, the binding is not checked).  Returns (status, version
    word after the call)."""
    if weights.dtype != np.uint16 or not weights.flags["C_CONTIGUOUS"]:
        raise TypeError("weights must be a C-contiguous uint16 array")
    pay = np.ascontiguousarray(payload, dtype=np.uint8).reshape(-1)
    ptr = pay.ctypes.data if pay.size else None
    word = None if version is None else np.array([version & 0xFFFFFFFFFFFFFFFF], np.uint64)
    st = _load().bf16d_ref_decompress_v2(weights.ctypes.data, weights.size, ptr, pay.size,
                                         checksum_value & 0xFFFFFFFFFFFFFFFF,
                                         None if word is None else word.ctypes.data)
    return int(st), (None if word is None else int(word[0]))
