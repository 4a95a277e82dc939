"""ctypes declarations of libbf16delta (include/bf16delta.h), and nothing else.

The library is loaded from this package directory.  torch is imported first so
that the library binds to the HIP runtime torch already uses.  A missing
library is an error: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime the library must share)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbf16delta.so")

OK, EINVAL, ECAPACITY, EFORMAT, ECHECKSUM, EHIP, ECODEC, EVERSION = 0, 1, 2, 3, 4, 5, 6, 7
BIND_OVERWRITE = 1
BLOCK_ELEMS = 8192
HEADER_BYTES = 64
FORMAT_VERSION = 1

EXPORTED = ("bf16d_max_payload_bytes", "bf16d_workspace_bytes",
            "bf16d_compress_workspace_bytes", "bf16d_compress",
            "bf16d_decompress", "bf16d_compress_ex", "bf16d_decompress_ex",
            "bf16d_delta_compress", "bf16d_delta_decompress", "bf16d_decompress_streamed",
            "bf16d_decompress_remapped", "bf16d_workspace_bytes_remapped",
            "bf16d_status_string", "bf16d_format_version", "bf16d_codec_available",
            "bf16d_race_bound", "bf16d_race_compress", "bf16d_race_frame_info",
            "bf16d_race_decompress", "bf16d_compress_bound", "bf16d_decompress_bound",
            "bf16d_decompress_noalloc", "bf16d_decompress_verified", "bf16d_remap_plan_bytes", "bf16d_remap_map_bytes",
            "bf16d_remap_prepare", "bf16d_decompress_remapped_prepared")
# the benchmark's measurement aids, in their own library (bf16delta_probe.h)
PROBE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbf16delta_probe.so")
PROBE_EXPORTED = ("bf16d_probe_read", "bf16d_probe_inplace", "bf16d_probe_write")
NOALLOC_SCRATCH_BYTES = 64 << 20

CODECS = {"stored": 0, "zstd": 1, "lz4": 2, "lz4hc": 3, "zlib": 4, "brotli": 5, "xz": 6}
RACE_FRAME_HEADER = 32


class Result(ctypes.Structure):
    _fields_ = [("status", ctypes.c_int32), ("reserved", ctypes.c_uint32),
                ("payload_bytes", ctypes.c_uint64), ("checksum", ctypes.c_uint64),
                ("n_changed", ctypes.c_uint64), ("n_rare", ctypes.c_uint64),
                ("n_bitmap_blocks", ctypes.c_uint64)]


class CompressJob(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("dst", ctypes.c_void_p), ("n", ctypes.c_uint64),
                ("payload", ctypes.c_void_p), ("capacity", ctypes.c_uint64)]


class DecompressJob(ctypes.Structure):
    _fields_ = [("weights", ctypes.c_void_p), ("n", ctypes.c_uint64),
                ("payload", ctypes.c_void_p), ("payload_bytes", ctypes.c_uint64),
                ("checksum", ctypes.c_uint64)]


class StreamJob(ctypes.Structure):
    _fields_ = [("weights", ctypes.c_void_p), ("n", ctypes.c_uint64),
                ("payload", ctypes.c_void_p), ("payload_bytes", ctypes.c_uint64),
                ("checksum", ctypes.c_uint64)]


class Segment(ctypes.Structure):
    _fields_ = [("first", ctypes.c_uint64), ("count", ctypes.c_uint64), ("dst", ctypes.c_void_p)]


class Remap(ctypes.Structure):
    _fields_ = [("segments", ctypes.POINTER(Segment)), ("count", ctypes.c_uint32)]


class Binding(ctypes.Structure):
    _fields_ = [("base_version", ctypes.c_uint64), ("target_version", ctypes.c_uint64),
                ("flags", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class Codec(ctypes.Structure):
    _fields_ = [("codec", ctypes.c_uint32), ("level", ctypes.c_int32)]


class RaceJob(ctypes.Structure):
    _fields_ = [("in_", ctypes.c_void_p), ("in_bytes", ctypes.c_uint64),
                ("out", ctypes.c_void_p), ("out_capacity", ctypes.c_uint64),
                ("out_bytes", ctypes.c_uint64), ("codec", ctypes.c_uint32),
                ("level", ctypes.c_int32), ("status", ctypes.c_int32),
                ("reserved", ctypes.c_uint32)]


class Events(ctypes.Structure):
    _fields_ = [("before", ctypes.c_void_p), ("after", ctypes.c_void_p)]


RESULT_BYTES = ctypes.sizeof(Result)
assert RESULT_BYTES == 48

_lib = None


class LibraryMissing(RuntimeError):
    pass


def lib():
    """The loaded library; raises LibraryMissing if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryMissing(
                f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        u64, u32, vp, sz = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_size_t
        L.bf16d_max_payload_bytes.argtypes = [u64]
        L.bf16d_max_payload_bytes.restype = u64
        L.bf16d_workspace_bytes.argtypes = [u64, u32]
        L.bf16d_workspace_bytes.restype = sz
        L.bf16d_compress_workspace_bytes.argtypes = [u64, u32, u32]
        L.bf16d_compress_workspace_bytes.restype = sz
        L.bf16d_compress.argtypes = [ctypes.POINTER(CompressJob), u32, vp, sz, vp, vp]
        L.bf16d_compress.restype = ctypes.c_int
        L.bf16d_decompress.argtypes = [ctypes.POINTER(DecompressJob), u32, vp, sz, vp, vp]
        L.bf16d_decompress.restype = ctypes.c_int
        L.bf16d_compress_ex.argtypes = [ctypes.POINTER(CompressJob), u32, vp, sz, vp, vp,
                                        ctypes.POINTER(Events)]
        L.bf16d_compress_ex.restype = ctypes.c_int
        L.bf16d_decompress_ex.argtypes = [ctypes.POINTER(DecompressJob), u32, vp, sz, vp, vp,
                                          ctypes.POINTER(Events)]
        L.bf16d_decompress_ex.restype = ctypes.c_int
        L.bf16d_decompress_streamed.argtypes = [ctypes.POINTER(StreamJob), u32,
                                                ctypes.POINTER(ctypes.c_uint32), u32, vp, sz, u32,
                                                vp, sz, vp, vp, ctypes.POINTER(vp), u32,
                                                ctypes.POINTER(vp), u32]
        L.bf16d_decompress_streamed.restype = ctypes.c_int
        L.bf16d_decompress_remapped.argtypes = [ctypes.POINTER(DecompressJob),
                                                ctypes.POINTER(Remap), u32, vp, sz, vp, vp]
        L.bf16d_decompress_remapped.restype = ctypes.c_int
        L.bf16d_workspace_bytes_remapped.argtypes = [u64, u32, u64]
        L.bf16d_workspace_bytes_remapped.restype = sz
        L.bf16d_delta_compress.argtypes = [vp, vp, u64, vp, u64, vp, sz, vp, vp]
        L.bf16d_delta_compress.restype = ctypes.c_int
        L.bf16d_delta_decompress.argtypes = [vp, u64, vp, u64, u64, vp, sz, vp, vp]
        L.bf16d_delta_decompress.restype = ctypes.c_int
        L.bf16d_status_string.argtypes = [ctypes.c_int]
        L.bf16d_status_string.restype = ctypes.c_char_p
        L.bf16d_format_version.argtypes = []
        L.bf16d_format_version.restype = ctypes.c_int
        L.bf16d_compress_bound.argtypes = [ctypes.POINTER(CompressJob), ctypes.POINTER(Binding),
                                           u32, vp, sz, vp, vp]
        L.bf16d_compress_bound.restype = ctypes.c_int
        L.bf16d_decompress_bound.argtypes = [ctypes.POINTER(DecompressJob), vp, u32, vp, sz, vp,
                                             vp]
        L.bf16d_decompress_bound.restype = ctypes.c_int
        L.bf16d_codec_available.argtypes = [u32]
        L.bf16d_codec_available.restype = ctypes.c_int
        L.bf16d_race_bound.argtypes = [u64]
        L.bf16d_race_bound.restype = u64
        L.bf16d_race_compress.argtypes = [ctypes.POINTER(RaceJob), u32, ctypes.POINTER(Codec),
                                          u32, u32]
        L.bf16d_race_compress.restype = ctypes.c_int
        L.bf16d_race_frame_info.argtypes = [vp, u64, ctypes.POINTER(ctypes.c_uint64),
                                            ctypes.POINTER(ctypes.c_uint32),
                                            ctypes.POINTER(ctypes.c_int32)]
        L.bf16d_race_frame_info.restype = ctypes.c_int
        L.bf16d_race_decompress.argtypes = [ctypes.POINTER(RaceJob), u32, u32]
        L.bf16d_race_decompress.restype = ctypes.c_int
        L.bf16d_decompress_verified.argtypes = [ctypes.POINTER(DecompressJob), u32, vp, sz, vp,
                                                vp, ctypes.POINTER(Events)]
        L.bf16d_decompress_verified.restype = ctypes.c_int
        L.bf16d_remap_plan_bytes.argtypes = [u32, u64]
        L.bf16d_remap_plan_bytes.restype = sz
        L.bf16d_remap_map_bytes.argtypes = [u64, u32]
        L.bf16d_remap_map_bytes.restype = sz
        L.bf16d_remap_prepare.argtypes = [ctypes.POINTER(DecompressJob), ctypes.POINTER(Remap),
                                          u32, vp, sz, vp, sz, vp]
        L.bf16d_remap_prepare.restype = ctypes.c_int
        L.bf16d_decompress_remapped_prepared.argtypes = [ctypes.POINTER(DecompressJob), u32, vp,
                                                         vp, vp, sz, vp, vp]
        L.bf16d_decompress_remapped_prepared.restype = ctypes.c_int
        L.bf16d_decompress_noalloc.argtypes = [ctypes.POINTER(DecompressJob), u32, vp, vp]
        L.bf16d_decompress_noalloc.restype = ctypes.c_int
        _lib = L
    return _lib


_probe_lib = None


def probe_lib():
    """The benchmark's measurement-aid library (bf16delta_probe.h)."""
    global _probe_lib
    if _probe_lib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise LibraryMissing(
                f"{PROBE_LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
        L = ctypes.CDLL(PROBE_LIB_PATH)
        u64, vp = ctypes.c_uint64, ctypes.c_void_p
        L.bf16d_probe_read.argtypes = [vp, vp, u64, vp, u64, vp]
        L.bf16d_probe_read.restype = ctypes.c_int
        L.bf16d_probe_inplace.argtypes = [vp, u64, vp, vp, u64, vp]
        L.bf16d_probe_inplace.restype = ctypes.c_int
        L.bf16d_probe_write.argtypes = [vp, u64, vp, vp]
        L.bf16d_probe_write.restype = ctypes.c_int
        _probe_lib = L
    return _probe_lib


def status_string(code: int) -> str:
    return lib().bf16d_status_string(code).decode()
