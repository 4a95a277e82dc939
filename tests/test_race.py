"""CPU tests of the codec race (bf16d_race_compress / bf16d_race_decompress).

"Every byte counts: ARCv3 and the case for cross-region RL", section "Deep
dive into ARCv3": general-purpose codecs race over each tensor's output on
the CPU and the smallest output is kept.  The race runs in the library, on
the host, so these tests need no GPU.

What pins it, apart from the library itself:
- every frame body decodes with an independent decoder of its standard
  format (Python's zlib and lzma modules, pyarrow's zstd, LZ4 and Brotli), and
  frames whose bodies those encoders made decode in the library;
- the zlib body equals Python's zlib output byte for byte (same level and
  stream parameters);
- the frame header is parsed field by field here, from its documented layout,
  and its hash is recomputed here in numpy from the documented definition;
- the winner of a race is the smallest of the single-candidate frames, the
  stored frame wins when nothing is smaller, and the choice does not depend on
  the thread count;
- structured payloads from the oracle survive the round trip and still
  rebuild the new weights in the oracle's decoder.
"""
import ctypes
import lzma
import struct
import zlib

import numpy as np
import pytest
import torch

import oracle
import lossless_bf16_weight_xor_amd as bd
from lossless_bf16_weight_xor_amd import _native, synth

pa = pytest.importorskip("pyarrow")

MAGIC = b"BF16DRC1"
CODECS = [("lz4", 1), ("lz4", 8), ("lz4hc", 4), ("zstd", 1), ("zstd", 9), ("zstd", -3),
          ("zlib", 1), ("zlib", 9), ("brotli", 0), ("brotli", 6), ("xz", 0), ("xz", 3)]


@pytest.fixture(scope="module")
def lib():
    import os
    if not os.path.exists(_native.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return _native.lib()


def _payload(shape=(300, 1000), seed=3, frac="0.02", placement="clustered"):
    src, dst = synth.make_pair(shape, frac, synth.MIX_DEFAULT, seed, "cpu", placement)
    a = synth.bits(src).numpy().astype(np.uint16).reshape(-1)
    b = synth.bits(dst).numpy().astype(np.uint16).reshape(-1)
    p, cs, _ = oracle.compress(a, b)
    return a, b, np.ascontiguousarray(p), cs


def _inputs():
    rng = np.random.default_rng(11)
    _, _, p, _ = _payload()
    return {
        "empty": np.zeros(0, np.uint8),
        "one": np.array([7], np.uint8),
        "zeros": np.zeros(1 << 20, np.uint8),
        "random": rng.integers(0, 256, 100_003, dtype=np.uint8),
        "text": np.frombuffer(b"the quick brown fox " * 5000, np.uint8).copy(),
        "payload": p,
    }


def _mix64(z):
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def _raw_hash(data: bytes) -> int:
    """The documented frame hash of the raw bytes, in numpy (wrapping u64)."""
    n = len(data)
    pad = np.zeros(-(-n // 8) * 8, np.uint8)
    pad[:n] = np.frombuffer(data, np.uint8)
    w = pad.view("<u8").astype(np.uint64)
    k1 = np.arange(1, w.size + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        S = int(_mix64(w ^ (k1 * np.uint64(0x9E3779B97F4A7C15))).sum(dtype=np.uint64)) if w.size else 0
        return int(_mix64(np.uint64(S) ^ np.uint64(n)))


def _header(frame: torch.Tensor):
    raw = frame.numpy().tobytes()
    magic, codec, level, n, h = struct.unpack_from("<8sIiQQ", raw, 0)
    assert h == _raw_hash(_independent_decode(codec, raw[32:], n)) if magic == MAGIC else True
    return magic, codec, level, n, raw[32:]


def _independent_decode(codec: int, body: bytes, n: int) -> bytes:
    name = {v: k for k, v in _native.CODECS.items()}[codec]
    if name == "stored":
        return body
    if name == "zlib":
        return zlib.decompress(body)
    if name == "xz":
        return lzma.decompress(body, format=lzma.FORMAT_XZ)
    pa_name = {"zstd": "zstd", "lz4": "lz4_raw", "lz4hc": "lz4_raw", "brotli": "brotli"}[name]
    return pa.Codec(pa_name).decompress(body, decompressed_size=n, asbytes=True)


@pytest.mark.parametrize("codec", CODECS, ids=lambda c: f"{c[0]}{c[1]}")
def test_each_codec_round_trips_and_decodes_independently(lib, codec):
    assert bd.codec_available(codec[0])
    for name, data in _inputs().items():
        f = bd.race_compress([data], [codec], threads=2)[0]
        magic, cid, level, n, body = _header(f.frame)
        assert magic == MAGIC and n == data.size, name
        assert (cid, level) == ((_native.CODECS[f.codec], f.level))
        assert f.codec in ("stored", codec[0]), name
        if f.codec == "stored":
            assert level == 0 and body == data.tobytes(), name
        else:
            assert len(body) < data.size, name   # a codec only wins when smaller
        assert _independent_decode(cid, body, n) == data.tobytes(), name
        back = bd.race_decompress([f], threads=2)[0]
        assert np.array_equal(back.numpy(), data), name


def test_zlib_body_equals_pythons_zlib(lib):
    data = _inputs()["payload"]
    for level in (1, 6, 9):
        f = bd.race_compress([data], [("zlib", level)], threads=1)[0]
        assert f.codec == "zlib"
        assert _header(f.frame)[4] == zlib.compress(data.tobytes(), level)


def _frame(codec: str, level: int, body: bytes, n: int, data: bytes) -> np.ndarray:
    head = struct.pack("<8sIiQQ", MAGIC, _native.CODECS[codec], level, n, _raw_hash(data))
    return np.frombuffer(head + body, np.uint8).copy()


def test_frames_made_by_independent_encoders_decode(lib):
    data = _inputs()["payload"].tobytes()
    n = len(data)
    frames = {
        "zlib": _frame("zlib", 6, zlib.compress(data, 6), n, data),
        "xz": _frame("xz", 1, lzma.compress(data, format=lzma.FORMAT_XZ, preset=1), n, data),
        "zstd": _frame("zstd", 5, pa.Codec("zstd", compression_level=5).compress(
            data, asbytes=True), n, data),
        "lz4": _frame("lz4", 1, pa.Codec("lz4_raw").compress(data, asbytes=True), n, data),
        "brotli": _frame("brotli", 4, pa.Codec("brotli", compression_level=4).compress(
            data, asbytes=True), n, data),
        "stored": _frame("stored", 0, data, n, data),
    }
    outs = bd.race_decompress(list(frames.values()), threads=3)
    for name, out in zip(frames, outs):
        assert out.numpy().tobytes() == data, name


def test_the_smallest_frame_wins_whatever_the_thread_count(lib):
    ins = list(_inputs().values()) + [_payload(seed=s)[2] for s in (4, 5)]
    cands = [("lz4", 1), ("zstd", 3), ("zlib", 6), ("brotli", 5), ("xz", 1)]
    single = [bd.race_compress(ins, [c], threads=4) for c in cands]
    for threads in (1, 3, 16):
        raced = bd.race_compress(ins, cands, threads=threads)
        for j, f in enumerate(raced):
            sizes = [s[j].frame.numel() for s in single]
            assert f.frame.numel() == min(sizes + [32 + ins[j].size])
            if f.codec == "stored":
                assert min(sizes) >= 32 + ins[j].size   # a tie goes to stored
            else:
                k = sizes.index(f.frame.numel())     # ties go to the earlier candidate
                assert (f.codec, f.level) == cands[k]
                assert torch.equal(f.frame, single[k][j].frame)


def test_incompressible_input_is_stored(lib):
    data = _inputs()["random"]
    f = bd.race_compress([data], [("lz4", 1), ("zstd", 19)], threads=2)[0]
    assert f.codec == "stored" and f.frame.numel() == 32 + data.size
    empty = bd.race_compress([np.zeros(0, np.uint8)], [("zstd", 3)])[0]
    assert empty.codec == "stored" and empty.frame.numel() == 32
    assert bd.race_decompress([empty])[0].numel() == 0


def test_no_candidates_stores_every_input(lib):
    ins = list(_inputs().values())
    for f, d in zip(bd.race_compress(ins, [], threads=2), ins):
        assert f.codec == "stored" and _header(f.frame)[4] == d.tobytes()


def test_raced_oracle_payloads_still_rebuild_the_weights(lib):
    cases = [_payload(shape, seed, frac, placement) for shape, seed, frac, placement in
             [((64, 8192), 21, "0.02", "clustered"), ((70001,), 22, "0.3", "uniform"),
              ((8191,), 23, "0.001", "uniform"), ((3, 8192), 24, "1.0", "uniform")]]
    frames = bd.race_compress([p for _, _, p, _ in cases], bd.DEFAULT_RACE, threads=4)
    payloads = bd.race_decompress(frames, threads=4)
    for (a, b, p, cs), q in zip(cases, payloads):
        assert np.array_equal(q.numpy(), p)
        w = a.copy()
        assert oracle.decompress_inplace(w, q.numpy(), cs) == oracle.OK
        assert np.array_equal(w, b)


def test_bad_frames_are_rejected(lib):
    data = _inputs()["payload"]
    good = bd.race_compress([data], [("zstd", 3)])[0].frame.clone()
    cases = {
        "short": good[:20].clone(),
        "magic": good.clone(),
        "codec": good.clone(),
        "level": good.clone(),
        "size": good.clone(),
        "body": good.clone(),
        "truncated body": good[:-7].clone(),
    }
    cases["magic"][0] ^= 1
    cases["codec"][8] = 9
    cases["level"][12:16] = torch.tensor([99, 0, 0, 0], dtype=torch.uint8)
    cases["size"][16] ^= 1
    cases["body"][good.numel() // 2 - 12:good.numel() // 2] ^= 0x5A
    # a stored body decodes whatever its bytes; only the hash catches a flip
    stored = bd.race_compress([data], [])[0].frame.clone()
    stored[32 + 1000] ^= 0x10
    cases["stored body"] = stored
    cases["hash"] = good.clone()
    cases["hash"][24] ^= 1
    for name, f in cases.items():
        with pytest.raises(bd.FormatError):
            bd.race_decompress([f])
            pytest.fail(name)


def test_per_job_statuses_and_argument_errors(lib):
    data = _inputs()["payload"]
    frame = bd.race_compress([data], [("zstd", 3)])[0].frame
    bad = frame.clone()
    bad[0] ^= 1
    small = torch.empty(data.size - 1, dtype=torch.uint8)
    good = torch.empty(data.size, dtype=torch.uint8)
    jobs = (_native.RaceJob * 3)()
    jobs[0] = _native.RaceJob(frame.data_ptr(), frame.numel(), small.data_ptr(), small.numel(),
                              0, 0, 0, -1, 0)
    jobs[1] = _native.RaceJob(bad.data_ptr(), bad.numel(), good.data_ptr(), good.numel(),
                              0, 0, 0, -1, 0)
    jobs[2] = _native.RaceJob(frame.data_ptr(), frame.numel(), good.data_ptr(), good.numel(),
                              0, 0, 0, -1, 0)
    assert lib.bf16d_race_decompress(jobs, 3, 2) == _native.OK
    assert [jobs[j].status for j in range(3)] == [_native.ECAPACITY, _native.EFORMAT,
                                                  _native.OK]
    assert jobs[2].out_bytes == data.size and np.array_equal(good.numpy(), data)
    # compress: argument errors, nothing written
    src = torch.from_numpy(data)
    out = torch.zeros(int(lib.bf16d_race_bound(data.size)), dtype=torch.uint8)
    cj = (_native.RaceJob * 1)(_native.RaceJob(src.data_ptr(), src.numel(), out.data_ptr(),
                                               out.numel() - 1, 0, 0, 0, -1, 0))
    one = (_native.Codec * 1)(_native.Codec(1, 3))
    assert lib.bf16d_race_compress(cj, 1, one, 1, 0) == _native.EINVAL   # output too short
    cj[0].out_capacity = out.numel()
    for codec, level in ((7, 0), (1, 23), (3, 13), (4, 0), (5, 12), (6, 7), (0, 1)):
        one[0] = _native.Codec(codec, level)
        assert lib.bf16d_race_compress(cj, 1, one, 1, 0) == _native.EINVAL, (codec, level)
    assert lib.bf16d_race_compress(cj, 1, one, 1, 2000) == _native.EINVAL   # threads
    assert not out.any()
    with pytest.raises(ValueError):
        bd.race_compress([data], [("snappy", 1)])
    with pytest.raises(TypeError):
        bd.race_compress([data.astype(np.uint16)])
    assert lib.bf16d_race_bound(10) == 42
