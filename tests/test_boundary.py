"""CPU checks of the C-ABI library.

These tests load libbf16delta and check that it exports every function that
include/bf16delta.h declares.  They also exercise the entry points that run
on the host only.  Nothing here launches a kernel.
"""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bf16delta.h")
PROBE_HEADER = os.path.join(ROOT, "include", "bf16delta_probe.h")


@pytest.fixture(scope="module")
def native():
    from lossless_bf16_weight_xor_amd import _native
    if not os.path.exists(_native.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return _native


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bf16d_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    assert "bf16d_compress" in names and "bf16d_decompress" in names
    assert "bf16d_delta_compress" in names and "bf16d_delta_decompress" in names


def test_every_declared_symbol_is_exported(native):
    lib = ctypes.CDLL(native.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(native.EXPORTED) == set(_declared_functions())


def test_the_measurement_aids_live_in_their_own_library(native):
    """The probes are declared in bf16delta_probe.h and exported by
    libbf16delta_probe.so only, not by the product library."""
    probe = ctypes.CDLL(native.PROBE_LIB_PATH)
    names = _declared_functions(PROBE_HEADER)
    assert set(names) == set(native.PROBE_EXPORTED) == {"bf16d_probe_read", "bf16d_probe_inplace",
                                                        "bf16d_probe_write"}
    product = ctypes.CDLL(native.LIB_PATH)
    for name in names:
        assert hasattr(probe, name), name
        assert not hasattr(product, name), name
    assert all(os.path.exists(p) for p in (HEADER, PROBE_HEADER))
    assert set(names).isdisjoint(_declared_functions())


def test_no_kernel_takes_an_address_space_qualified_parameter():
    """A kernel's name must be the same in the host and device passes.  The
    global-memory qualifier is empty in the host pass, so a kernel parameter
    carrying it would give the device kernel a name the host never registers
    (the launch then fails with a missing-symbol abort)."""
    csrc = os.path.join(ROOT, "lossless_bf16_weight_xor_amd", "csrc")
    kernels = 0
    for f in sorted(os.listdir(csrc)):
        if not f.endswith(".hip"):
            continue
        text = re.sub(r"//[^\n]*", "", open(os.path.join(csrc, f)).read())
        for m in re.finditer(r"__global__[^;{]*?\b(\w+)\s*\(([^)]*)\)\s*\{", text):
            kernels += 1
            assert "BF16D_GMEM" not in m.group(2), f"{f}: kernel {m.group(1)}"
    assert kernels >= 10


def test_struct_sizes_match_the_header(native):
    assert ctypes.sizeof(native.Result) == 48
    assert ctypes.sizeof(native.CompressJob) == 40
    assert ctypes.sizeof(native.DecompressJob) == 40


def test_host_only_entry_points(native):
    lib = native.lib()
    assert lib.bf16d_format_version() == 1
    assert native.status_string(native.ECHECKSUM).startswith("ECHECKSUM")
    for n in (0, 1, 7, 8191, 8192, 8193, 3 * 8192 + 5, 10 ** 7 + 3):
        assert lib.bf16d_max_payload_bytes(n) == oracle.max_payload_bytes(n)
    assert lib.bf16d_workspace_bytes(10 ** 9, 300) > lib.bf16d_workspace_bytes(10 ** 6, 3)


def test_invalid_arguments_are_rejected_before_any_gpu_work(native):
    lib = native.lib()
    res = (native.Result * 1)()
    ws = ctypes.create_string_buffer(1 << 16)
    ws_ptr = (ctypes.addressof(ws) + 15) // 16 * 16
    job = native.CompressJob(None, None, 5, None, 0)
    # count == 0, null jobs, null results, null workspace, null src with n > 0
    assert lib.bf16d_compress(ctypes.byref(job), 0, ws_ptr, 1 << 15, ctypes.addressof(res), None) \
        == native.EINVAL
    assert lib.bf16d_compress(None, 1, ws_ptr, 1 << 15, ctypes.addressof(res), None) == native.EINVAL
    assert lib.bf16d_compress(ctypes.byref(job), 1, ws_ptr, 1 << 15, None, None) == native.EINVAL
    assert lib.bf16d_compress(ctypes.byref(job), 1, None, 1 << 15, ctypes.addressof(res), None) \
        == native.EINVAL
    assert lib.bf16d_compress(ctypes.byref(job), 1, ws_ptr, 1 << 15, ctypes.addressof(res), None) \
        == native.EINVAL
    # misaligned src
    job = native.CompressJob(ws_ptr + 2, ws_ptr + 64, 4, ws_ptr + 4096, 128)
    assert lib.bf16d_compress(ctypes.byref(job), 1, ws_ptr + 8192, 1 << 14,
                              ctypes.addressof(res), None) == native.EINVAL
    # payload overlapping dst
    job = native.CompressJob(ws_ptr, ws_ptr + 64, 16, ws_ptr + 80, 128)
    assert lib.bf16d_compress(ctypes.byref(job), 1, ws_ptr + 8192, 1 << 14,
                              ctypes.addressof(res), None) == native.EINVAL
    # workspace too small
    job = native.CompressJob(ws_ptr, ws_ptr + 64, 16, ws_ptr + 128, 128)
    assert lib.bf16d_compress(ctypes.byref(job), 1, ws_ptr + 8192, 16,
                              ctypes.addressof(res), None) == native.EINVAL
    # decompress: null payload, weights overlapping payload
    djob = native.DecompressJob(ws_ptr, 16, None, 64, 0)
    assert lib.bf16d_decompress(ctypes.byref(djob), 1, ws_ptr + 8192, 1 << 14,
                                ctypes.addressof(res), None) == native.EINVAL
    djob = native.DecompressJob(ws_ptr, 64, ws_ptr + 64, 64, 0)
    assert lib.bf16d_decompress(ctypes.byref(djob), 1, ws_ptr + 8192, 1 << 14,
                                ctypes.addressof(res), None) == native.EINVAL
    # results overlapping a buffer the call writes (otherwise valid calls: the
    # workspace is large enough, so only the overlap refuses them)
    need = lib.bf16d_workspace_bytes(16, 1)
    assert need <= (1 << 16) - 16384
    job = native.CompressJob(ws_ptr, ws_ptr + 64, 16, ws_ptr + 128, 128)
    assert lib.bf16d_compress(ctypes.byref(job), 1, ws_ptr + 8192, need,
                              ws_ptr + 8192 + 64, None) == native.EINVAL      # in the workspace
    assert lib.bf16d_compress(ctypes.byref(job), 1, ws_ptr + 8192, need,
                              ws_ptr + 160, None) == native.EINVAL            # in the payload
    djob = native.DecompressJob(ws_ptr, 16, ws_ptr + 128, 64, 0)
    assert lib.bf16d_decompress(ctypes.byref(djob), 1, ws_ptr + 8192, need,
                                ws_ptr + 16, None) == native.EINVAL          # in the weights


def test_sizes_beyond_two_to_the_62_are_refused(native):
    """A capacity or payload size so large that buffer + size wraps the
    address space would slip past the overlap checks (and compress stages
    records just below `capacity`): such sizes are refused before any GPU
    work.  Without the check these calls would go on to the runtime."""
    lib = native.lib()
    res = (native.Result * 1)()
    ws = ctypes.create_string_buffer(1 << 16)
    ws_ptr = (ctypes.addressof(ws) + 15) // 16 * 16
    need = lib.bf16d_workspace_bytes(16, 1)
    wrap = (1 << 64) - 4096
    job = native.CompressJob(ws_ptr, ws_ptr + 64, 16, ws_ptr + 128, wrap)
    assert lib.bf16d_compress(ctypes.byref(job), 1, ws_ptr + 8192, need,
                              ctypes.addressof(res), None) == native.EINVAL
    job = native.CompressJob(ws_ptr, ws_ptr + 64, 16, ws_ptr + 128, (1 << 62) + 1)
    assert lib.bf16d_compress(ctypes.byref(job), 1, ws_ptr + 8192, need,
                              ctypes.addressof(res), None) == native.EINVAL
    djob = native.DecompressJob(ws_ptr, 16, ws_ptr + 128, wrap, 0)
    assert lib.bf16d_decompress(ctypes.byref(djob), 1, ws_ptr + 8192, need,
                                ctypes.addressof(res), None) == native.EINVAL
    djob = native.DecompressJob(ws_ptr, (1 << 62) + 1, ws_ptr + 128, 64, 0)
    assert lib.bf16d_decompress(ctypes.byref(djob), 1, ws_ptr + 8192, need,
                                ctypes.addressof(res), None) == native.EINVAL


def test_python_api_refuses_cpu_tensors(native):
    import torch
    from lossless_bf16_weight_xor_amd import delta_compress
    src = torch.zeros(16, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        delta_compress(src, src.clone())
    with pytest.raises(ValueError):
        delta_compress(src, src.clone(), compression_format="arc_v3")


def test_streamed_arguments_are_rejected_before_any_gpu_work(native):
    """bf16d_decompress_streamed checks every argument before it enqueues
    anything, so these calls need no GPU (the pointers are never touched)."""
    lib = native.lib()
    assert ctypes.sizeof(native.StreamJob) == 40
    res = (native.Result * 4)()
    payload = ctypes.create_string_buffer(64)
    base = 1 << 40                     # fake 16-byte aligned device addresses
    w0, w1, staging, ws = base, base + (1 << 24), base + (2 << 24), base + (3 << 24)
    WS = 1 << 22
    jobs = (native.StreamJob * 2)(native.StreamJob(w0, 100, ctypes.addressof(payload), 64, 0),
                                  native.StreamJob(w1, 100, ctypes.addressof(payload), 64, 0))

    copies = (ctypes.c_void_p * 2)(None, None)

    lanes = (ctypes.c_void_p * 2)(None, None)

    def call(jobs=jobs, count=2, ends=(1, 2), staging=staging, slot=4096, slots=2, ws=ws,
             ws_bytes=WS, results=ctypes.addressof(res), copy=copies, n_copy=1, lanes=None,
             n_lanes=0):
        ge = (ctypes.c_uint32 * max(1, len(ends)))(*ends) if ends is not None else None
        return lib.bf16d_decompress_streamed(jobs, count, ge, len(ends) if ends else 0, staging,
                                             slot, slots, ws, ws_bytes, results, None, copy,
                                             n_copy, lanes, n_lanes)

    E = native.EINVAL
    assert call(count=0) == E
    assert call(ends=None) == E
    assert call(ends=(1,)) == E                 # groups must end at count
    assert call(ends=(2, 2)) == E               # strictly increasing
    assert call(ends=(1, 2, 2)) == E            # more groups than jobs
    assert call(staging=staging + 8) == E       # staging alignment
    assert call(slot=4100) == E                 # slot size not a multiple of 16
    assert call(slot=48) == E                   # a payload larger than a slot
    assert call(ends=(2,), slot=112) == E       # a group that does not fit (2 x 64 > 112)
    assert call(ws_bytes=16) == E               # workspace too small
    assert call(results=None) == E
    assert call(staging=w0 + 64) == E           # staging overlaps the weights
    assert call(results=ws + 64) == E           # results inside the workspace
    assert call(slots=1) == E                   # a ring needs two slots at least
    assert call(slots=65) == E                  # and at most 64
    assert call(copy=None) == E                 # no copy streams
    assert call(n_copy=0) == E
    assert call(n_copy=9) == E                  # at most 8
    assert call(n_lanes=1) == E                 # a lane count without lanes
    assert call(lanes=lanes, n_lanes=2) == E    # at most one extra lane
    # the third slot of a ring of three overlaps the second job's weights
    assert call(staging=w1 - 2 * 4096 - 16, slots=3) == E
    bad = (native.StreamJob * 2)(native.StreamJob(w0 + 2, 100, ctypes.addressof(payload), 64, 0),
                                 native.StreamJob(w1, 100, ctypes.addressof(payload), 64, 0))
    assert call(jobs=bad) == E                  # weights alignment
    nopay = (native.StreamJob * 2)(native.StreamJob(w0, 100, None, 64, 0),
                                   native.StreamJob(w1, 100, ctypes.addressof(payload), 64, 0))
    assert call(jobs=nopay) == E                # a payload of 64 bytes at NULL


def test_remapped_arguments_are_rejected_before_any_gpu_work(native):
    """bf16d_decompress_remapped checks the segments before it enqueues
    anything; none of these calls reaches the GPU."""
    lib = native.lib()
    assert ctypes.sizeof(native.Segment) == 24
    res = (native.Result * 2)()
    base = 1 << 40
    ws, pay = base, base + (1 << 30)
    WS = int(lib.bf16d_workspace_bytes_remapped(3 * 8192, 1, 4))
    job = native.DecompressJob(None, 3 * 8192, pay, 64, 0)
    A, B = base + (2 << 30), base + (3 << 30)

    def call(segs, job=job, ws_bytes=WS):
        arr = (native.Segment * len(segs))(*[native.Segment(*s) for s in segs])
        remap = (native.Remap * 1)(native.Remap(arr, len(segs)))
        return lib.bf16d_decompress_remapped(ctypes.byref(job), remap, 1, ws, ws_bytes,
                                            ctypes.addressof(res), None)

    E = native.EINVAL
    ok = [(0, 8192, A), (8192, 2 * 8192, B)]
    assert call(ok, ws_bytes=16) == E                                # workspace too small
    assert call(ok, job=native.DecompressJob(A, 3 * 8192, pay, 64, 0)) == E   # weights set too
    assert call([(0, 8192, A), (8192, 8192, B)]) == E                # covers less than n
    assert call([(0, 8192, A), (16384, 8192, B)]) == E               # a gap
    assert call([(8192, 3 * 8192, A)]) == E                          # does not start at 0
    assert call([(0, 100, A), (100, 3 * 8192 - 100, B)]) == E        # not block-aligned
    assert call([(0, 8192, A + 8), (8192, 2 * 8192, B)]) == E        # dst alignment
    assert call([(0, 8192, A), (8192, 2 * 8192, A + 4096)]) == E     # segments overlap
    assert call([(0, 8192, A), (8192, 2 * 8192, None)]) == E         # no destination


def test_bound_arguments_are_rejected_before_any_gpu_work(native):
    lib = native.lib()
    assert ctypes.sizeof(native.Binding) == 24
    ws = ctypes.create_string_buffer(1 << 16)
    jobs = (native.CompressJob * 1)(native.CompressJob(None, None, 0, None, 0))
    res = ctypes.create_string_buffer(64)
    ws_ptr = (ctypes.addressof(ws) + 15) // 16 * 16
    # no bindings array
    assert lib.bf16d_compress_bound(jobs, None, 1, ws_ptr, 1 << 15, ctypes.addressof(res),
                                    None) == native.EINVAL
    for flags, reserved in ((2, 0), (1 | 4, 0), (0, 1)):
        b = (native.Binding * 1)(native.Binding(0, 1, flags, reserved))
        assert lib.bf16d_compress_bound(jobs, b, 1, ws_ptr, 1 << 15, ctypes.addressof(res),
                                        None) == native.EINVAL, (flags, reserved)
    dj = (native.DecompressJob * 1)(native.DecompressJob(None, 0, None, 0, 0))
    # version words must be 8-byte aligned and may not overlap the workspace
    assert lib.bf16d_decompress_bound(dj, ws_ptr + 3, 1, ws_ptr, 1 << 15, ctypes.addressof(res),
                                      None) == native.EINVAL
    assert lib.bf16d_decompress_bound(dj, ws_ptr + 64, 1, ws_ptr, 1 << 15,
                                      ctypes.addressof(res), None) == native.EINVAL
    assert native.status_string(native.EVERSION).startswith("EVERSION")


def test_remap_prepare_refuses_bad_layouts_before_any_gpu_work(native):
    """bf16d_remap_prepare checks the layout before it uploads the block map,
    so these calls need no GPU (the pointers are never touched)."""
    lib = native.lib()
    base = 1 << 40
    n = 4 * 8192
    plan = ctypes.create_string_buffer(int(lib.bf16d_remap_plan_bytes(2, 8)))
    map_bytes = int(lib.bf16d_remap_map_bytes(2 * n, 2))
    mp = base + (1 << 30)

    def segs(*spec):
        arr = (native.Segment * len(spec))(*[native.Segment(f, c, d) for f, c, d in spec])
        return arr, native.Remap(arr, len(spec))

    def call(spec0, spec1, plan_len=len(plan), m=mp, mb=map_bytes):
        a0, r0 = segs(*spec0)
        a1, r1 = segs(*spec1)
        jobs = (native.DecompressJob * 2)(native.DecompressJob(None, n, None, 0, 0),
                                          native.DecompressJob(None, n, None, 0, 0))
        remaps = (native.Remap * 2)(r0, r1)
        return lib.bf16d_remap_prepare(jobs, remaps, 2, plan, plan_len, m, mb, None)

    half = 2 * 8192
    good0 = [(0, half, base), (half, half, base + 4 * half)]
    good1 = [(0, half, base + 2 * half), (half, half, base + 6 * half)]
    E = native.EINVAL
    # segments of the two tensors overlapping each other
    assert call(good0, [(0, half, base + 2 * half), (half, half, base + 4 * half)]) == E
    # not block-aligned, not in order, not covering n
    assert call([(0, 8000, base), (8000, n - 8000, base + 2 * 8192 * 8)], good1) == E
    assert call([(half, half, base), (0, half, base + 4 * half)], good1) == E
    assert call([(0, half, base)], good1) == E
    # a misaligned segment
    assert call([(0, half, base + 2), (half, half, base + 4 * half)], good1) == E
    # short plan, short or misaligned map, the map inside the weights
    assert call(good0, good1, plan_len=16) == E
    assert call(good0, good1, mb=8) == E
    assert call(good0, good1, m=mp + 4) == E
    assert call(good0, good1, m=base + 8) == E
    # the prepared call refuses a plan that was never prepared
    jobs = (native.DecompressJob * 2)()
    ws = base + (1 << 31)
    assert lib.bf16d_decompress_remapped_prepared(jobs, 2, plan, mp, ws, 1 << 20, ws + (1 << 21),
                                                  None) == E
