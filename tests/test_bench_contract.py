"""bench.py's command-line contract, on the CPU: more than one GPU is refused
with a one-line JSON message and a non-zero exit before anything touches a
device, and the helpers that shape the report behave as documented."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for n in (2, 8):
        p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                           capture_output=True, text=True, timeout=300, cwd=ROOT)
        assert p.returncode != 0
        line = json.loads(p.stdout.strip().splitlines()[-1])
        assert line["n_gpus"] == n and "one GPU" in line["error"]


def test_layer_groups_follow_the_transformer_layers():
    sys.path.insert(0, ROOT)
    import bench
    names = ["embed", "layers.0.q", "layers.0.k", "layers.1.q", "layers.1.k", "norm", "lm_head"]
    assert bench.layer_groups(names, 1) == [1, 2, 2, 1, 1]
    assert bench.layer_groups(names, 2) == [3, 3, 1]
    assert sum(bench.layer_groups(names, 4)) == len(names)


def test_counter_traffic_is_reported_only_for_the_profiled_workload():
    sys.path.insert(0, ROOT)
    import bench
    fields = {}
    with open(bench.TRAFFIC_PROFILE) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    current = fields.get("source_sha256") == bench.kernel_source_hash()
    # the profiled pair: reported while the kernel sources are those profiled
    assert (bench.measured_traffic(int(fields["elements_per_call"])) is not None) == current
    assert bench.measured_traffic(34_226_176_000) is None       # another workload
    assert bench.measured_traffic(1) is None


def test_dirty_chunk_bitmap_of_the_in_place_probe():
    """bench.dirty_chunks marks chunk c (elements 8c .. 8c + 7 of the tensors
    laid end to end) in bit c & 31 of word c >> 5 exactly when old and new
    differ in it, also for chunks that straddle two tensors, and covers whole
    8192-element blocks only."""
    sys.path.insert(0, ROOT)
    import numpy as np
    import torch
    import bench
    g = torch.Generator().manual_seed(11)
    pairs = []
    for m in (8192 * 3 + 5, 3, 100, 8192 * 2 - 3, 8192):
        s = torch.randint(-1000, 1000, (m,), generator=g, dtype=torch.int16)
        d = s.clone()
        d[torch.randint(0, m, (m // 40 + 1,), generator=g)] += 1
        pairs.append((s, d))
    pairs.append((torch.zeros(8192, dtype=torch.int16), torch.zeros(8192, dtype=torch.int16)))
    n = sum(s.numel() for s, _ in pairs)
    words, chunk_pct, line_pct = bench.dirty_chunks(pairs, n, torch.device("cpu"))
    full = n // 8192 * 8192
    assert words.dtype == torch.int32 and words.numel() == full // 8192 * 32
    old = torch.cat([s for s, _ in pairs]).numpy()[:full]
    new = torch.cat([d for _, d in pairs]).numpy()[:full]
    want = (old != new).reshape(-1, 8).any(1)
    w = words.numpy().view(np.uint32)
    got = (w[np.arange(want.size) >> 5] >> (np.arange(want.size) & 31)) & 1
    assert np.array_equal(got.astype(bool), want)
    assert abs(chunk_pct - 100 * want.mean()) < 1e-3
    assert abs(line_pct - 100 * want.reshape(-1, 8).any(1).mean()) < 1e-3
    start = n - 8192   # the all-zero last pair: its chunks are all clean
    assert want[-(-start // 8):].sum() == 0


def test_flat_receiver_lays_the_tensors_end_to_end():
    """bench.flat_receiver: copies of the tensors as views into one buffer,
    back to back in order (so the in-place probe's bitmap of the tensors laid
    end to end describes it), each starting 16-byte aligned; plain clones when
    a size would break that alignment."""
    sys.path.insert(0, ROOT)
    import torch
    import bench
    g = torch.Generator().manual_seed(3)
    ts = [torch.randint(-9, 9, (m,), generator=g, dtype=torch.int16).view(torch.bfloat16)
          for m in (8192, 4096, 24, 8192 * 3)]
    buf, views = bench.flat_receiver(ts, torch.device("cpu"))
    assert buf.numel() == sum(t.numel() for t in ts)
    at = 0
    for t, v in zip(ts, views):
        assert v.dtype == t.dtype and torch.equal(v.view(torch.int16), t.view(torch.int16))
        assert v.data_ptr() == buf.data_ptr() + 2 * at and v.data_ptr() % 16 == buf.data_ptr() % 16
        at += t.numel()
    assert torch.equal(buf, torch.cat([t.view(torch.int16) for t in ts]))
    buf2, views2 = bench.flat_receiver(ts + [torch.zeros(5, dtype=torch.bfloat16)],
                                       torch.device("cpu"))
    assert buf2 is None and len(views2) == 5
    assert all(torch.equal(a.view(torch.int16), b.view(torch.int16))
               for a, b in zip(views2, ts))
