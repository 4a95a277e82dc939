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
