"""Host-side parts of the benchmark's output contract, checked without a GPU:
more than one GPU is refused with a message (the path is measured on one
GPU; the batch would shard as data parallelism over sequences), and the HBM
byte counts that the JSON line reports as `traffic` come from committed
rocprofv3 summaries whose recorded source hash matches the kernel sources
they were taken on, so a kernel edited after its counters were taken shows
up here instead of as a silently stale figure."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


@pytest.mark.parametrize("key", sorted(bench.TRAFFIC))
def test_traffic_summaries_match_their_sources(key):
    name, files = bench.TRAFFIC[key]
    text = open(os.path.join(ROOT, "profiles", name)).read()
    fields = dict(l.split(": ", 1) for l in text.splitlines() if ": " in l and not l.startswith(("-", "|", "#")))
    assert fields["source_sha256_16"].strip() == bench.source_hash(files), \
        f"profiles/{name} was taken on other sources than these; take its counters again"
    n = bench.profiled_traffic(key)
    assert n is not None and n == int(fields["traffic_bytes_per_launch"]) and n > 0
