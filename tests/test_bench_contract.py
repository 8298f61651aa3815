"""CPU checks of the benchmark's command-line contract (no GPU needed)."""

import json
import os
import subprocess
import sys

from conftest import ROOT


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_decode_traffic_summary_is_machine_readable():
    sys.path.insert(0, ROOT)
    import bench

    fields = {}
    for line in open(bench.TRAFFIC_FILE):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    assert float(fields["traffic_bytes_per_launch"]) > 1_000_000
    assert len(fields["source_sha256"]) == 64
    json.dumps(bench.committed_traffic())  # a number while the decode sources match, else None
