"""Host-side pieces of bench.py that need no GPU: the committed counter
records are found (or rejected) for every workload and call kind the bench
asks for, and a request for more than one GPU exits with a message."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_counter_records_are_looked_up_for_every_workload():
    for workload, record in bench.PROFILE_RECORDS.items():
        for call in ("pa_decode_step", "pa_decode"):
            r = bench.counter_traffic(record, workload, call)
            assert r is None or r > 0
        assert bench.counter_traffic(record, "another_workload", "pa_decode_step") is None
    r = bench.counter_traffic("prefill_llama3_8b", "prefill_llama3_8b")
    assert r is None or r > 0


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "single GPU" in json.loads(p.stdout.strip().splitlines()[-1])["error"]
