"""Host-side logic of bench.py (no GPU): the code hash that keys the committed
traffic figures, and the JSON contract's refusal of more than one GPU."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_tokens_ignore_comments_and_whitespace():
    a = 'int a = 1; // note\n/* block\n comment */ const char* s = "x // kept";\n  int   b;'
    b = 'int a = 1;\nconst char* s = "x // kept"; int b; // other note'
    assert bench._code_tokens(a) == bench._code_tokens(b) == 'int a = 1; const char* s = "x // kept"; int b;'
    assert bench._code_tokens("int a = 1;") != bench._code_tokens("int a = 2;")


def test_traffic_figures_are_used_only_for_the_code_they_were_taken_on():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    got = bench.traffic_for("bwd_grads")
    if t["source_sha256"] == bench.kernel_source_hash():
        assert got == t["kernels"]["bwd_grads"]["bytes_per_launch"] > 0
    else:
        assert got is None
    assert bench.traffic_for("no_such_kernel") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
