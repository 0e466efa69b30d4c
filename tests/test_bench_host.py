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


def test_profile_figures_follow_the_code_hash(tmp_path, monkeypatch):
    """MFMA utilisation and HBM GB/s are read from the counter summaries only
    while they were taken on the current code; otherwise null and marked stale."""
    sha = bench.kernel_source_hash()
    mf, tf = tmp_path / "mfma.json", tmp_path / "traffic.json"
    mf.write_text(json.dumps({"source_sha256": sha, "kernels": {"bwd_g": {"mfma_util": 0.5, "engine_ghz": 2.0}}}))
    tf.write_text(json.dumps({"source_sha256": sha, "kernels": {"bwd_g": {"bytes_per_launch": 7.0e8}}}))
    monkeypatch.setattr(bench, "MFMA_FILE", str(mf))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    got = bench.profile_figures("bwd_g", 0.35)
    assert got["mfma_util"] == 0.5 and got["engine_ghz"] == 2.0
    assert got["hbm_gbs"] == round(7.0e8 / 0.35e-3 / 1e9, 1) and got["stale"] == []
    assert bench.profile_figures("nothing", 0.35)["mfma_util"] is None
    mf.write_text(json.dumps({"source_sha256": "0" * 64, "kernels": {"bwd_g": {"mfma_util": 0.5}}}))
    got = bench.profile_figures("bwd_g", 0.35)
    assert got["mfma_util"] is None and got["hbm_gbs"] is not None
    assert len(got["stale"]) == 1 and got["stale"][0].startswith("mfma")


def test_counter_summary_ratios(tmp_path):
    """--summarize-counters: per-dispatch averages over two dispatches and the
    cycle ratios (bank-conflict share of LDS cycles, issue waits, L2 hit rate)."""
    rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
    for did in (7, 9):
        for name, v in (("SQ_INSTS_MFMA", 1000), ("SQ_INSTS_VALU", 1500), ("SQ_INSTS_LDS", 300),
                        ("SQ_LDS_BANK_CONFLICT", 10), ("SQ_LDS_IDX_ACTIVE", 100), ("GRBM_GUI_ACTIVE", 8000),
                        ("SQ_WAVE_CYCLES", 400), ("SQ_WAIT_INST_ANY", 40), ("SQ_WAIT_INST_LDS", 4),
                        ("TCC_HIT_sum", 90), ("TCC_MISS_sum", 10)):
            rows.append(f"{did},fkl::k_bwd_g(Params),{name},{v}")
    csv = tmp_path / "c.csv"
    csv.write_text("\n".join(rows) + "\n")
    md = bench.summarize_counters(str(csv), "cmd")
    line = [l for l in md.splitlines() if l.startswith("| k_bwd_g |")]
    assert line[0].startswith("| k_bwd_g | 2 | 8000 | 300 | 1000 | 1500 | 10 | 100 | 40 | 4 | 400 | 90 | 10 |")
    # 10/100 conflicts; 100 LDS cycles over 1000 x 256 CU cycles; 40/400 and
    # 4/400 of wave cycles waiting; 0.3 LDS and 0.5 other VALU per MFMA; 0.9 hits
    assert line[1] == "| k_bwd_g | 0.100 | 0.0 | 10.0 | 1.0 | 0.30 | 0.50 | 0.900 |"
