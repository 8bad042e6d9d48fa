"""Host-side pieces of bench.py: the one-GPU refusal, the algorithmic work
per head-token, and the source-hash guard on committed counter summaries."""
import hashlib
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus"] == 2


def test_algorithmic_flops_per_head_token():
    # forward: causal scores and P V average C d_k + C d_v, plus the readout and
    # the state update (2 d_k d_v each) and the gate's two dot products
    assert bench.FWD_FLOPS_HT == 128 * 96 + 128 * 192 + 2 * 96 * 192 * 2 + 2 * 96 + 2 * 192 == 111_168
    assert bench.BWD_FLOPS_HT == 271_872
    # bytes per head-token of the forward: q, k (d_k) and v, o (d_v) in bf16
    assert bench.HT_BYTES == 1152


def test_profile_values_follow_the_source_hash(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("int x; // a comment\n\n    int y;   \n")
    # the digest covers the code lines alone: "int x;" and "    int y;"
    digest = hashlib.sha256(b"int x;\n    int y;\n").hexdigest()[:16]
    assert bench.code_digest([str(src)]) == digest
    prof = tmp_path / "p.txt"
    prof.write_text(f"# comment: ignored\nx_executed_flops: 123\nsources_sha256: {digest}\n")
    assert bench._profile_values(str(prof), [str(src)])["x_executed_flops"] == "123"
    # comments and blank lines may change
    src.write_text("// header\nint x; // another comment\n    int y;\n\n")
    assert bench._profile_values(str(prof), [str(src)])["x_executed_flops"] == "123"
    # code may not
    src.write_text("int x;\n    int y = 1;\n")
    assert bench._profile_values(str(prof), [str(src)]) is None
    src.write_text("int x;\n  int y;\n")      # indentation is part of the code line
    assert bench._profile_values(str(prof), [str(src)]) is None
    assert bench._profile_values(str(tmp_path / "missing.txt"), [str(src)]) is None


def test_counter_byte_map_names_real_summaries():
    # every leg's counter bytes come from a committed summary that holds the
    # keys the map names and a source hash (checked or not, the keys must exist)
    for name, (fname, sources, keys) in bench.COUNTER_BYTES.items():
        path = os.path.join(ROOT, "profiles", fname)
        text = open(path).read()
        for k in keys:
            assert f"\n{k}: " in text, (name, k)
        assert "\nsources_sha256: " in text, name
        for f in sources:
            assert os.path.exists(f), f
    assert bench.counter_bytes("no such leg") is None


def test_call_seconds_per_leg_kind():
    assert bench.call_seconds({"us_per_step": 500.0, "ms": 9.0}) == 500e-6
    assert abs(bench.call_seconds({"ms_fwd": 0.07, "ms_bwd": 0.13}) - 0.2e-3) < 1e-12
    assert bench.call_seconds({"ms": 0.05}) == 0.05e-3
