"""The benchmark's contract: one JSON line with the required fields, one GPU
only, and the HBM-traffic figure reported only for the code it was measured
on.  The CPU tests need no GPU; the GPU test runs a reduced bench (2 layers,
short oracle sample) in a child process and checks the line it prints."""

import importlib.util
import json
import os
import subprocess
import sys

import pytest

from gpu_common import needs_gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", BENCH)
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert r.stdout == ""
    assert "one GPU" in r.stderr


def test_source_hash_sees_code_not_comments(tmp_path, monkeypatch):
    b = _bench_module()
    src = tmp_path / "k.h"
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    monkeypatch.setattr(b, "GEMM_SOURCES", ("k.h",))
    src.write_text("int f(int x) {  // doubles\n    return 2 * x;\n}\n")
    h0 = b.gemm_source_hash()
    src.write_text("// a new note\nint f(int x) {  // twice x\n  return 2 * x;  /* same */\n}\n")
    assert b.gemm_source_hash() == h0
    src.write_text("int f(int x) {  // doubles\n    return 3 * x;\n}\n")
    assert b.gemm_source_hash() != h0


def test_traffic_reported_only_for_the_measured_code(tmp_path, monkeypatch):
    b = _bench_module()
    prof = tmp_path / "traffic.md"
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(prof))
    assert b.measured_traffic()[0] is None                      # no summary
    h = b.gemm_source_hash()
    prof.write_text(f"x\ntraffic_bytes_per_call: 12345\nsource_sha256_16: {h}\n")
    assert b.measured_traffic()[0] == 12345
    prof.write_text("traffic_bytes_per_call: 12345\nsource_sha256_16: 0000000000000000\n")
    value, why = b.measured_traffic()
    assert value is None and "changed" in why


@pytest.mark.gpu
@needs_gpu
def test_reduced_bench_prints_the_contract_line():
    cmd = [sys.executable, BENCH, "--steps", "2", "--warmup", "1", "--layers", "2",
           "--load-reps", "1", "--no-sweep", "--no-formats", "--no-xf32", "--mmq-steps", "0",
           "--grouped-steps", "0", "--fused-steps", "1", "--cpu-rows", "64", "--cpu-layers", "1"]
    print("case: reduced bench.py run", flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for k, t in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int),
                 ("steps", int), ("warmup", int), ("ms_per_step", float),
                 ("higher_is_better", bool), ("scaling", str), ("dtype", str),
                 ("data", str), ("config", dict), ("roofline", dict), ("cpu_baseline", dict)):
        assert isinstance(d[k], t), k
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["vs_baseline"] is None
    assert d["config"]["workload"] and d["config"]["layers"] == 2
    assert abs(d["value"] - d["config"]["M"] / (d["ms_per_step"] / 1e3)) < 1e-3 * d["value"]
    rl = d["roofline"]
    assert rl["bound"] == "mfma" and rl["unit"] == "TFLOP/s" and rl["peak"] == 2500.0
    assert 0 < rl["frac"] < 1 and abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    assert rl["traffic"] is None or rl["traffic"] > rl["algorithmic_bytes_per_call"]
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    assert cpu["dequant_parallel_gbs"] > 0 and cpu["dequant_parallel_procs"] >= 1
    fc = d["forward_check"]
    assert fc["pass"] and fc["cache_bit_exact"] and fc["gemms"] == 4
    assert fc["outputs_checked"] == 4 * 64 * 256
    assert d["config"]["gemms_per_step"] == 4 * 2 and d["config"]["products_per_step"] == 7 * 2
    assert d["forward_196"]["ms_per_step"] > 0
    dq = d["dequant_roofline"]
    assert dq["hbm_copy_gbs"] > 0 and abs(dq["frac_of_copy"] - dq["achieved"] / dq["hbm_copy_gbs"]) < 1e-3
    assert d["fused"]["expansions_per_s"] > 0
