"""bench.py's command line without a GPU: one GPU only, and the traffic record.

A request for more than one GPU exits with status 2 and a message before any
GPU work; the committed traffic records parse, and one taken on other kernel
source is not reported.
"""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL, WORKLOAD = "pa_balanced_kernel", "llama70b-gqa8-bf16-b64-l128to4096"


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def _fields(path):
    return dict(line.split() for line in open(path) if len(line.split()) == 2 and not line.startswith("#"))


def test_traffic_records_parse():
    recs = [f for f in os.listdir(bench.PROFILES) if f.startswith("traffic_")]
    assert f"traffic_{KERNEL}_{WORKLOAD}.txt" in recs
    for f in recs:
        kv = _fields(os.path.join(bench.PROFILES, f))
        for key in ("kernel_source_sha256_16", "fetch_kib_per_dispatch", "write_kib_per_dispatch",
                    "read_factor", "write_factor", "hbm_bytes_per_dispatch"):
            assert key in kv, (f, key)
        assert float(kv["hbm_bytes_per_dispatch"]) > 0
        assert abs(float(kv["read_factor"]) - 2.0) < 0.01 and abs(float(kv["write_factor"]) - 1.0) < 0.01


def test_a_record_of_other_kernel_source_is_not_reported(tmp_path, monkeypatch):
    name = f"traffic_{KERNEL}_{WORKLOAD}.txt"
    lines = open(os.path.join(bench.PROFILES, name)).read().splitlines()
    for tag, expect_none in (("0000000000000000", True), (bench.kernel_source_hash(), False)):
        out = [f"kernel_source_sha256_16 {tag}" if l.startswith("kernel_source_sha256_16") else l for l in lines]
        (tmp_path / name).write_text("\n".join(out) + "\n")
        monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
        got = bench.read_traffic(KERNEL, WORKLOAD)
        assert (got is None) == expect_none, (tag, got)


def test_step_description_names_the_append_each_cache_takes():
    assert bench.step_description(True, "", 0).endswith("decode partitions (fused K/V append) + merge")
    assert "fused quantized int8 K/V append" in bench.step_description(True, "i8", 0)
    assert "fused quantized fp8 K/V append" in bench.step_description(True, "fp8", 0)
    assert "prefix attention + decode partitions" in bench.step_description(True, "", 32)
    assert "reshape_and_cache_fp8 + decode partitions" in bench.step_description(False, "fp8", 0)
    assert "reshape_and_cache + decode partitions" in bench.step_description(False, "", 0)
