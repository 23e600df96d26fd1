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


def test_timing_stats_reports_mean_median_and_percentiles():
    st = bench.timing_stats([0.001 * k for k in range(1, 101)])   # 1 .. 100 us
    assert st["timed_launches"] == 100
    assert abs(st["mean_us"] - 50.5) < 1e-9 and abs(st["median_us"] - 50.5) < 1e-9
    assert abs(st["p10_us"] - 10.9) < 1e-6 and abs(st["p90_us"] - 90.1) < 1e-6


def test_oracle_sample_rebuilds_the_rows_a_replica_attends():
    """bench's parity check rebuilds sampled sequences from the workload's rows
    (prompt, then the rows of the steps that replica appended); with every step
    it must equal the oracle's decode of the whole pool after those steps, bit
    for bit (the fp64 table walk does not depend on block placement)."""
    import numpy as np
    from paged_kv_cache_65_amd import workloads
    from tests import oracle_side
    for cache in ("", "i8"):
        spec = workloads.custom(seed=81, dtype="bf16", lens=(3, 40, 17, 100), num_q_heads=8, num_kv_heads=2,
                                head_dim=64, decode_steps=5, prefix_len=16, cache=cache)
        wl = workloads.generate(spec)
        ost = oracle_side.build(wl, steps=5)
        mb = oracle_side.max_blocks_for(wl)
        full = oracle_side.decode(wl, ost, mb)
        got = bench.oracle_sample(wl, [0, 2, 3], list(range(5)))
        assert np.array_equal(got, full[[0, 2, 3]]), cache
        # a replica that took every other step attends to those rows only
        part = bench.oracle_sample(wl, [1], [1, 3])
        assert not np.array_equal(part[0], full[1])


def test_wave_trace_summary_reads_the_records():
    # records as the traced build writes them: entry, inputs ready, first block,
    # stream end, exit (100 MHz ticks), XCD, blocks, written flag
    import numpy as np
    rec = np.zeros((6, 8), dtype=np.uint64)
    for w in range(4):
        rec[w] = [1000 + w, 1100 + w, 1500 + w, 9000 + 100 * w, 9050 + 100 * w, w % 2, 10, 1]
    rec[4] = [1200, 1300, 0, 0, 1400, 1, 0, 1]     # a wave without units
    # rec[5] never written (flag 0): ignored
    s = bench.summarize_waves(rec)
    assert s["waves"] == 5 and s["working_waves"] == 4
    assert s["span_us"] == (9350 - 1000) / 100.0
    assert abs(s["first_block_us"]["median"] - 5.015) <= 0.006   # (rounded to 0.01 us)
    assert s["stream_end_us"]["max"] == (9300 - 1000) / 100.0
    assert s["stream_end_median_us_by_xcd"][0] == (9100 - 1000) / 100.0   # waves 0 and 2
    assert s["stream_end_median_us_by_xcd"][1] == (9200 - 1000) / 100.0   # waves 1 and 3
    assert s["stream_end_median_us_by_xcd"][2] is None


def test_warmup_runs_for_both_the_calls_and_the_time_asked():
    calls, syncs = [], []
    n = bench.warm_past_transient(calls.append, 7, seconds=0.05, sync=lambda: syncs.append(1))
    assert n == len(calls) >= 7 and calls == list(range(n))
    assert syncs  # the GPU is synchronized, so the time is GPU time, not queueing
    t = bench.time.perf_counter()
    assert bench.warm_past_transient(lambda i: None, 1000, seconds=0.0, sync=lambda: None) == 1000
    assert bench.time.perf_counter() - t < 5
