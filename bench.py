#!/usr/bin/env python3
"""Paged decode attention on one MI355X: decode tokens/s and achieved HBM GB/s.

One step is one pass of the whole hot path over the batch:
  1. host block pool: append one token to every sequence (a new block at each
     16-token boundary; copy-on-write pairs if a shared block is written),
  2. the step's slots, block tables and context lengths go to the device
     (pinned staging; copied on a second stream while the previous step's
     kernels run),
  3. pa_copy_blocks (only when the pool asked for a copy),
  4. pa_decode_partitions: one launch that appends the new tokens' K/V
     through the slots and attends (with --append separate,
     pa_reshape_and_cache runs first instead),
  5. pa_decode_merge: log-sum-exp merge of split contexts.
Steps rotate over --replicas independent pools (own caches, tables, block
placement) so the working set is several times the 256 MB Infinity Cache.

Prints one JSON line.  value = decode tokens/s (one token per sequence per
step) over the timed steps, wall clock between device synchronizations.
roofline = the decode: the attention launch (balanced split or partitions;
  with a shared prefix, the prefix kernel and the split together) and the
  merge launch, from the first dispatch's start to the merge's end, taken
  with HIP events on the dispatches of at least 10 timed steps: algorithmic
  bytes per step / that duration.  roofline.kernel_only is the attention
  launch alone.  max_abs_err compares sampled rows of the last timed step's
  output with the fp64 oracle, which rebuilds those sequences from the
  workload's rows.
cpu_baseline = the fp64 CPU oracle on whole-batch passes of the same workload
  (OpenMP), plus a single-threaded figure on a sample of its sequences.

A workload that is a decode loop (workload 5: 4 x 32768 tokens, 128 steps,
512-token partitions) runs exactly its steps on one pool (its 537 MB per step
is twice the Infinity Cache), after --warmup decode launches without appends,
and adds the whole loop's tokens/s and GB/s.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from paged_kv_cache_65_amd import accounting, workloads  # noqa: E402

METRIC = "paged decode-attention tokens/s + achieved HBM GB/s (% of 8 TB/s peak)"
HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "paged_kv_cache_65_amd", "csrc", "pa_kernels.hip")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from committed rocprofv3
    counter runs, or None when the kernel source changed since they were taken.
    With the counter run's own algorithmic bytes per launch in the record, the
    result is a dict {"hbm": bytes, "algorithmic": bytes}; else just the bytes."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        parts = line.split()
        if len(parts) == 2 and not line.startswith("#"):
            kv[parts[0]] = parts[1]
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        hbm = float(kv["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None
    try:
        return {"hbm": hbm, "algorithmic": float(kv["algorithmic_bytes_per_dispatch"])}
    except (KeyError, ValueError):
        return hbm


def traffic_bytes(rec):
    return None if rec is None else (rec["hbm"] if isinstance(rec, dict) else rec)


def timing_stats(ms) -> dict:
    """mean, median, p10 and p90 in microseconds of launch durations in ms."""
    us = np.asarray(ms, dtype=np.float64) * 1e3
    return {"mean_us": round(float(us.mean()), 2), "median_us": round(float(np.median(us)), 2),
            "p10_us": round(float(np.percentile(us, 10)), 2), "p90_us": round(float(np.percentile(us, 90)), 2),
            "timed_launches": int(us.size)}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------- GPU side
class Hip:
    """The few HIP runtime calls the step loop needs, called directly (streams and
    events of default priority; pinned host -> device copies)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        for name in ("hipStreamCreate", "hipEventCreateWithFlags", "hipEventRecord",
                     "hipStreamWaitEvent", "hipEventSynchronize", "hipMemcpyAsync",
                     "hipDeviceSynchronize", "hipEventElapsedTime"):
            getattr(self.lib, name).restype = ctypes.c_int
        self.lib.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_int, ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def stream(self):
        h = ctypes.c_void_p()
        self._ok(self.lib.hipStreamCreate(ctypes.byref(h)), "hipStreamCreate")
        return h.value

    def event(self, timing=False):
        h = ctypes.c_void_p()
        self._ok(self.lib.hipEventCreateWithFlags(ctypes.byref(h), 0 if timing else 2),
                 "hipEventCreateWithFlags")
        return h.value

    def record(self, ev, stream):
        self._ok(self.lib.hipEventRecord(ev, stream), "hipEventRecord")

    def wait(self, stream, ev):
        self._ok(self.lib.hipStreamWaitEvent(stream, ev, 0), "hipStreamWaitEvent")

    def sync_event(self, ev):
        self._ok(self.lib.hipEventSynchronize(ev), "hipEventSynchronize")

    def h2d(self, dst, src, nbytes, stream):
        self._ok(self.lib.hipMemcpyAsync(dst, src, nbytes, 1, stream), "hipMemcpyAsync")

    def sync_device(self):
        self._ok(self.lib.hipDeviceSynchronize(), "hipDeviceSynchronize")

    def elapsed_ms(self, a, b):
        out = ctypes.c_float()
        self._ok(self.lib.hipEventElapsedTime(ctypes.byref(out), a, b), "hipEventElapsedTime")
        return out.value


@dataclasses.dataclass
class Replica:
    pool: object
    seq_ids: np.ndarray
    k_cache: object
    v_cache: object
    params: object
    out: object
    max_ctx: int
    lens_host: np.ndarray


@dataclasses.dataclass
class Slot:
    """One step descriptor in flight: pinned host staging and its device copy."""
    stage: object          # pinned int32 staging: slots(int64) | lens | tables | cows
    desc: object           # device copy of the staging buffer
    copied: object = None  # copy-stream event: desc holds this slot's step


def stage_layout(S, MB):
    """int32-word offsets of the step descriptor: slots (int64), lens, tables, cow
    pairs; every region starts on a 16-byte boundary."""
    def up(w):
        return (w + 3) // 4 * 4
    lens = up(2 * S)
    tab = up(lens + S)
    cows = up(tab + S * MB)
    return {"slots": 0, "lens": lens, "tables": tab, "cows": cows, "words": up(cows + 2 * S)}


def build_replica(pa, torch, wl, order, k_rows_d, v_rows_d, MB, S, dev):
    spec = wl.spec
    nb = len(order)
    pool = pa.BlockPool(nb, 16, order)
    slots_all = []
    owner = -1
    if spec.prefix_len:
        owner = pool.seq_create()
        s_, _ = pool.seq_append(owner, spec.prefix_len)
        slots_all.append(s_)
    ids = []
    for s in range(S):
        sid = pool.seq_fork(owner) if spec.prefix_len else pool.seq_create()
        ids.append(sid)
        n = int(wl.token_offsets[s + 1] - wl.token_offsets[s])
        s_, cow = pool.seq_append(sid, n)
        assert cow is None  # prefixes are block-aligned in the named workloads
        slots_all.append(s_)
    slots = torch.from_numpy(np.concatenate(slots_all)).to(dev)
    n_elems = nb * spec.num_kv_heads * 16 * spec.head_dim
    if spec.cache in ("i8", "fp8"):
        # byte caches: every tile holds its 16 rows' codes (0x7F unwritten), then their scales (NaN)
        code_t = torch.uint8 if spec.cache == "fp8" else torch.int8
        D = spec.head_dim
        caches = []
        for _ in range(2):
            c = torch.full((nb * spec.num_kv_heads * 16 * (D + 4),), 127, dtype=code_t, device=dev)
            c.view(-1, 16 * (D + 4))[:, 16 * D:].view(torch.float32).fill_(float("nan"))
            caches.append(c)
        kc, vc = caches
        quantize = pa.pa_reshape_and_cache_fp8 if spec.cache == "fp8" else pa.pa_reshape_and_cache_int8
        quantize(k_rows_d, v_rows_d, kc, vc, slots)
    else:
        dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[spec.dtype]
        kc = torch.full((n_elems,), float("nan"), dtype=dt, device=dev)
        vc = torch.full((n_elems,), float("nan"), dtype=dt, device=dev)
        pa.pa_reshape_and_cache(k_rows_d, v_rows_d, kc, vc, slots)
    ids = np.array(ids, dtype=np.int32)
    tab, lens = pool.seq_export(ids, MB)
    return Replica(pool, ids, kc, vc, None, None, int(lens.max()), lens.copy())


def run_gpu(args, wl, loop=False):
    """loop: the workload is a decode loop -- the --warmup launches decode the
    prompt state without appending, then exactly --steps steps append and attend."""
    import torch
    from paged_kv_cache_65_amd import binding as pa
    L = pa.lib()
    spec = wl.spec
    dev = torch.device("cuda:0")
    S, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    K, R = args.steps, args.replicas
    W = 0 if loop else args.warmup          # warmup steps of the step loop (they append too)
    MB = int(-(-(int(wl.prompt_lens.max()) + W + K) // 16))
    dt_code = {"f32": pa.PA_F32, "f16": pa.PA_F16, "bf16": pa.PA_BF16}[spec.dtype]

    def to_dev(a):
        if spec.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    k_rows = np.concatenate([wl.prefix_k, wl.k_tokens]) if spec.prefix_len else wl.k_tokens
    v_rows = np.concatenate([wl.prefix_v, wl.v_tokens]) if spec.prefix_len else wl.v_tokens
    k_rows_d, v_rows_d = to_dev(k_rows), to_dev(v_rows)
    step_k_d, step_v_d = to_dev(wl.step_k), to_dev(wl.step_v)
    q_d = to_dev(wl.q)
    reps = []
    # A pool sized exactly for the prompts (the 7B MHA workload) gets slack blocks
    # for the timed decode steps, at the bottom of the free stack so the
    # workload's own placement is used first.
    grow = int(np.sum(-(-(wl.prompt_lens + W + K) // 16) - (-(-wl.prompt_lens // 16))))
    slack = max(0, grow - (wl.num_blocks - int(np.sum(-(-(wl.prompt_lens - spec.prefix_len) // 16)))
                           - spec.prefix_len // 16))
    nb_pool = wl.num_blocks + slack
    for r in range(R):
        order = wl.free_order if r == 0 else \
            np.random.default_rng(spec.seed * 1000 + r).permutation(wl.num_blocks).astype(np.int32)
        order = np.concatenate([np.arange(wl.num_blocks, nb_pool, dtype=np.int32), order])
        reps.append(build_replica(pa, torch, wl, order, k_rows_d, v_rows_d, MB, S, dev))
        log(f"replica {r} built: {nb_pool} blocks, max context {reps[-1].max_ctx}")
    del k_rows_d, v_rows_d
    out_dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[spec.out_dtype]
    ws_need = 0
    lay = stage_layout(S, MB)
    # Step descriptors travel through a ring of NS staging slots (pinned host
    # buffer + device copy), independent of the R replicas, so the host needs a
    # completion event only every DONE_EVERY steps.
    NS, DONE_EVERY = 32, 16
    slots = [Slot(torch.empty(lay["words"], dtype=torch.int32, pin_memory=True),
                  torch.empty(lay["words"], dtype=torch.int32, device=dev)) for _ in range(NS)]

    def views(slot):
        return (slot.desc[0:2 * S].view(torch.int64), slot.desc[lay["lens"]:lay["lens"] + S],
                slot.desc[lay["tables"]:lay["tables"] + S * MB].view(S, MB))

    # every sequence forks the prefix owner: its blocks lead every table
    shared_prefix = spec.prefix_len // 16 if (spec.prefix_len and not args.no_shared_prefix) else 0
    for rep in reps:
        slots_v, lens_v, tab_v = views(slots[0])
        rep.out = torch.empty((S, Hq, D), dtype=out_dt, device=dev)
        rep.params = pa.make_decode_params(rep.out, q_d, rep.k_cache, rep.v_cache, tab_v, lens_v,
                                           Hkv, rep.max_ctx + W + K, spec.fp32_scale(),
                                           args.partition_tokens, args.kernel,
                                           sliding_window=spec.window,
                                           shared_prefix_blocks=shared_prefix)
        ws_need = max(ws_need, pa.pa_decode_workspace_bytes(rep.params))
        rep.params.max_context_len = rep.max_ctx
        if args.append == "fused":
            rep.params.k_new = step_k_d.data_ptr()
            rep.params.v_new = step_v_d.data_ptr()
            rep.params.slot_mapping = slots_v.data_ptr()
    ws = torch.empty(max(ws_need, 16), dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = ctypes.c_void_p(ws.data_ptr()), ws.numel()
    part_tokens = pa.pa_decode_partition_tokens(reps[0].params)

    hip = Hip()
    # Two streams of default priority.  Step i+1's inputs are prepared on the
    # host and copied on the copy stream while step i's kernels run; the host
    # then waits for that copy (an event that is normally already complete)
    # before launching step i+1, so the compute queue holds only kernels and
    # never waits on the copy engine.  No GPU-side cross-stream waits are used:
    # a copy that waited on a compute-stream event blocked the host for most
    # of a step.  Events on the compute stream ride on the kernel dispatches
    # (no marker packets) and are attached to few steps: each one makes that
    # dispatch's completion visible to the host, which costs stream time.
    compute = hip.stream()
    copy = hip.stream()
    for sl in slots:
        sl.copied = hip.event()
        hip.record(sl.copied, copy)        # start "complete"
    done_events = {}                       # step -> event attached to its merge
    done_pool = [hip.event(timing=True) for _ in range(NS // DONE_EVERY + 3)]
    cs = ctypes.c_void_p(compute)
    ids_ptr = [rep.seq_ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) for rep in reps]
    ncow = [0] * NS
    ncow_c = ctypes.c_int32()
    row_bytes = S * Hkv * D * step_k_d.element_size()
    nb_rep = nb_pool
    # events ride on the dispatches of every `every`-th step: at least 10 timed
    # launches whatever --steps is (each event costs a few us of stream time)
    every = args.time_every if args.time_every > 0 else max(1, min(10, K // 10))
    markers = args.event_markers
    n_timed = (K + every - 1) // every
    ev_a = [hip.event(timing=True) for _ in range(n_timed)]
    ev_b = [hip.event(timing=True) for _ in range(n_timed)]
    ev_c = [hip.event(timing=True) for _ in range(n_timed)]   # end of the timed steps' merge
    borrowed = set()                       # timing events that also served as a step's completion
    lens_log = []
    waited = [0.0]
    stage_bytes = lay["words"] * 4
    ptrs = []
    for sl in slots:
        base = sl.stage.data_ptr()
        slots_v, lens_v, tab_v = views(sl)
        ptrs.append(dict(
            slots=ctypes.cast(base, ctypes.POINTER(ctypes.c_int64)),
            lens=ctypes.cast(base + 4 * lay["lens"], ctypes.POINTER(ctypes.c_int32)),
            tab=ctypes.cast(base + 4 * lay["tables"], ctypes.POINTER(ctypes.c_int32)),
            cow=ctypes.cast(base + 4 * lay["cows"], ctypes.POINTER(ctypes.c_int32)),
            stage=ctypes.c_void_p(base), desc=ctypes.c_void_p(sl.desc.data_ptr()),
            slots_d=slots_v.data_ptr(), lens_d=lens_v.data_ptr(), tab_d=tab_v.data_ptr(),
            cows_d=ctypes.c_void_p(sl.desc.data_ptr() + 4 * lay["cows"]),
            lens_np=np.ctypeslib.as_array(ctypes.cast(base + 4 * lay["lens"], ctypes.POINTER(ctypes.c_int32)),
                                          shape=(S,))))
    rp = []
    for rep in reps:
        rp.append(dict(
            kc=ctypes.c_void_p(rep.k_cache.data_ptr()), vc=ctypes.c_void_p(rep.v_cache.data_ptr())))
    pool_h = [rep.pool._h for rep in reps]
    i8 = spec.cache in ("i8", "fp8")             # byte caches: codes + row scales
    append_codes = L.pa_reshape_and_cache_fp8 if spec.cache == "fp8" else L.pa_reshape_and_cache_int8
    fused = args.append == "fused"              # byte caches: the new rows are quantized in the launch
    k0, v0 = step_k_d.data_ptr(), step_v_d.data_ptr()
    torch.cuda.synchronize()

    def prepare(i):
        """Host pool append for step i and the copy of its inputs (copy stream)."""
        r, j = i % R, i % NS
        rep, pp = reps[r], ptrs[j]
        if i >= NS:                                    # slot j was last used by step i - NS
            w0 = time.perf_counter()
            s_done = min(s for s in done_events if s >= i - NS)
            hip.sync_event(done_events[s_done])
            waited[0] += time.perf_counter() - w0
            for s in [s for s in done_events if s < s_done]:
                e = done_events.pop(s)
                if id(e) not in borrowed:
                    done_pool.append(e)
        st = L.pa_seq_append_batch(pool_h[r], ids_ptr[r], S, pp["slots"], pp["cow"], ctypes.byref(ncow_c))
        if st:
            pa._check(st)
        ncow[j] = ncow_c.value
        st = L.pa_seq_export(pool_h[r], ids_ptr[r], S, MB, pp["tab"], pp["lens"])
        if st:
            pa._check(st)
        rep.max_ctx += 1
        hip.h2d(pp["desc"], pp["stage"], stage_bytes, copy)
        hip.record(slots[j].copied, copy)

    def launch(i, timed_idx):
        """Step i's kernels (compute stream), once its inputs are on the device."""
        r, j = i % R, i % NS
        rep, pp, q = reps[r], ptrs[j], rp[r]
        w0 = time.perf_counter()
        hip.sync_event(slots[j].copied)
        waited[0] += time.perf_counter() - w0
        prm = rep.params
        prm.block_tables, prm.context_lens = pp["tab_d"], pp["lens_d"]
        prm.max_context_len = rep.max_ctx
        if ncow[j]:
            if i8:
                pa._check(L.pa_copy_blocks_int8(q["kc"], q["vc"], pp["cows_d"], ncow[j], Hkv, D, nb_rep, cs))
            else:
                pa._check(L.pa_copy_blocks(q["kc"], q["vc"], pp["cows_d"], ncow[j], Hkv, D,
                                           nb_rep, dt_code, cs))
        if fused:
            prm.k_new = k0 + i * row_bytes
            prm.v_new = v0 + i * row_bytes
            prm.slot_mapping = pp["slots_d"]
        elif i8:
            pa._check(append_codes(ctypes.c_void_p(k0 + i * row_bytes), ctypes.c_void_p(v0 + i * row_bytes),
                                   q["kc"], q["vc"], ctypes.c_void_p(pp["slots_d"]), S, Hkv, D, nb_rep, dt_code,
                                   cs))
        else:
            pa._check(L.pa_reshape_and_cache(ctypes.c_void_p(k0 + i * row_bytes),
                                             ctypes.c_void_p(v0 + i * row_bytes), q["kc"], q["vc"],
                                             ctypes.c_void_p(pp["slots_d"]), S, Hkv, D, nb_rep, dt_code, cs))
        done = None
        if i % DONE_EVERY == DONE_EVERY - 1 or i == total - 1:
            if timed_idx >= 0 and not markers:   # the merge's timing event marks completion too
                done = ev_c[timed_idx]
                borrowed.add(id(done))
            else:
                done = done_pool.pop()
            done_events[i] = done
        if markers:
            if timed_idx >= 0:
                hip.record(ev_a[timed_idx], compute)
            pa._check(L.pa_decode_partitions(ctypes.byref(prm), ws_ptr, ws_bytes, cs))
            if timed_idx >= 0:
                hip.record(ev_b[timed_idx], compute)
            pa._check(L.pa_decode_merge(ctypes.byref(prm), ws_ptr, ws_bytes, cs))
            if done is not None:
                hip.record(done, compute)
        else:
            prm.start_event = ev_a[timed_idx] if timed_idx >= 0 else None
            prm.stop_event = ev_b[timed_idx] if timed_idx >= 0 else None
            pa._check(L.pa_decode_partitions(ctypes.byref(prm), ws_ptr, ws_bytes, cs))
            prm.start_event = None
            prm.stop_event = ev_c[timed_idx] if timed_idx >= 0 else done
            pa._check(L.pa_decode_merge(ctypes.byref(prm), ws_ptr, ws_bytes, cs))
        lens_log.append((timed_idx >= 0, pp["lens_np"].copy()))

    if loop and args.warmup > 0:
        # decode launches on the prompt state (no append), for warm code and caches
        for rep in reps:
            tab, lens = rep.pool.seq_export(rep.seq_ids, MB)
            tab_d, lens_d = torch.from_numpy(tab).to(dev), torch.from_numpy(lens).to(dev)
            for _ in range(args.warmup):
                pa.pa_decode(rep.out, q_d, rep.k_cache, rep.v_cache, tab_d, lens_d, Hkv, int(lens.max()),
                             spec.fp32_scale(), partition_tokens=args.partition_tokens, kernel=args.kernel,
                             sliding_window=spec.window,
                             shared_prefix_blocks=shared_prefix)
        torch.cuda.synchronize()
    total = W + K
    prepare(0)
    for i in range(W):
        launch(i, -1)
        prepare(i + 1)
    hip.sync_device()
    log(f"warmup done ({args.warmup} {'decode launches' if loop else 'steps'}); timing {K} steps")
    waited[0] = 0.0
    t0 = time.perf_counter()
    host = 0.0
    for k in range(K):
        h0 = time.perf_counter()
        launch(W + k, k // every if k % every == 0 else -1)
        if W + k + 1 < total:
            prepare(W + k + 1)
        host += time.perf_counter() - h0
    hip.sync_device()
    t1 = time.perf_counter()
    log(f"host time inside the step loop: {host / K * 1e6:.1f} us per step, of which "
        f"{waited[0] / K * 1e6:.1f} us blocked on the device")
    elapsed = t1 - t0
    part_ms = np.array([hip.elapsed_ms(ev_a[k], ev_b[k]) for k in range(n_timed)])
    decode_ms = None if markers else np.array([hip.elapsed_ms(ev_a[k], ev_c[k]) for k in range(n_timed)])

    def alg_of(lens):
        return accounting.decode_algorithmic_bytes(lens, Hq, Hkv, D, spec.dtype, spec.out_dtype, cache=spec.cache,
                                                   shared_tokens=spec.prefix_len, window=spec.window)
    alg_bytes = [alg_of(l) for timed, l in lens_log if timed]
    alg_timed_steps = [alg_of(l) for timed, l in lens_log[W:]]   # every step of the timed region
    # per attention launch over every step, warmup included: what a counter run sees
    log(f"algorithmic bytes per attention launch over all {len(lens_log)} steps: "
        f"{np.mean([alg_of(l)['total'] for _, l in lens_log]):.0f}")
    log(f"timed {K} steps in {elapsed * 1e3:.2f} ms; attention launch mean {part_ms.mean() * 1e3:.1f} us")
    # the last step's output (its replica's out was last written by it) and the
    # steps whose rows that replica's sequences appended, for the oracle check
    last = total - 1
    last_out = reps[last % R].out.float().cpu().numpy()
    return {
        "elapsed": elapsed, "part_ms": part_ms, "decode_ms": decode_ms, "alg": alg_bytes,
        "alg_all": alg_timed_steps, "part_tokens": part_tokens,
        "max_blocks": MB, "S": S,
        "append_bytes": accounting.append_bytes(S, Hkv, D, spec.dtype, spec.cache),
        "device": torch.cuda.get_device_name(0),
        "last_out": last_out, "last_steps": list(range(last % R, last + 1, R)), "every": every,
    }


# ---------------------------------------------------------------- CPU oracle leg
class OracleCaches:
    """The oracle's K/V pool of a workload's cache type (16-bit, INT8 or FP8)."""

    def __init__(self, spec, num_blocks):
        import oracle
        self.o, self.spec, self.nb = oracle, spec, num_blocks
        Hkv, D, dt = spec.num_kv_heads, spec.head_dim, spec.dtype
        self.i8, self.fp8 = spec.cache in ("i8", "fp8"), spec.cache == "fp8"
        if self.i8:
            empty = oracle.empty_cache_fp8 if self.fp8 else oracle.empty_cache_i8
            self.kc, self.vc = empty(num_blocks, Hkv, D), empty(num_blocks, Hkv, D)
        else:
            self.kc = oracle.empty_cache(num_blocks, Hkv, D, dt)
            self.vc = oracle.empty_cache(num_blocks, Hkv, D, dt)

    def put(self, k, v, slots):
        o, sp = self.o, self.spec
        if self.i8:
            (o.reshape_and_cache_fp8 if self.fp8 else o.reshape_and_cache_i8)(
                k, v, self.kc, self.vc, slots, sp.num_kv_heads, sp.head_dim, self.nb, sp.dtype)
        else:
            o.reshape_and_cache(k, v, self.kc, self.vc, slots, sp.num_kv_heads, sp.head_dim, self.nb, sp.dtype)

    def decode(self, q, tab, lens, nthreads=0):
        """(fp64 output, threads used)."""
        o, sp = self.o, self.spec
        if self.i8:
            return o.decode_i8(q, sp.dtype, self.kc, self.vc, tab, lens, sp.num_kv_heads, sp.fp32_scale(),
                               nthreads=nthreads, return_threads=True, window=sp.window, fp8=self.fp8)
        return o.decode(q, self.kc, self.vc, tab, lens, sp.num_kv_heads, sp.fp32_scale(), sp.dtype,
                        nthreads=nthreads, return_threads=True, window=sp.window)


def oracle_sample(wl, seqs, step_ids):
    """The fp64 oracle's output rows of sequences `seqs` after the decode steps
    `step_ids` appended their rows: each sequence is rebuilt alone from the
    workload's rows (prompt, then one row per step) in an oracle pool and
    decoded by the oracle's table walk."""
    import oracle
    from oracle.pool_model import PoolModel
    oracle.build()
    spec = wl.spec
    outs = []
    for s in seqs:
        k = np.concatenate([wl.seq_rows(s, "k")] + [wl.step_k[j, s][None] for j in step_ids])
        v = np.concatenate([wl.seq_rows(s, "v")] + [wl.step_v[j, s][None] for j in step_ids])
        n = len(k)
        mb = -(-n // 16)
        pool = PoolModel(mb + 1, 16, np.arange(mb + 1, dtype=np.int32))
        sid = pool.seq_create()
        slots, _ = pool.seq_append(sid, n)
        caches = OracleCaches(spec, mb + 1)
        caches.put(np.ascontiguousarray(k), np.ascontiguousarray(v), slots)
        tab, lens = pool.export([sid], mb)
        out, _ = caches.decode(np.ascontiguousarray(wl.q[s:s + 1]), np.array(tab, np.int32).reshape(1, mb),
                               np.array(lens, np.int32))
        outs.append(out[0])
    return np.stack(outs)


def run_cpu_baseline(wl, seconds):
    import oracle
    from oracle.pool_model import PoolModel
    oracle.build()
    spec = wl.spec
    pool = PoolModel(wl.num_blocks, 16, wl.free_order)
    caches = OracleCaches(spec, wl.num_blocks)
    put = caches.put
    owner = -1
    if spec.prefix_len:
        owner = pool.seq_create()
        sl, _ = pool.seq_append(owner, spec.prefix_len)
        put(wl.prefix_k, wl.prefix_v, sl)
    ids = []
    for s in range(spec.num_seqs):
        sid = pool.seq_fork(owner) if spec.prefix_len else pool.seq_create()
        ids.append(sid)
        lo, hi = wl.token_offsets[s], wl.token_offsets[s + 1]
        sl, _ = pool.seq_append(sid, int(hi - lo))
        put(wl.k_tokens[lo:hi], wl.v_tokens[lo:hi], sl)
    mb = int(-(-int(wl.prompt_lens.max()) // 16))
    tab, lens = pool.export(ids, mb)
    tab, lens = np.array(tab, np.int32), np.array(lens, np.int32)
    passes, used = 0, 0
    t0 = time.perf_counter()
    while True:
        _, used = caches.decode(wl.q, tab, lens)
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    # one thread: the leading sequences holding about an eighth of the batch's tokens
    m = int(np.searchsorted(np.cumsum(lens), max(1, int(lens.sum()) // 8))) + 1
    m = min(max(m, 1), spec.num_seqs)
    q1 = np.ascontiguousarray(wl.q[:m])
    passes1 = 0
    t1 = time.perf_counter()
    while True:
        caches.decode(q1, tab[:m], lens[:m], nthreads=1)
        passes1 += 1
        el1 = time.perf_counter() - t1
        if el1 >= seconds / 2:
            break
    return {
        "value": round(spec.num_seqs * passes / el, 3), "unit": "tokens/s", "cores": int(used),
        "kind": "oracle",
        "sample": f"{passes} whole-batch fp64 decode passes of the same workload "
                  f"({spec.num_seqs} sequences, prompt contexts, sum L={int(lens.sum())}) "
                  f"in {el:.1f} s, OpenMP over (sequence, head)",
        "single_thread": {"value": round(m * passes1 / el1, 3), "unit": "tokens/s", "cores": 1,
                          "sample": f"{passes1} passes over sequences 0-{m - 1} (sum L={int(lens[:m].sum())}) "
                                    f"in {el1:.1f} s on one thread"},
        "cpu_model": cpu_model(),
    }


# ---------------------------------------------------------------- copy calibration
def summarize_waves(rec):
    """Per-launch summary of the traced build's wave records (uint64 [n][8]: entry,
    inputs ready, first block, stream end, exit, XCD, blocks, written), times in
    microseconds from the first wave's entry."""
    rec = rec[rec[:, 7] == 1].astype(np.int64)
    base = rec[:, 0].min()
    us = lambda c: (rec[:, c] - base) / 100.0   # 100 MHz real-time counter
    t0, t1, t2, t3, t4 = (us(c) for c in range(5))
    work = rec[:, 6] > 0
    med = lambda x: round(float(np.median(x)), 2)
    pct = lambda x, q: round(float(np.percentile(x, q)), 2)
    xcd = [med(t3[work & (rec[:, 5] == x)]) if np.any(work & (rec[:, 5] == x)) else None for x in range(8)]
    return {"waves": int(len(rec)), "working_waves": int(work.sum()), "span_us": round(float(t4.max()), 2),
            "entry_us": {"median": med(t0), "max": round(float(t0.max()), 2)},
            "inputs_ready_us": {"median": med(t1), "p90": pct(t1, 90)},
            "first_block_us": {"median": med(t2[work]), "p90": pct(t2[work], 90)},
            "stream_end_us": {"median": med(t3[work]), "p10": pct(t3[work], 10), "p90": pct(t3[work], 90),
                              "max": round(float(t3[work].max()), 2)},
            "exit_us": {"median": med(t4[work]), "max": round(float(t4.max()), 2)},
            "blocks_per_wave": {"median": med(rec[work, 6]), "max": int(rec[work, 6].max())},
            "stream_end_median_us_by_xcd": xcd}


def run_wave_trace(args, wl):
    """--wave-trace: per-wave timeline of the attention launch of the workload
    (the decode without a fused append, or pa_extend with --extend K), from the
    traced build libpa_trace.so; one JSON line with a summary per launch."""
    import torch
    from paged_kv_cache_65_amd import binding as pa
    from paged_kv_cache_65_amd import build as pa_build
    if not os.path.exists(pa_build.TRACE_LIB):
        sys.exit("bench.py --wave-trace needs the traced build: python -m paged_kv_cache_65_amd.build --trace")
    pa.use_library(pa_build.TRACE_LIB)
    L = pa.lib()
    L.pa_trace_read.argtypes, L.pa_trace_read.restype = [ctypes.c_void_p, ctypes.c_size_t], ctypes.c_int
    L.pa_trace_clear.argtypes, L.pa_trace_clear.restype = [], ctypes.c_int
    L.pa_trace_bytes.argtypes, L.pa_trace_bytes.restype = [], ctypes.c_size_t
    spec = wl.spec
    dev = torch.device("cuda:0")
    S, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    MB = int(-(-int(wl.prompt_lens.max()) // 16))

    def to_dev(a):
        if spec.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    k_rows = np.concatenate([wl.prefix_k, wl.k_tokens]) if spec.prefix_len else wl.k_tokens
    v_rows = np.concatenate([wl.prefix_v, wl.v_tokens]) if spec.prefix_len else wl.v_tokens
    rep = build_replica(pa, torch, wl, wl.free_order, to_dev(k_rows), to_dev(v_rows), MB, S, dev)
    tab, lens = rep.pool.seq_export(rep.seq_ids, MB)
    tab_d, lens_d = torch.from_numpy(tab).to(dev), torch.from_numpy(lens).to(dev)
    out_dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[spec.out_dtype]
    k = args.extend
    if k:
        q = to_dev(workloads.round_to(np.random.default_rng(spec.seed + 77).standard_normal(
            (S * k, Hq, D), dtype=np.float32), spec.dtype))
        qs = torch.arange(0, S * k + 1, k, dtype=torch.int32, device=dev)
        out = torch.empty((S * k, Hq, D), dtype=q.dtype, device=dev)

        def call():
            pa.pa_extend(out, q, rep.k_cache, rep.v_cache, tab_d, lens_d, qs, Hkv, int(lens.max()), k,
                         spec.fp32_scale(), partition_tokens=args.partition_tokens or 0)
        kernel, what = "pa_extend_kernel", f"pa_extend, {k} new tokens per sequence"
    else:
        q = to_dev(wl.q)
        out = torch.empty((S, Hq, D), dtype=out_dt, device=dev)
        sp = (spec.prefix_len // 16) if spec.prefix_len else 0

        def call():
            pa.pa_decode(out, q, rep.k_cache, rep.v_cache, tab_d, lens_d, Hkv, int(lens.max()),
                         spec.fp32_scale(), partition_tokens=-1, sliding_window=spec.window,
                         shared_prefix_blocks=sp)
        kernel, what = "pa_balanced_kernel", "pa_decode (balanced split, no fused append)"
    buf = np.zeros(L.pa_trace_bytes() // 8, dtype=np.uint64)
    if k:
        warm_past_transient(lambda i: call(), args.warmup)
    launches = []
    for r in range(max(1, args.steps or 3)):
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        assert L.pa_trace_clear() == 0
        call()
        torch.cuda.synchronize()
        assert L.pa_trace_read(buf.ctypes.data, buf.nbytes) == 0
        launches.append(summarize_waves(buf.reshape(-1, 8)))
        log(f"traced launch {r}: span {launches[-1]['span_us']} us")
    print(json.dumps({"wave_trace": kernel, "launch": what, "workload": spec.name,
                      "clock": "s_memrealtime, 100 MHz, from the first wave's entry", "launches": launches}),
          flush=True)


def run_extend_ramp(args, L, params, ws_ptr, ws_bytes, stream, hip, spec, k, n=1000):
    """--extend K --ramp: per-call times of n pa_extend calls started from an idle
    GPU (one second of sleep first), as means over windows of call indices."""
    from paged_kv_cache_65_amd import binding as pa
    ev_a = [hip.event(timing=True) for _ in range(n)]
    ev_b = [hip.event(timing=True) for _ in range(n)]
    time.sleep(1.0)
    for i in range(n):
        prm = params[i % len(params)]
        prm.start_event, prm.stop_event = ev_a[i], ev_b[i]
        pa._check(L.pa_extend(ctypes.byref(prm), ws_ptr, ws_bytes, stream))
        prm.start_event = prm.stop_event = None
    hip.sync_event(ev_b[-1])
    t = np.array([hip.elapsed_ms(ev_a[i], ev_b[i]) * 1e3 for i in range(n)])
    print(json.dumps({"ramp": "pa_extend per-call time from idle", "workload": spec.name, "draft_tokens": k,
                      "calls": n, "windows": ramp_windows(t)}), flush=True)


def ramp_windows(t):
    edges = [0, 5, 15, 35, 60, 100, 200, 400, 700, len(t)]
    return [{"calls": [a, b], "mean_us": round(float(t[a:b].mean()), 2)} for a, b in zip(edges[:-1], edges[1:])]


def run_decode_ramp(args, wl, n=1000):
    """--ramp without --extend: per-call times of n pa_decode calls (balanced split
    and merge, no append; three replicas in turn) started from an idle GPU, with
    timing events recorded between the calls."""
    import torch
    from paged_kv_cache_65_amd import binding as pa
    spec = wl.spec
    dev = torch.device("cuda:0")
    S, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    MB = int(-(-int(wl.prompt_lens.max()) // 16))

    def to_dev(a):
        if spec.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    k_rows = np.concatenate([wl.prefix_k, wl.k_tokens]) if spec.prefix_len else wl.k_tokens
    v_rows = np.concatenate([wl.prefix_v, wl.v_tokens]) if spec.prefix_len else wl.v_tokens
    k_rows, v_rows = to_dev(k_rows), to_dev(v_rows)
    reps = []
    for r in range(3):
        order = wl.free_order if r == 0 else \
            np.random.default_rng(spec.seed * 1000 + r).permutation(wl.num_blocks).astype(np.int32)
        rep = build_replica(pa, torch, wl, order, k_rows, v_rows, MB, S, dev)
        tab, lens = rep.pool.seq_export(rep.seq_ids, MB)
        reps.append((rep, torch.from_numpy(tab).to(dev), torch.from_numpy(lens).to(dev), int(lens.max())))
    del k_rows, v_rows
    q = to_dev(wl.q)
    out = torch.empty((S, Hq, D), dtype={"f32": torch.float32, "f16": torch.float16,
                                         "bf16": torch.bfloat16}[spec.out_dtype], device=dev)
    sp = (spec.prefix_len // 16) if spec.prefix_len else 0
    need = max(pa.pa_decode_workspace_bytes(pa.make_decode_params(
        out, q, rep.k_cache, rep.v_cache, tab_d, lens_d, Hkv, mx, spec.fp32_scale(), args.partition_tokens, "auto",
        None, None, None, sliding_window=spec.window, shared_prefix_blocks=sp)) for rep, tab_d, lens_d, mx in reps)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    torch.cuda.synchronize()
    time.sleep(1.0)
    for i in range(n):
        rep, tab_d, lens_d, mx = reps[i % 3]
        ev_a[i].record()
        pa.pa_decode(out, q, rep.k_cache, rep.v_cache, tab_d, lens_d, Hkv, mx, spec.fp32_scale(),
                     partition_tokens=args.partition_tokens, sliding_window=spec.window, shared_prefix_blocks=sp,
                     workspace=ws)
        ev_b[i].record()
    torch.cuda.synchronize()
    t = np.array([ev_a[i].elapsed_time(ev_b[i]) * 1e3 for i in range(n)])
    print(json.dumps({"ramp": "pa_decode per-call time from idle", "workload": spec.name, "calls": n,
                      "windows": ramp_windows(t)}), flush=True)


def run_read_probe(args, wl, reps=20):
    """--read-probe: the read rate of the balanced split's access pattern with none
    of its math (the traced build's pa_read_probe) over the workload's cache: every
    (sequence, KV head, block) unit's K and V tiles once, in the split's order."""
    import torch
    from paged_kv_cache_65_amd import binding as pa
    from paged_kv_cache_65_amd import build as pa_build
    if not os.path.exists(pa_build.TRACE_LIB):
        sys.exit("bench.py --read-probe needs the traced build: python -m paged_kv_cache_65_amd.build --trace")
    spec = wl.spec
    if spec.head_dim != 128 or spec.dtype == "f32" or spec.cache in ("i8", "fp8"):
        sys.exit("bench.py --read-probe reads 4 KiB tiles: a D = 128 16-bit cache")
    pa.use_library(pa_build.TRACE_LIB)
    L = pa.lib()
    L.pa_read_probe.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t] + \
        [ctypes.c_void_p] * 3
    L.pa_read_probe.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    S, Hkv = spec.num_seqs, spec.num_kv_heads
    MB = int(-(-int(wl.prompt_lens.max()) // 16))

    def to_dev(a):
        if spec.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    rep = build_replica(pa, torch, wl, wl.free_order, to_dev(wl.k_tokens), to_dev(wl.v_tokens), MB, S, dev)
    tab, lens = rep.pool.seq_export(rep.seq_ids, MB)
    units = []   # (sequence, KV head, block) order: tile index block * Hkv + head
    for s in range(S):
        blocks = tab[s, :-(-int(lens[s]) // 16)].astype(np.int64)
        units += [blocks * Hkv + g for g in range(Hkv)]
    tiles = np.concatenate(units).astype(np.int32)
    tiles_d = torch.from_numpy(tiles).to(dev)
    n = int(tiles.size)
    sink = torch.zeros(4 * 1024, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    hip = Hip()
    ev = [(hip.event(timing=True), hip.event(timing=True)) for _ in range(reps)]
    args_of = lambda e0, e1: (ctypes.c_void_p(rep.k_cache.data_ptr()), ctypes.c_void_p(rep.v_cache.data_ptr()),
                              ctypes.c_void_p(tiles_d.data_ptr()), n, ctypes.c_void_p(sink.data_ptr()),
                              sink.numel(), e0, e1, stream)
    for _ in range(5):
        pa._check(L.pa_read_probe(*args_of(None, None)))
    torch.cuda.synchronize()
    for e0, e1 in ev:
        pa._check(L.pa_read_probe(*args_of(e0, e1)))
    torch.cuda.synchronize()
    us = np.array([hip.elapsed_ms(e0, e1) for e0, e1 in ev]) * 1e3
    nbytes = n * 2 * 4096
    print(json.dumps({"read_probe": "pa_read_probe (balanced split access pattern, no math)", "workload": spec.name,
                      "units": n, "bytes": nbytes, "launches": reps,
                      "median_us": round(float(np.median(us)), 2), "p10_us": round(float(np.percentile(us, 10)), 2),
                      "p90_us": round(float(np.percentile(us, 90)), 2),
                      "GBps": round(nbytes / float(np.median(us)) / 1e3, 1),
                      "frac_of_8TBps": round(nbytes / float(np.median(us)) / 1e3 / HBM_PEAK_GBPS, 4)}), flush=True)


def run_copy_calibration(nbytes):
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    src.fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 5}), flush=True)


def run_read_ceiling(nbytes, reps=20):
    """--read-ceiling: what plain library kernels reach on this GPU's HBM, as a
    reference beside the 8 TB/s peak: a full reduction reading nbytes (torch.sum
    over float32, result 4 bytes) and a device copy of nbytes / 2 (read + write),
    each timed with events over `reps` launches."""
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    src = torch.ones(nbytes // 8, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    out = {}
    for name, fn, moved in (("sum_read", lambda: torch.sum(x), nbytes),
                            ("copy_read_write", lambda: dst.copy_(src), nbytes)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for i in range(reps):
            ev[2 * i].record()
            fn()
            ev[2 * i + 1].record()
        torch.cuda.synchronize()
        ms = np.array([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(reps)])
        out[name] = {"bytes": moved, "median_us": round(float(np.median(ms)) * 1e3, 2),
                     "GBps": round(moved / (float(np.median(ms)) / 1e3) / 1e9, 1),
                     "frac_of_8TBps": round(moved / (float(np.median(ms)) / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)}
    print(json.dumps({"read_ceiling": out, "device": torch.cuda.get_device_name(0)}), flush=True)


# pa_extend launches with several query tiles per wave (k >= 8 at G = 8) keep the
# matrix cores busy enough that, from idle, the GPU's clock management settles
# only after a transient: per-call times over a long run of calls (--ramp) go
# 110 -> 135 -> 105 us at k = 8 over the first ~200 calls (~25 ms), while the
# decode and k = 1 launches are flat from the start.  Their timing warms up past it.
EXTEND_WARMUP_S = 0.1


def warm_past_transient(call, min_calls, seconds=EXTEND_WARMUP_S, sync=None):
    """Runs call(i) for i = 0, 1, ... until at least min_calls calls and `seconds`
    of wall time (synchronized every 20 calls) have passed; returns the count."""
    import torch
    t0, i = time.perf_counter(), 0
    while i < min_calls or time.perf_counter() - t0 < seconds:
        call(i)
        i += 1
        if i % 20 == 0:
            (sync or torch.cuda.synchronize)()
    (sync or torch.cuda.synchronize)()
    return i


def run_extend_bench(args, wl, k):
    """Speculative verification on the workload: the last k cached tokens of every
    sequence are the drafted ones, each attending causally (pa_extend), over R
    replicas in rotation.  Events ride on the dispatches of the timed calls."""
    import torch
    from paged_kv_cache_65_amd import binding as pa
    spec = wl.spec
    dev = torch.device("cuda:0")
    S, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    R, K, W = args.replicas, args.steps, args.warmup
    MB = int(-(-int(wl.prompt_lens.max()) // 16))

    def to_dev(a):
        if spec.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    k_rows_d, v_rows_d = to_dev(wl.k_tokens), to_dev(wl.v_tokens)
    reps = []
    for r in range(R):
        order = wl.free_order if r == 0 else \
            np.random.default_rng(spec.seed * 1000 + r).permutation(wl.num_blocks).astype(np.int32)
        reps.append(build_replica(pa, torch, wl, order, k_rows_d, v_rows_d, MB, S, dev))
    del k_rows_d, v_rows_d
    T = S * k
    rng = np.random.default_rng(spec.seed + 77)
    q = to_dev(workloads.round_to(rng.standard_normal((T, Hq, D), dtype=np.float32), spec.dtype))
    qs = torch.arange(0, T + 1, k, dtype=torch.int32, device=dev)
    hip = Hip()
    params, outs, tabs = [], [], []
    for rep in reps:
        tab, lens = rep.pool.seq_export(rep.seq_ids, MB)
        tab_d, lens_d = torch.from_numpy(tab).to(dev), torch.from_numpy(lens).to(dev)
        out = torch.empty((T, Hq, D), dtype=q.dtype, device=dev)
        prm = pa.make_extend_params(out, q, rep.k_cache, rep.v_cache, tab_d, lens_d, qs, Hkv, int(lens.max()), k,
                                    spec.fp32_scale(), partition_tokens=args.partition_tokens)
        params.append(prm)
        outs.append(out)
        tabs.append((tab_d, lens_d, lens))
    need = max(pa.pa_extend_workspace_bytes(p_) for p_ in params)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = ctypes.c_void_p(ws.data_ptr()), ws.numel()
    L = pa.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ev_a = [hip.event(timing=True) for _ in range(K)]
    ev_b = [hip.event(timing=True) for _ in range(K)]
    if args.ramp:
        run_extend_ramp(args, L, params, ws_ptr, ws_bytes, stream, hip, wl.spec, k)
        return
    W = warm_past_transient(lambda i: pa._check(L.pa_extend(ctypes.byref(params[i % R]), ws_ptr, ws_bytes, stream)), W)
    t0 = time.perf_counter()
    for i in range(K):
        prm = params[i % R]
        prm.start_event, prm.stop_event = ev_a[i], ev_b[i]
        pa._check(L.pa_extend(ctypes.byref(prm), ws_ptr, ws_bytes, stream))
        prm.start_event = prm.stop_event = None
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    call_ms = np.array([hip.elapsed_ms(ev_a[i], ev_b[i]) for i in range(K)])
    lens = tabs[0][2]
    eb = accounting.ELEM_BYTES[spec.dtype]
    kv = int(np.sum(lens)) * 2 * Hkv * D * eb
    small = 2 * T * Hq * D * eb + 4 * int(np.sum(-(-lens // 16))) + 4 * S + 4 * (S + 1)
    alg = kv + small
    call_s = float(call_ms.mean()) / 1e3
    rec = {"metric": "speculative-verify attention tokens/s (k drafted tokens per sequence, pa_extend)",
           "value": round(T * K / elapsed, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
           "ms_per_step": round(elapsed / K * 1e3, 5), "higher_is_better": True, "dtype": spec.dtype,
           "data": "synthetic", "warmup_note": f"{W} calls, at least {EXTEND_WARMUP_S} s (clock transient)",
           "config": {"workload": spec.name, "draft_tokens": k, "query_rows": T,
                      "partition_tokens": pa.pa_extend_partition_tokens(params[0]), "replicas": R,
                      "device": torch.cuda.get_device_name(0)},
           "roofline": {"kernel": "pa_extend (attention + merge)", "bound": "hbm",
                        "achieved": round(alg / call_s / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(alg / call_s / 1e9 / HBM_PEAK_GBPS, 4),
                        "algorithmic_bytes_per_launch": alg, "mean_call_us": round(call_s * 1e6, 2)}}
    print(json.dumps(rec), flush=True)


def run_swap_bench(blocks, reps):
    """Swap-out (device -> pinned host) and swap-in (host -> device) of `blocks`
    scattered blocks of the 70B-GQA cache shape (8 KV heads, D = 128, bf16:
    64 KiB of K+V per block) through pa_swap_blocks, against plain DMA copies
    of the same bytes between contiguous buffers.  One JSON line."""
    import torch
    from paged_kv_cache_65_amd import binding as pa
    Hkv, D, NB = 8, 128, 20000
    per = Hkv * 16 * D
    g = torch.Generator(device="cuda").manual_seed(11)
    kc = torch.randn(NB * per, dtype=torch.bfloat16, device="cuda", generator=g)
    vc = torch.randn(NB * per, dtype=torch.bfloat16, device="cuda", generator=g)
    ids = torch.from_numpy(np.random.default_rng(12).permutation(NB)[:2 * blocks].astype(np.int32))
    hk = torch.empty(blocks * per, dtype=torch.bfloat16).pin_memory()
    hv = torch.empty(blocks * per, dtype=torch.bfloat16).pin_memory()
    ar = torch.arange(blocks, dtype=torch.int32)
    out_pairs = torch.stack([ids[:blocks], ar], 1).contiguous().cuda()
    in_pairs = torch.stack([ar, ids[blocks:]], 1).contiguous().cuda()   # back into other blocks
    nbytes = 2 * blocks * per * 2
    dev_flat = torch.empty(2 * blocks * per, dtype=torch.bfloat16, device="cuda")
    host_flat = torch.empty(2 * blocks * per, dtype=torch.bfloat16).pin_memory()

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) / 1e3 / reps

    t_out = timed(lambda: pa.pa_swap_blocks(kc, vc, hk, hv, out_pairs, Hkv, D))
    t_in = timed(lambda: pa.pa_swap_blocks(hk, hv, kc, vc, in_pairs, Hkv, D))
    t_d2h = timed(lambda: host_flat.copy_(dev_flat, non_blocking=True))
    t_h2d = timed(lambda: dev_flat.copy_(host_flat, non_blocking=True))
    # the round trip restores the blocks bit for bit
    torch.cuda.synchronize()
    same = bool(torch.equal(kc.view(NB, per)[ids[blocks:].long()], kc.view(NB, per)[ids[:blocks].long()]))
    rec = {"metric": "KV swap bandwidth, device <-> pinned host (pa_swap_blocks)", "unit": "GB/s",
           "blocks": blocks, "bytes_per_direction": nbytes, "reps": reps,
           "swap_out_GBps": round(nbytes / t_out / 1e9, 2), "swap_in_GBps": round(nbytes / t_in / 1e9, 2),
           "memcpy_d2h_GBps": round(nbytes / t_d2h / 1e9, 2), "memcpy_h2d_GBps": round(nbytes / t_h2d / 1e9, 2),
           "swap_out_ms": round(t_out * 1e3, 3), "swap_in_ms": round(t_in * 1e3, 3),
           "round_trip_bitwise": same,
           "config": {"workload": "70B-GQA cache blocks (8 KV heads, D=128, bf16), scattered over 20000",
                      "device": torch.cuda.get_device_name(0)}}
    print(json.dumps(rec), flush=True)


def step_description(fused, cache, shared_prefix):
    append = {"i8": "quantized int8 ", "fp8": "quantized fp8 "}.get(cache, "")
    attend = "prefix attention + decode partitions" if shared_prefix else "decode partitions"
    if fused:
        return f"pool append + H2D slots/tables/lens + {attend} (fused {append}K/V append) + merge"
    kern = {"i8": "reshape_and_cache_int8", "fp8": "reshape_and_cache_fp8"}.get(cache, "reshape_and_cache")
    return f"pool append + H2D slots/tables/lens + {kern} + {attend} + merge"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 200; a decode-loop workload: its own step count)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3, choices=list(range(1, 12)))
    ap.add_argument("--replicas", type=int, default=None,
                    help="independent pools in rotation (default 3; a decode-loop workload: 1)")
    ap.add_argument("--kernel", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--partition-tokens", type=int, default=None,
                    help="0 = automatic, -1 = balanced split, else a multiple of 16 (default: the workload's)")
    ap.add_argument("--append", default="fused", choices=["fused", "separate"],
                    help="append the step's K/V inside the decode launch, or with pa_reshape_and_cache")
    ap.add_argument("--time-every", type=int, default=0, metavar="N",
                    help="bracket every N-th step's launches with timing events (default: often enough "
                         "for at least 10 timed launches; the events themselves cost stream time)")
    ap.add_argument("--event-markers", action="store_true",
                    help="record the timing and completion events as separate stream markers "
                         "(hipEventRecord) instead of on the kernel dispatches")
    ap.add_argument("--no-shared-prefix", action="store_true",
                    help="with a shared-prefix workload, stream the prefix blocks per sequence instead of "
                         "computing their attention once (shared_prefix_blocks = 0)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    ap.add_argument("--extend", type=int, default=0, metavar="K",
                    help="only measure multi-query attention with K new tokens per sequence of the workload")
    ap.add_argument("--ramp", action="store_true",
                    help="only print per-call times of 1000 attention calls (pa_decode, or pa_extend with "
                         "--extend) started from an idle GPU")
    ap.add_argument("--read-ceiling", type=int, default=0, metavar="BYTES",
                    help="only time plain library kernels over BYTES of HBM (a reduction and a copy)")
    ap.add_argument("--read-probe", action="store_true",
                    help="only time the traced build's read probe over the workload's cache (its K / V tiles "
                         "in the balanced split's order, no math)")
    ap.add_argument("--wave-trace", action="store_true",
                    help="only print the per-wave timeline of --steps traced attention launches (default 3), "
                         "from the traced build (python -m paged_kv_cache_65_amd.build --trace)")
    ap.add_argument("--swap", type=int, default=0, metavar="BLOCKS",
                    help="only measure swap-out / swap-in of BLOCKS scattered cache blocks")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py times one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}); the "
              f"decode path shards by sequence and KV head with no exchange, so run it once per GPU.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        run_copy_calibration(args.copy_calibration)
        return
    if args.read_ceiling:
        run_read_ceiling(args.read_ceiling)
        return
    if args.swap:
        run_swap_bench(args.swap, 10)
        return
    base = workloads.named(args.workload)
    loop = base.decode_steps > 0 and not args.extend   # a decode loop: its own steps, one pool
    if args.steps is None:
        args.steps = 3 if args.wave_trace else base.decode_steps if loop else 200
    if args.replicas is None:
        args.replicas = 1 if loop else 3
    if args.partition_tokens is None:
        args.partition_tokens = base.partition_tokens
    spec = dataclasses.replace(base, decode_steps=args.steps if loop else args.warmup + args.steps)
    t = time.perf_counter()
    wl = workloads.generate(spec)
    log(f"workload {spec.name} generated in {time.perf_counter() - t:.1f} s "
        f"(sum of prompt lengths {int(wl.prompt_lens.sum())})")
    if args.wave_trace:
        run_wave_trace(args, wl)
        return
    if args.read_probe:
        run_read_probe(args, wl)
        return
    if args.ramp and not args.extend:
        run_decode_ramp(args, wl)
        return
    if args.extend:
        run_extend_bench(args, wl, args.extend)
        return
    g = run_gpu(args, wl, loop=loop)
    K = args.steps
    tok_s = spec.num_seqs * K / g["elapsed"]
    mean_alg = float(np.mean([a["total"] for a in g["alg"]]))
    row_bytes = (spec.head_dim + accounting.I8_SCALE_BYTES) if spec.cache in ("i8", "fp8") else \
        spec.head_dim * accounting.ELEM_BYTES[spec.dtype]
    mean_kv_tokens = float(np.mean([a["kv_logical"] for a in g["alg"]])) / (2 * spec.num_kv_heads * row_bytes)
    part = timing_stats(g["part_ms"])
    step_bytes = mean_alg + g["append_bytes"]
    step_gbps = step_bytes * K / g["elapsed"] / 1e9
    shared_prefix = (spec.prefix_len // 16) if (spec.prefix_len and not args.no_shared_prefix) else 0
    balanced = g["part_tokens"] == 0
    kernel_name = "pa_balanced_kernel" if balanced else "pa_partition_kernel"
    if shared_prefix:   # the prefix kernel runs beside the split on a second stream
        kernel_name = kernel_name + " (pa_prefix_kernel beside it)"
    merge_name = "pa_merge_balanced_kernel" if balanced else "pa_merge_kernel"
    t_attn = read_traffic(kernel_name.split(" ")[0], spec.name)
    t_merge = read_traffic(merge_name, spec.name)

    def gbps(nbytes, us):
        return round(nbytes / (us * 1e-6) / 1e9, 1)

    kernel_only = {"kernel": kernel_name, **part, "achieved": gbps(mean_alg, part["mean_us"]),
                   "frac": round(gbps(mean_alg, part["mean_us"]) / HBM_PEAK_GBPS, 4),
                   "traffic": traffic_bytes(t_attn)}
    if isinstance(t_attn, dict):
        kernel_only["traffic_ratio"] = round(t_attn["hbm"] / t_attn["algorithmic"], 4)
    if g["decode_ms"] is not None:
        dec = timing_stats(g["decode_ms"])
        # the merge launches only when some context was split; its traffic joins the attention's
        decode_traffic = None
        if t_attn is not None and t_merge is not None:
            decode_traffic = traffic_bytes(t_attn) + traffic_bytes(t_merge)
        roofline = {"kernel": f"{kernel_name}+{merge_name} (decode: attention and merge launches)",
                    "bound": "hbm", "achieved": gbps(mean_alg, dec["mean_us"]), "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(gbps(mean_alg, dec["mean_us"]) / HBM_PEAK_GBPS, 4),
                    "traffic": decode_traffic, "algorithmic_bytes_per_launch": round(mean_alg),
                    "mean_launch_us": dec["mean_us"], **{k: v for k, v in dec.items() if k != "mean_us"},
                    "kernel_only": kernel_only}
        if isinstance(t_attn, dict) and isinstance(t_merge, dict):
            roofline["traffic_ratio"] = round(decode_traffic / t_attn["algorithmic"], 4)
    else:                # marker events: the attention launch alone
        roofline = {**kernel_only, "bound": "hbm", "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "algorithmic_bytes_per_launch": round(mean_alg), "mean_launch_us": part["mean_us"]}
    # parity of a timed step: sampled rows of the last step's output against the oracle
    S = spec.num_seqs
    sample = sorted({0, S // 3, (2 * S) // 3, S - 1})
    log(f"oracle check: sequences {sample} of step {args.warmup + K - 1 if not loop else K - 1}")
    ref = oracle_sample(wl, sample, g["last_steps"])
    err = float(np.max(np.abs(g["last_out"][sample].astype(np.float64) - ref)))
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: fp64 oracle")
        cpu = run_cpu_baseline(wl, args.cpu_seconds)
    rec = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(g["elapsed"] / K * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic",
        "achieved_GBps": round(step_gbps, 1),
        "hbm_frac": round(step_gbps / HBM_PEAK_GBPS, 4),
        "kv_tokens_per_s": round(mean_kv_tokens * K / g["elapsed"], 1),
        "max_abs_err": err,
        "max_abs_err_rows": f"sequences {sample} of the last timed step, all heads, {spec.out_dtype} output "
                            f"vs the fp64 oracle",
        "config": {
            "workload": spec.name, "num_seqs": spec.num_seqs, "num_q_heads": spec.num_q_heads,
            "num_kv_heads": spec.num_kv_heads, "head_dim": spec.head_dim, "block_size": 16,
            "kv_dtype": {"i8": "int8 + f32 row scales", "fp8": "fp8 e4m3 + f32 row scales"}.get(spec.cache, spec.dtype),
            "pool_blocks": int(wl.num_blocks),
            "sliding_window": int(spec.window),
            "shared_prefix_blocks": shared_prefix,
            "mean_context": round(mean_kv_tokens / spec.num_seqs, 1),
            "partition_tokens": g["part_tokens"], "replicas": args.replicas,
            "kernel": args.kernel, "seed": spec.seed, "timed_every": g["every"],
            "step": step_description(args.append == "fused", spec.cache, shared_prefix),
            "device": g["device"],
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if loop:   # the whole decode loop: every step's tokens and bytes over the loop's wall time
        loop_bytes = float(sum(a["total"] for a in g["alg_all"])) + g["append_bytes"] * K
        rec["loop"] = {"steps": K, "decode_tokens": S * K, "total_ms": round(g["elapsed"] * 1e3, 3),
                       "tokens_per_s": round(tok_s, 1), "per_step_us": round(g["elapsed"] / K * 1e6, 2),
                       "GBps": round(loop_bytes / g["elapsed"] / 1e9, 1),
                       "algorithmic_bytes": round(loop_bytes)}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
