"""GPU parity for groups of more than 16 query heads per KV head, up to
multi-query attention (every query head on one KV head: "Inference serving:
the KV-cache machine", section "The KV cache: attention's memory bill,
derived", names one shared head for the 32-head 8B model).

The matrix-core kernels hold ceil(G/16) score tiles per wave and feed every
K/V fragment to all of them; the vector-ALU kernel splits the group into
16-head workgroups.  Bars as for the other decode tests: max-abs <= 2e-3
against the fp64 oracle for fp16/bf16 inputs and byte caches, <= 1e-5 for
fp32; an empty context gives a zero row, a one-token context V exactly; a
16-bit output is the float32 output rounded to nearest even; caches written
by the fused append equal the oracle's bit for bit.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from paged_kv_cache_65_amd import binding as pa  # noqa: E402
from paged_kv_cache_65_amd import workloads  # noqa: E402
from tests import gpu_side, oracle_side  # noqa: E402

BAL = pa.PA_PARTITION_BALANCED
pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
LENS = (1, 15, 16, 17, 0, 511, 512, 513, 100, 1000)


@pytest.fixture(scope="module", autouse=True)
def _gpu(oracle_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _f32(out):
    return out.float().cpu().numpy().astype(np.float64)


def _both(spec, steps=0):
    wl = workloads.generate(spec)
    _say(f"[case] {spec.name} seed={spec.seed} dtype={spec.dtype} cache={spec.cache or spec.dtype} "
         f"S={spec.num_seqs} Hq={spec.num_q_heads} Hkv={spec.num_kv_heads} D={spec.head_dim}")
    return wl, gpu_side.build(wl, steps), oracle_side.build(wl, steps)


# (dtype, D, Hq, Hkv): G = 32 and 64 (two and four full tiles), 24 / 40 / 48
# (a last tile only partly used), fp32 caches on the vector-ALU kernel
SWEEP = [("bf16", 128, 32, 1), ("f16", 64, 32, 1), ("bf16", 128, 64, 2), ("f16", 128, 64, 1),
         ("bf16", 64, 64, 1), ("bf16", 128, 24, 1), ("f16", 128, 48, 1), ("bf16", 64, 80, 2),
         ("f32", 64, 32, 1), ("f32", 128, 64, 2)]


@pytest.mark.parametrize("dtype,D,Hq,Hkv", SWEEP)
def test_mqa_decode_sweep(dtype, D, Hq, Hkv):
    spec = workloads.custom(name="mqa-sweep", seed=500 + Hq + D, dtype=dtype, lens=LENS, num_q_heads=Hq,
                            num_kv_heads=Hkv, head_dim=D)
    wl, gst, ost = _both(spec)
    mb = oracle_side.max_blocks_for(wl)
    ref = oracle_side.decode(wl, ost, mb)
    G = Hq // Hkv
    kernels = ["valu"] if dtype == "f32" else ["valu", "mfma"]
    v0 = oracle.to_float64(wl.v_tokens[wl.token_offsets[0]], dtype)
    for kern in kernels:
        for pt in ((0, BAL, 16, 64, 512) if kern == "mfma" else (0, 16, 512)):
            _say(f"  kernel={kern} partition_tokens={pt}")
            got = _f32(gpu_side.decode(wl, gst, mb, out_dtype="f32", kernel=kern, partition_tokens=pt))
            err = np.max(np.abs(got - ref))
            assert np.all(np.isfinite(got)), (kern, pt)
            assert err <= TOL[dtype], (kern, pt, err)
            assert np.all(got[4] == 0)
            for h in range(Hq):
                assert np.array_equal(got[0, h], v0[h // G]), (kern, pt, h)
    if dtype != "f32":
        o32 = gpu_side.decode(wl, gst, mb, out_dtype="f32", partition_tokens=BAL)
        o16 = gpu_side.decode(wl, gst, mb, out_dtype=dtype, partition_tokens=BAL)
        assert torch.equal(o16.cpu().view(torch.int16), o32.cpu().to(gpu_side.TORCH[dtype]).view(torch.int16))


def test_mqa_equals_gqa_with_the_kv_head_replicated():
    # 32 q heads on 1 KV head == the same q heads on 2 KV heads holding the same rows
    spec = workloads.custom(name="mqa-rep", seed=520, dtype="bf16", lens=(29, 513, 1200), num_q_heads=32,
                            num_kv_heads=1, head_dim=128)
    wl = workloads.generate(spec)
    gst = gpu_side.build(wl)
    mb = oracle_side.max_blocks_for(wl)
    rep = workloads.Workload(
        workloads.custom(name="mqa-rep2", seed=520, dtype="bf16", lens=(29, 513, 1200), num_q_heads=32,
                         num_kv_heads=2, head_dim=128),
        wl.prompt_lens, wl.free_order, wl.q, wl.prefix_k, wl.prefix_v,
        np.repeat(wl.k_tokens, 2, axis=1), np.repeat(wl.v_tokens, 2, axis=1), wl.token_offsets,
        wl.step_k, wl.step_v)
    rst = gpu_side.build(rep)
    for kern, pt in (("mfma", BAL), ("mfma", 128), ("valu", 128)):
        a = gpu_side.decode(wl, gst, mb, out_dtype="f32", kernel=kern, partition_tokens=pt)
        b = gpu_side.decode(rep, rst, mb, out_dtype="f32", kernel=kern, partition_tokens=pt)
        assert np.max(np.abs(_f32(a) - _f32(b))) <= 1e-6, (kern, pt)


BYTE = [("i8", "bf16", 128, 32, 1), ("i8", "f16", 64, 64, 1), ("fp8", "bf16", 128, 64, 2),
        ("fp8", "f16", 128, 32, 1), ("i8", "bf16", 128, 48, 1)]


@pytest.mark.parametrize("cache,dtype,D,Hq,Hkv", BYTE)
def test_mqa_byte_cache_decode(cache, dtype, D, Hq, Hkv):
    spec = workloads.custom(name="mqa-bytes", seed=530 + Hq + D, dtype=dtype, lens=LENS, num_q_heads=Hq,
                            num_kv_heads=Hkv, head_dim=D, cache=cache)
    wl, gst, ost = _both(spec)
    mb = oracle_side.max_blocks_for(wl)
    ref = oracle_side.decode(wl, ost, mb)
    out = gpu_side.decode(wl, gst, mb, out_dtype="f32")
    got = _f32(out)
    err = np.max(np.abs(got - ref))
    _say(f"  max_abs_err={err:.3e}")
    assert np.all(np.isfinite(got)) and err <= 2e-3, err
    assert np.all(got[4] == 0)
    o16 = gpu_side.decode(wl, gst, mb, out_dtype=dtype)
    assert torch.equal(o16.cpu().view(torch.int16), out.cpu().to(gpu_side.TORCH[dtype]).view(torch.int16))


@pytest.mark.parametrize("cache,pt", [("", 0), ("", BAL), ("", 16), ("", 128), ("i8", 0), ("fp8", 0)])
def test_mqa_sliding_window(cache, pt):
    lens = (1, 40, 130, 600, 1000, 17)
    spec = workloads.custom(name="mqa-window", seed=540, dtype="bf16", lens=lens, num_q_heads=32,
                            num_kv_heads=1, head_dim=128, cache=cache)
    wl, gst, ost = _both(spec)
    mb = oracle_side.max_blocks_for(wl)
    for W in (100, 300):
        ref = oracle_side.decode(wl, ost, mb, window=W)
        got = _f32(gpu_side.decode(wl, gst, mb, out_dtype="f32", partition_tokens=pt, window=W))
        err = np.max(np.abs(got - ref))
        _say(f"  window={W} partition_tokens={pt} max_abs_err={err:.3e}")
        assert err <= 2e-3, (W, err)


@pytest.mark.parametrize("cache,D,Hq,Hkv,kern,pt", [("", 128, 32, 1, "mfma", 0), ("", 128, 32, 1, "mfma", BAL),
                                                   ("", 64, 64, 1, "mfma", 32), ("", 128, 64, 2, "valu", 0),
                                                   ("i8", 128, 32, 1, "auto", 0), ("fp8", 64, 64, 1, "auto", 0)])
def test_mqa_fused_append_steps(cache, D, Hq, Hkv, kern, pt):
    """pa_decode with k_new / v_new for several steps (a copy-on-write on the
    first one): rows against the oracle, caches bit for bit afterwards."""
    spec = workloads.custom(name="mqa-fused", seed=550 + Hq, dtype="bf16", lens=(5, 40, 16, 300, 33),
                            num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, prefix_len=20, decode_steps=18,
                            cache=cache)
    wl, gst, ost = _both(spec)
    assert gst.pool.seq_fork(gst.seq_ids[0]) == ost.pool.seq_fork(ost.seq_ids[0])
    mb = oracle_side.max_blocks_for(wl)
    q = gpu_side.to_device(wl.q, "bf16")
    byte = cache in ("i8", "fp8")
    saw_cow = False
    for step in range(spec.decode_steps):
        slots, cows = gst.pool.seq_append_batch(gst.seq_ids)
        if len(cows):
            saw_cow = True
            pairs = torch.from_numpy(cows.copy()).cuda()
            if byte:
                pa.pa_copy_blocks_int8(gst.k_cache, gst.v_cache, pairs, Hkv, D)
            else:
                pa.pa_copy_blocks(gst.k_cache, gst.v_cache, pairs, Hkv, D)
        oracle_side.advance(wl, ost, step)
        assert slots.tolist() == ost.step_slots[-1]
        tab_d, lens_d, _, lh = gpu_side.tables(gst, mb)
        out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        pa.pa_decode(out, q, gst.k_cache, gst.v_cache, tab_d, lens_d, Hkv, int(lh.max()), spec.fp32_scale(),
                     partition_tokens=pt, kernel=kern, k_new=gpu_side.to_device(wl.step_k[step], "bf16"),
                     v_new=gpu_side.to_device(wl.step_v[step], "bf16"),
                     slot_mapping=torch.from_numpy(slots.copy()).cuda())
        ref = oracle_side.decode(wl, ost, mb)
        err = np.max(np.abs(_f32(out) - ref))
        assert err <= 2e-3, (step, err)
    assert saw_cow
    torch.cuda.synchronize()
    for g, o in ((gst.k_cache, ost.k_cache), (gst.v_cache, ost.v_cache)):
        gb = gpu_side.to_host_bits(g)
        if byte:
            assert np.array_equal(gb.view(np.uint8), o.view(np.uint8))
        else:
            ob = o.view(np.uint16)
            written = ~(((ob & 0x7F80) == 0x7F80) & ((ob & 0x007F) != 0))
            assert np.array_equal(gb.view(np.uint16)[written], ob[written])


PREFIX = [("bf16", 128, 32, 1, 256, (1, 15, 16, 17, 300, 40)), ("f16", 64, 64, 1, 64, (5, 100, 33)),
          ("bf16", 128, 64, 2, 128, (20, 700, 3)), ("bf16", 128, 48, 1, 32, (7, 90))]


@pytest.mark.parametrize("case", range(len(PREFIX)))
def test_mqa_shared_prefix(case):
    dtype, D, Hq, Hkv, P, suffix = PREFIX[case]
    spec = workloads.custom(name="mqa-prefix", seed=560 + case, dtype=dtype, lens=suffix, num_q_heads=Hq,
                            num_kv_heads=Hkv, head_dim=D, prefix_len=P)
    wl, gst, ost = _both(spec)
    mb = oracle_side.max_blocks_for(wl)
    ref = oracle_side.decode(wl, ost, mb)
    tab_d, lens_d, _, lh = gpu_side.tables(gst, mb)
    q = gpu_side.to_device(wl.q, dtype)
    out = torch.full(q.shape, -9.0, dtype=torch.float32, device="cuda")
    pa.pa_decode(out, q, gst.k_cache, gst.v_cache, tab_d, lens_d, Hkv, int(lh.max()), spec.fp32_scale(),
                 shared_prefix_blocks=P // 16)
    err = np.max(np.abs(_f32(out) - ref))
    _say(f"  max_abs_err={err:.3e}")
    assert err <= 2e-3, err


EXTEND = [("bf16", 128, 32, 1, (130, 700, 33), (4, 4, 4)), ("f16", 64, 64, 1, (50, 300), (8, 33)),
          ("bf16", 128, 64, 2, (90, 260, 1000), (2, 7, 1)), ("bf16", 128, 40, 1, (100, 20), (5, 20))]


@pytest.mark.parametrize("case", range(len(EXTEND)))
def test_mqa_extend(case):
    dtype, D, Hq, Hkv, lens, news = EXTEND[case]
    spec = workloads.custom(name="mqa-extend", seed=570 + case, dtype=dtype, lens=lens, num_q_heads=Hq,
                            num_kv_heads=Hkv, head_dim=D)
    wl, gst, ost = _both(spec)
    mb = oracle_side.max_blocks_for(wl)
    qs = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    T = int(qs[-1])
    qh = workloads.round_to(np.random.default_rng(spec.seed + 1).standard_normal((T, Hq, D), dtype=np.float32),
                            dtype)
    tab, l = oracle_side.tables(ost, mb)
    ref = oracle.extend(qh, ost.k_cache, ost.v_cache, tab, l, qs, Hkv, spec.fp32_scale(), dtype)
    tab_d, lens_d, _, lh = gpu_side.tables(gst, mb)
    qd = gpu_side.to_device(qh, dtype)
    for pt in (0, 16, 64, 512):
        out = torch.full(qd.shape, -5.0, dtype=torch.float32, device="cuda")
        pa.pa_extend(out, qd, gst.k_cache, gst.v_cache, tab_d, lens_d, torch.from_numpy(qs).cuda(), Hkv,
                     int(lh.max()), max(news), spec.fp32_scale(), partition_tokens=pt)
        err = np.max(np.abs(_f32(out) - ref))
        _say(f"  partition_tokens={pt} max_abs_err={err:.3e}")
        assert err <= 2e-3, (pt, err)


def test_workload_11_mqa_sampled():
    spec = workloads.named(11)
    wl, gst, ost = _both(spec)
    mb = oracle_side.max_blocks_for(wl)
    sample = [0, 50, 101, 200, 255]
    ref = oracle_side.decode(wl, ost, mb, seq_subset=sample)
    for kern in ("auto", "valu"):
        out = gpu_side.decode(wl, gst, mb, out_dtype="f32", kernel=kern)
        err = np.max(np.abs(_f32(out)[sample] - ref))
        _say(f"  {spec.name} kernel={kern} max_abs_err={err:.3e}")
        assert err <= 2e-3, (kern, err)
        o16 = gpu_side.decode(wl, gst, mb, kernel=kern)
        assert torch.equal(o16.cpu().view(torch.int16), out.cpu().to(torch.bfloat16).view(torch.int16))
