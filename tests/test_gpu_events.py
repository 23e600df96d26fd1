"""Launch events on the decode entry points (start_event / stop_event).

The events are recorded from the kernel dispatches themselves; the outputs
must be bitwise those of calls without events, the stop event must complete
after the call's work, and a call that launches nothing must still record
the events it was given.
"""
import ctypes

import pytest

torch = pytest.importorskip("torch")

from paged_kv_cache_65_amd import binding as pa  # noqa: E402
from paged_kv_cache_65_amd import workloads  # noqa: E402
from tests import gpu_side, oracle_side  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(oracle_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()


class _Events:
    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        for n in ("hipEventCreateWithFlags", "hipEventSynchronize", "hipEventElapsedTime",
                  "hipEventDestroy", "hipEventQuery"):
            getattr(self.hip, n).restype = ctypes.c_int
        self.made = []

    def new(self):
        h = ctypes.c_void_p()
        assert self.hip.hipEventCreateWithFlags(ctypes.byref(h), 0) == 0
        self.made.append(h.value)
        return h.value

    def ms(self, a, b):
        assert self.hip.hipEventSynchronize(ctypes.c_void_p(b)) == 0
        t = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return t.value

    def close(self):
        for h in self.made:
            self.hip.hipEventDestroy(ctypes.c_void_p(h))


@pytest.fixture()
def events():
    e = _Events()
    yield e
    e.close()


def _case():
    spec = workloads.custom(seed=66, dtype="bf16", lens=(1500, 20, 700, 33), num_q_heads=16,
                            num_kv_heads=2, head_dim=128)
    wl = workloads.generate(spec)
    return spec, wl, gpu_side.build(wl), oracle_side.max_blocks_for(wl)


def _params(spec, wl, gst, mb, out, pt, start=None, stop=None):
    tab_d, lens_d, _, l = gpu_side.tables(gst, mb)
    q = gpu_side.to_device(wl.q, "bf16")
    prm = pa.make_decode_params(out, q, gst.k_cache, gst.v_cache, tab_d, lens_d, spec.num_kv_heads,
                                int(l.max()), spec.fp32_scale(), partition_tokens=pt,
                                start_event=start, stop_event=stop)
    return prm, (tab_d, lens_d, q)


# 256: partitions + merge kernel; 0: automatic; -1: balanced split + merge; 2048: one
# partition, no merge launch
@pytest.mark.parametrize("pt", [256, 0, -1, 2048])
def test_decode_with_events_is_bitwise_the_same(events, pt):
    spec, wl, gst, mb = _case()
    print(f"[case] events pt={pt}", flush=True)
    ref = gpu_side.decode(wl, gst, mb, out_dtype="f32", partition_tokens=pt)
    out = torch.full(ref.shape, -3.0, dtype=torch.float32, device="cuda")
    a, b = events.new(), events.new()
    prm, keep = _params(spec, wl, gst, mb, out, pt, a, b)
    need = pa.pa_decode_workspace_bytes(prm)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
    ptr, n = pa._ws(ws)
    pa._check(pa.lib().pa_decode(ctypes.byref(prm), ptr, n, pa._stream(None)))
    t = events.ms(a, b)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert 0.0 < t < 1000.0


@pytest.mark.parametrize("pt", [256, 0, -1, 2048])
def test_split_launches_with_events(events, pt):
    spec, wl, gst, mb = _case()
    print(f"[case] split events pt={pt}", flush=True)
    ref = gpu_side.decode(wl, gst, mb, out_dtype="f32", partition_tokens=pt)
    out = torch.full(ref.shape, -3.0, dtype=torch.float32, device="cuda")
    a, b, c, d = events.new(), events.new(), events.new(), events.new()
    prm, keep = _params(spec, wl, gst, mb, out, pt, a, b)
    need = pa.pa_decode_workspace_bytes(prm)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
    pa.pa_decode_partitions(prm, ws if need else None)
    prm.start_event, prm.stop_event = c, d
    pa.pa_decode_merge(prm, ws if need else None)
    t_part, t_merge, t_all = events.ms(a, b), events.ms(c, d), events.ms(a, d)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert t_part > 0.0 and t_merge >= 0.0
    assert t_all >= t_part


def test_empty_batch_still_records_events(events):
    spec, wl, gst, mb = _case()
    out = torch.zeros((spec.num_seqs, spec.num_q_heads, spec.head_dim), dtype=torch.float32, device="cuda")
    a, b = events.new(), events.new()
    prm, keep = _params(spec, wl, gst, mb, out, 0, a, b)
    prm.num_seqs = 0
    ws = torch.zeros(max(pa.pa_decode_workspace_bytes(prm), 16), dtype=torch.uint8, device="cuda")
    ptr, n = pa._ws(ws)
    pa._check(pa.lib().pa_decode(ctypes.byref(prm), ptr, n, pa._stream(None)))
    assert events.ms(a, b) >= 0.0
    c, d = events.new(), events.new()
    prm.start_event, prm.stop_event = c, d
    pa._check(pa.lib().pa_decode_partitions(ctypes.byref(prm), ptr, n, pa._stream(None)))
    pa._check(pa.lib().pa_decode_merge(ctypes.byref(prm), ptr, n, pa._stream(None)))
    assert events.ms(c, d) >= 0.0
    torch.cuda.synchronize()
    assert not out.any()
