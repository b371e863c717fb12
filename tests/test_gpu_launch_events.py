"""The per-kernel timing hook (mla_debug_set_launch_events) on the GPU: a
registered call records a pair of events at the start and end of each
kernel it launches, in launch order, and leaves the outputs bit for bit as
an unregistered call makes them; every kernel ends before the next starts
(one stream) and their durations fit in the call's span."""
import ctypes

import pytest

import workloads
from workloads import V2LITE, R1

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from parity import run_lib, upload  # noqa: E402


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_attention_kv_amd as mla

    mla.lib()
    return torch.device("cuda:0")


# (dims, T, kind, dtype, kernels per call): the decode family's two
# launches at T = 1, the fp16 prefill family's three, W8A8's four
CASES = [(V2LITE, 1, "fp", "f16", 2), (V2LITE, 300, "fp", "f16", 3),
         (R1, 40, "w8a8", "bf16", 4)]


@pytest.mark.parametrize("case", CASES, ids=["decode_T1", "prefill_T300", "w8a8_T40"])
def test_launch_events_one_per_kernel(dev, case):
    import mla_attention_kv_amd as mla

    dims, T, kind, dtype, nk = case
    print(f"launch events: {kind} {dtype} T={T}", flush=True)
    w = workloads.make_custom(dims, T, kind=kind, dtype=dtype, seed=11)
    t = upload(w, dev)
    ref, _ = run_lib(w, t)
    torch.cuda.synchronize()
    L = mla.lib()
    maxk = 8
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * maxk)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    arr = (ctypes.c_void_p * (2 * maxk))(*[e.cuda_event for e in evs])
    assert L.mla_debug_set_launch_events(arr, 2 * maxk) == 0
    try:
        got, _ = run_lib(w, t)
    finally:
        used = L.mla_debug_set_launch_events(None, 0)
    torch.cuda.synchronize()
    assert used == 2 * nk
    for a, b in zip(ref, got):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    durs = [evs[2 * k].elapsed_time(evs[2 * k + 1]) for k in range(nk)]
    gaps = [evs[2 * k + 1].elapsed_time(evs[2 * k + 2]) for k in range(nk - 1)]
    assert all(d > 0.0 for d in durs), durs
    assert all(x >= -1e-3 for x in gaps), gaps
    span = evs[0].elapsed_time(evs[2 * nk - 1])
    assert sum(durs) <= span + 1e-3
    # an unregistered call records nothing more
    run_lib(w, t)
    torch.cuda.synchronize()
    assert L.mla_debug_set_launch_events(None, 0) == 0
