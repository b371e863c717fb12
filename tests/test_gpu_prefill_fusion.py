"""The fp16 / bf16 prefill's finish and kv_b_proj in one launch, the
normalised latent staged in LDS (``mla_debug_set_prefill_fusion(1)``).

Every case runs the call with the one-launch finish + kv_b_proj and with the
two launches through compressed_kv, and checks:
- every output row of the one-launch call against the CPU oracle
  (1e-2 + 1e-2 |ref|);
- from 2048 tokens (where the separate finish adds kv_a_proj's K splits in
  ascending order, as the one-launch kernel always does), all four outputs
  bit for bit equal to the two-launch call's.

Shapes: the V2-Lite prefill at full size (T = 4096), ragged last row blocks
(T = 4100, 2050, 777, 100), bf16, head counts that give head groups of one
(nh = 1, 3, 5), the decode family's tiling forced past 64 tokens, the
paged-cache write of the first head group's workgroups, and replays of the
call captured in a HIP graph.
"""
import numpy as np
import pytest

import workloads
from workloads import V2LITE, Dims

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from parity import compare, gpu_rows, run_oracle, upload  # noqa: E402


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_attention_kv_amd as mla

    mla.lib()
    return torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _reset_hooks():
    yield
    import mla_attention_kv_amd as mla

    mla.mla_debug_set_prefill_fusion(-1)
    mla.mla_kv_prolog_force_path(-1)


def _both(w, t, path=None):
    """(one-launch outputs, two-launch outputs) of the same call."""
    import mla_attention_kv_amd as mla

    mla.mla_kv_prolog_force_path(-1 if path is None else path)
    res = {}
    for mode in (1, 0):
        assert mla.mla_debug_set_prefill_fusion(mode) in (-1, 0, 1)
        res[mode] = mla.mla_kv_prolog(t["X"], t["Wa"], t["gamma"], t["Wb"], t["pos"], w.eps,
                                      w.theta)
    torch.cuda.synchronize()
    return res[1], res[0]


def _bit_equal(a_outs, b_outs, label):
    for a, b, n in zip(a_outs, b_outs, ("k_nope", "value", "k_pe", "ckv")):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{label} {n}"


CASES = [
    # dims, dtype, T, forced path (None: the dispatcher's), seed
    (V2LITE, "f16", 4096, None, 1),   # the V2-Lite prefill workload's shape
    (V2LITE, "bf16", 4100, None, 2),  # last row block of 4 rows
    (V2LITE, "f16", 2050, None, 3),   # last row block of 2 rows, 2 K splits
    (V2LITE, "f16", 777, None, 4),    # under 2048 tokens: more K splits
    (V2LITE, "bf16", 100, None, 5),   # two row blocks, 16 K splits
    (Dims(H=2048, nh=1), "f16", 4096, None, 6),
    (Dims(H=2048, nh=3), "bf16", 3000, None, 7),
    (Dims(H=1024, nh=5), "f16", 2100, None, 8),
    (V2LITE, "f16", 200, 0, 9),       # the decode family's tiling past 64 tokens
]


@pytest.mark.parametrize("dims,dtype,T,path,seed", CASES)
def test_one_launch_finish_kv_b_every_row(dev, dims, dtype, T, path, seed):
    w = workloads.make_custom(dims, T, dtype=dtype, seed=1100 + seed, max_pos=32768)
    print(f"[prefill-fusion] H={dims.H} nh={dims.nh} {dtype} T={T} path={path}", flush=True)
    t = upload(w, dev)
    fused, split = _both(w, t, path)
    compare(gpu_rows(fused), run_oracle(w), f"one launch T={T}")
    if T >= 2048:
        _bit_equal(fused, split, f"one launch vs two, T={T}")


def test_one_launch_cached_write(dev):
    """The fused cache write (mla_kv_prolog_cached): only the first head
    group's workgroups write compressed_kv, k_pe and the cache rows; the
    cache and the outputs equal the two-launch call's bit for bit, and
    unmapped slots keep their contents."""
    import mla_attention_kv_amd as mla

    w = workloads.make_custom(V2LITE, 4100, dtype="bf16", seed=1150, max_pos=32768)
    slots, n = workloads.paged_slot_mapping(w, block_size=64, seed=3)
    slots = slots.copy()
    slots[::7] = -1  # some tokens write no slot
    print(f"[prefill-fusion] cached T={w.T} slots={n}", flush=True)
    t = upload(w, dev)
    sl = torch.from_numpy(slots).to(dev)
    res = {}
    for mode in (1, 0):
        mla.mla_debug_set_prefill_fusion(mode)
        cache = torch.full((n // 64, 64, 576), -1.75, dtype=t["X"].dtype, device=dev)
        outs = mla.mla_kv_prolog_cached(t["X"], t["Wa"], t["gamma"], t["Wb"], t["pos"], sl,
                                        cache, w.eps, w.theta)
        res[mode] = (outs, cache)
    torch.cuda.synchronize()
    _bit_equal(res[1][0], res[0][0], "cached")
    assert torch.equal(res[1][1].view(torch.int16), res[0][1].view(torch.int16)), "cache"
    ok = slots >= 0
    rows = torch.from_numpy(np.nonzero(ok)[0]).to(dev)
    got = res[1][1].view(n, 576)[torch.from_numpy(slots[ok]).to(dev)]
    mine = torch.cat([res[1][0][3][rows], res[1][0][2][rows]], dim=1)
    assert torch.equal(got.view(torch.int16), mine.view(torch.int16)), "cache != returned rows"
    compare(gpu_rows(res[1][0]), run_oracle(w), "one launch cached")


def test_one_launch_graph_replays(dev):
    """The one-launch call captured in a HIP graph: three replays, with new
    hidden rows and unrelated eager work between them, each give the bits of
    an eager call on the same inputs (the launch records no memset and
    allocates nothing)."""
    import mla_attention_kv_amd as mla

    w = workloads.make_custom(V2LITE, 4100, dtype="f16", seed=1170, max_pos=32768)
    print(f"[prefill-fusion] graph replays T={w.T}", flush=True)
    t = upload(w, dev)
    mla.mla_debug_set_prefill_fusion(1)
    x0 = t["X"].clone()
    args = (t["X"], t["Wa"], t["gamma"], t["Wb"], t["pos"], w.eps, w.theta)
    cap = torch.cuda.Stream(device=dev)
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        mla.mla_kv_prolog(*args)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        outs = mla.mla_kv_prolog(*args)
    for i in range(3):
        t["X"].copy_(x0 * (1.0 + 0.25 * i))
        junk = torch.randn(1 << 20, device=dev).abs().sum()
        g.replay()
        torch.cuda.synchronize()
        ref = mla.mla_kv_prolog(*args)
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        _bit_equal(outs, ref, f"replay {i}")
