"""GPU parity at sizes where output offsets pass 2^31 (elements and bytes).

V2-Lite fp16 at T = 2^20 + 4099 puts k_nope / value element offsets
(T x 16 heads x 128) past 2^31; R1 W8A8 at T = 2^17 + 1029 does the same
for its [T, 128, 128] outputs and puts the int8 activation copy past 2^29
bytes.  Inputs are drawn on the device from a seeded generator (the host
would need tens of GB for them); the oracle runs on sampled rows copied
back, so every checked value is the oracle's.
"""
import numpy as np
import pytest

import workloads
from workloads import R1, V2LITE

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from parity import compare, gpu_rows, run_oracle, upload  # noqa: E402


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_attention_kv_amd as mla

    mla.lib()
    return torch.device("cuda:0")


def device_inputs(T, H, dtype, seed, dev, max_pos):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    X = torch.randn((T, H), generator=g, device=dev, dtype=torch.float32).to(dtype)
    pos = torch.randint(0, max_pos, (T,), generator=g, device=dev, dtype=torch.int32)
    return X, pos


def sampled(T, extra, seed):
    rng = np.random.default_rng(seed)
    rows = {0, 1, T // 2, T - 2, T - 1, *extra}
    rows.update(int(r) for r in rng.integers(0, T, 10))
    return np.array(sorted(r for r in rows if 0 <= r < T))


def host_rows(w, X, pos, rows):
    """The workload w (weights from it) with the sampled token rows of the
    device inputs."""
    idx = torch.from_numpy(rows).to(X.device)
    xr = X[idx].cpu()
    if X.dtype == torch.float16:
        xs = xr.numpy()
    else:
        xs = xr.view(torch.int16).numpy().view(np.uint16)
    w.X, w.positions, w.T = xs, pos[idx].cpu().numpy().astype(np.int32), len(rows)
    return w


def test_v2lite_fp16_past_2_31_elements(dev):
    import mla_attention_kv_amd as mla

    T = (1 << 20) + 4099
    print(f"[large] V2-Lite fp16 T={T}", flush=True)
    w = workloads.make_custom(V2LITE, 1, dtype="f16", seed=901)
    t = upload(w, dev)
    X, pos = device_inputs(T, V2LITE.H, torch.float16, 902, dev, 1 << 16)
    outs = mla.mla_kv_prolog(X, t["Wa"], t["gamma"], t["Wb"], pos, w.eps, w.theta)
    torch.cuda.synchronize()
    # rows whose k_nope / value offsets lie past 2^31 elements: t * 2048 >= 2^31
    rows = sampled(T, [(1 << 20) - 1, 1 << 20, (1 << 20) + 1], 903)
    ref = run_oracle(host_rows(w, X, pos, rows))
    compare(gpu_rows(outs, rows), ref, "v2lite T>2^20")
    del outs, X


def test_r1_w8a8_past_2_31_elements(dev):
    import mla_attention_kv_amd as mla

    T = (1 << 17) + 1029
    print(f"[large] R1 W8A8 T={T}", flush=True)
    w = workloads.make_custom(R1, 1, kind="w8a8", dtype="bf16", seed=911, wstd=0.01)
    t = upload(w, dev)
    X, pos = device_inputs(T, R1.H, torch.bfloat16, 912, dev, 1 << 15)
    rows = sampled(T, [(1 << 16) - 1, 1 << 16, (1 << 17) - 1, 1 << 17], 913)
    b = T - 6
    d1 = torch.full((4, R1.N1), -7, dtype=torch.int32, device=dev)
    d2 = torch.full((4, R1.N2), -7, dtype=torch.int32, device=dev)
    outs = mla.mla_kv_prolog_w8a8(X, t["Wqa"], t["swa"], t["gamma"], t["Wqb"], t["swb"], pos,
                                  w.eps, w.theta, dbg_acc1=d1, dbg_acc2=d2, dbg_row_begin=b,
                                  dbg_rows=4)
    torch.cuda.synchronize()
    ref = run_oracle(host_rows(w, X, pos, rows))
    compare(gpu_rows(outs, rows), ref, "r1 w8a8 T>2^17")
    # the exact int32 accumulators of four consecutive rows near the end
    w4 = host_rows(w, X, pos, np.arange(b, b + 4))
    ref4 = run_oracle(w4)
    np.testing.assert_array_equal(d1.cpu().numpy(), ref4["acc1"])
    np.testing.assert_array_equal(d2.cpu().numpy(), ref4["acc2"])
    del outs, X
