"""GPU parity over a seeded sweep of shapes away from the five workloads:
small and uneven hidden sizes (partial last K splits of the decode family,
one-slab K ranges), odd head counts, ragged token counts on both sides of
the dispatcher's threshold, fp16 / bf16 and W8A8 (exact accumulators)."""
import numpy as np
import pytest

import workloads
from workloads import Dims



torch = pytest.importorskip("torch")

from parity import compare, gpu_rows, run_lib, run_oracle, upload  # noqa: E402


def sweep(n, seed):
    # W8A8 needs H % 128 == 0; it is drawn here from H >= 512
    rng = np.random.default_rng(seed)
    Hs = [128, 192, 320, 704, 1536, 2112, 4096]
    Hq = [512, 768, 1536, 4096]
    nhs = [1, 2, 5, 8, 17, 33, 64]
    Ts = [1, 2, 5, 16, 31, 48, 64, 65, 100, 257]
    out = []
    i = 0
    while len(out) < n:
        kind = "w8a8" if i % 3 == 2 else "fp"
        H = int(rng.choice(Hq if kind == "w8a8" else Hs))
        nh = int(rng.choice(nhs))
        T = int(rng.choice(Ts))
        dtype = "bf16" if (kind == "w8a8" or i % 2) else "f16"
        i += 1
        if (H, nh, T, kind, dtype) not in out:
            out.append((H, nh, T, kind, dtype))
    return out


CASES = sweep(24, 2024)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_attention_kv_amd as mla

    mla.lib()
    return torch.device("cuda:0")


def test_sweep_is_supported():
    # every drawn shape is one the library accepts (checked without a GPU)
    import mla_attention_kv_amd as mla

    for H, nh, T, kind, dtype in CASES:
        d = mla.Dims(H=H, nh=nh)
        code = mla.MLA_F16 if dtype == "f16" else mla.MLA_BF16
        nb = (mla.mla_kv_prolog_w8a8_workspace_size(T, d) if kind == "w8a8"
              else mla.mla_kv_prolog_workspace_size(T, d, code))
        assert nb > 0, (H, nh, T, kind, dtype)


@pytest.mark.gpu
@pytest.mark.parametrize("H,nh,T,kind,dtype", CASES)
def test_shape_sweep(dev, H, nh, T, kind, dtype):
    print(f"[shapes] H={H} nh={nh} T={T} {kind} {dtype}", flush=True)
    w = workloads.make_custom(Dims(H=H, nh=nh), T, kind=kind, dtype=dtype,
                              seed=H * 7 + nh * 131 + T, wstd=0.5 / np.sqrt(H),
                              max_pos=1 << 20)
    t = upload(w, dev)
    outs, accs = run_lib(w, t, dbg_rows=(0, T) if kind == "w8a8" else None)
    torch.cuda.synchronize()
    ref = run_oracle(w)
    compare(gpu_rows(outs), ref, f"H{H} nh{nh} T{T} {kind} {dtype}")
    if kind == "w8a8":
        np.testing.assert_array_equal(accs[0].cpu().numpy(), ref["acc1"])
        np.testing.assert_array_equal(accs[1].cpu().numpy(), ref["acc2"])
