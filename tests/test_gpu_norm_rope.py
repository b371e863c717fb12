"""GPU parity of the standalone RMSNorm and RoPE against the CPU oracle.

Tolerance: both kernels compute in fp32 and round once to the model dtype,
so each value must lie within one unit in the last place of the dtype
(2^-10 relative for fp16, 2^-7 for bf16) of the oracle's fp32 value, plus,
for RoPE, 1e-6 of the inputs' magnitude for the fp32 rotation (cos and sin
to about 1e-7); this is tighter than the prolog's 1e-2 + 1e-2 |ref|, which
is asserted as well.  In-place calls must give the same bits.
"""
import numpy as np
import pytest

import oracle
from workloads import to_storage, widen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ULP = {"f16": 2.0 ** -10, "bf16": 2.0 ** -7}
TINY = {"f16": 2.0 ** -24, "bf16": 2.0 ** -133}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_attention_kv_amd as mla

    mla.lib()
    return torch.device("cuda:0")


def to_dev(a32, dtype, dev):
    st = to_storage(a32, dtype)
    if dtype == "f16":
        t = torch.from_numpy(st)
    else:
        t = torch.from_numpy(st.view(np.int16)).view(torch.bfloat16)
    return t.to(dev), widen(st, dtype).astype(np.float64)


def check(got, ref, dtype, extra=0.0, label=""):
    g = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(g - ref)
    bound = ULP[dtype] * np.abs(ref) + TINY[dtype] + extra
    bad = ~(err <= bound)
    assert not bad.any(), (f"{label}: {int(bad.sum())} of {bad.size} beyond one ulp; "
                           f"worst {float((err - bound).max())}")
    assert np.all(err <= 1e-2 + 1e-2 * np.abs(ref)), label


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("rows,n", [(1, 512), (5, 512), (257, 512), (3, 8), (7, 520),
                                    (4, 4096), (3, 8192), (4096, 512)])
def test_rms_norm(dev, dtype, rows, n):
    import mla_attention_kv_amd as mla

    print(f"[norm] rms {dtype} rows={rows} n={n}", flush=True)
    rng = np.random.default_rng(rows * 7 + n)
    scale = rng.uniform(0.05, 20.0, (rows, 1))
    xt, x = to_dev((rng.standard_normal((rows, n)) * scale).astype(np.float32), dtype, dev)
    gt, g = to_dev(rng.uniform(0.5, 1.5, n).astype(np.float32), dtype, dev)
    if rows > 2:
        xt[2] = 0  # zero row: output zeros
        x[2] = 0
    y = mla.mla_rms_norm(xt, gt, 1e-6)
    ref = oracle.rms_norm(x, g, 1e-6)
    torch.cuda.synchronize()
    check(y, ref, dtype, label=f"rms {rows}x{n}")
    xi = xt.clone()
    mla.mla_rms_norm(xi, gt, 1e-6, out=xi)
    torch.cuda.synchronize()
    assert torch.equal(xi.view(torch.int16), y.view(torch.int16)), "in place differs"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,heads", [(1, 1), (7, 1), (33, 16), (256, 128), (4096, 1),
                                     (5, 3)])
def test_rope(dev, dtype, T, heads):
    import mla_attention_kv_amd as mla

    print(f"[norm] rope {dtype} T={T} heads={heads}", flush=True)
    rng = np.random.default_rng(T * 13 + heads)
    xt, x = to_dev((rng.standard_normal((T, heads, 64)) * 3).astype(np.float32), dtype, dev)
    pos = rng.integers(0, 32768, T).astype(np.int32)
    if T >= 3:
        pos[0], pos[1], pos[2] = 0, (1 << 24) + 3, (1 << 31) - 1  # identity and huge angles
    pt = torch.from_numpy(pos).to(dev)
    y = mla.mla_rope(xt, pt, 1e4)
    ref = oracle.rope(x, pos, 1e4)
    torch.cuda.synchronize()
    mag = np.abs(x) + np.abs(np.concatenate([x[..., 32:], x[..., :32]], axis=-1))
    check(y, ref, dtype, extra=1e-6 * mag, label=f"rope T{T} h{heads}")
    if T >= 1:
        assert torch.equal(y[0].view(torch.int16), xt[0].view(torch.int16)) or pos[0] != 0
    yi = xt.clone()
    mla.mla_rope(yi, pt, 1e4, out=yi)
    torch.cuda.synchronize()
    assert torch.equal(yi.view(torch.int16), y.view(torch.int16)), "in place differs"
    if heads == 1:
        y2 = mla.mla_rope(xt[:, 0].contiguous(), pt, 1e4)  # [T, 64] form
        torch.cuda.synchronize()
        assert torch.equal(y2.view(torch.int16), y[:, 0].view(torch.int16))


@pytest.mark.parametrize("T,heads", [(1100, 128), (30001, 9), (4200, 128), (70001, 8)])
def test_rope_many_rows_sampled(dev, T, heads):
    # launches that give each wave 2, 4 or 8 row groups (the cos / sin reuse
    # across a token's heads, tokens changing inside a wave's rows, a ragged
    # last workgroup); all heads of sampled tokens are compared
    import mla_attention_kv_amd as mla

    print(f"[norm] rope bf16 T={T} heads={heads} sampled", flush=True)
    rng = np.random.default_rng(T + heads)
    xt, x = to_dev(rng.standard_normal((T, heads, 64)).astype(np.float32), "bf16", dev)
    pos = rng.integers(0, 1 << 20, T).astype(np.int32)
    pt = torch.from_numpy(pos).to(dev)
    y = mla.mla_rope(xt, pt, 1e4)
    torch.cuda.synchronize()
    tok = np.unique(np.concatenate([rng.choice(T, 48, replace=False), [0, 1, T - 2, T - 1]]))
    ref = oracle.rope(x[tok], pos[tok], 1e4)
    xs = x[tok]
    mag = np.abs(xs) + np.abs(np.concatenate([xs[..., 32:], xs[..., :32]], axis=-1))
    check(y[torch.from_numpy(tok).to(dev)], ref, "bf16", extra=1e-6 * mag,
          label=f"rope T{T} h{heads}")


def test_rope_alternating_theta(dev):
    # calls with different bases in a row (the frequencies of the last base
    # are kept per host thread and must be recomputed when it changes),
    # through the standalone RoPE and the prolog's k_pe
    import mla_attention_kv_amd as mla
    import workloads
    from parity import compare, gpu_rows, run_oracle, upload

    rng = np.random.default_rng(77)
    xt, x = to_dev(rng.standard_normal((40, 4, 64)).astype(np.float32), "bf16", dev)
    pos = rng.integers(0, 1 << 20, 40).astype(np.int32)
    pt = torch.from_numpy(pos).to(dev)
    w = workloads.make_custom(workloads.V2LITE, 5, dtype="f16", seed=78)
    t = upload(w, dev)
    mag = np.abs(x) + np.abs(np.concatenate([x[..., 32:], x[..., :32]], axis=-1))
    for theta in (1e4, 5e5, 1e4, 10.0, 5e5):
        print(f"[norm] rope theta={theta}", flush=True)
        y = mla.mla_rope(xt, pt, theta)
        outs = mla.mla_kv_prolog(t["X"], t["Wa"], t["gamma"], t["Wb"], t["pos"], w.eps, theta)
        torch.cuda.synchronize()
        check(y, oracle.rope(x, pos, theta), "bf16", extra=1e-6 * mag, label=f"theta {theta}")
        w.theta = theta
        compare(gpu_rows(outs), run_oracle(w), f"prolog theta {theta}")
