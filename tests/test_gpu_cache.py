"""GPU parity of the paged KV-cache append against the CPU oracle, bit for
bit (the fp cache holds copies; the int8 codes and scales are decided in
fp32 with the same operations on both sides).  Inputs are seeded synthetic
rows in the model dtype; every cache starts from a fill pattern that both
sides see, so untouched slots are checked too."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
R, DR = 512, 64


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_attention_kv_amd as mla

    mla.lib()
    return torch.device("cuda:0")


def inputs(T, S, dtype, seed, skips=True):
    rng = np.random.default_rng(seed)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    ckv = torch.from_numpy(rng.standard_normal((T, R)).astype(np.float32)).to(tdt)
    kpe = torch.from_numpy((rng.standard_normal((T, DR)) * 3).astype(np.float32)).to(tdt)
    if T:
        ckv[T // 2] = 0  # a zero latent row (int8: only the rope part sets the scale)
    slots = rng.permutation(S)[:T].astype(np.int64)
    if skips and T >= 8:
        slots[1], slots[3], slots[5], slots[7] = -1, S, S + 3, 1 << 40  # not cached
    return ckv, kpe, slots


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,S", [(1, 4), (37, 100), (64, 64), (517, 2048)])
def test_fp_cache_append(dev, dtype, T, S):
    import mla_attention_kv_amd as mla

    print(f"[cache] fp {dtype} T={T} S={S}", flush=True)
    ckv, kpe, slots = inputs(T, S, dtype, seed=600 + T)
    fill = torch.full((S, R + DR), -1.75, dtype=ckv.dtype)
    cache = fill.to(dev)
    mla.mla_kv_cache_append(ckv.to(dev), kpe.to(dev), torch.from_numpy(slots).to(dev), cache)
    torch.cuda.synchronize()
    ref = oracle.kv_cache_append(ckv.double().numpy(), kpe.double().numpy(), slots,
                                 fill.double().numpy())
    np.testing.assert_array_equal(cache.cpu().double().numpy(), ref)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,S", [(1, 4), (37, 100), (517, 2048)])
def test_int8_cache_append_exact(dev, dtype, T, S):
    import mla_attention_kv_amd as mla

    print(f"[cache] int8 {dtype} T={T} S={S}", flush=True)
    ckv, kpe, slots = inputs(T, S, dtype, seed=700 + T)
    q0 = np.full((S, R + DR), 99, np.int8)
    s0 = np.full(S, -2.0, np.float32)
    q = torch.from_numpy(q0.copy()).to(dev)
    sc = torch.from_numpy(s0.copy()).to(dev)
    mla.mla_kv_cache_append_int8(ckv.to(dev), kpe.to(dev), torch.from_numpy(slots).to(dev), q, sc)
    torch.cuda.synchronize()
    rq, rs = oracle.kv_cache_append_int8(ckv.float().numpy(), kpe.float().numpy(), slots, q0, s0)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
    np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def test_cache_append_large_sampled(dev):
    # decode-cache sized: 4096 tokens into 1M slots (1.2 GB fp16 cache); the
    # written slots and a sample of the untouched ones are compared
    import mla_attention_kv_amd as mla

    T, S = 4096, 1 << 20
    print(f"[cache] large T={T} S={S}", flush=True)
    ckv, kpe, slots = inputs(T, S, "f16", seed=800, skips=False)
    cache = torch.full((S, R + DR), 0.5, dtype=torch.float16, device=dev)
    mla.mla_kv_cache_append(ckv.to(dev), kpe.to(dev), torch.from_numpy(slots).to(dev), cache)
    q = torch.zeros((S, R + DR), dtype=torch.int8, device=dev)
    sc = torch.zeros(S, dtype=torch.float32, device=dev)
    mla.mla_kv_cache_append_int8(ckv.to(dev), kpe.to(dev), torch.from_numpy(slots).to(dev), q, sc)
    torch.cuda.synchronize()
    got = cache[torch.from_numpy(slots).to(dev)].cpu().double().numpy()
    np.testing.assert_array_equal(got[:, :R], ckv.double().numpy())
    np.testing.assert_array_equal(got[:, R:], kpe.double().numpy())
    others = np.setdiff1d(np.random.default_rng(1).integers(0, S, 2000), slots)
    assert torch.all(cache[torch.from_numpy(others).to(dev)] == 0.5)
    rq, rs = oracle.kv_cache_append_int8(ckv.float().numpy(), kpe.float().numpy(),
                                         np.arange(T, dtype=np.int64),
                                         np.zeros((T, R + DR), np.int8), np.zeros(T, np.float32))
    np.testing.assert_array_equal(q[torch.from_numpy(slots).to(dev)].cpu().numpy(), rq)
    np.testing.assert_array_equal(sc[torch.from_numpy(slots).to(dev)].cpu().numpy(), rs)
