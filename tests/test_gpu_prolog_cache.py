"""GPU parity of the prolog with the paged KV-cache append fused into its
finish (mla_kv_prolog_cached, mla_kv_prolog_w8a8_cached).

Each case checks, on seeded synthetic inputs and a paged slot mapping:
  * the four returned outputs against the CPU oracle's prolog (the
    1e-2 + 1e-2 |ref| tolerance of the other parity tests);
  * the cache against the oracle's prolog outputs placed by the oracle's
    append (same tolerance on written slots; untouched slots keep their fill
    bit for bit);
  * that every written slot holds exactly the bits of the returned rows, and
    that the returned outputs equal those of the plain prolog bit for bit
    (the fused write changes no arithmetic).
The int8 cache of the W8A8 prolog is checked bit for bit against the
standalone int8 append of the returned rows, and dequantised against the
oracle's values.
"""
import numpy as np
import pytest

import oracle
import workloads
from workloads import V2LITE, Dims

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
FILL = -1.75  # untouched slots keep this value


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_attention_kv_amd as mla

    mla.lib()
    return torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _reset_path():
    yield
    try:
        import mla_attention_kv_amd as mla

        mla.mla_kv_prolog_force_path(-1)
    except Exception:
        pass


from parity import ATOL, RTOL, compare, gpu_rows, run_oracle, sample_rows, upload  # noqa: E402


def skip_some(slots, num_slots):
    """Padding tokens: a few mapped outside [0, num_slots) (not cached)."""
    s = slots.copy()
    if len(s) >= 8:
        s[1], s[4], s[6] = -1, num_slots, 1 << 40
    return s


def run_cached(w, dev, slots, num_slots, block_size=64, path=None):
    import mla_attention_kv_amd as mla

    if path is not None:
        mla.mla_kv_prolog_force_path(path)
    t = upload(w, dev)
    tdt = t["X"].dtype
    W = w.dims.r + w.dims.dr
    cache = torch.full((num_slots // block_size, block_size, W), FILL, dtype=tdt, device=dev)
    sl = torch.from_numpy(slots).to(dev)
    outs = mla.mla_kv_prolog_cached(t["X"], t["Wa"], t["gamma"], t["Wb"], t["pos"], sl, cache,
                                    w.eps, w.theta)
    plain = mla.mla_kv_prolog(t["X"], t["Wa"], t["gamma"], t["Wb"], t["pos"], w.eps, w.theta)
    torch.cuda.synchronize()
    for a, b, n in zip(outs, plain, ("k_nope", "value", "k_pe", "ckv")):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{n}: fused != plain"
    return outs, cache.view(num_slots, W)


def check_cache_rows(outs, cache, slots, num_slots, ref, rows):
    """Written slots: the returned rows' exact bits, and the oracle within
    tolerance.  ``ref`` holds the oracle outputs of token rows ``rows``."""
    k_pe, ckv = outs[2], outs[3]
    rows = np.asarray(rows)
    ok = (slots[rows] >= 0) & (slots[rows] < num_slots)
    r_ok = rows[ok]
    s_dev = torch.from_numpy(slots[r_ok]).to(cache.device)
    got = cache[s_dev]
    mine = torch.cat([ckv[torch.from_numpy(r_ok).to(cache.device)],
                      k_pe[torch.from_numpy(r_ok).to(cache.device)]], dim=1)
    assert torch.equal(got.view(torch.int16), mine.view(torch.int16)), "cache != returned rows"
    # the oracle: its own outputs placed by its own append into a cache of
    # just the checked slots
    refc = oracle.kv_cache_append(ref["ckv"][ok], ref["k_pe"][ok],
                                  np.arange(len(r_ok), dtype=np.int64),
                                  np.full((len(r_ok), cache.shape[1]), FILL))
    g = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(g - refc)
    bad = ~(err <= ATOL + RTOL * np.abs(refc))
    assert not bad.any(), f"{int(bad.sum())} cache values out of tolerance"


def check_untouched(cache, slots, num_slots):
    """Slots no token maps to still hold the fill, bit for bit."""
    mapped = slots[(slots >= 0) & (slots < num_slots)]
    changed = (cache != FILL).any(dim=1).nonzero().flatten().cpu().numpy()
    extra = np.setdiff1d(changed, mapped)
    assert extra.size == 0, f"slots written that no token maps to: {extra[:8]}"
    assert changed.size == np.unique(mapped).size, "a mapped slot was not written"


CASES = [
    # (dims, dtype, T, path, wstd): the decode family with the fused finish +
    # kv_b_proj launch, the decode family with a separate finish launch
    # (more than 256 sixteen-token items), and the tiled family
    (V2LITE, "f16", 1, 0, 0.02),
    (V2LITE, "f16", 17, 0, 0.02),
    (V2LITE, "f16", 64, 0, 0.02),
    (Dims(H=1024, nh=64), "bf16", 17, 0, 0.03),
    (V2LITE, "f16", 1, 1, 0.02),
    (V2LITE, "f16", 130, 1, 0.02),
    (Dims(H=1024, nh=8), "bf16", 300, 1, 0.03),
]


@pytest.mark.parametrize("dims,dtype,T,path,wstd", CASES)
def test_prolog_cached_small(dev, dims, dtype, T, path, wstd):
    w = workloads.make_custom(dims, T, dtype=dtype, seed=900 + T + path, wstd=wstd)
    slots, n = workloads.paged_slot_mapping(w, block_size=16, seed=T)
    slots = skip_some(slots, n)
    print(f"[prolog-cache] H={dims.H} nh={dims.nh} {dtype} T={T} path={path} slots={n}",
          flush=True)
    outs, cache = run_cached(w, dev, slots, n, block_size=16, path=path)
    ref = run_oracle(w)
    compare(gpu_rows(outs), ref, f"cached T{T}")
    check_cache_rows(outs, cache, slots, n, ref, np.arange(T))
    check_untouched(cache, slots, n)


@pytest.mark.parametrize("idx", [0, 1])
def test_prolog_cached_decode_configs(dev, idx):
    w = workloads.make_config(idx)
    slots, n = workloads.paged_slot_mapping(w, seed=idx)
    print(f"[prolog-cache] config{idx} T={w.T} slots={n}", flush=True)
    outs, cache = run_cached(w, dev, slots, n)
    ref = run_oracle(w)
    compare(gpu_rows(outs), ref, f"cached config{idx}")
    check_cache_rows(outs, cache, slots, n, ref, np.arange(w.T))
    check_untouched(cache, slots, n)


@pytest.mark.parametrize("idx,nsample", [(2, 24), (3, 16)])
def test_prolog_cached_large_sampled(dev, idx, nsample):
    w = workloads.make_config(idx)
    slots, n = workloads.paged_slot_mapping(w, seed=idx)
    slots = skip_some(slots, n)
    print(f"[prolog-cache] config{idx} T={w.T} slots={n} sampled {nsample}", flush=True)
    outs, cache = run_cached(w, dev, slots, n)
    rows = np.unique(np.concatenate([sample_rows(w.T, nsample, seed=idx), [0, 1, 4, 6]]))
    ref = run_oracle(w, rows)
    compare(gpu_rows(outs, rows), ref, f"cached config{idx}")
    check_cache_rows(outs, cache, slots, n, ref, rows)
    # every token's slot holds its returned rows, bit for bit
    ok = (slots >= 0) & (slots < n)
    allr = torch.from_numpy(np.nonzero(ok)[0]).to(dev)
    mine = torch.cat([outs[3][allr], outs[2][allr]], dim=1)
    got = cache[torch.from_numpy(slots[ok]).to(dev)]
    assert torch.equal(got.view(torch.int16), mine.view(torch.int16))
    check_untouched(cache, slots, n)


def test_prolog_cached_without_slots(dev):
    # num_slots == 0: the plain prolog, nothing written
    import mla_attention_kv_amd as mla

    w = workloads.make_custom(V2LITE, 5, seed=3)
    t = upload(w, dev)
    empty = torch.empty((0, 576), dtype=t["X"].dtype, device=dev)
    sl = torch.zeros(5, dtype=torch.int64, device=dev)
    outs = mla.mla_kv_prolog_cached(t["X"], t["Wa"], t["gamma"], t["Wb"], t["pos"], sl, empty,
                                    w.eps, w.theta)
    torch.cuda.synchronize()
    compare(gpu_rows(outs), run_oracle(w), "cached no slots")


# ---------------------------------------------------------------------------
# W8A8 prolog with a bf16 cache or the int8 ("C8") cache
# ---------------------------------------------------------------------------

def run_w8_cached(w, dev, slots, num_slots, q8):
    import mla_attention_kv_amd as mla

    t = upload(w, dev)
    W = w.dims.r + w.dims.dr
    sl = torch.from_numpy(slots).to(dev)
    args = (t["X"], t["Wqa"], t["swa"], t["gamma"], t["Wqb"], t["swb"], t["pos"])
    if q8:
        cq = torch.full((num_slots, W), 99, dtype=torch.int8, device=dev)
        cs = torch.full((num_slots,), -2.0, dtype=torch.float32, device=dev)
        outs = mla.mla_kv_prolog_w8a8_cached(*args, sl, w.eps, w.theta, kv_cache_q=cq,
                                             kv_scale=cs)
        cache = (cq, cs)
    else:
        cb = torch.full((num_slots, W), FILL, dtype=torch.bfloat16, device=dev)
        outs = mla.mla_kv_prolog_w8a8_cached(*args, sl, w.eps, w.theta, kv_cache=cb)
        cache = cb
    plain = mla.mla_kv_prolog_w8a8(*args, w.eps, w.theta)
    torch.cuda.synchronize()
    for a, b, n in zip(outs, plain, ("k_nope", "value", "k_pe", "ckv")):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{n}: fused != plain"
    return outs, cache


def check_c8(outs, cq, cs, slots, num_slots, ref, rows):
    """The int8 cache: bit for bit what the standalone int8 append makes of
    the returned rows (that kernel is pinned bit-exact to the oracle), and,
    dequantised, within half a quantisation step of the oracle's values plus
    the output tolerance.  Untouched slots keep their fill."""
    import mla_attention_kv_amd as mla

    dev = cq.device
    W = cq.shape[1]
    q2 = torch.full_like(cq, 99)
    s2 = torch.full_like(cs, -2.0)
    mla.mla_kv_cache_append_int8(outs[3], outs[2], torch.from_numpy(slots).to(dev), q2, s2)
    torch.cuda.synchronize()
    assert torch.equal(cq, q2), "int8 codes differ from the standalone append"
    assert torch.equal(cs.view(torch.int32), s2.view(torch.int32)), "scales differ"
    rows = np.asarray(rows)
    ok = (slots[rows] >= 0) & (slots[rows] < num_slots)
    sidx = torch.from_numpy(slots[rows][ok]).to(dev)
    codes = cq[sidx].cpu().numpy().astype(np.float64)
    scale = cs[sidx].cpu().numpy().astype(np.float64)
    deq = codes * scale[:, None]
    refv = np.concatenate([ref["ckv"][ok], ref["k_pe"][ok]], axis=1)
    bound = 0.5 * scale[:, None] * (1 + 1e-6) + ATOL + RTOL * np.abs(refv)
    bad = ~(np.abs(deq - refv) <= bound)
    assert not bad.any(), f"{int(bad.sum())} dequantised cache values out of bound"
    assert np.all(np.abs(codes).max(axis=1) == 127), "each slot's largest code is 127"
    mapped = slots[(slots >= 0) & (slots < num_slots)]
    untouched = np.setdiff1d(np.arange(num_slots), mapped)
    if untouched.size:
        u = torch.from_numpy(untouched).to(dev)
        assert bool((cq[u] == 99).all()) and bool((cs[u] == -2.0).all())


@pytest.mark.parametrize("q8", [False, True])
@pytest.mark.parametrize("T", [5, 12, 40, 131])
def test_prolog_w8a8_cached_small(dev, T, q8):
    # T = 5: quantiser folded into kv_a_proj and finish fused into kv_b_proj;
    # 12: the fused finish alone; 40: four launches; 131: the prefill family
    w = workloads.make_custom(Dims(H=1024, nh=8), T, kind="w8a8", dtype="bf16", seed=950 + T,
                              wstd=0.03)
    slots, n = workloads.paged_slot_mapping(w, block_size=16, seed=T)
    slots = skip_some(slots, n)
    print(f"[prolog-cache] w8a8 T={T} q8={q8} slots={n}", flush=True)
    outs, cache = run_w8_cached(w, dev, slots, n, q8)
    ref = run_oracle(w)
    compare(gpu_rows(outs), ref, f"w8a8 cached T{T}")
    if q8:
        check_c8(outs, cache[0], cache[1], slots, n, ref, np.arange(T))
    else:
        check_cache_rows(outs, cache, slots, n, ref, np.arange(T))
        check_untouched(cache, slots, n)


@pytest.mark.parametrize("q8", [False, True])
def test_prolog_w8a8_cached_config4_sampled(dev, q8):
    w = workloads.make_config(4)
    slots, n = workloads.paged_slot_mapping(w, seed=4)
    slots = skip_some(slots, n)
    print(f"[prolog-cache] config4 T={w.T} q8={q8} slots={n}", flush=True)
    outs, cache = run_w8_cached(w, dev, slots, n, q8)
    rows = np.unique(np.concatenate([sample_rows(w.T, 12, seed=44), [0, 1, 4, 6]]))
    ref = run_oracle(w, rows)
    compare(gpu_rows(outs, rows), ref, "w8a8 cached config4")
    if q8:
        check_c8(outs, cache[0], cache[1], slots, n, ref, rows)
    else:
        check_cache_rows(outs, cache, slots, n, ref, rows)
        check_untouched(cache, slots, n)
