"""GPU tests of the captured decode buckets (mla_prolog_graphs_*).

A graph set records one prolog call per token-count bucket over static
buffers.  Each step here writes T token rows into those buffers, launches
the set (the smallest bucket >= T runs) and checks:
  * bit for bit, every output row of the bucket against a direct call of the
    same entry point over the same buffer contents (a graph replays exactly
    the launches of that call);
  * the first T rows against the CPU oracle (the 1e-2 + 1e-2 |ref| bar);
  * with a cache: the slots equal those the direct cached call writes, the
    padding rows (slot -1) write nothing.
Steps replay every graph several times with eager torch work between them,
each replay checked on its own.
"""
import numpy as np
import pytest

import workloads
from workloads import V2LITE, Dims

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from parity import compare, gpu_rows, run_oracle, sample_rows, upload  # noqa: E402

FILL = -1.75


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_attention_kv_amd as mla

    mla.lib()
    return torch.device("cuda:0")


def bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int8)


def outputs(g, n):
    return (g.k_nope[:n], g.value[:n], g.k_pe[:n], g.compressed_kv[:n])


def head(ref, n):
    return {k: ref[k][:n] for k in ("k_nope", "value", "k_pe", "ckv")}


def eager_noise(dev):
    # unrelated eager work between replays
    a = torch.randn(4096, device=dev)
    return float((a * a).sum())


def direct_fp(g, t, b, w, cache=None):
    """The plain entry point over the first b rows of the set's buffers."""
    import mla_attention_kv_amd as mla

    args = (g.hidden[:b].clone(), t["Wa"], t["gamma"], t["Wb"], g.positions[:b].clone())
    if cache is None:
        return mla.mla_kv_prolog(*args, w.eps, w.theta)
    return mla.mla_kv_prolog_cached(*args, g.slot_mapping[:b].clone(), cache, w.eps, w.theta)


def test_graphs_fp16_buckets(dev):
    import mla_attention_kv_amd as mla

    buckets = (1, 2, 4, 8, 16, 32, 64, 128)
    w = workloads.make_custom(V2LITE, 128, dtype="f16", seed=1201)
    t = upload(w, dev)
    ref = run_oracle(w)
    g = mla.PrologGraphs((t["Wa"], t["gamma"], t["Wb"]), buckets, w.eps, w.theta)
    assert [g.bucket(T) for T in (1, 3, 5, 64, 65, 128, 129)] == [1, 4, 8, 64, 128, 128, 0]
    for rep in range(2):
        for T in (1, 3, 17, 64, 100, 128):
            print(f"[graphs] fp16 V2-Lite rep={rep} T={T}", flush=True)
            g.hidden[:T] = t["X"][:T]
            g.positions[:T] = t["pos"][:T]
            b = g.run(T)
            assert b == g.bucket(T)
            d = direct_fp(g, t, b, w)
            torch.cuda.synchronize()
            for x, y, n in zip(outputs(g, b), d, ("k_nope", "value", "k_pe", "ckv")):
                assert torch.equal(bits(x), bits(y)), f"T={T} {n}: graph != direct call"
            compare(gpu_rows(outputs(g, T)), head(ref, T),
                    f"graphs T{T}")
            eager_noise(dev)
    g.close()


def test_graphs_r1_bf16_sampled(dev):
    import mla_attention_kv_amd as mla

    w = workloads.make_config(3)
    t = upload(w, dev)
    g = mla.PrologGraphs((t["Wa"], t["gamma"], t["Wb"]), (64, 256), w.eps, w.theta)
    for T in (256, 40, 256):
        print(f"[graphs] R1 bf16 T={T}", flush=True)
        g.hidden[:T] = t["X"][:T]
        g.positions[:T] = t["pos"][:T]
        b = g.run(T)
        d = direct_fp(g, t, b, w)
        torch.cuda.synchronize()
        for x, y in zip(outputs(g, b), d):
            assert torch.equal(bits(x), bits(y))
        rows = sample_rows(T, 12, seed=T)
        compare(gpu_rows(outputs(g, T), rows), run_oracle(w, rows), f"graphs R1 T{T}")
        eager_noise(dev)


def test_graphs_cached_padding(dev):
    import mla_attention_kv_amd as mla

    w = workloads.make_custom(V2LITE, 64, dtype="f16", seed=1202)
    slots, nsl = workloads.paged_slot_mapping(w, block_size=16, seed=5)
    t = upload(w, dev)
    W = w.dims.r + w.dims.dr
    cache = torch.full((nsl, W), FILL, dtype=torch.float16, device=dev)
    g = mla.PrologGraphs((t["Wa"], t["gamma"], t["Wb"]), (16, 64), w.eps, w.theta, cache=cache)
    ref = run_oracle(w)
    sl = torch.from_numpy(slots).to(dev)
    for T in (50, 9, 64):
        print(f"[graphs] cached T={T}", flush=True)
        g.hidden[:T] = t["X"][:T]
        g.positions[:T] = t["pos"][:T]
        g.slot_mapping[:T] = sl[:T]
        g.slot_mapping[T:] = -1  # padding rows write no slot
        cache.fill_(FILL)
        b = g.run(T)
        torch.cuda.synchronize()
        got = cache.clone()
        cache2 = torch.full_like(cache, FILL)
        d = direct_fp(g, t, b, w, cache=cache2)
        torch.cuda.synchronize()
        assert torch.equal(bits(got), bits(cache2)), f"T={T}: cache differs from the direct call"
        for x, y in zip(outputs(g, b), d):
            assert torch.equal(bits(x), bits(y))
        written = (got != FILL).any(dim=1).nonzero().flatten().cpu().numpy()
        assert np.array_equal(np.sort(written), np.sort(slots[:T])), "slots written"
        mine = torch.cat([g.compressed_kv[:T], g.k_pe[:T]], dim=1)
        assert torch.equal(bits(got[sl[:T]]), bits(mine))
        compare(gpu_rows(outputs(g, T)), head(ref, T), f"cached T{T}")
        eager_noise(dev)


def test_graphs_w8a8_int8_cache(dev):
    import mla_attention_kv_amd as mla

    dims = Dims(H=1024, nh=8)
    w = workloads.make_custom(dims, 16, kind="w8a8", dtype="bf16", seed=1203, wstd=0.03)
    slots, nsl = workloads.paged_slot_mapping(w, block_size=16, seed=6)
    t = upload(w, dev)
    W = dims.r + dims.dr
    cq = torch.full((nsl, W), 99, dtype=torch.int8, device=dev)
    cs = torch.full((nsl,), -2.0, dtype=torch.float32, device=dev)
    weights = (t["Wqa"], t["swa"], t["gamma"], t["Wqb"], t["swb"])
    g = mla.PrologGraphs(weights, (4, 16), w.eps, w.theta, w8a8=True, cache=(cq, cs))
    ref = run_oracle(w)
    sl = torch.from_numpy(slots).to(dev)
    # each bucket replayed twice, with eager work in between
    for T in (3, 16, 11, 4):
        print(f"[graphs] w8a8 T={T}", flush=True)
        g.hidden[:T] = t["X"][:T]
        g.positions[:T] = t["pos"][:T]
        g.slot_mapping[:T] = sl[:T]
        g.slot_mapping[T:] = -1
        cq.fill_(99)
        cs.fill_(-2.0)
        b = g.run(T)
        torch.cuda.synchronize()
        q1, s1 = cq.clone(), cs.clone()
        q2 = torch.full_like(cq, 99)
        s2 = torch.full_like(cs, -2.0)
        d = mla.mla_kv_prolog_w8a8_cached(
            g.hidden[:b].clone(), *weights[:2], weights[2], *weights[3:],
            g.positions[:b].clone(), g.slot_mapping[:b].clone(), w.eps, w.theta,
            kv_cache_q=q2, kv_scale=s2)
        torch.cuda.synchronize()
        for x, y in zip(outputs(g, b), d):
            assert torch.equal(bits(x), bits(y))
        assert torch.equal(q1, q2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32))
        compare(gpu_rows(outputs(g, T)), head(ref, T), f"w8a8 T{T}")
        eager_noise(dev)


def test_graphs_update_layers(dev):
    # two "layers": other weights and another cache, rebound in place
    import mla_attention_kv_amd as mla

    ws = [workloads.make_custom(V2LITE, 32, dtype="f16", seed=1300 + i) for i in range(2)]
    ts = [upload(w, dev) for w in ws]
    refs = [run_oracle(w) for w in ws]
    W = 576
    caches = [torch.full((64, W), FILL, dtype=torch.float16, device=dev) for _ in range(2)]
    g = mla.PrologGraphs((ts[0]["Wa"], ts[0]["gamma"], ts[0]["Wb"]), (8, 32), cache=caches[0])
    for step, layer in enumerate((0, 1, 0, 1)):
        w, t = ws[layer], ts[layer]
        if step > 0:
            g.update((t["Wa"], t["gamma"], t["Wb"]), w.eps, w.theta, cache=caches[layer])
        T = 32 if step % 2 == 0 else 7
        print(f"[graphs] update step={step} layer={layer} T={T}", flush=True)
        g.hidden[:T] = t["X"][:T]
        g.positions[:T] = t["pos"][:T]
        g.slot_mapping[:T] = torch.arange(T, device=dev) + 32 * layer
        g.slot_mapping[T:] = -1
        b = g.run(T)
        d = direct_fp(g, t, b, w)
        torch.cuda.synchronize()
        for x, y in zip(outputs(g, b), d):
            assert torch.equal(bits(x), bits(y))
        compare(gpu_rows(outputs(g, T)), head(refs[layer], T),
                f"layer {layer} T{T}")
        mine = torch.cat([g.compressed_kv[:T], g.k_pe[:T]], dim=1)
        assert torch.equal(bits(caches[layer][32 * layer:32 * layer + T]), bits(mine))
    # the other layer's cache rows were written by its own steps only
    assert bool((caches[0][32:] == FILL).all()) and bool((caches[1][:32] == FILL).all())


def test_graphs_launch_errors(dev):
    import mla_attention_kv_amd as mla

    w = workloads.make_custom(V2LITE, 4, dtype="f16", seed=1204)
    t = upload(w, dev)
    g = mla.PrologGraphs((t["Wa"], t["gamma"], t["Wb"]), (4,))
    assert g.run(0) == 0
    with pytest.raises(mla.MlaError) as e:
        g.run(5)
    assert e.value.status == mla.MLA_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        g.update((t["Wa"], t["gamma"][:256].contiguous(), t["Wb"]))
    g.close()
    g.close()


def test_graphs_multi_layer(dev):
    """One set over three layers, each with its own weights and cache: one
    launch replays all three prologs in layer order.  Every layer's outputs
    equal a direct call of that layer, bit for bit, and the oracle within
    tolerance; its cache rows hold its own returned rows.  Then the set is
    rebound to the layers in reverse order and checked again; every graph is
    replayed several times with eager work in between."""
    import mla_attention_kv_amd as mla

    L = 3
    ws = [workloads.make_custom(V2LITE, 64, dtype="f16", seed=1400 + i) for i in range(L)]
    ts = [upload(w, dev) for w in ws]
    # one shared hidden / positions input (the set's static rows): every
    # layer reads layer 0's token rows
    refs = [run_oracle(dataclasses_replace(ws[l], X=ws[0].X, positions=ws[0].positions))
            for l in range(L)]
    caches = [torch.full((64, 576), FILL, dtype=torch.float16, device=dev) for _ in range(L)]
    weights = [(t["Wa"], t["gamma"], t["Wb"]) for t in ts]
    g = mla.PrologGraphs(weights, (4, 16, 64), ws[0].eps, ws[0].theta, cache=caches)
    assert mla.lib().mla_prolog_graphs_layers(g.handle) == L
    assert tuple(g.k_nope.shape) == (L, 64, 16, 128)
    order = list(range(L))
    for step, T in enumerate((5, 64, 16, 64)):
        if step == 2:
            order = order[::-1]
            g.update([weights[l] for l in order], cache=[caches[l] for l in order])
        print(f"[graphs] {L} layers step={step} T={T} order={order}", flush=True)
        g.hidden[:T] = ts[0]["X"][:T]
        g.positions[:T] = ts[0]["pos"][:T]
        g.slot_mapping[:T] = torch.arange(T, device=dev)
        g.slot_mapping[T:] = -1
        for rep in range(2):
            b = g.run(T)
            torch.cuda.synchronize()
            for i, l in enumerate(order):
                t = ts[l]
                d = mla.mla_kv_prolog(g.hidden[:b].clone(), t["Wa"], t["gamma"], t["Wb"],
                                      g.positions[:b].clone(), ws[l].eps, ws[l].theta)
                torch.cuda.synchronize()
                mine = (g.k_nope[i, :b], g.value[i, :b], g.k_pe[i, :b], g.compressed_kv[i, :b])
                for x, y in zip(mine, d):
                    assert torch.equal(bits(x), bits(y)), f"layer {l} T={T}"
                compare(gpu_rows(tuple(m[:T] for m in mine)), head(refs[l], T),
                        f"layer {l} T{T}")
                row = torch.cat([g.compressed_kv[i, :T], g.k_pe[i, :T]], dim=1)
                assert torch.equal(bits(caches[l][:T]), bits(row))
            eager_noise(dev)
    g.close()


def dataclasses_replace(w, **kw):
    import dataclasses

    return dataclasses.replace(w, **kw)
