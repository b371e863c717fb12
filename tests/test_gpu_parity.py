"""GPU parity: the HIP library against the CPU oracle, element by element.

Every case is a seeded synthetic workload from ``workloads``, and every
case compares every output row, the five benchmark workloads at full size
included (the R1 W8A8 prefill in chunks of rows).  The W8A8 int32
accumulators are compared bit for bit.
"""
import numpy as np
import pytest

import workloads
from workloads import V2LITE, R1, Dims

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


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


from parity import compare, gpu_rows, run_lib, run_oracle, sample_rows, upload  # noqa: E402


def check_full(w, dev, label, path=None, dbg=False):
    import mla_attention_kv_amd as mla

    if path is not None:
        mla.mla_kv_prolog_force_path(path)
    print(f"[parity] {label} T={w.T} path={path}", flush=True)
    t = upload(w, dev)
    outs, accs = run_lib(w, t, dbg_rows=(0, w.T) if dbg else None)
    torch.cuda.synchronize()
    ref = run_oracle(w)
    stats = compare(gpu_rows(outs), ref, label)
    if dbg:
        np.testing.assert_array_equal(accs[0].cpu().numpy(), ref["acc1"])
        np.testing.assert_array_equal(accs[1].cpu().numpy(), ref["acc2"])
    return stats, outs


# ---------------------------------------------------------------------------
# the five benchmark workloads at full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("idx", [0, 1])
def test_config_decode_full(dev, idx):
    w = workloads.make_config(idx)
    check_full(w, dev, f"config{idx}")


@pytest.mark.parametrize("idx", [2, 3])
def test_config_large_every_row(dev, idx):
    """V2-Lite prefill (T = 4096) and R1 decode (T = 256) at full size:
    every output row against the oracle."""
    w = workloads.make_config(idx)
    print(f"[parity] config{idx} T={w.T} every row", flush=True)
    t = upload(w, dev)
    outs, _ = run_lib(w, t)
    torch.cuda.synchronize()
    compare(gpu_rows(outs), run_oracle(w), f"config{idx}")


def test_config4_w8a8_every_row_and_exact_accumulators(dev):
    """The R1 W8A8 ragged prefill at full size (T = 12,874): every output row
    of the production launch against the oracle, and the int32 accumulators
    of both projections, from a second launch with the accumulator exports
    on, bit for bit on every row.  Compared in chunks of rows to bound host
    memory; the oracle runs once per chunk."""
    w = workloads.make_config(4)
    print(f"[parity] config4 T={w.T} lens={list(w.seq_lens)} every row", flush=True)
    t = upload(w, dev)
    outs, _ = run_lib(w, t)
    outs2, (d1, d2) = run_lib(w, t, dbg_rows=(0, w.T))
    torch.cuda.synchronize()
    chunk = 1024
    for b in range(0, w.T, chunk):
        rows = np.arange(b, min(w.T, b + chunk))
        ref = run_oracle(w, rows)
        compare(gpu_rows(outs, rows), ref, f"config4 rows {b}..")
        np.testing.assert_array_equal(d1[b:b + len(rows)].cpu().numpy(), ref["acc1"],
                                      err_msg=f"acc1 rows {b}..")
        np.testing.assert_array_equal(d2[b:b + len(rows)].cpu().numpy(), ref["acc2"],
                                      err_msg=f"acc2 rows {b}..")
        if b == 0:
            # the launch with the exports on computes the same outputs
            for x, y in zip(outs, outs2):
                assert torch.equal(x.view(torch.int16), y.view(torch.int16))


# ---------------------------------------------------------------------------
# ragged token counts, both kernel families
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("path", [0, 1])
@pytest.mark.parametrize("T", [1, 2, 3, 15, 16, 17, 33, 63, 64, 65, 127, 129])
def test_v2lite_fp16_token_counts(dev, T, path):
    w = workloads.make_custom(V2LITE, T, dtype="f16", seed=100 + T)
    check_full(w, dev, f"v2lite_f16_T{T}", path=path)


@pytest.mark.parametrize("path", [0, 1])
@pytest.mark.parametrize("T", [1, 2, 7, 64, 130])
def test_bf16_token_counts(dev, T, path):
    d = Dims(H=1024, nh=8)
    w = workloads.make_custom(d, T, dtype="bf16", seed=200 + T, wstd=0.03)
    check_full(w, dev, f"bf16_T{T}", path=path)


@pytest.mark.parametrize("path", [0, 1])
@pytest.mark.parametrize("T", [1, 5, 8, 9, 16, 17, 64, 131])
def test_w8a8_token_counts_exact(dev, T, path):
    # on the decode family: the quantiser folded into kv_a_proj up to 8
    # tokens, the finish fused into kv_b_proj up to 16, four launches beyond
    d = Dims(H=1024, nh=4)
    w = workloads.make_custom(d, T, kind="w8a8", dtype="bf16", seed=300 + T, wstd=0.02)
    check_full(w, dev, f"w8a8_T{T}", path=path, dbg=True)


# ---------------------------------------------------------------------------
# edge shapes
# ---------------------------------------------------------------------------

def test_minimal_hidden_single_head(dev):
    d = Dims(H=64, nh=1)
    w = workloads.make_custom(d, 5, dtype="f16", seed=400, wstd=0.1)
    check_full(w, dev, "H64_nh1")


def test_w8a8_long_prefill_ragged_tail_exact(dev):
    # W8A8 at a long token count: both projections on the pipelined kernel;
    # int32 accumulators of every row bit-exact
    d = Dims(H=512, nh=2)
    w = workloads.make_custom(d, 4100, kind="w8a8", dtype="bf16", seed=450, wstd=0.02,
                              max_pos=8192)
    check_full(w, dev, "w8a8_T4100", path=1, dbg=True)


@pytest.mark.parametrize("kind", ["fp16", "w8a8"])
def test_tall_kv_a_tiles(dev, kind):
    # 12000 tokens with a short K: the dispatcher takes 160-row kv_a_proj
    # tiles (225 tiles, one round over the CUs) and a ragged last tile
    d = Dims(H=256, nh=2)
    if kind == "w8a8":
        w = workloads.make_custom(d, 12000, kind="w8a8", dtype="bf16", seed=480, wstd=0.02,
                                  max_pos=16384)
        check_full(w, dev, "w8a8_T12000", path=1, dbg=True)
    else:
        w = workloads.make_custom(d, 12000, dtype="f16", seed=481, wstd=0.05, max_pos=16384)
        check_full(w, dev, "f16_T12000", path=1)


@pytest.mark.parametrize("nh,T", [(16, 5000), (3, 2049), (5, 3001), (1, 2080)])
def test_w8a8_weight_stationary_kv_b(dev, nh, T):
    # token counts that take the weight-stationary kv_b_proj kernel: row
    # ranges of more blocks than its ring has stages (nh = 16: 10 blocks of
    # 32 rows each), odd and single head counts, ragged last blocks (5000 =
    # 156 x 32 + 8, 2049, 3001), an odd and an even block count per range.
    # The production launch against the oracle on every row, then a launch
    # with the accumulator exports: bit-exact int32 accumulators and the same
    # outputs.
    d = Dims(H=512, nh=nh)
    w = workloads.make_custom(d, T, kind="w8a8", dtype="bf16", seed=490 + nh, wstd=0.02,
                              max_pos=8192)
    print(f"[parity] w8a8 weight-stationary kv_b nh={nh} T={T}", flush=True)
    t = upload(w, dev)
    outs, _ = run_lib(w, t)
    outs2, (d1, d2) = run_lib(w, t, dbg_rows=(0, w.T))
    torch.cuda.synchronize()
    ref = run_oracle(w)
    compare(gpu_rows(outs), ref, f"w8a8_ws_nh{nh}_T{T}")
    np.testing.assert_array_equal(d1.cpu().numpy(), ref["acc1"])
    np.testing.assert_array_equal(d2.cpu().numpy(), ref["acc2"])
    for x, y in zip(outs, outs2):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("dtype,nh,T", [("f16", 128, 4100), ("bf16", 257, 2049)])
def test_fp_weight_stationary_kv_b(dev, dtype, nh, T):
    # fp16 / bf16 prefills that take the weight-stationary kv_b_proj kernel
    # (row ranges of at least 2048 rows): two ranges of 2050 rows at R1's
    # head count with a ragged 4-row last block; an odd head count above the
    # CU count (more workgroups than fit at once) with one range and a
    # 1-row last block.  Every row against the oracle.
    d = Dims(H=512, nh=nh)
    w = workloads.make_custom(d, T, dtype=dtype, seed=520 + nh, wstd=0.03, max_pos=8192)
    check_full(w, dev, f"{dtype}_ws_nh{nh}_T{T}", path=1)


@pytest.mark.parametrize("H,T,path,nh", [(7168, 1, 0, 8), (7168, 5, 0, 8), (7168, 64, 0, 8),
                                         (2304, 3, 0, 4), (12288, 1, 1, 2), (16384, 2, 1, 2)])
def test_w8a8_many_splits_exact(dev, H, T, path, nh):
    # W8A8 calls whose kv_a_proj is split over K more than 8 ways (9 to 64
    # splits: H = 2304 on path 0 gives 9, R1's H = 7168 on path 0 gives 28,
    # H = 12288 and 16384 on path 1 give 48 and 64): the finish sums the
    # splits over four waves per token.  int32 accumulators of both
    # projections bit-exact, outputs within tolerance, every row.
    d = Dims(H=H, nh=nh)
    w = workloads.make_custom(d, T, kind="w8a8", dtype="bf16", seed=530 + T + H % 97,
                              wstd=0.01)
    check_full(w, dev, f"w8a8_H{H}_T{T}_p{path}", path=path, dbg=True)


@pytest.mark.parametrize("H,T", [(640, 7), (8320, 6)])
def test_w8a8_hidden_sizes_exact(dev, H, T):
    # the activation quantiser: H = 640 leaves lanes with a partial last chunk
    # (one wave per row), H = 8320 takes the long-row workgroup kernel; token
    # counts that are not a multiple of the four rows per workgroup
    d = Dims(H=H, nh=2)
    w = workloads.make_custom(d, T, kind="w8a8", dtype="bf16", seed=470 + T, wstd=0.02)
    check_full(w, dev, f"w8a8_H{H}_T{T}", path=1, dbg=True)


@pytest.mark.parametrize("T", [9, 40])
def test_decode_many_k_splits(dev, T):
    # more than 16 kv_a_proj K splits: the finish reads its later splits in
    # a second round of partial loads
    d = Dims(H=4096, nh=2)
    w = workloads.make_custom(d, T, dtype="f16", seed=440 + T, wstd=0.02)
    check_full(w, dev, f"H4096_T{T}", path=0)


def test_long_prefill_ragged_tail(dev):
    # long prefill (kv_a_proj without split-K, pipelined kv_b_proj) with a
    # token count that leaves partial tiles; every row checked
    d = Dims(H=512, nh=2)
    w = workloads.make_custom(d, 4100, dtype="f16", seed=430, wstd=0.03, max_pos=8192)
    check_full(w, dev, "prefill_T4100", path=1)


@pytest.mark.parametrize("T", [17, 40, 64])
def test_odd_head_count_multi_tile(dev, T):
    # kv_b_proj work items over an odd number of 64-column slab pairs with
    # several token tiles: every item must map to an existing slab
    d = Dims(H=256, nh=3)
    w = workloads.make_custom(d, T, dtype="f16", seed=410 + T, wstd=0.05)
    check_full(w, dev, f"nh3_T{T}", path=0)


@pytest.mark.parametrize("nh", [1, 3, 64])
@pytest.mark.parametrize("T", [1, 2])
def test_tiny_T_head_counts(dev, T, nh):
    # one or two tokens through the fused finish + kv_b_proj launch: with 1
    # or 3 heads some workgroups of the rounded-up grid have no slab but
    # still finish their token, with 64 heads the launch holds 256
    # workgroups (the most it runs fused)
    d = Dims(H=512, nh=nh)
    w = workloads.make_custom(d, T, dtype="f16", seed=430 + 10 * nh + T, wstd=0.04)
    check_full(w, dev, f"tiny_nh{nh}_T{T}", path=0)


@pytest.mark.parametrize("H,nh,T,dtype", [(7168, 8, 65, "bf16"), (7168, 8, 300, "f16"),
                                           (20480, 2, 65, "bf16"), (2048, 16, 100, "f16")])
def test_many_split_finish_prefill(dev, H, nh, T, dtype):
    # prefill-family calls whose kv_a_proj is split over K more than 8 ways
    # (16, 28 and 40 splits at these shapes) with under 2048 tokens: the
    # finish sums the splits over four waves per token.  Every row.
    d = Dims(H=H, nh=nh)
    w = workloads.make_custom(d, T, dtype=dtype, seed=720 + T + H % 101, wstd=0.01,
                              max_pos=32768)
    check_full(w, dev, f"wide_finish_H{H}_T{T}_{dtype}", path=1)


@pytest.mark.parametrize("dtype,T", [("bf16", 16), ("bf16", 64), ("f16", 33)])
def test_r1_decode_family(dev, dtype, T):
    # the decode family at R1 shape: the weight-streaming kv_a_proj over
    # H = 7168 and the fused finish + kv_b_proj over 512 slabs of W_kv_b (two
    # workgroups per CU when the device holds them all at once).  Every row
    # against the oracle, and no workgroup runs out of polls.
    import mla_attention_kv_amd as mla

    w = workloads.make_custom(R1, T, dtype=dtype, seed=740 + T, wstd=0.01, max_pos=32768)
    assert mla.mla_debug_handoff_fallbacks(reset=True) >= 0
    check_full(w, dev, f"r1_decode_{dtype}_T{T}", path=0)
    assert mla.mla_debug_handoff_fallbacks() == 0


def test_r1_shapes_small_T(dev):
    w = workloads.make_custom(R1, 3, dtype="bf16", seed=401, wstd=0.01, max_pos=32768)
    check_full(w, dev, "r1_T3")


def test_large_positions(dev):
    T = 32
    pos = np.array([0, 1, 2, 4095, 32767, 65535, 1 << 20, (1 << 31) - 1] * 4, np.int32)
    w = workloads.make_custom(V2LITE, T, dtype="f16", seed=402, positions=pos)
    check_full(w, dev, "large_positions")


def test_zero_tokens_is_noop(dev):
    import mla_attention_kv_amd as mla

    w = workloads.make_custom(V2LITE, 1, dtype="f16", seed=403)
    t = upload(w, dev)
    X0 = t["X"][:0]
    outs = mla.mla_kv_prolog(X0, t["Wa"], t["gamma"], t["Wb"], t["pos"][:0])
    assert all(o.shape[0] == 0 for o in outs)


@pytest.mark.parametrize("path", [0, 1])
@pytest.mark.parametrize("kind,dtype", [("fp", "f16"), ("fp", "bf16"), ("w8a8", "bf16")])
def test_signed_gamma_and_wide_activations(dev, kind, dtype, path):
    """gamma of both signs with exact zeros among its entries (the W8A8 path
    quantises z = c * gamma, so a sign or a zero must reach the codes the
    same way on both sides), and hidden rows whose scale spans 2^-6 .. 2^6
    from token to token.  Every row against the oracle; W8A8 accumulators
    bit-exact."""
    d = Dims(H=1024, nh=4)
    T = 40 if path == 0 else 200
    w = workloads.make_custom(d, T, kind=kind, dtype=dtype, seed=700 + T + len(dtype), wstd=0.02)
    rng = np.random.default_rng(701)
    g = rng.uniform(-1.5, 1.5, d.r).astype(np.float32)
    g[::37] = 0.0
    w.gamma = workloads.to_storage(g, dtype)
    x = workloads.widen(w.X, dtype) * np.exp2(rng.integers(-6, 7, (T, 1))).astype(np.float32)
    w.X = workloads.to_storage(x, dtype)
    check_full(w, dev, f"signed_gamma_{kind}_{dtype}_p{path}", path=path, dbg=(kind == "w8a8"))


def test_zero_row_w8a8(dev):
    """A token whose hidden row is all zeros: codes 0, scale 0, outputs 0."""
    d = Dims(H=256, nh=2)
    w = workloads.make_custom(d, 4, kind="w8a8", dtype="bf16", seed=404)
    w.X[2, :] = 0
    check_full(w, dev, "w8a8_zero_row", dbg=True)


def test_deterministic(dev):
    w = workloads.make_config(1)
    t = upload(w, dev)
    a, _ = run_lib(w, t)
    b, _ = run_lib(w, t)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_nondefault_stream_and_reused_workspace(dev):
    import mla_attention_kv_amd as mla

    w = workloads.make_config(1)
    t = upload(w, dev)
    ws = torch.zeros(mla.mla_kv_prolog_workspace_size(w.T, mla.Dims(H=2048, nh=16)),
                     dtype=torch.uint8, device=dev)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        outs1 = mla.mla_kv_prolog(t["X"], t["Wa"], t["gamma"], t["Wb"], t["pos"], workspace=ws)
        outs2 = mla.mla_kv_prolog(t["X"], t["Wa"], t["gamma"], t["Wb"], t["pos"], workspace=ws)
    s.synchronize()
    for x, y in zip(outs1, outs2):
        assert torch.equal(x, y)
    compare(gpu_rows(outs2), run_oracle(w), "stream")


@pytest.mark.parametrize("kind", ["fp", "w8a8"])
@pytest.mark.parametrize("path", [0, 1])
def test_garbage_workspace(dev, path, kind):
    """The result does not depend on what the workspace held before the call."""
    import mla_attention_kv_amd as mla

    d = Dims(H=1024, nh=4)
    T = 40
    w = workloads.make_custom(d, T, kind=kind, dtype="bf16", seed=520 + path, wstd=0.03)
    t = upload(w, dev)
    mla.mla_kv_prolog_force_path(path)
    try:
        md = mla.Dims(H=d.H, nh=d.nh)
        nb = (mla.mla_kv_prolog_workspace_size(T, md, mla.MLA_BF16) if kind == "fp"
              else mla.mla_kv_prolog_w8a8_workspace_size(T, md))
        res = []
        for fill in (0x00, 0xFF, 0x3C):
            ws = torch.full((nb,), fill, dtype=torch.uint8, device=dev)
            outs, _ = run_lib(w, t, workspace=ws)
            torch.cuda.synchronize()
            res.append([o.clone() for o in outs])
    finally:
        mla.mla_kv_prolog_force_path(-1)
    for other in res[1:]:
        for x, y in zip(res[0], other):
            assert torch.equal(x, y)
    compare(gpu_rows(res[0]), run_oracle(w), f"garbage_ws_{kind}_p{path}")


@pytest.mark.parametrize("T", [1, 64])
def test_decode_many_calls_one_workspace(dev, T):
    """Many back-to-back decode calls on one workspace that starts out filled
    with garbage (inputs changing between calls) all give the oracle's
    result."""
    import mla_attention_kv_amd as mla

    ws = torch.full((mla.mla_kv_prolog_workspace_size(T, mla.Dims(H=2048, nh=16)),), 0xA5,
                    dtype=torch.uint8, device=dev)
    cases = [workloads.make_custom(V2LITE, T, dtype="f16", seed=500 + T + i) for i in range(3)]
    ups = [upload(w, dev) for w in cases]
    refs = [run_oracle(w) for w in cases]
    outs = None
    for it in range(60):
        i = it % 3
        t = ups[i]
        outs = mla.mla_kv_prolog(t["X"], t["Wa"], t["gamma"], t["Wb"], t["pos"], workspace=ws)
        if it == 0 or it >= 57:
            torch.cuda.synchronize()
            compare(gpu_rows(outs), refs[i], f"repeat{it}")


# ---------------------------------------------------------------------------
# the decode family's finish + kv_b_proj hand-off
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 2, 17, 64])
def test_decode_handoff_normal_run_needs_no_fallback(dev, T):
    """On a normal call every latent row arrives through the hand-off: the
    fallback count stays at zero, and the outputs match the oracle."""
    import mla_attention_kv_amd as mla

    w = workloads.make_custom(V2LITE, T, dtype="f16", seed=600 + T)
    t = upload(w, dev)
    assert mla.mla_debug_handoff_fallbacks(reset=True) >= 0
    outs, _ = run_lib(w, t)
    torch.cuda.synchronize()
    assert mla.mla_debug_handoff_fallbacks() == 0
    compare(gpu_rows(outs), run_oracle(w), f"handoff_T{T}")


@pytest.mark.parametrize("T", [1, 2, 17, 64])
def test_decode_handoff_fallback_rebuilds_rows(dev, T):
    """With the poll bound set to 0 from the host, every kv_b_proj workgroup
    of the one-launch finish rebuilds its tile's latent rows itself from the
    split-K partials (no workgroup waits, every kernel exits normally).  The
    outputs are the same bits as the hand-off's, and match the oracle."""
    import mla_attention_kv_amd as mla

    w = workloads.make_custom(V2LITE, T, dtype="f16", seed=610 + T)
    t = upload(w, dev)
    ref_outs, _ = run_lib(w, t)
    torch.cuda.synchronize()
    prev = mla.mla_debug_set_handoff_spin(0)
    try:
        mla.mla_debug_handoff_fallbacks(reset=True)
        outs, _ = run_lib(w, t)
        torch.cuda.synchronize()
        n = mla.mla_debug_handoff_fallbacks(reset=True)
    finally:
        mla.mla_debug_set_handoff_spin(prev)
    ntile = (T + 15) // 16
    assert n == ntile * (V2LITE.N2 // 64), n   # every workgroup with a tile
    for a, b in zip(ref_outs, outs):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    compare(gpu_rows(outs), run_oracle(w), f"handoff_fallback_T{T}")


# W8A8 at decode sizes: the finish fused into kv_b_proj (up to 16 tokens)
W8DEC = Dims(H=7168, nh=128)   # R1: 28 kv_a_proj splits, 512 kv_b_proj slabs


@pytest.mark.parametrize("T", [1, 2, 7, 16])
def test_w8a8_decode_fused_handoff_exact(dev, T):
    """R1-shaped W8A8 calls of up to 16 tokens run the finish inside
    kv_b_proj's launch and hand the latent codes and scales over between
    workgroups.  On a normal call no workgroup falls back; the int32
    accumulators of both projections are bit-exact and the outputs match
    the oracle on every row; the launch with the accumulator exports gives
    the same outputs."""
    import mla_attention_kv_amd as mla

    w = workloads.make_custom(W8DEC, T, kind="w8a8", dtype="bf16", seed=640 + T, wstd=0.01,
                              max_pos=32768)
    print(f"[parity] w8a8 decode fused T={T}", flush=True)
    t = upload(w, dev)
    assert mla.mla_debug_handoff_fallbacks(reset=True) >= 0
    outs, _ = run_lib(w, t)
    torch.cuda.synchronize()
    assert mla.mla_debug_handoff_fallbacks() == 0
    outs2, (d1, d2) = run_lib(w, t, dbg_rows=(0, w.T))
    torch.cuda.synchronize()
    ref = run_oracle(w)
    compare(gpu_rows(outs), ref, f"w8a8_decode_T{T}")
    np.testing.assert_array_equal(d1.cpu().numpy(), ref["acc1"])
    np.testing.assert_array_equal(d2.cpu().numpy(), ref["acc2"])
    for x, y in zip(outs, outs2):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("dims,T", [(W8DEC, 1), (W8DEC, 16), (Dims(H=1024, nh=4), 5)])
def test_w8a8_decode_fallback_rebuilds_codes(dev, dims, T):
    """With the poll bound set to 0 from the host, every kv_b_proj workgroup
    of the fused W8A8 launch rebuilds its tile's latent codes and scales from
    the split-K partials (no workgroup waits).  The outputs and accumulators
    are the same bits as the hand-off's, and match the oracle."""
    import mla_attention_kv_amd as mla

    w = workloads.make_custom(dims, T, kind="w8a8", dtype="bf16", seed=650 + T, wstd=0.01)
    t = upload(w, dev)
    ref_outs, (r1, r2) = run_lib(w, t, dbg_rows=(0, w.T))
    torch.cuda.synchronize()
    prev = mla.mla_debug_set_handoff_spin(0)
    try:
        mla.mla_debug_handoff_fallbacks(reset=True)
        outs, (d1, d2) = run_lib(w, t, dbg_rows=(0, w.T))
        torch.cuda.synchronize()
        n = mla.mla_debug_handoff_fallbacks(reset=True)
    finally:
        mla.mla_debug_set_handoff_spin(prev)
    assert n == dims.N2 // 64, n   # every slab's workgroup
    for a, b in zip(ref_outs, outs):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(r2, d2) and torch.equal(r1, d1)
    ref = run_oracle(w)
    compare(gpu_rows(outs), ref, f"w8a8_decode_fallback_T{T}")
    np.testing.assert_array_equal(d2.cpu().numpy(), ref["acc2"])


@pytest.mark.parametrize("H,T,nh", [(3456, 4, 4), (128, 3, 2), (7168, 8, 128)])
def test_w8a8_decode_folded_quantiser_exact(dev, H, T, nh):
    """W8A8 calls of up to 8 tokens quantise their activations inside
    kv_a_proj: splits of 384 rows (H = 3456, 9 splits: a split narrower than
    the kernel's LDS slab), of 128 rows (H = 128, one split) and R1's 256
    rows at the largest such token count.  The int32 accumulators of both
    projections are bit-exact on every row, the outputs match the oracle."""
    d = Dims(H=H, nh=nh)
    w = workloads.make_custom(d, T, kind="w8a8", dtype="bf16", seed=660 + H % 89 + T,
                              wstd=0.01)
    check_full(w, dev, f"w8a8_fold_H{H}_T{T}", path=0, dbg=True)
