"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: numpy's /
torch's own format conversions, closed forms, invariants of RMSNorm and of
the rotary encoding, special weight matrices that turn a step into a known
permutation, and exact integer brute force for the W8A8 accumulators.  The
set is chosen so that a plausible slip anywhere in the oracle (a dropped
term, a wrong sign, a swapped index, a transposed operand, a wrong split
order, a missing rounding) fails at least one of them.

The method: the seven-step KV prolog of the DeepSeek-V2-Lite MLA migration
guide (section "Background"), with the data flow of its "Source-level
principle" section and the RoPE form and shapes of its "Precision
verification" section.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from workloads import Dims, bf16_bits_to_f32, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

TINY = Dims(H=12, nh=2, r=8, dr=4, dn=3, dv=5)
U32 = 2.0 ** -24  # unit roundoff of fp32


def run_fp(X, Wa, g, Wb, pos, dims, eps=1e-6, theta=10000.0, dtype="f16"):
    return oracle.kv_prolog_fp(X, Wa, g, Wb, pos, r=dims.r, dr=dims.dr, nh=dims.nh,
                               dn=dims.dn, dv=dims.dv, eps=eps, theta=theta,
                               dtype=dtype)


def f16v(a):
    """Values rounded to fp16 (as float64): the model dtype of the inputs."""
    return np.asarray(a, np.float64).astype(np.float16).astype(np.float64)


def sum_bound(n, absdot):
    """Rigorous bound on the error of an n-term fp32 sum of exact products
    (recursive summation): gamma_n * sum |x_k w_k|, gamma_n = n u / (1 - n u)."""
    return n * U32 / (1 - n * U32) * absdot


def rand_case(dims, T, seed, pos=None):
    rng = np.random.default_rng(seed)
    X = f16v(rng.standard_normal((T, dims.H)))
    Wa = f16v(rng.standard_normal((dims.H, dims.N1)) * 0.3)
    g = f16v(rng.uniform(0.5, 1.5, dims.r))
    Wb = f16v(rng.standard_normal((dims.r, dims.N2)) * 0.3)
    if pos is None:
        pos = rng.integers(0, 4096, T)
    return X, Wa, g, Wb, np.asarray(pos, np.int32)


def identity_Wa(dims):
    """W_kv_a = [I | 0]: latent c = X[:, :r], rope input p = X[:, r:r+dr]."""
    assert dims.H >= dims.N1
    Wa = np.zeros((dims.H, dims.N1))
    Wa[np.arange(dims.N1), np.arange(dims.N1)] = 1.0
    return Wa


# ----------------------------------------------------------------------------
# storage-format rounding
# ----------------------------------------------------------------------------

def test_round_fp16_matches_numpy():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000),
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -24, 2.0 ** -25,
         3 * 2.0 ** -26, 2.0 ** -14, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 1e9],
    ])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).astype(np.float64)
    got = oracle.round_to_dtype(x, "f16")
    np.testing.assert_array_equal(got, ref)


def test_round_bf16_matches_torch_and_double_ties():
    rng = np.random.default_rng(2)
    x32 = (rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000)).astype(np.float32)
    ref = bf16_bits_to_f32(f32_to_bf16_bits(x32)).astype(np.float64)
    got = oracle.round_to_dtype(x32.astype(np.float64), "bf16")
    np.testing.assert_array_equal(got, ref)
    # ties to even and a value just above a tie (only visible from double)
    cases = {
        1 + 2.0 ** -8: 1.0,
        1 + 3 * 2.0 ** -8: 1 + 2.0 ** -6,
        1 + 2.0 ** -8 + 2.0 ** -40: 1 + 2.0 ** -7,
        -(1 + 2.0 ** -8): -1.0,
    }
    got = oracle.round_to_dtype(np.array(list(cases)), "bf16")
    np.testing.assert_array_equal(got, np.array(list(cases.values())))


# ----------------------------------------------------------------------------
# kv_a_proj and split
# ----------------------------------------------------------------------------

def test_kv_a_proj_and_split_order_against_library_matmul():
    """At position 0 the rope output is the rope slice of X @ W_kv_a itself
    (RoPE at angle 0 is the identity), so k_pe pins kv_a_proj, its operand
    order (W_kv_a stored [H, r+dr]) and that the rope columns are the LAST dr,
    to within the fp32 summation bound."""
    d = TINY
    X, Wa, g, Wb, _ = rand_case(d, 5, 3)
    out = run_fp(X, Wa, g, Wb, np.zeros(5, np.int32), d)
    A = X @ Wa
    bound = sum_bound(d.H, np.abs(X) @ np.abs(Wa))
    assert np.all(np.abs(out["k_pe"] - A[:, d.r:]) <= bound[:, d.r:])


def test_integer_projections_are_exact():
    """Small integer inputs keep every fp32 partial sum exact (|sum| < 2^24),
    so both projections must equal the integer matrix products exactly: this
    pins indexing and layout of kv_a_proj and kv_b_proj bit for bit."""
    d = Dims(H=40, nh=3, r=8, dr=4, dn=2, dv=3)
    rng = np.random.default_rng(21)
    X = rng.integers(-20, 21, (4, d.H)).astype(np.float64)
    Wa = rng.integers(-20, 21, (d.H, d.N1)).astype(np.float64)
    # one-hot rows make the RMSNorm output a known set of fp16 values, and
    # an integer W_kv_b keeps kv_b_proj's sums exact
    Wb = rng.integers(-8, 9, (d.r, d.N2)).astype(np.float64)
    out = run_fp(X, Wa, np.ones(d.r), Wb, np.zeros(4, np.int32), d)
    A = (X.astype(np.int64) @ Wa.astype(np.int64)).astype(np.float64)
    np.testing.assert_array_equal(out["k_pe"], A[:, d.r:])
    yq = out["ckv"].astype(np.float16).astype(np.float64)
    B = (yq @ Wb).reshape(4, d.nh, d.dn + d.dv)
    bound = sum_bound(d.r, (np.abs(yq) @ np.abs(Wb))).reshape(4, d.nh, d.dn + d.dv)
    assert np.all(np.abs(out["k_nope"] - B[:, :, :d.dn]) <= bound[:, :, :d.dn])
    assert np.all(np.abs(out["value"] - B[:, :, d.dn:]) <= bound[:, :, d.dn:])


def test_fp32_accumulator_runs_in_ascending_order():
    """The sums are single fp32 accumulators in ascending k.  Rope column 0
    sums the products 2^24, 1, -2^24 (bf16 values) in that order: 2^24 + 1
    rounds to 2^24 (a tie, to even), so the sum is 0.  Rope column 1 sums the
    same terms reversed, -2^24 + 1 = -(2^24 - 1) is exact, so the sum is 1.
    A wider accumulator gives [1, 1]; a descending loop gives [1, 0]."""
    d = Dims(H=3, nh=1, r=2, dr=2, dn=1, dv=1)
    X = np.ones((1, 3))
    Wa = np.zeros((3, 4))
    Wa[:, 0] = [1.0, 0.0, 0.0]
    Wa[:, 1] = [0.0, 1.0, 0.0]
    Wa[:, 2] = [2.0 ** 24, 1.0, -(2.0 ** 24)]
    Wa[:, 3] = [-(2.0 ** 24), 1.0, 2.0 ** 24]
    out = run_fp(X, Wa, np.ones(2), np.zeros((2, 2)), np.zeros(1, np.int32), d,
                 dtype="bf16")
    np.testing.assert_array_equal(out["k_pe"][0], [0.0, 1.0])


def test_identity_weight_split_is_exact():
    d = Dims(H=16, nh=2, r=8, dr=4, dn=3, dv=5)
    rng = np.random.default_rng(4)
    X = f16v(rng.standard_normal((3, d.H)))
    out = run_fp(X, identity_Wa(d), np.ones(d.r), np.zeros((d.r, d.N2)),
                 np.zeros(3, np.int32), d, eps=0.0)
    np.testing.assert_array_equal(out["k_pe"], X[:, d.r:d.N1])
    c = X[:, :d.r]
    rms = np.sqrt(np.mean(c * c, axis=1, keepdims=True))
    np.testing.assert_allclose(out["ckv"], c / rms, rtol=4e-7)


# ----------------------------------------------------------------------------
# RMSNorm
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("v,eps", [(1.0, 0.5), (-0.37, 1e-6), (3.0, 2.0), (1e-4, 1e-6)])
def test_rmsnorm_constant_row_closed_form(v, eps):
    """A latent row of constant value v maps to gamma * v / sqrt(v^2 + eps):
    the mean runs over the r latent columns only (the rope columns of the
    row hold a different value), eps sits inside the root, gamma multiplies
    after the normalisation."""
    d = Dims(H=16, nh=1, r=8, dr=4, dn=2, dv=2)
    v = float(f16v(v))
    X = np.zeros((1, d.H))
    X[0, :d.r] = v
    X[0, d.r:d.N1] = f16v(7.0 * v + 1.0)
    g = f16v(np.linspace(0.5, 1.5, d.r))
    out = run_fp(X, identity_Wa(d), g, np.zeros((d.r, d.N2)), np.zeros(1, np.int32),
                 d, eps=eps)
    e32 = float(np.float32(eps))
    expect = g * v / math.sqrt(v * v + e32)
    np.testing.assert_allclose(out["ckv"][0], expect, rtol=5e-7)


def test_rmsnorm_unit_rms_and_scale_invariance():
    d = TINY
    X, Wa, g, Wb, pos = rand_case(d, 6, 5)
    o = run_fp(X, Wa, g, Wb, pos, d, eps=0.0)
    rms = np.sqrt(np.mean((o["ckv"] / g) ** 2, axis=1))
    np.testing.assert_allclose(rms, 1.0, rtol=1e-6)
    o2 = run_fp(X * 32.0, Wa, g, Wb, pos, d, eps=0.0)
    np.testing.assert_allclose(o2["ckv"], o["ckv"], rtol=2e-6, atol=1e-7)
    # with eps, RMS of y/gamma is sqrt(ms / (ms + eps)) for ms = mean(c^2)
    eps = 0.3
    o3 = run_fp(X, Wa, g, Wb, pos, d, eps=eps)
    c = (X @ Wa)[:, :d.r]
    ms = np.mean(c * c, axis=1)
    rms3 = np.sqrt(np.mean((o3["ckv"] / g) ** 2, axis=1))
    np.testing.assert_allclose(rms3, np.sqrt(ms / (ms + np.float32(eps))), rtol=2e-6)


# ----------------------------------------------------------------------------
# kv_b_proj, reshape + split
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_kv_b_proj_slices_of_rounded_latent(dtype):
    """k_nope / value are the per-head [dn | dv] column slices of
    round_dtype(ckv) @ W_kv_b (kv_b_proj consumes the stored latent)."""
    d = TINY
    X, Wa, g, Wb, pos = rand_case(d, 4, 6)
    if dtype == "bf16":
        X, Wa, g, Wb = (oracle.round_to_dtype(a, "bf16") for a in (X, Wa, g, Wb))
    o = run_fp(X, Wa, g, Wb, pos, d, dtype=dtype)
    ckv = o["ckv"].astype(np.float64)
    if dtype == "f16":
        yq = ckv.astype(np.float16).astype(np.float64)
    else:
        yq = oracle.round_to_dtype(ckv, "bf16")
    assert not np.array_equal(yq, ckv)  # the rounding is visible
    B = (yq @ Wb).reshape(4, d.nh, d.dn + d.dv)
    bound = sum_bound(d.r, np.abs(yq) @ np.abs(Wb)).reshape(4, d.nh, d.dn + d.dv)
    assert np.all(np.abs(o["k_nope"] - B[:, :, :d.dn]) <= bound[:, :, :d.dn])
    assert np.all(np.abs(o["value"] - B[:, :, d.dn:]) <= bound[:, :, d.dn:])


def test_one_hot_kv_b_is_known_permutation():
    """W_kv_b with one 1 per column routes latent j to a known (head, slot):
    column m = h*(dn+dv) + s holds k_nope[h, s] for s < dn and value[h, s-dn]
    otherwise."""
    d = Dims(H=16, nh=3, r=8, dr=4, dn=2, dv=3)
    rng = np.random.default_rng(7)
    X = f16v(rng.standard_normal((2, d.H)))
    src = rng.integers(0, d.r, d.N2)
    Wb = np.zeros((d.r, d.N2))
    Wb[src, np.arange(d.N2)] = 1.0
    o = run_fp(X, identity_Wa(d), np.ones(d.r), Wb, np.zeros(2, np.int32), d)
    yq = o["ckv"].astype(np.float16).astype(np.float64)
    for h in range(d.nh):
        for s in range(d.dn + d.dv):
            m = h * (d.dn + d.dv) + s
            got = o["k_nope"][:, h, s] if s < d.dn else o["value"][:, h, s - d.dn]
            np.testing.assert_array_equal(got, yq[:, src[m]])


# ----------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------

def rope_case(d, P, pos):
    """Feed rope input P [T, dr] straight through (identity W_kv_a)."""
    T = P.shape[0]
    X = np.zeros((T, d.H))
    X[:, :d.r] = 1.0
    X[:, d.r:d.N1] = P
    o = run_fp(X, identity_Wa(d), np.ones(d.r), np.zeros((d.r, d.N2)),
               np.asarray(pos, np.int32), d)
    return o["k_pe"].astype(np.float64)


RD = Dims(H=72, nh=1, r=4, dr=64, dn=1, dv=1)


def f32v(a):
    return np.asarray(a, np.float64).astype(np.float32).astype(np.float64)


def test_rope_position_zero_is_identity_bit_exact():
    P = f16v(np.random.default_rng(8).standard_normal((3, RD.dr)))
    np.testing.assert_array_equal(rope_case(RD, P, [0, 0, 0]), P)


def test_rope_preserves_pair_norms():
    rng = np.random.default_rng(9)
    P = f16v(rng.standard_normal((5, RD.dr)))
    out = rope_case(RD, P, [1, 17, 4095, 32766, 123456])
    h = RD.dr // 2
    n_in = np.hypot(P[:, :h], P[:, h:])
    n_out = np.hypot(out[:, :h], out[:, h:])
    np.testing.assert_allclose(n_out, n_in, rtol=4e-7)


@pytest.mark.parametrize("i", [0, 1, 5, 31])
@pytest.mark.parametrize("pos", [1, 3, 1000, 32767])
def test_rope_unit_vector_closed_form(i, pos):
    """e_i rotates to (cos a) e_i + (sin a) e_{i+dr/2} and e_{i+dr/2} to
    -(sin a) e_i + (cos a) e_{i+dr/2}, with a = pos * theta^(-2i/dr): the
    rotate-half pairing (i, i + dr/2), the sign convention and the
    frequency ladder all show here (cos a, sin a rounded to fp32)."""
    h = RD.dr // 2
    P = np.zeros((2, RD.dr))
    P[0, i] = 1.0
    P[1, i + h] = 1.0
    out = rope_case(RD, P, [pos, pos])
    a = pos * 10000.0 ** (-2.0 * i / RD.dr)
    e0 = np.zeros(RD.dr)
    e0[i], e0[i + h] = math.cos(a), math.sin(a)
    e1 = np.zeros(RD.dr)
    e1[i], e1[i + h] = -math.sin(a), math.cos(a)
    np.testing.assert_allclose(out[0], e0, atol=6e-8)
    np.testing.assert_allclose(out[1], e1, atol=6e-8)


def test_rope_composition_and_relative_position():
    rng = np.random.default_rng(10)
    P = f16v(rng.standard_normal((1, RD.dr)))
    a, b = 37, 1201
    once = rope_case(RD, f32v(rope_case(RD, P, [a])), [b])
    direct = rope_case(RD, P, [a + b])
    np.testing.assert_allclose(once, direct, atol=2e-6)
    # <R_m q, R_n k> = <R_{m-n} q, k>
    q = f16v(rng.standard_normal((1, RD.dr)))
    k = f16v(rng.standard_normal((1, RD.dr)))
    m, n = 2050, 777
    lhs = (rope_case(RD, q, [m]) @ rope_case(RD, k, [n]).T).item()
    rhs = (rope_case(RD, q, [m - n]) @ k.T).item()
    assert abs(lhs - rhs) < 2e-5 * max(1.0, abs(rhs))


def test_rope_per_token_positions():
    """Each token is rotated by its own position."""
    rng = np.random.default_rng(11)
    P = f16v(rng.standard_normal((4, RD.dr)))
    pos = [5, 0, 99, 5]
    out = rope_case(RD, P, pos)
    for t in range(4):
        np.testing.assert_array_equal(out[t], rope_case(RD, P[t:t + 1], [pos[t]])[0])


# ----------------------------------------------------------------------------
# the pages' published case
# ----------------------------------------------------------------------------

def test_published_case_shapes():
    with open(os.path.join(GOLDEN, "mla_prolog_001_shapes.json")) as f:
        gold = json.load(f)
    b, s, H = gold["hidden_states"]
    r, dr, nh = gold["kv_lora_rank"], gold["rope_dim"], gold["num_heads"]
    dn, dv = gold["qk_nope_head_dim"], gold["v_head_dim"]
    assert gold["kv_a_weight"] == [H, r + dr]
    assert gold["kv_b_weight"] == [r, nh * (dn + dv)]
    d = Dims(H=H, nh=nh, r=r, dr=dr, dn=dn, dv=dv)
    X, Wa, g, Wb, pos = rand_case(d, b * s, 12)
    o = run_fp(X, f16v(Wa * 0.05), g, f16v(Wb * 0.05), pos, d, eps=gold["eps"])
    T = b * s
    # token-major outputs, transposed to the page's [b, heads, s, dim] order
    kn = o["k_nope"].reshape(b, s, nh, dn).transpose(0, 2, 1, 3)
    vv = o["value"].reshape(b, s, nh, dv).transpose(0, 2, 1, 3)
    kp = o["k_pe"].reshape(b, s, 1, dr).transpose(0, 2, 1, 3)
    assert list(kn.shape) == gold["k_nope"]
    assert list(vv.shape) == gold["value"]
    assert list(kp.shape) == gold["k_pe"]
    assert o["ckv"].shape == (T, r)
    for v in o.values():
        assert np.all(np.isfinite(v))


# ----------------------------------------------------------------------------
# W8A8
# ----------------------------------------------------------------------------

def run_w8(X, Wqa, swa, g, Wqb, swb, pos, d, eps=1e-6, codes=True):
    return oracle.kv_prolog_w8a8(X, Wqa, swa, g, Wqb, swb, pos, r=d.r, dr=d.dr,
                                 nh=d.nh, dn=d.dn, dv=d.dv, eps=eps, theta=10000.0,
                                 want_codes=codes)


def w8_case(d, T, seed):
    rng = np.random.default_rng(seed)
    X = bf16_bits_to_f32(f32_to_bf16_bits(rng.standard_normal((T, d.H)).astype(np.float32)))
    Wqa = rng.integers(-127, 128, (d.H, d.N1)).astype(np.int8)
    swa = (rng.uniform(0.5, 2.0, d.N1) / 127 * 0.02).astype(np.float32)
    g = bf16_bits_to_f32(f32_to_bf16_bits(rng.uniform(0.5, 1.5, d.r).astype(np.float32)))
    Wqb = rng.integers(-127, 128, (d.r, d.N2)).astype(np.int8)
    swb = (rng.uniform(0.5, 2.0, d.N2) / 127 * 0.02).astype(np.float32)
    pos = rng.integers(0, 4096, T).astype(np.int32)
    return X, Wqa, swa, g, Wqb, swb, pos


def test_w8a8_accumulators_equal_integer_brute_force():
    d = TINY
    X, Wqa, swa, g, Wqb, swb, pos = w8_case(d, 3, 13)
    o = run_w8(X, Wqa, swa, g, Wqb, swb, pos, d)
    for t in range(3):
        qx = [int(v) for v in o["qx"][t]]
        for n in range(d.N1):
            assert o["acc1"][t, n] == sum(qx[k] * int(Wqa[k, n]) for k in range(d.H))
        qz = [int(v) for v in o["qz"][t]]
        for m in range(d.N2):
            assert o["acc2"][t, m] == sum(qz[j] * int(Wqb[j, m]) for j in range(d.r))


def test_w8a8_quantiser_special_cases():
    """amax = 127 makes the reciprocal scale exactly 1: integer rows come
    back unchanged, halves round to even; a zero row gives code 0, scale 0."""
    d = Dims(H=8, nh=1, r=4, dr=2, dn=1, dv=1)
    X = np.array([
        [127, -3, 5, 0, 1, -127, 64, 2],
        [127, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5],
        [0, 0, 0, 0, 0, 0, 0, 0],
    ], np.float32)
    Wqa = np.zeros((d.H, d.N1), np.int8)
    Wqb = np.zeros((d.r, d.N2), np.int8)
    o = run_w8(X, Wqa, np.ones(d.N1, np.float32), np.ones(d.r, np.float32), Wqb,
               np.ones(d.N2, np.float32), np.zeros(3, np.int32), d)
    np.testing.assert_array_equal(o["qx"][0], X[0].astype(np.int8))
    np.testing.assert_array_equal(o["qx"][1], [127, 2, 4, -2, -4, 0, 2, 0])
    np.testing.assert_array_equal(o["qx"][2], 0)
    np.testing.assert_array_equal(o["sx"], [1.0, 1.0, 0.0])


def test_w8a8_no_overflow_at_r1_bound():
    """H = 7168 with every code at +-127: |acc1| = 7168 * 127 * 127 exactly."""
    d = Dims(H=7168, nh=1, r=512, dr=64, dn=1, dv=1)
    X = np.ones((1, d.H), np.float32)
    Wqa = np.full((d.H, d.N1), 127, np.int8)
    Wqa[:, 1] = -127
    Wqb = np.full((d.r, d.N2), -127, np.int8)
    o = run_w8(X, Wqa, np.ones(d.N1, np.float32), np.ones(d.r, np.float32), Wqb,
               np.ones(d.N2, np.float32), np.zeros(1, np.int32), d)
    assert o["acc1"][0, 0] == 7168 * 127 * 127
    assert o["acc1"][0, 1] == -7168 * 127 * 127
    # c is constant 7168*127*127 (except column 1) -> z = c, codes +-127
    assert np.all(np.abs(o["acc2"][0]) <= 512 * 127 * 127)


def test_w8a8_unit_scales_closed_form():
    """Integer activations with amax 127, unit weight scales and gamma = 1:
    every quantisation is exact, so A = X @ Wqa in integers, z = c, the
    kv_b_proj codes are c itself when max|c| = 127, and the outputs are the
    exact rational results scaled by the RMS factor."""
    d = Dims(H=8, nh=1, r=4, dr=2, dn=1, dv=3)
    X = np.array([[127, 1, 0, 0, 0, 0, 0, 0]], np.float32)
    Wqa = np.zeros((d.H, d.N1), np.int8)
    # c = [127, -5, 3, 1]; p = [2, -7]
    Wqa[0, 0] = 1
    Wqa[1, 1] = -5
    Wqa[1, 2] = 3
    Wqa[1, 3] = 1
    Wqa[1, 4] = 2
    Wqa[1, 5] = -7
    Wqb = np.array([[1, 0, 2, -1], [0, 1, 1, 3], [5, 0, 0, 1], [0, -2, 1, 0]], np.int8)
    o = run_w8(X, Wqa, np.ones(d.N1, np.float32), np.ones(d.r, np.float32), Wqb,
               np.ones(d.N2, np.float32), np.zeros(1, np.int32), d, eps=0.0)
    c = np.array([127, -5, 3, 1])
    np.testing.assert_array_equal(o["acc1"][0], [127, -5, 3, 1, 2, -7])
    np.testing.assert_array_equal(o["qz"][0], c)
    assert o["sz"][0] == 1.0
    inv = 1.0 / math.sqrt(sum(int(v) ** 2 for v in c) / 4.0)
    B = [sum(int(c[j]) * int(Wqb[j, m]) for j in range(4)) for m in range(4)]
    np.testing.assert_allclose(o["k_nope"][0, 0], [B[0] * inv], rtol=4e-7)
    np.testing.assert_allclose(o["value"][0, 0], np.array(B[1:]) * inv, rtol=4e-7)
    np.testing.assert_allclose(o["ckv"][0], c * inv, rtol=4e-7)
    np.testing.assert_array_equal(o["k_pe"][0], [2.0, -7.0])


def real_prolog(X, Wa, g, Wb, pos, d, eps, theta=10000.0):
    """The prolog as real-valued mathematics, in float64 with numpy: no
    quantisation, no storage rounding.  Used as the closed form the W8A8
    path must reproduce when its quantisations are lossless."""
    A = X @ Wa
    c, p = A[:, :d.r], A[:, d.r:]
    inv = 1.0 / np.sqrt(np.mean(c * c, axis=1, keepdims=True) + eps)
    y = c * inv * g
    B = (y @ Wb).reshape(len(X), d.nh, d.dn + d.dv)
    h = d.dr // 2
    f = theta ** (-2.0 * np.arange(h) / d.dr)
    a = np.asarray(pos, np.float64)[:, None] * f[None, :]
    kpe = np.concatenate([p[:, :h] * np.cos(a) - p[:, h:] * np.sin(a),
                          p[:, h:] * np.cos(a) + p[:, :h] * np.sin(a)], axis=1)
    return {"k_nope": B[:, :, :d.dn], "value": B[:, :, d.dn:], "k_pe": kpe, "ckv": y}


def lossless_w8a8_case():
    """Inputs for which both W8A8 activation quantisations are exact.

    Token t has int8 codes qx_t (one of them +-127) and a power-of-two scale
    sx_t, and X_t = qx_t * sx_t, so quantising X_t gives back qx_t and sx_t.
    W_kv_a is a signed permutation (int8), so acc1 is a signed permutation of
    qx_t.  Per-column power-of-two weight scales s_a[n] and gamma[j] are all
    different (scaling by the wrong column's factor changes the result), and
    c * gamma = acc1 * sx_t * s_a * gamma lands on multiples of a power of
    two sz_t with max |.| = 127 sz_t, so quantising z is exact too.  Then the
    W8A8 prolog must equal the real-valued prolog with the dequantised weights
    (Wq * s), up to fp32 rounding."""
    d = Dims(H=8, nh=2, r=4, dr=2, dn=1, dv=3)
    s_a = np.array([0.25, 0.5, 2.0, 1.0, 0.125, 4.0], np.float32)
    gamma = np.array([0.5, 2.0, 0.25, 1.0], np.float32)
    # signed permutation: acc1[n] = sign[n] * qx[perm[n]]
    perm = np.array([3, 0, 6, 1, 7, 2])
    sign = np.array([1, -1, 1, 1, -1, 1])
    Wqa = np.zeros((d.H, d.N1), np.int8)
    Wqa[perm, np.arange(d.N1)] = sign
    # latent factors f = s_a * gamma = [1/8, 1, 1/2, 1]; with sx = 2 and
    # sz = 2: qz = acc1 * f, so acc1[0] must be a multiple of 8, acc1[2] even
    want_acc1 = np.array([[-96, 127, 50, -7, 9, -33],     # token 0, sx = 2
                          [40, -20, 127, 3, -5, 64]])     # token 1, sx = 4
    sx = np.array([2.0, 4.0], np.float32)
    qx = np.zeros((2, d.H), np.int64)
    for t in range(2):
        for n in range(d.N1):
            qx[t, perm[n]] = sign[n] * want_acc1[t, n]
    qx[0, 4], qx[0, 5] = 11, -127   # the two unused hidden columns
    qx[1, 4], qx[1, 5] = -3, 2
    X = (qx * sx[:, None]).astype(np.float32)
    rng = np.random.default_rng(31)
    Wqb = rng.integers(-127, 128, (d.r, d.N2)).astype(np.int8)
    s_b = np.array([0.5, 4.0, 0.25, 2.0, 1.0, 0.125, 8.0, 0.0625], np.float32)
    pos = np.array([0, 1234], np.int32)
    return d, X, Wqa, s_a, gamma, Wqb, s_b, pos, want_acc1, sx


def test_w8a8_lossless_quantisation_equals_real_prolog():
    """Pins the dequantisation (acc1 * sx * s_a[n], acc2 * sz * inv * s_b[m]),
    gamma, the per-token scales and the RMS factor of the W8A8 path: on the
    lossless case every output must equal the real-valued prolog.  Dropping
    sx changes k_pe by 2x; dropping or mis-indexing s_a, gamma or s_b scales
    columns by different powers of two; dropping sz or inv scales k_nope /
    value by 2x or by the RMS factor."""
    d, X, Wqa, s_a, gamma, Wqb, s_b, pos, want_acc1, sx = lossless_w8a8_case()
    eps = 1e-6
    o = run_w8(X, Wqa, s_a, gamma, Wqb, s_b, pos, d, eps=eps)
    # the construction itself: exact codes and power-of-two scales
    np.testing.assert_array_equal(o["sx"], sx)
    np.testing.assert_array_equal(o["acc1"], want_acc1)
    np.testing.assert_array_equal(o["sz"], [2.0, 2.0])
    z = want_acc1[:, :d.r] * sx[:, None] * s_a[None, :d.r] * gamma[None, :]
    np.testing.assert_array_equal(o["qz"].astype(np.float64) * 2.0, z)
    ref = real_prolog(X.astype(np.float64), Wqa * s_a[None, :].astype(np.float64),
                      gamma.astype(np.float64), Wqb * s_b[None, :].astype(np.float64),
                      pos, d, np.float32(eps))
    for name in ("k_nope", "value", "k_pe", "ckv"):
        np.testing.assert_allclose(o[name], ref[name], rtol=2e-6, atol=1e-6 * np.abs(ref[name]).max(),
                                   err_msg=name)


def test_w8a8_close_to_real_prolog_on_random_inputs():
    """On random inputs of the synthetic workloads' distributions the W8A8
    prolog approximates the real-valued prolog with the dequantised weights:
    the only differences are the two per-token activation quantisations (a
    half step of amax / 127 each).  Bounded loosely (3 % of each output's
    largest magnitude), it catches any transposed operand, lost scale or
    wrong head split even where the exact pins use tiny shapes."""
    d = Dims(H=256, nh=4, r=512, dr=64, dn=128, dv=128)
    rng = np.random.default_rng(32)
    T = 5
    X = bf16_bits_to_f32(f32_to_bf16_bits(rng.standard_normal((T, d.H)).astype(np.float32)))
    Wa32 = (rng.standard_normal((d.H, d.N1)) * 0.01).astype(np.float32)
    Wb32 = (rng.standard_normal((d.r, d.N2)) * 0.01).astype(np.float32)
    from workloads import quantize_weight_per_column
    Wqa, swa = quantize_weight_per_column(Wa32)
    Wqb, swb = quantize_weight_per_column(Wb32)
    g = bf16_bits_to_f32(f32_to_bf16_bits(rng.uniform(0.5, 1.5, d.r).astype(np.float32)))
    pos = rng.integers(0, 4096, T).astype(np.int32)
    o = run_w8(X, Wqa, swa, g, Wqb, swb, pos, d, codes=False)
    ref = real_prolog(X.astype(np.float64), Wqa * swa[None, :].astype(np.float64),
                      g.astype(np.float64), Wqb * swb[None, :].astype(np.float64), pos, d, 1e-6)
    for name in ("k_nope", "value", "k_pe", "ckv"):
        err = np.abs(o[name] - ref[name]).max()
        assert err <= 0.03 * np.abs(ref[name]).max(), (name, err)
