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


def run_fp(X, Wa, g, Wb, pos, dims, eps=1e-6, theta=10000.0, dtype="f16"):
    return oracle.kv_prolog_fp(X, Wa, g, Wb, pos, r=dims.r, dr=dims.dr, nh=dims.nh,
                               dn=dims.dn, dv=dims.dv, eps=eps, theta=theta,
                               dtype=dtype)


def rand_case(dims, T, seed, pos=None):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, dims.H))
    Wa = rng.standard_normal((dims.H, dims.N1)) * 0.3
    g = rng.uniform(0.5, 1.5, dims.r)
    Wb = rng.standard_normal((dims.r, dims.N2)) * 0.3
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
    order (W_kv_a stored [H, r+dr]) and that the rope columns are the LAST dr."""
    d = TINY
    X, Wa, g, Wb, _ = rand_case(d, 5, 3)
    out = run_fp(X, Wa, g, Wb, np.zeros(5, np.int32), d)
    A = X @ Wa
    np.testing.assert_allclose(out["k_pe"], A[:, d.r:], rtol=1e-12, atol=1e-12)


def test_identity_weight_split_is_exact():
    d = Dims(H=16, nh=2, r=8, dr=4, dn=3, dv=5)
    rng = np.random.default_rng(4)
    X = rng.standard_normal((3, d.H))
    out = run_fp(X, identity_Wa(d), np.ones(d.r), np.zeros((d.r, d.N2)),
                 np.zeros(3, np.int32), d, eps=0.0)
    np.testing.assert_array_equal(out["k_pe"], X[:, d.r:d.N1])
    c = X[:, :d.r]
    rms = np.sqrt(np.mean(c * c, axis=1, keepdims=True))
    np.testing.assert_allclose(out["ckv"], c / rms, rtol=1e-13)


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
    X = np.zeros((1, d.H))
    X[0, :d.r] = v
    X[0, d.r:d.N1] = 7.0 * v + 1.0
    g = np.linspace(0.5, 1.5, d.r)
    out = run_fp(X, identity_Wa(d), g, np.zeros((d.r, d.N2)), np.zeros(1, np.int32),
                 d, eps=eps)
    expect = g * v / math.sqrt(v * v + eps)
    np.testing.assert_allclose(out["ckv"][0], expect, rtol=1e-14)


def test_rmsnorm_unit_rms_and_scale_invariance():
    d = TINY
    X, Wa, g, Wb, pos = rand_case(d, 6, 5)
    o = run_fp(X, Wa, g, Wb, pos, d, eps=0.0)
    rms = np.sqrt(np.mean((o["ckv"] / g) ** 2, axis=1))
    np.testing.assert_allclose(rms, 1.0, rtol=1e-13)
    o2 = run_fp(X * 37.5, Wa, g, Wb, pos, d, eps=0.0)
    np.testing.assert_allclose(o2["ckv"], o["ckv"], rtol=1e-12)
    # with eps, RMS of y/gamma is sqrt(ms / (ms + eps)) for ms = mean(c^2)
    eps = 0.3
    o3 = run_fp(X, Wa, g, Wb, pos, d, eps=eps)
    c = (X @ Wa)[:, :d.r]
    ms = np.mean(c * c, axis=1)
    rms3 = np.sqrt(np.mean((o3["ckv"] / g) ** 2, axis=1))
    np.testing.assert_allclose(rms3, np.sqrt(ms / (ms + eps)), rtol=1e-12)


# ----------------------------------------------------------------------------
# kv_b_proj, reshape + split
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_kv_b_proj_slices_of_rounded_latent(dtype):
    """k_nope / value are the per-head [dn | dv] column slices of
    round_dtype(ckv) @ W_kv_b (kv_b_proj consumes the stored latent)."""
    d = TINY
    X, Wa, g, Wb, pos = rand_case(d, 4, 6)
    o = run_fp(X, Wa, g, Wb, pos, d, dtype=dtype)
    if dtype == "f16":
        yq = o["ckv"].astype(np.float16).astype(np.float64)
    else:
        yq = oracle.round_to_dtype(o["ckv"], "bf16")
    assert not np.array_equal(yq, o["ckv"])  # the rounding is visible
    B = (yq @ Wb).reshape(4, d.nh, d.dn + d.dv)
    np.testing.assert_allclose(o["k_nope"], B[:, :, :d.dn], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o["value"], B[:, :, d.dn:], rtol=1e-12, atol=1e-12)


def test_one_hot_kv_b_is_known_permutation():
    """W_kv_b with one 1 per column routes latent j to a known (head, slot):
    column m = h*(dn+dv) + s holds k_nope[h, s] for s < dn and value[h, s-dn]
    otherwise."""
    d = Dims(H=16, nh=3, r=8, dr=4, dn=2, dv=3)
    rng = np.random.default_rng(7)
    X = rng.standard_normal((2, d.H))
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
    return o["k_pe"]


RD = Dims(H=72, nh=1, r=4, dr=64, dn=1, dv=1)


def test_rope_position_zero_is_identity_bit_exact():
    P = np.random.default_rng(8).standard_normal((3, RD.dr))
    np.testing.assert_array_equal(rope_case(RD, P, [0, 0, 0]), P)


def test_rope_preserves_pair_norms():
    rng = np.random.default_rng(9)
    P = rng.standard_normal((5, RD.dr))
    out = rope_case(RD, P, [1, 17, 4095, 32766, 123456])
    h = RD.dr // 2
    n_in = np.hypot(P[:, :h], P[:, h:])
    n_out = np.hypot(out[:, :h], out[:, h:])
    np.testing.assert_allclose(n_out, n_in, rtol=1e-13)


@pytest.mark.parametrize("i", [0, 1, 5, 31])
@pytest.mark.parametrize("pos", [1, 3, 1000, 32767])
def test_rope_unit_vector_closed_form(i, pos):
    """e_i rotates to (cos a) e_i + (sin a) e_{i+dr/2} and e_{i+dr/2} to
    -(sin a) e_i + (cos a) e_{i+dr/2}, with a = pos * theta^(-2i/dr): the
    rotate-half pairing (i, i + dr/2), the sign convention and the
    frequency ladder all show here."""
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
    np.testing.assert_allclose(out[0], e0, atol=1e-12)
    np.testing.assert_allclose(out[1], e1, atol=1e-12)


def test_rope_composition_and_relative_position():
    rng = np.random.default_rng(10)
    P = rng.standard_normal((1, RD.dr))
    a, b = 37, 1201
    once = rope_case(RD, rope_case(RD, P, [a]), [b])
    direct = rope_case(RD, P, [a + b])
    np.testing.assert_allclose(once, direct, atol=1e-10)
    # <R_m q, R_n k> = <R_{m-n} q, k>
    q = rng.standard_normal((1, RD.dr))
    k = rng.standard_normal((1, RD.dr))
    m, n = 2050, 777
    lhs = (rope_case(RD, q, [m]) @ rope_case(RD, k, [n]).T).item()
    rhs = (rope_case(RD, q, [m - n]) @ k.T).item()
    assert abs(lhs - rhs) < 1e-10 * max(1.0, abs(rhs))


def test_rope_per_token_positions():
    """Each token is rotated by its own position."""
    rng = np.random.default_rng(11)
    P = rng.standard_normal((4, RD.dr))
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
    o = run_fp(X, Wa * 0.05, g, Wb * 0.05, pos, d, eps=gold["eps"])
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
    np.testing.assert_allclose(o["k_nope"][0, 0], [B[0] * inv], rtol=1e-14)
    np.testing.assert_allclose(o["value"][0, 0], np.array(B[1:]) * inv, rtol=1e-14)
    np.testing.assert_allclose(o["ckv"][0], c * inv, rtol=1e-14)
    np.testing.assert_array_equal(o["k_pe"][0], [2.0, -7.0])
