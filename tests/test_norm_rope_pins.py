"""Pins of the oracle's standalone RMSNorm and RoPE, on the CPU: closed
forms, invariants and special cases, plus agreement with the (separately
pinned) prolog oracle, whose steps 3 and 6 these operators are."""
import numpy as np
import pytest

import oracle
from workloads import to_storage, widen

EPS = 1e-6


def f16v(a):
    """Values rounded to fp16 (as float64): the operators' model dtype."""
    return np.asarray(a, np.float64).astype(np.float16).astype(np.float64)


# ---------------------------------------------------------------------------
# RMSNorm: y[j] = x[j] / sqrt(mean x^2 + eps) * gamma[j]
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [8, 64, 512, 1000])
def test_rms_alternating_row_is_plus_minus_gamma(n):
    # x = (+a, -a, +a, ...), eps = 0: mean x^2 = a^2, so y = +-gamma exactly
    a = 3.0
    x = np.where(np.arange(n) % 2 == 0, a, -a)[None, :]
    gamma = f16v(np.random.default_rng(n).uniform(0.5, 1.5, n))
    y = oracle.rms_norm(x, gamma, 0.0)
    # inv = 1/3 rounded to fp32, so x * inv is +-1 to within one fp32 rounding
    np.testing.assert_allclose(y[0], np.where(np.arange(n) % 2 == 0, gamma, -gamma),
                               rtol=2.5e-7, atol=0)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.5])
def test_rms_mean_square_closed_form(eps):
    # y / gamma = x / sqrt(ms + eps), hence mean((y / gamma)^2) = ms / (ms + eps):
    # fails for a wrong mean (n - 1, or over the wrong axis), eps outside the
    # root, or gamma applied to the wrong index
    rng = np.random.default_rng(1)
    x = f16v(rng.standard_normal((5, 512)) * np.array([[0.1], [1.0], [7.0], [0.01], [2.0]]))
    gamma = f16v(rng.uniform(0.5, 1.5, 512))
    y = oracle.rms_norm(x, gamma, eps)
    ms = np.mean(x * x, axis=1)
    e32 = float(np.float32(eps))
    np.testing.assert_allclose(np.mean((y / gamma) ** 2, axis=1), ms / (ms + e32), rtol=2e-6)
    # signs follow x, and each value scales with its own gamma
    assert np.all(np.sign(y) == np.sign(x))


def test_rms_scale_invariance_and_zero_row():
    rng = np.random.default_rng(2)
    x = f16v(rng.standard_normal((3, 256)))
    gamma = f16v(rng.uniform(0.5, 1.5, 256))
    np.testing.assert_allclose(oracle.rms_norm(37.0 * x, gamma, 0.0),
                               oracle.rms_norm(x, gamma, 0.0), rtol=2e-6)
    z = oracle.rms_norm(np.zeros((2, 64)), np.ones(64), EPS)
    assert np.all(z == 0.0)


def test_rms_permutation_equivariance():
    # permuting x and gamma together permutes y (no index mix-up)
    rng = np.random.default_rng(3)
    x = f16v(rng.standard_normal((4, 128)))
    gamma = f16v(rng.uniform(0.5, 1.5, 128))
    perm = rng.permutation(128)
    # the sum of squares is taken in another order: equal to fp32 rounding
    np.testing.assert_allclose(oracle.rms_norm(x[:, perm], gamma[perm], EPS),
                               oracle.rms_norm(x, gamma, EPS)[:, perm], rtol=2e-6)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_rms_equals_prolog_compressed_kv(dtype):
    # the prolog with W_kv_a = [I | 0] makes c = x: its compressed_kv is the
    # standalone RMSNorm of x
    rng = np.random.default_rng(4)
    T, r, dr = 6, 512, 64
    x = widen(to_storage(rng.standard_normal((T, r)).astype(np.float32), dtype), dtype)
    gamma = widen(to_storage(rng.uniform(0.5, 1.5, r).astype(np.float32), dtype), dtype)
    Wa = np.zeros((r, r + dr))
    Wa[:, :r] = np.eye(r)
    ref = oracle.kv_prolog_fp(x, Wa, gamma, np.zeros((r, 256)), np.zeros(T, np.int32), r=r,
                              dr=dr, nh=1, dn=128, dv=128, eps=EPS, theta=1e4, dtype=dtype)
    np.testing.assert_array_equal(oracle.rms_norm(x, gamma, EPS), ref["ckv"])


# ---------------------------------------------------------------------------
# RoPE (rotate-half, f_i = theta^(-2i/dr)), rows of dr = 64 per head
# ---------------------------------------------------------------------------

def test_rope_position_zero_is_identity():
    x = f16v(np.random.default_rng(5).standard_normal((3, 4, 64)))
    assert np.array_equal(oracle.rope(x, np.zeros(3, np.int32), 1e4), x)


@pytest.mark.parametrize("i,pos", [(0, 1), (0, 7), (16, 100), (31, 12345)])
def test_rope_unit_vectors_closed_form(i, pos):
    # e_i -> cos a at i, sin a at i + 32; e_(i+32) -> -sin a at i, cos a at
    # i + 32, with a = pos * theta^(-2i/64) (for i = 16, theta = 1e4:
    # f = 1e-2, so pos 100 is one radian)
    theta = 1e4
    a = pos * theta ** (-2.0 * i / 64)
    x = np.zeros((1, 2, 64))
    x[0, 0, i] = 1.0
    x[0, 1, i + 32] = 1.0
    y = oracle.rope(x, np.array([pos], np.int32), theta)
    # cos a and sin a rounded to fp32: within half an fp32 ulp of 1
    np.testing.assert_allclose([y[0, 0, i], y[0, 0, i + 32]], [np.cos(a), np.sin(a)],
                               rtol=0, atol=6e-8)
    np.testing.assert_allclose([y[0, 1, i], y[0, 1, i + 32]], [-np.sin(a), np.cos(a)],
                               rtol=0, atol=6e-8)
    others = np.delete(y[0, 0], [i, i + 32])
    assert np.all(others == 0.0)


def test_rope_norms_composition_and_heads():
    rng = np.random.default_rng(6)
    T, heads = 5, 3
    x = f16v(rng.standard_normal((T, heads, 64)))
    p1 = rng.integers(0, 5000, T).astype(np.int32)
    p2 = rng.integers(0, 5000, T).astype(np.int32)
    y = oracle.rope(x, p1, 1e4)
    # each (i, i + 32) pair keeps its norm (to fp32 rounding)
    np.testing.assert_allclose(y[..., :32] ** 2 + y[..., 32:] ** 2,
                               x[..., :32] ** 2 + x[..., 32:] ** 2, rtol=1e-6, atol=1e-7)
    # rotations compose: rope(rope(x, p1), p2) = rope(x, p1 + p2)
    np.testing.assert_allclose(oracle.rope(y, p2, 1e4), oracle.rope(x, p1 + p2, 1e4),
                               rtol=0, atol=2e-6)
    # every head of a token takes that token's position, independently
    for h in range(heads):
        np.testing.assert_array_equal(y[:, h], oracle.rope(x[:, h], p1, 1e4))


def test_rope_equals_prolog_k_pe():
    # the prolog with W_kv_a = [0 | I] makes its rope part p = x: its k_pe is
    # the standalone RoPE of x
    rng = np.random.default_rng(7)
    T, r, dr = 9, 512, 64
    x = f16v(rng.standard_normal((T, dr)))
    Wa = np.zeros((dr, r + dr))
    Wa[:, r:] = np.eye(dr)
    pos = rng.integers(0, 30000, T).astype(np.int32)
    ref = oracle.kv_prolog_fp(x, Wa, np.ones(r), np.zeros((r, 256)), pos, r=r, dr=dr, nh=1,
                              dn=128, dv=128, eps=EPS, theta=1e4, dtype="bf16")
    np.testing.assert_array_equal(oracle.rope(x, pos, 1e4), ref["k_pe"])
