"""Pins of the oracle's paged KV-cache append (the step after "assemble"),
on the CPU: closed forms, invariants and special cases.  The pages name paged
attention and an int8 cache mode without a layout or formula; the reading
(slot = [compressed_kv row | k_pe row], skip outside [0, num_slots), one
symmetric int8 scale per slot) is documented in oracle/oracle.c."""
import numpy as np
import pytest

import oracle

R, DR = 512, 64


def rows(T, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    ckv = oracle.round_to_dtype(rng.standard_normal((T, R)) * scale, "bf16")
    kpe = oracle.round_to_dtype(rng.standard_normal((T, DR)) * scale, "bf16")
    return ckv, kpe


def test_fp_append_places_rows_and_skips():
    T, S = 9, 40
    ckv, kpe = rows(T, 1)
    slots = np.array([5, -1, 39, 0, 40, 12, -7, 1 << 40, 7])
    cache0 = np.full((S, R + DR), -3.25)
    out = oracle.kv_cache_append(ckv, kpe, slots, cache0)
    written = set()
    for t, s in enumerate(slots):
        if 0 <= s < S:
            assert np.array_equal(out[s, :R], ckv[t]) and np.array_equal(out[s, R:], kpe[t])
            written.add(int(s))
    for s in range(S):
        if s not in written:
            assert np.all(out[s] == -3.25)  # untouched


def test_fp_append_permutation_round_trip():
    T = 33
    ckv, kpe = rows(T, 2)
    perm = np.random.default_rng(3).permutation(T)
    out = oracle.kv_cache_append(ckv, kpe, perm, np.zeros((T, R + DR)))
    # reading the slots back in mapping order recovers the tokens
    assert np.array_equal(out[perm, :R], ckv) and np.array_equal(out[perm, R:], kpe)


def test_int8_zero_row():
    q, s = oracle.kv_cache_append_int8(np.zeros((1, R)), np.zeros((1, DR)), [2],
                                       np.full((3, R + DR), 9, np.int8), np.full(3, 5.0, np.float32))
    assert np.all(q[2] == 0) and s[2] == 0.0
    assert np.all(q[0] == 9) and s[0] == 5.0  # untouched


def test_int8_integer_row_is_exact():
    # amax = 127: inverse 1, every integer value is its own code, scale 1
    rng = np.random.default_rng(4)
    c = rng.integers(-127, 128, (1, R)).astype(float)
    c[0, 17] = -127.0
    p = rng.integers(-126, 127, (1, DR)).astype(float)
    q, s = oracle.kv_cache_append_int8(c, p, [0], np.zeros((1, R + DR), np.int8),
                                       np.zeros(1, np.float32))
    assert s[0] == 1.0
    assert np.array_equal(q[0, :R], c[0].astype(np.int8)) and np.array_equal(q[0, R:], p[0].astype(np.int8))


def test_int8_ties_to_even():
    c = np.zeros((1, R))
    c[0, :6] = [127.0, 0.5, 1.5, 2.5, -0.5, -2.5]
    p = np.zeros((1, DR))
    p[0, :2] = [3.5, -3.5]
    q, s = oracle.kv_cache_append_int8(c, p, [0], np.zeros((1, R + DR), np.int8),
                                       np.zeros(1, np.float32))
    assert list(q[0, :6]) == [127, 0, 2, 2, 0, -2] and list(q[0, R:R + 2]) == [4, -4]


@pytest.mark.parametrize("scale", [1e-3, 1.0, 300.0])
def test_int8_error_bound_and_extremes(scale):
    T = 16
    ckv, kpe = rows(T, 5, scale)
    q, s = oracle.kv_cache_append_int8(ckv, kpe, np.arange(T), np.zeros((T, R + DR), np.int8),
                                       np.zeros(T, np.float32))
    v = np.concatenate([ckv, kpe], axis=1)
    amax = np.abs(v).max(axis=1)
    assert np.allclose(s, (amax / 127.0).astype(np.float32), rtol=0, atol=0)
    deq = q.astype(np.float64) * s[:, None].astype(np.float64)
    # round to nearest: within half a step (plus fp32 rounding of the scaled value)
    assert np.all(np.abs(deq - v) <= s[:, None] * (0.5 + 1e-5))
    assert np.all(np.abs(q).max(axis=1) == 127)
    am = np.abs(v).argmax(axis=1)
    assert np.all(np.abs(q[np.arange(T), am]) == 127)
