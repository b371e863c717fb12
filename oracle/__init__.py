"""CPU oracle for the MLA KV prolog -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does, and
this package never imports the product library.

The arithmetic lives in ``oracle.c`` (plain C, fp32 with fp32
accumulators in ascending order, built by ``oracle/build_oracle.py``); this
module only converts numpy arrays to the pointer form that file takes.  What each step computes, and from which
passage of the pages, is documented in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MLA_ORACLE_LIB names another build of oracle.c (the mutation tests load
# deliberately broken copies through it); by default the in-tree build.
LIB_PATH = os.environ.get("MLA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build_oracle

        build_oracle.build()
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    lib.oracle_round_to_dtype.argtypes = [vp, vp, i64, i32]
    lib.oracle_round_to_dtype.restype = i32
    lib.oracle_kv_prolog_fp.argtypes = (
        [i64] * 7 + [vp] * 5 + [dbl, dbl, i32] + [vp] * 4 + [i32]
    )
    lib.oracle_kv_prolog_fp.restype = i32
    lib.oracle_kv_prolog_w8a8.argtypes = (
        [i64] * 7 + [vp] * 7 + [dbl, dbl] + [vp] * 4 + [vp] * 6 + [i32]
    )
    lib.oracle_kv_prolog_w8a8.restype = i32
    lib.oracle_kv_cache_append.argtypes = [i64, i64, i64, vp, vp, vp, i64, vp]
    lib.oracle_kv_cache_append.restype = i32
    lib.oracle_kv_cache_append_int8.argtypes = [i64, i64, i64, vp, vp, vp, i64, vp, vp]
    lib.oracle_kv_cache_append_int8.restype = i32
    lib.oracle_rms_norm.argtypes = [i64, i64, vp, vp, dbl, vp]
    lib.oracle_rms_norm.restype = i32
    lib.oracle_rope.argtypes = [i64, i64, i64, vp, vp, dbl, vp]
    lib.oracle_rope.restype = i32
    lib.oracle_num_threads.argtypes = [i32]
    lib.oracle_num_threads.restype = i32
    _lib = lib
    return lib


DTYPE_CODE = {"f16": 1, "bf16": 2}


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def _f32(a):
    """float32 copy of an array whose values must be exactly representable
    in float32 (model-dtype values); raises if converting would round."""
    a64 = np.asarray(a)
    out = np.ascontiguousarray(a64, dtype=np.float32)
    if a64.dtype != np.float32 and a64.size and not np.array_equal(
            out.astype(np.float64), np.asarray(a64, np.float64), equal_nan=True):
        raise ValueError("oracle inputs must be exactly representable in float32")
    return out


def round_to_dtype(x, dtype: str) -> np.ndarray:
    """Round float64 values to the nearest fp16 / bf16 value (ties to even);
    returns float64 holding the rounded values."""
    x = _c(x, np.float64)
    out = np.empty_like(x)
    rc = _load().oracle_round_to_dtype(_ptr(x), _ptr(out), x.size, DTYPE_CODE[dtype])
    if rc != 0:
        raise ValueError(f"oracle_round_to_dtype failed: {rc}")
    return out


def num_threads(n: int = 0) -> int:
    return _load().oracle_num_threads(int(n))


def kv_prolog_fp(X, Wa, gamma, Wb, pos, *, r, dr, nh, dn, dv, eps, theta,
                 dtype: str, nthreads: int = 0, want_kv: bool = True):
    """fp16/bf16 KV prolog in fp32.  Inputs are arrays of the stored values
    (any float dtype holding fp16 / bf16 values; they are widened exactly to
    float32).  Returns a dict of float32 arrays k_nope [T,nh,dn],
    value [T,nh,dv], k_pe [T,dr], ckv [T,r], all before the final rounding
    to the output dtype."""
    X = _f32(X)
    T, H = X.shape
    Wa = _f32(Wa)
    gamma = _f32(gamma)
    Wb = _f32(Wb)
    pos = _c(pos, np.int32)
    assert Wa.shape == (H, r + dr) and gamma.shape == (r,)
    assert Wb.shape == (r, nh * (dn + dv)) and pos.shape == (T,)
    f = np.float32
    out = {
        "k_nope": np.empty((T, nh, dn), f) if want_kv else None,
        "value": np.empty((T, nh, dv), f) if want_kv else None,
        "k_pe": np.empty((T, dr), f),
        "ckv": np.empty((T, r), f),
    }
    rc = _load().oracle_kv_prolog_fp(
        T, H, r, dr, nh, dn, dv, _ptr(X), _ptr(Wa), _ptr(gamma), _ptr(Wb),
        _ptr(pos), float(eps), float(theta), DTYPE_CODE[dtype],
        _ptr(out["k_nope"]), _ptr(out["value"]), _ptr(out["k_pe"]),
        _ptr(out["ckv"]), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_kv_prolog_fp failed: {rc}")
    return out


def kv_prolog_w8a8(X, Wqa, swa, gamma, Wqb, swb, pos, *, r, dr, nh, dn, dv,
                   eps, theta, nthreads: int = 0, want_kv: bool = True,
                   want_acc: bool = True, want_codes: bool = False):
    """W8A8 KV prolog.  X and gamma hold bf16 values (widened exactly to
    float32 here); Wqa/Wqb int8 with float32 per-output-column scales.
    Returns float32 references (before the final rounding to bf16) plus the
    exact int32 accumulators."""
    X = _c(X, np.float32)
    T, H = X.shape
    N1 = r + dr
    N2 = nh * (dn + dv)
    Wqa = _c(Wqa, np.int8)
    swa = _c(swa, np.float32)
    gamma = _c(gamma, np.float32)
    Wqb = _c(Wqb, np.int8)
    swb = _c(swb, np.float32)
    pos = _c(pos, np.int32)
    assert Wqa.shape == (H, N1) and swa.shape == (N1,) and gamma.shape == (r,)
    assert Wqb.shape == (r, N2) and swb.shape == (N2,) and pos.shape == (T,)
    f = np.float32
    out = {
        "k_nope": np.empty((T, nh, dn), f) if want_kv else None,
        "value": np.empty((T, nh, dv), f) if want_kv else None,
        "k_pe": np.empty((T, dr), f),
        "ckv": np.empty((T, r), f),
        "acc1": np.empty((T, N1), np.int32) if want_acc else None,
        "acc2": np.empty((T, N2), np.int32) if (want_acc and want_kv) else None,
        "qx": np.empty((T, H), np.int8) if want_codes else None,
        "sx": np.empty((T,), np.float32) if want_codes else None,
        "qz": np.empty((T, r), np.int8) if want_codes else None,
        "sz": np.empty((T,), np.float32) if want_codes else None,
    }
    rc = _load().oracle_kv_prolog_w8a8(
        T, H, r, dr, nh, dn, dv, _ptr(X), _ptr(Wqa), _ptr(swa), _ptr(gamma),
        _ptr(Wqb), _ptr(swb), _ptr(pos), float(eps), float(theta),
        _ptr(out["k_nope"]), _ptr(out["value"]), _ptr(out["k_pe"]),
        _ptr(out["ckv"]), _ptr(out["acc1"]), _ptr(out["acc2"]),
        _ptr(out["qx"]), _ptr(out["sx"]), _ptr(out["qz"]), _ptr(out["sz"]),
        int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_kv_prolog_w8a8 failed: {rc}")
    return out


def kv_cache_append(ckv, kpe, slots, cache) -> np.ndarray:
    """Paged KV-cache append (fp): returns a copy of ``cache`` [num_slots,
    r + dr] with token t's [ckv row | kpe row] in slot ``slots[t]`` (slots
    outside [0, num_slots) skip the token)."""
    ckv, kpe = _c(ckv, np.float64), _c(kpe, np.float64)
    slots = _c(slots, np.int64)
    out = _c(cache, np.float64).copy()
    T, r = ckv.shape
    dr = kpe.shape[1]
    rc = _load().oracle_kv_cache_append(T, r, dr, _ptr(ckv), _ptr(kpe), _ptr(slots),
                                        out.shape[0], _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_kv_cache_append failed: {rc}")
    return out


def kv_cache_append_int8(ckv, kpe, slots, cache_q, scale):
    """Paged KV-cache append into an int8 cache with one fp32 scale per slot
    (the W8A8 activation scheme over the slot's r + dr values); returns
    copies of ``cache_q`` [num_slots, r + dr] and ``scale`` [num_slots]."""
    ckv, kpe = _c(ckv, np.float32), _c(kpe, np.float32)
    slots = _c(slots, np.int64)
    q = _c(cache_q, np.int8).copy()
    sc = _c(scale, np.float32).copy()
    T, r = ckv.shape
    dr = kpe.shape[1]
    rc = _load().oracle_kv_cache_append_int8(T, r, dr, _ptr(ckv), _ptr(kpe), _ptr(slots),
                                             q.shape[0], _ptr(q), _ptr(sc))
    if rc != 0:
        raise ValueError(f"oracle_kv_cache_append_int8 failed: {rc}")
    return q, sc


def rms_norm(x, gamma, eps: float) -> np.ndarray:
    """Standalone RMSNorm over the last axis of ``x`` (fp32, before the final
    rounding).  ``x`` and ``gamma`` hold model-dtype values."""
    x = _f32(x)
    gamma = _f32(gamma)
    n = x.shape[-1]
    rows = x.size // n if n else 0
    y = np.empty_like(x)
    rc = _load().oracle_rms_norm(rows, n, _ptr(x), _ptr(gamma), float(eps), _ptr(y))
    if rc != 0:
        raise ValueError(f"oracle_rms_norm failed: {rc}")
    return y


def rope(x, pos, theta: float) -> np.ndarray:
    """Standalone rotate-half RoPE of ``x`` [T, dr] or [T, heads, dr], every
    head of token t rotated by ``pos[t]`` (fp32 rotation of fp32-rounded
    cos / sin of a double angle, before the final rounding)."""
    x = _f32(x)
    pos = _c(pos, np.int32)
    T, dr = x.shape[0], x.shape[-1]
    heads = x.shape[1] if x.ndim == 3 else 1
    y = np.empty_like(x)
    rc = _load().oracle_rope(T, heads, dr, _ptr(x), _ptr(pos), float(theta), _ptr(y))
    if rc != 0:
        raise ValueError(f"oracle_rope failed: {rc}")
    return y
