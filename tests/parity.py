"""Helpers shared by the parity tests: move a seeded workload to the GPU, run
the library through its Python binding, run the CPU oracle on the same
inputs, and compare element by element.

Tolerance (fp16 / bf16 outputs): |gpu - ref| <= 1e-2 + 1e-2 * |ref|, with
ref the oracle's fp32 value before the final rounding -- the rtol = atol =
1e-2 bar of the migration guide's golden test ("Precision verification"
section).  W8A8 int32 accumulators must match bit for bit.
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads
from workloads import Workload, widen

ATOL = 1e-2
RTOL = 1e-2


def torch_dev(a: np.ndarray, kind: str, device):
    import torch

    if kind == "f16":
        return torch.from_numpy(np.ascontiguousarray(a, np.float16)).to(device)
    if kind == "bf16":
        bits = np.ascontiguousarray(a, np.uint16).view(np.int16)
        return torch.from_numpy(bits).view(torch.bfloat16).to(device)
    if kind == "i8":
        return torch.from_numpy(np.ascontiguousarray(a, np.int8)).to(device)
    if kind == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
    if kind == "i32":
        return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(device)
    raise ValueError(kind)


def upload(w: Workload, device):
    t = dict(X=torch_dev(w.X, w.dtype, device), gamma=torch_dev(w.gamma, w.dtype, device),
             pos=torch_dev(w.positions, "i32", device))
    if w.kind == "fp":
        t["Wa"] = torch_dev(w.Wa, w.dtype, device)
        t["Wb"] = torch_dev(w.Wb, w.dtype, device)
    else:
        t["Wqa"] = torch_dev(w.Wqa, "i8", device)
        t["swa"] = torch_dev(w.swa, "f32", device)
        t["Wqb"] = torch_dev(w.Wqb, "i8", device)
        t["swb"] = torch_dev(w.swb, "f32", device)
    return t


def run_lib(w: Workload, t, dbg_rows=None, **kw):
    """Run the library; returns the four output tensors (on the GPU) and,
    for W8A8 with dbg_rows=(begin, n), the int32 accumulators."""
    import mla_attention_kv_amd as mla
    import torch

    if w.kind == "fp":
        return mla.mla_kv_prolog(t["X"], t["Wa"], t["gamma"], t["Wb"], t["pos"], w.eps,
                                 w.theta, **kw), None
    d1 = d2 = None
    b, n = (0, 0) if dbg_rows is None else dbg_rows
    if dbg_rows is not None:
        dev = t["X"].device
        d1 = torch.full((n, w.dims.N1), -7, dtype=torch.int32, device=dev)
        d2 = torch.full((n, w.dims.N2), -7, dtype=torch.int32, device=dev)
    outs = mla.mla_kv_prolog_w8a8(t["X"], t["Wqa"], t["swa"], t["gamma"], t["Wqb"], t["swb"],
                                  t["pos"], w.eps, w.theta, dbg_acc1=d1, dbg_acc2=d2,
                                  dbg_row_begin=b, dbg_rows=n, **kw)
    return outs, (d1, d2)


def run_oracle(w: Workload, rows=None, nthreads: int = 0):
    """Oracle outputs (fp32, before the final rounding) for all rows or the
    given subset of token rows."""
    sub = w if rows is None else w.rows(rows)
    d = w.dims
    if w.kind == "fp":
        return oracle.kv_prolog_fp(widen(sub.X, w.dtype), widen(w.Wa, w.dtype),
                                   widen(w.gamma, w.dtype), widen(w.Wb, w.dtype),
                                   sub.positions, r=d.r, dr=d.dr, nh=d.nh, dn=d.dn, dv=d.dv,
                                   eps=w.eps, theta=w.theta, dtype=w.dtype, nthreads=nthreads)
    return oracle.kv_prolog_w8a8(widen(sub.X, "bf16"), w.Wqa, w.swa, widen(w.gamma, "bf16"),
                                 w.Wqb, w.swb, sub.positions, r=d.r, dr=d.dr, nh=d.nh,
                                 dn=d.dn, dv=d.dv, eps=w.eps, theta=w.theta,
                                 nthreads=nthreads)


def gpu_rows(outs, rows=None):
    """GPU outputs as float64 numpy (optionally only some token rows)."""
    import torch

    names = ("k_nope", "value", "k_pe", "ckv")
    res = {}
    for n, o in zip(names, outs):
        if rows is not None:
            o = o[torch.as_tensor(np.asarray(rows), device=o.device)]
        res[n] = o.float().cpu().numpy().astype(np.float64)
    return res


def compare(gpu: dict, ref: dict, label: str = ""):
    """Element-wise tolerance check; returns per-output (max_abs, max_rel)."""
    stats = {}
    for n in ("k_nope", "value", "k_pe", "ckv"):
        g, r = gpu[n], ref[n]
        assert g.shape == r.shape, f"{label} {n}: shape {g.shape} vs {r.shape}"
        err = np.abs(g - r)
        bound = ATOL + RTOL * np.abs(r)
        bad = ~(err <= bound)
        if bad.any():
            idx = np.argwhere(bad)[:5]
            samples = [(tuple(i), float(g[tuple(i)]), float(r[tuple(i)])) for i in idx]
            raise AssertionError(
                f"{label} {n}: {int(bad.sum())} of {bad.size} elements out of tolerance; "
                f"first (index, gpu, ref): {samples}")
        stats[n] = (float(err.max(initial=0.0)),
                    float((err / np.maximum(np.abs(r), 1e-30)).max(initial=0.0)))
    return stats


def sample_rows(T: int, n: int, seed: int = 0, tile: int = 128):
    """Token rows for sampled parity: first, last, around tile edges, and
    random ones."""
    rng = np.random.default_rng(seed)
    rows = {0, T - 1}
    for e in (15, 16, 63, 64, 127, 128, tile - 1, tile, T // 2):
        if 0 <= e < T:
            rows.add(e)
    while len(rows) < min(n, T):
        rows.add(int(rng.integers(0, T)))
    return np.array(sorted(rows))


__all__ = ["upload", "run_lib", "run_oracle", "gpu_rows", "compare", "sample_rows",
           "workloads"]
