#!/usr/bin/env python3
"""Benchmark of the MLA KV prolog on one MI355X.

One step = one call of the whole prolog (kv_a_proj, split, RMSNorm,
kv_b_proj, reshape/split, RoPE, assemble) over one batch of seeded synthetic
input.  The headline workload is the largest single-GPU one: the
DeepSeek-R1-sized W8A8 packed prefill of 8 sequences (T = 12,874 for its
seed).  The same JSON line carries the four other workloads (V2-Lite fp16
decode at T = 1 and 64, V2-Lite fp16 prefill at T = 4096, R1 bf16 decode at
T = 256) under "configs", each with its time per call and roofline
fraction; --config N makes workload N the headline and measures it alone.

Timing: inputs, weights, outputs and workspace are replicated over enough
distinct buffers (>= 512 MB in total) that the 256 MB last-level cache
cannot serve a repeated call; successive steps rotate through them.  The K
timed steps run on one stream, bracketed by synchronisation and HIP events
on that stream, two ways: as HIP graph replays (launch overhead removed, as
a decode loop would run them) and as direct, stream-ordered calls (as a
prefill would); value = T * K / elapsed (tokens/s) of the faster, and the
JSON names it and gives both.

The binding roof of a workload is the one its algorithmic arithmetic
intensity (operations per algorithmic byte) puts it under: HBM below the
ridge point (peak operations / 8 TB/s), MFMA above; both fractions are
reported.

Prints ONE JSON line on stdout.

--op prolog_cached times the prolog with the paged KV-cache append fused
into its finish (each token's compressed_kv and k_pe rows also land in its
slot of a paged cache; the rotated input sets map to disjoint blocks of one
cache; for the W8A8 workload the int8 cache with one scale per slot);
--op prolog_then_append times the same work as two calls (the prolog, then
the append), for comparison.

--op rms_norm / rope time the standalone operators on the workload's shapes:
RMSNorm over [T, 512] (the latent), RoPE over [T, heads, 64] (a rope key per
head, the query-side shape).

--op graph_buckets times the library's captured decode buckets
(mla_prolog_graphs_*): one graph set per rotated input set, one
mla_prolog_graphs_launch per step issued from the host (the serving-loop
cost, launch included), against direct calls on the same sets.

--op graph_layers --layers L times a stack of L layers' prologs per step
(V2-Lite decode by default): one multi-layer graph launch
(mla_prolog_graphs_create_layers) against L direct calls, per layer.

--op vendor_gemm times the vendor library's GEMM (torch.matmul) on the two
projections' shapes, as a reference for the MFMA fractions (not the prolog).

--op cache_append / cache_append_int8 times the paged KV-cache append
instead (the step after "assemble"): the workload's T rows of
compressed_kv and k_pe (seeded, model dtype) written into a cache by a slot
mapping, rotating over input sets that map to disjoint slot ranges of one
cache.
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "i8": 5000.0}
ROTATE_BYTES = 512e6


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash(files=None) -> str:
    """Hash of the kernel sources: the given repository-relative files, or
    every file under the package's csrc/."""
    if files is None:
        paths = sorted(glob.glob(os.path.join(ROOT, "mla_attention_kv_amd", "csrc", "*")))
    else:
        paths = [os.path.join(ROOT, f) for f in sorted(files)]
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per call and per kernel (launch order) from committed
    rocprofv3 counter runs, or None when they are absent or any source file
    of the kernels they measured (listed in the file as "sources") has
    changed since."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("src_hash") != kernel_source_hash(t.get("sources")):
        return None
    return {"call": t.get("hbm_bytes_per_launch"), "kernels": t.get("kernel_hbm_bytes")}


class Sets:
    """n_sets device copies of one workload's tensors plus output buffers and
    workspace, with ready-made C argument tuples."""

    def __init__(self, w, n_sets, dev, cache_mode=None):
        import torch

        import mla_attention_kv_amd as mla
        from tests.parity import upload

        self.mla = mla
        self.w = w
        d = w.dims
        self.dims = mla.Dims(H=d.H, nh=d.nh, r=d.r, dr=d.dr, dn=d.dn, dv=d.dv)
        base = upload(w, dev)
        odt = torch.float16 if w.dtype == "f16" else torch.bfloat16
        if w.kind == "fp":
            code = mla.MLA_F16 if w.dtype == "f16" else mla.MLA_BF16
            nbytes = mla.mla_kv_prolog_workspace_size(w.T, self.dims, code)
        else:
            code = None
            nbytes = mla.mla_kv_prolog_w8a8_workspace_size(w.T, self.dims)
        self.keep = []
        self.args = []
        self.cache_mode = cache_mode
        self.append_args = []
        if cache_mode is not None:
            import workloads

            slots, nsl = workloads.paged_slot_mapping(w, seed=7)
            # fp16 / bf16 prolog: a cache of the model dtype; W8A8: the int8
            # cache with one scale per slot
            cdt = odt if w.kind == "fp" else torch.int8
            self.cache = torch.zeros((nsl * n_sets, d.r + d.dr), dtype=cdt, device=dev)
            self.scale = torch.zeros(nsl * n_sets, dtype=torch.float32, device=dev)
            self.slot_sets = [torch.from_numpy(slots + i * nsl).to(dev) for i in range(n_sets)]
        for i in range(n_sets):
            t = {k: v.clone() for k, v in base.items()}
            outs = (torch.empty((w.T, d.nh, d.dn), dtype=odt, device=dev),
                    torch.empty((w.T, d.nh, d.dv), dtype=odt, device=dev),
                    torch.empty((w.T, d.dr), dtype=odt, device=dev),
                    torch.empty((w.T, d.r), dtype=odt, device=dev))
            ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
            self.keep.append((t, outs, ws))
            if w.kind == "fp":
                a = (t["X"].data_ptr(), t["Wa"].data_ptr(), t["gamma"].data_ptr(),
                     t["Wb"].data_ptr(), t["pos"].data_ptr(), w.T, self.dims.c(), code,
                     w.eps, w.theta, outs[0].data_ptr(), outs[1].data_ptr(),
                     outs[2].data_ptr(), outs[3].data_ptr(), ws.data_ptr(), ws.numel())
                if cache_mode == "fused":
                    a = a[:14] + (self.slot_sets[i].data_ptr(), self.cache.data_ptr(),
                                  self.cache.shape[0]) + a[14:]
                elif cache_mode == "separate":
                    self.append_args.append(
                        (outs[3].data_ptr(), outs[2].data_ptr(), self.slot_sets[i].data_ptr(),
                         w.T, self.dims.c(), code, self.cache.data_ptr(), self.cache.shape[0]))
            else:
                a = (t["X"].data_ptr(), t["Wqa"].data_ptr(), t["swa"].data_ptr(),
                     t["gamma"].data_ptr(), t["Wqb"].data_ptr(), t["swb"].data_ptr(),
                     t["pos"].data_ptr(), w.T, self.dims.c(), w.eps, w.theta,
                     outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(),
                     outs[3].data_ptr(), None, None, 0, 0, ws.data_ptr(), ws.numel())
                if cache_mode == "fused":
                    a = a[:15] + (self.slot_sets[i].data_ptr(), None, self.cache.data_ptr(),
                                  self.scale.data_ptr(), self.cache.shape[0]) + a[19:]
                elif cache_mode == "separate":
                    self.append_args.append(
                        (outs[3].data_ptr(), outs[2].data_ptr(), self.slot_sets[i].data_ptr(),
                         w.T, self.dims.c(), mla.MLA_BF16, self.cache.data_ptr(),
                         self.scale.data_ptr(), self.cache.shape[0]))
            self.args.append(a)
        self.fn = mla.lib().mla_kv_prolog if w.kind == "fp" else mla.lib().mla_kv_prolog_w8a8
        if cache_mode == "fused":
            self.fn = (mla.lib().mla_kv_prolog_cached if w.kind == "fp"
                       else mla.lib().mla_kv_prolog_w8a8_cached)
        self.append_fn = (mla.lib().mla_kv_cache_append if w.kind == "fp"
                          else mla.lib().mla_kv_cache_append_int8)

    def call(self, i, stream_ptr):
        st = self.fn(*self.args[i % len(self.args)], ctypes.c_void_p(stream_ptr))
        if st == 0 and self.cache_mode == "separate":
            st = self.append_fn(*self.append_args[i % len(self.args)],
                                ctypes.c_void_p(stream_ptr))
        if st != 0:
            raise RuntimeError(f"library call failed: {self.mla.mla_status_string(st)}")


def time_graph(sets, steps, warmup, dev):
    """Capture one rotation cycle (and the remainder) as HIP graphs, replay
    so that exactly `steps` calls run; return elapsed ms (events)."""
    import torch

    n = len(sets.args)
    cap = torch.cuda.Stream(device=dev)
    graphs = {}

    def make(count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            sp = torch.cuda.current_stream(dev).cuda_stream
            for i in range(count):
                sets.call(i, sp)
        return g

    full = make(n)
    rem = steps % n
    part = make(rem) if rem else None
    torch.cuda.synchronize()
    wfull = max(1, math.ceil(warmup / n)) if warmup > 0 else 0
    for _ in range(wfull):
        full.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps // n):
        full.replay()
    if part is not None:
        part.replay()
    e1.record()
    torch.cuda.synchronize()
    del graphs
    return e0.elapsed_time(e1)


class GraphBucketSets:
    """The library's own captured decode buckets (mla_prolog_graphs_*): one
    graph set per rotated input set, each with buckets 1, 2, 4, ... up to the
    first power of two >= T, over static buffers filled with that set's
    inputs.  A step is one mla_prolog_graphs_launch (one hipGraphLaunch)."""

    def __init__(self, sets, T):
        import mla_attention_kv_amd as mla

        self.mla = mla
        buckets = [1]
        while buckets[-1] < T:
            buckets.append(buckets[-1] * 2)
        self.buckets = tuple(buckets)
        self.graphs = []
        w = sets.w
        for t, _outs, _ws in sets.keep:
            weights = ((t["Wa"], t["gamma"], t["Wb"]) if w.kind == "fp" else
                       (t["Wqa"], t["swa"], t["gamma"], t["Wqb"], t["swb"]))
            g = mla.PrologGraphs(weights, self.buckets, w.eps, w.theta, w8a8=w.kind != "fp")
            g.hidden[:T] = t["X"]
            g.positions[:T] = t["pos"]
            self.graphs.append(g)
        self.T = T
        self.launch = mla.lib().mla_prolog_graphs_launch

    def call(self, i, stream_ptr):
        g = self.graphs[i % len(self.graphs)]
        st = self.launch(g.handle, self.T, ctypes.c_void_p(stream_ptr), None)
        if st != 0:
            raise RuntimeError(f"library call failed: {self.mla.mla_status_string(st)}")


class LayerStack:
    """n_models stand-ins of an L-layer model for one workload: each model
    holds L layers' weights (copies of the workload's, at distinct
    addresses) and one multi-layer graph set over them (one bucket, the
    workload's T).  call() is one step of the stack: either one
    mla_prolog_graphs_launch replaying all L prologs (graph=True), or L
    direct prolog calls over the same buffers."""

    def __init__(self, w, L, n_models, dev, graph):
        import mla_attention_kv_amd as mla
        from tests.parity import upload

        self.mla, self.w, self.L, self.graph = mla, w, L, graph
        base = upload(w, dev)
        fp = w.kind == "fp"
        names = ("Wa", "gamma", "Wb") if fp else ("Wqa", "swa", "gamma", "Wqb", "swb")
        self.models = []
        for _ in range(n_models):
            layers = [tuple(base[n].clone() for n in names) for _ in range(L)]
            g = mla.PrologGraphs(layers, (w.T,), w.eps, w.theta, w8a8=not fp)
            g.hidden[:w.T] = base["X"]
            g.positions[:w.T] = base["pos"]
            self.models.append((g, layers))
        d = w.dims
        self.dims = mla.Dims(H=d.H, nh=d.nh).c()
        self.code = mla.MLA_F16 if w.dtype == "f16" else mla.MLA_BF16
        self.launch = mla.lib().mla_prolog_graphs_launch
        self.fn = mla.lib().mla_kv_prolog if fp else mla.lib().mla_kv_prolog_w8a8
        self.args = self.models  # the rotation (time_graph's cycle length)

    def call(self, i, stream_ptr):
        g, layers = self.models[i % len(self.models)]
        sp = ctypes.c_void_p(stream_ptr)
        if self.graph:
            st = self.launch(g.handle, self.w.T, sp, None)
        else:
            st = 0
            T = self.w.T
            for l in range(self.L):
                outs = (g.k_nope[l].data_ptr(), g.value[l].data_ptr(), g.k_pe[l].data_ptr(),
                        g.compressed_kv[l].data_ptr())
                if self.w.kind == "fp":
                    Wa, gamma, Wb = layers[l]
                    st = self.fn(g.hidden.data_ptr(), Wa.data_ptr(), gamma.data_ptr(),
                                 Wb.data_ptr(), g.positions.data_ptr(), T, self.dims, self.code,
                                 self.w.eps, self.w.theta, *outs, g.workspace.data_ptr(),
                                 g.workspace.numel(), sp)
                else:
                    Wqa, swa, gamma, Wqb, swb = layers[l]
                    st = self.fn(g.hidden.data_ptr(), Wqa.data_ptr(), swa.data_ptr(),
                                 gamma.data_ptr(), Wqb.data_ptr(), swb.data_ptr(),
                                 g.positions.data_ptr(), T, self.dims, self.w.eps, self.w.theta,
                                 *outs, None, None, 0, 0, g.workspace.data_ptr(),
                                 g.workspace.numel(), sp)
                if st != 0:
                    break
        if st != 0:
            raise RuntimeError(f"library call failed: {self.mla.mla_status_string(st)}")


def main_layers(args, headline, dev):
    """--op graph_layers: an L-layer stack of prologs per step, as one
    multi-layer graph launch against L direct calls; reports time per layer."""
    import torch

    import workloads

    cfg = workloads.CONFIGS[headline]
    w = workloads.make_config(headline)
    L = args.layers
    per_layer = workloads.algorithmic_bytes(w.dims, w.T, w.kind, w.dtype)
    n_models = max(2, math.ceil(ROTATE_BYTES / (L * per_layer)))
    log(f"{cfg['name']}: {L} layers per step, {n_models} rotated models")
    res = {}
    for graph in (True, False):
        stack = LayerStack(w, L, n_models, dev, graph)
        torch.cuda.synchronize()
        ms = time_eager(stack, args.steps, args.warmup, dev)
        res["graph" if graph else "direct"] = ms / args.steps / L * 1e3
        if not graph:
            # the same direct calls captured into one replayed graph per rotation
            res["direct_replayed"] = time_graph(stack, args.steps, args.warmup, dev) / args.steps / L * 1e3
        del stack
        torch.cuda.empty_cache()
    log(f"per layer: one multi-layer graph launch {res['graph']:.2f} us, direct calls "
        f"{res['direct']:.2f} us, direct calls replayed as a captured graph "
        f"{res['direct_replayed']:.2f} us")
    out = {"metric": "MLA KV prolog time per layer of an L-layer stack", "unit": "us",
           "value": res["graph"], "higher_is_better": False, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "data": "synthetic (seeded; no public dataset exists for this path)",
           "config": {"workload": cfg["name"] + f"_{L}_layers", "T": w.T, "layers": L,
                      "rotated_models": n_models,
                      "timing": "events around K host-issued steps (launches included)"},
           "us_per_layer": res}
    print(json.dumps(out), flush=True)


def vendor_gemm_reference(dev, steps):
    """The vendor library's GEMM (torch.matmul, i.e. hipBLASLt) on the
    prolog's two projections at the workloads' shapes: a reference point for
    the MFMA fractions, not part of the prolog.  Rotates over buffer sets,
    times with events on the current stream."""
    import torch

    shapes = [("v2lite_prefill_kv_b", 4096, 512, 4096, torch.float16),
              ("v2lite_prefill_kv_a", 4096, 2048, 576, torch.float16),
              ("r1_T256_kv_b", 256, 512, 32768, torch.bfloat16),
              ("r1_T256_kv_a", 256, 7168, 576, torch.bfloat16),
              ("r1_T12874_kv_b_bf16", 12874, 512, 32768, torch.bfloat16),
              ("r1_T12874_kv_a_bf16", 12874, 7168, 576, torch.bfloat16)]
    out = []
    for name, M, K, N, dt in shapes:
        nsets = max(2, min(8, int(512e6 // ((M * K + K * N + M * N) * 2))))
        A = [torch.randn(M, K, device=dev).to(dt) for _ in range(nsets)]
        B = [(torch.randn(K, N, device=dev) * 0.02).to(dt) for _ in range(nsets)]
        C = [torch.empty(M, N, device=dev, dtype=dt) for _ in range(nsets)]
        reps = max(10, min(steps, int(2e5 // max(1, M * N * K // 10**7))))
        for i in range(10):
            torch.matmul(A[i % nsets], B[i % nsets], out=C[i % nsets])
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            torch.matmul(A[i % nsets], B[i % nsets], out=C[i % nsets])
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        tf = 2.0 * M * K * N / us / 1e6
        log(f"{name}: {us:.2f} us, {tf:.0f} TFLOP/s")
        out.append({"gemm": name, "M": M, "K": K, "N": N, "dtype": str(dt).split(".")[-1],
                    "us": us, "tflops": tf, "frac_of_2.5PF": tf / 2500.0})
        del A, B, C
    print(json.dumps({"metric": "vendor GEMM (torch.matmul) on the prolog's projection shapes",
                      "unit": "us", "higher_is_better": False, "results": out}), flush=True)


def time_eager(sets, steps, warmup, dev):
    import torch

    sp = torch.cuda.current_stream(dev).cuda_stream
    for i in range(warmup):
        sets.call(i, sp)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        sets.call(i, sp)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def cpu_baseline(w, seconds):
    """The CPU oracle, as it stands, on a bounded sample of the same
    workload: whole batches (or the first 256 token rows) repeated until
    about `seconds` have elapsed.  The inputs are widened to the oracle's
    fp32 form once, outside the timed loop."""
    import numpy as np

    import oracle
    from workloads import widen

    nthreads = oracle.num_threads(0)
    rows = None if w.T <= 256 else np.arange(256)
    sub = w if rows is None else w.rows(rows)
    d = w.dims
    kw = dict(r=d.r, dr=d.dr, nh=d.nh, dn=d.dn, dv=d.dv, eps=w.eps, theta=w.theta)
    if w.kind == "fp":
        args = (widen(sub.X, w.dtype), widen(w.Wa, w.dtype), widen(w.gamma, w.dtype),
                widen(w.Wb, w.dtype), sub.positions)
        f = lambda: oracle.kv_prolog_fp(*args, dtype=w.dtype, **kw)  # noqa: E731
    else:
        args = (widen(sub.X, "bf16"), w.Wqa, w.swa, widen(w.gamma, "bf16"), w.Wqb, w.swb,
                sub.positions)
        f = lambda: oracle.kv_prolog_w8a8(*args, want_acc=False, **kw)  # noqa: E731
    ntok = sub.T
    t0 = time.perf_counter()
    f()
    one = time.perf_counter() - t0
    reps = max(1, min(100000, int(seconds / max(one, 1e-6))))
    t0 = time.perf_counter()
    for _ in range(reps):
        f()
    dt = time.perf_counter() - t0
    sample = (f"{reps} x {'all ' if rows is None else 'the first '}{ntok} token rows of the "
              f"same seeded workload ({dt:.1f} s)")
    return {"value": ntok * reps / dt, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": sample}


class CacheSets:
    """Rotated inputs of the paged KV-cache append: n_sets of (compressed_kv,
    k_pe, slot mapping) over disjoint slot ranges of one shared cache, with
    the same call interface as Sets."""

    def __init__(self, T, dtype, int8, n_sets, dev, seed):
        import numpy as np
        import torch

        import mla_attention_kv_amd as mla

        self.mla = mla
        tdt = torch.float16 if dtype == "f16" else torch.bfloat16
        code = mla.MLA_F16 if dtype == "f16" else mla.MLA_BF16
        rng = np.random.default_rng(seed)
        S = T * n_sets
        if int8:
            self.cache = (torch.zeros((S, 576), dtype=torch.int8, device=dev),
                          torch.zeros(S, dtype=torch.float32, device=dev))
        else:
            self.cache = (torch.zeros((S, 576), dtype=tdt, device=dev),)
        self.keep, self.args = [], []
        d = mla.Dims(H=64, nh=1).c()
        for i in range(n_sets):
            ckv = torch.from_numpy(rng.standard_normal((T, 512)).astype(np.float32)).to(tdt).to(dev)
            kpe = torch.from_numpy(rng.standard_normal((T, 64)).astype(np.float32)).to(tdt).to(dev)
            slots = torch.from_numpy(i * T + rng.permutation(T).astype(np.int64)).to(dev)
            self.keep.append((ckv, kpe, slots))
            if int8:
                a = (ckv.data_ptr(), kpe.data_ptr(), slots.data_ptr(), T, d, code,
                     self.cache[0].data_ptr(), self.cache[1].data_ptr(), S)
            else:
                a = (ckv.data_ptr(), kpe.data_ptr(), slots.data_ptr(), T, d, code,
                     self.cache[0].data_ptr(), S)
            self.args.append(a)
        self.fn = mla.lib().mla_kv_cache_append_int8 if int8 else mla.lib().mla_kv_cache_append

    def call(self, i, stream_ptr):
        st = self.fn(*self.args[i % len(self.args)], ctypes.c_void_p(stream_ptr))
        if st != 0:
            raise RuntimeError(f"library call failed: {self.mla.mla_status_string(st)}")


class ElemSets:
    """Rotated inputs of the standalone RMSNorm / RoPE: n_sets of (x, out)
    plus gamma / positions, same call interface as Sets."""

    def __init__(self, op, T, heads, dtype, n_sets, dev, seed):
        import numpy as np
        import torch

        import mla_attention_kv_amd as mla

        self.mla = mla
        tdt = torch.float16 if dtype == "f16" else torch.bfloat16
        code = mla.MLA_F16 if dtype == "f16" else mla.MLA_BF16
        rng = np.random.default_rng(seed)
        shape = (T, 512) if op == "rms_norm" else (T, heads, 64)
        self.keep, self.args = [], []
        for _ in range(n_sets):
            x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(tdt).to(dev)
            y = torch.empty_like(x)
            if op == "rms_norm":
                g = torch.from_numpy(rng.uniform(0.5, 1.5, 512).astype(np.float32)).to(tdt).to(dev)
                a = (x.data_ptr(), g.data_ptr(), T, 512, code, 1e-6, y.data_ptr())
            else:
                g = torch.from_numpy(rng.integers(0, 32768, T).astype(np.int32)).to(dev)
                a = (x.data_ptr(), g.data_ptr(), T, heads, 64, code, 1e4, y.data_ptr())
            self.keep.append((x, y, g))
            self.args.append(a)
        self.fn = mla.lib().mla_rms_norm if op == "rms_norm" else mla.lib().mla_rope

    def call(self, i, stream_ptr):
        st = self.fn(*self.args[i % len(self.args)], ctypes.c_void_p(stream_ptr))
        if st != 0:
            raise RuntimeError(f"library call failed: {self.mla.mla_status_string(st)}")


def elem_cpu_baseline(op, T, heads, dtype, seconds, seed):
    """The CPU oracle of RMSNorm / RoPE on (a prefix of) the same shapes,
    repeated for about `seconds`."""
    import numpy as np

    import oracle

    rng = np.random.default_rng(seed)
    rows = min(T, 1024)
    if op == "rms_norm":
        x = oracle.round_to_dtype(rng.standard_normal((rows, 512)), dtype)
        g = oracle.round_to_dtype(rng.uniform(0.5, 1.5, 512), dtype)
        f = lambda: oracle.rms_norm(x, g, 1e-6)  # noqa: E731
    else:
        x = oracle.round_to_dtype(rng.standard_normal((rows, heads, 64)), dtype)
        pos = rng.integers(0, 32768, rows).astype(np.int32)
        f = lambda: oracle.rope(x, pos, 1e4)  # noqa: E731
    t0 = time.perf_counter()
    f()
    one = time.perf_counter() - t0
    reps = max(1, min(100000, int(seconds / max(one, 1e-6))))
    t0 = time.perf_counter()
    for _ in range(reps):
        f()
    dt = time.perf_counter() - t0
    return {"value": rows * reps / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} x the first {rows} token rows ({dt:.1f} s; single-threaded)"}


def main_elem(args, cfg, w, dev):
    import torch

    op = args.op
    heads = w.dims.nh
    per_tok = 512 * 2 * 2 if op == "rms_norm" else heads * 64 * 2 * 2 + 4
    alg_bytes = w.T * per_tok + (512 * 2 if op == "rms_norm" else 0)
    n_sets = max(2, math.ceil(ROTATE_BYTES / alg_bytes))
    log(f"{op}: T={w.T} heads={heads} bytes/step={alg_bytes} sets={n_sets}")
    sets = ElemSets(op, w.T, heads, w.dtype, n_sets, dev, seed=1000 + args.config)
    torch.cuda.synchronize()
    steps, warmup = args.steps, args.warmup
    ms = time_graph(sets, steps, warmup, dev)
    ms_per_step = ms / steps
    step_s = ms_per_step / 1e3
    value = w.T * steps / (ms / 1e3)
    log(f"{ms_per_step * 1e3:.2f} us/step, {value:.4g} tokens/s")
    roof = {"bound": "hbm", "achieved": alg_bytes / step_s / 1e9, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "traffic": None,
            "kernel": ("rms_norm_kernel" if op == "rms_norm" else "rope_kernel") +
                      " (one launch per call)"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    cpu = None
    if not args.no_cpu_baseline:
        cpu = elem_cpu_baseline(op, w.T, heads, w.dtype, args.cpu_seconds, 1000 + args.config)
    shape = [w.T, 512] if op == "rms_norm" else [w.T, heads, 64]
    out = {
        "metric": f"MLA standalone {op} tokens/s + % HBM roofline",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded; no public dataset exists for this path)",
        "config": {"workload": f"{cfg['name']}_{op}", "T": w.T, "shape": shape,
                   "timing": "HIP graph replays", "rotated_sets": n_sets,
                   "algorithmic_bytes_per_step": alg_bytes},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cache_cpu_baseline(T, dtype, int8, seconds, seed):
    """The CPU oracle of the append on the same shapes, repeated for about
    `seconds`."""
    import numpy as np

    import oracle

    rng = np.random.default_rng(seed)
    ckv = oracle.round_to_dtype(rng.standard_normal((T, 512)), dtype)
    kpe = oracle.round_to_dtype(rng.standard_normal((T, 64)), dtype)
    slots = rng.permutation(T).astype(np.int64)
    if int8:
        q, sc = np.zeros((T, 576), np.int8), np.zeros(T, np.float32)
        f = lambda: oracle.kv_cache_append_int8(ckv, kpe, slots, q, sc)  # noqa: E731
    else:
        cache = np.zeros((T, 576))
        f = lambda: oracle.kv_cache_append(ckv, kpe, slots, cache)  # noqa: E731
    t0 = time.perf_counter()
    f()
    one = time.perf_counter() - t0
    reps = max(1, min(100000, int(seconds / max(one, 1e-6))))
    t0 = time.perf_counter()
    for _ in range(reps):
        f()
    dt = time.perf_counter() - t0
    return {"value": T * reps / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} x all {T} token rows ({dt:.1f} s; the append is single-threaded)"}


def main_cache(args, cfg, w, dev):
    import torch

    int8 = args.op == "cache_append_int8"
    es = 2
    per_tok = 576 * es + 8 + (576 + 4 if int8 else 576 * es)  # read rows + slot, write slot
    alg_bytes = w.T * per_tok
    n_sets = max(2, math.ceil(ROTATE_BYTES / alg_bytes))
    log(f"cache append{' int8' if int8 else ''}: T={w.T} bytes/step={alg_bytes} sets={n_sets}")
    sets = CacheSets(w.T, w.dtype, int8, n_sets, dev, seed=1000 + args.config)
    torch.cuda.synchronize()
    steps, warmup = args.steps, args.warmup
    ms = time_graph(sets, steps, warmup, dev)
    ms_per_step = ms / steps
    step_s = ms_per_step / 1e3
    value = w.T * steps / (ms / 1e3)
    log(f"{ms_per_step * 1e3:.2f} us/step, {value:.4g} tokens/s")
    roof = {"bound": "hbm", "achieved": alg_bytes / step_s / 1e9, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "traffic": None,
            "kernel": "kv_cache_append_kernel (one launch per call)"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cache_cpu_baseline(w.T, w.dtype, int8, args.cpu_seconds, 1000 + args.config)
    out = {
        "metric": "MLA KV cache append tokens/s + % HBM roofline",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8" if int8 else w.dtype,
        "data": "synthetic (seeded; no public dataset exists for this path)",
        "config": {"workload": f"{cfg['name']}_{args.op}", "T": w.T, "slot_width": 576,
                   "cache_slots": w.T * n_sets, "timing": "HIP graph replays",
                   "rotated_sets": n_sets, "algorithmic_bytes_per_step": alg_bytes},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def kernel_parts(w, path, n_kernels):
    """Names and algorithmic (bytes, operations) of the kernels one call
    launches, in launch order: what each kernel must read and write at least
    once as a stand-alone step (its inputs and its result; the kv_a_proj
    result counted once in fp32, [T, 576]) and the multiply-adds it does
    (2 operations each)."""
    d, T = w.dims, w.T
    D = 2
    fp = w.kind == "fp"
    wa = d.H * d.N1 * (D if fp else 1) + (0 if fp else 4 * d.N1)
    wb = d.r * d.N2 * (D if fp else 1) + (0 if fp else 4 * d.N2)
    xin = T * d.H * D + 4 * T
    a_out = T * d.N1 * 4
    fin_out = T * (d.r + d.dr) * D + (0 if fp else T * (d.r + 8))
    kv_out = T * d.N2 * D
    lat_in = T * d.r * (D if fp else 1) + (0 if fp else 8 * T)
    f1, f2 = 2 * T * d.H * d.N1, 2 * T * d.r * d.N2
    kv_a = ("kv_a_proj GEMM", (T * d.H * (D if fp else 1) + wa + a_out, f1))
    finish = ("finish (split, RMSNorm, RoPE)", (a_out + d.r * D + 4 * T + fin_out, 0))
    kv_b = ("kv_b_proj GEMM", (lat_in + wb + kv_out, f2))
    if not fp:
        quant = ("activation quantiser", (xin + T * d.H + 4 * T, 0))
        fused = ("finish fused into kv_b_proj (W8A8 decode)",
                 (a_out + d.r * D + 4 * T + fin_out + wb + kv_out, f2))
        if n_kernels == 2:  # up to 8 tokens: the quantiser folded into kv_a_proj too
            return [("kv_a_proj with the activation quantiser folded in (W8A8 decode)",
                     (xin + wa + a_out, f1)), fused]
        if n_kernels == 3:  # decode sizes: the finish fused into kv_b_proj
            return [quant, kv_a, fused]
        return [quant, kv_a, finish, kv_b]
    if path == 1 and n_kernels == 2:  # the finish and kv_b_proj in one launch
        return [kv_a, ("finish + kv_b_proj in one launch (latent staged in LDS)",
                       (a_out + d.r * D + 4 * T + fin_out + wb + kv_out, f2))]
    if path == 0 and n_kernels == 2:
        return [("dec_kv_a (kv_a_proj, split-K)", (xin + wa + a_out, f1)),
                ("dec_fin_kv_b (finish fused into kv_b_proj)",
                 (a_out + d.r * D + 4 * T + fin_out + wb + kv_out, f2))]
    if path == 0:
        return [("dec_kv_a (kv_a_proj, split-K)", (xin + wa + a_out, f1)),
                ("dec_finish", finish[1]), ("dec_kv_b", kv_b[1])]
    return [kv_a, finish, kv_b]


def kernel_times(sets, reps, dev):
    """Average duration of each kernel of a call, live: pairs of events
    registered with the library (mla_debug_set_launch_events) are recorded
    at each kernel's own start and end (its dispatch timestamps); eager
    calls rotating over the input sets."""
    import torch

    L = sets.mla.lib()
    sp = torch.cuda.current_stream(dev).cuda_stream
    maxk = 8
    sums = None
    for i in range(reps + 3):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * maxk)]
        for e in evs:
            e.record()
        torch.cuda.synchronize()
        arr = (ctypes.c_void_p * (2 * maxk))(*[e.cuda_event for e in evs])
        L.mla_debug_set_launch_events(arr, 2 * maxk)
        sets.call(i, sp)
        used = L.mla_debug_set_launch_events(None, 0)
        torch.cuda.synchronize()
        ms = [evs[2 * k].elapsed_time(evs[2 * k + 1]) for k in range(used // 2)]
        if i < 3:
            continue  # warm-up calls
        sums = ms if sums is None else [a + x for a, x in zip(sums, ms)]
    return [s / reps * 1e3 for s in sums]  # microseconds


def roofline(w, step_s, alg_bytes, alg_flops):
    """Roofline of one call: the binding roof is HBM when the algorithmic
    arithmetic intensity is below the ridge point of the workload's MFMA
    dtype, MFMA above it; both fractions are given."""
    dt = "i8" if w.kind == "w8a8" else w.dtype
    hbm = alg_bytes / step_s / 1e9
    mfma = alg_flops / step_s / 1e12
    ridge = MFMA_PEAK_TFLOPS[dt] * 1e12 / (HBM_PEAK_GBS * 1e9)
    ai = alg_flops / alg_bytes
    if ai < ridge:
        roof = {"bound": "hbm", "achieved": hbm, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": mfma, "peak": MFMA_PEAK_TFLOPS[dt],
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["hbm_frac"] = hbm / HBM_PEAK_GBS
    roof["mfma_frac"] = mfma / MFMA_PEAK_TFLOPS[dt]
    roof["mfma_dtype"] = dt
    roof["arith_intensity"] = ai
    roof["ridge"] = ridge
    return roof


def kernel_names(w, path, cache_mode):
    fused_decode = path == 0 and w.kind == "fp" and w.T <= 64
    if fused_decode:
        k = "dec_kv_a + dec_fin_kv_b (finish fused into kv_b_proj)"
    elif w.kind == "w8a8":
        k = "kv_a_proj GEMM + finish + kv_b_proj GEMM (+ activation quantiser)"
    else:
        k = "kv_a_proj GEMM + finish + kv_b_proj GEMM"
    k = "one library call = every launch of the step: " + k
    k += {None: "", "fused": "; paged-cache write fused into the finish",
          "separate": "; then kv_cache_append"}[cache_mode]
    if cache_mode is not None and w.kind != "fp":
        k += " (int8 cache)"
    return k


def measure_prolog(idx, steps, warmup, dev, args, cache_mode=None, graph_buckets=False):
    """Time one workload's prolog over rotated input sets; returns a dict of
    the measurements (the workload is returned too, for the CPU baseline)."""
    import torch

    import mla_attention_kv_amd as mla
    import workloads

    cfg = dict(workloads.CONFIGS[idx])
    if getattr(args, "tokens", None):
        # the configuration's model, dtype and value distributions at another
        # token count (positions uniform over [0, 32768))
        cfg["name"] = f"{cfg['name']}_at_T{args.tokens}"
        log(f"generating workload {cfg['name']}")
        w = workloads.make_custom(cfg["dims"], args.tokens, kind=cfg["kind"], dtype=cfg["dtype"],
                                  seed=1000 + idx, wstd=cfg["wstd"], max_pos=32768)
    else:
        log(f"generating workload {cfg['name']}")
        w = workloads.make_config(idx)
    d = w.dims
    alg_bytes = workloads.algorithmic_bytes(d, w.T, w.kind, w.dtype)
    if cache_mode is not None:
        # each token's cache slot (int8 codes + scale for W8A8) and its slot index
        alg_bytes += w.T * ((d.r + d.dr) * (2 if w.kind == "fp" else 1) +
                            (0 if w.kind == "fp" else 4) + 8)
    alg_flops = workloads.algorithmic_flops(d, w.T)
    n_sets = max(1, math.ceil(ROTATE_BYTES / alg_bytes))
    log(f"T={w.T} algorithmic bytes/step={alg_bytes} flops/step={alg_flops} sets={n_sets}")
    sets = Sets(w, n_sets, dev, cache_mode)
    torch.cuda.synchronize()

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    buckets = None
    eager_steps = min(steps, 2000)
    if graph_buckets:
        # the library's captured buckets, one graph launch per step from the
        # host, against direct calls on the same rotated sets
        buckets = GraphBucketSets(sets, w.T)
        torch.cuda.synchronize()
        ms = time_eager(buckets, steps, warmup, dev)
        eager_ms = time_eager(sets, eager_steps, min(warmup, 200), dev) * steps / eager_steps
    elif args.eager:
        ms = time_eager(sets, steps, warmup, dev)
        eager_ms = ms
    else:
        ms = time_graph(sets, steps, warmup, dev)
        eager_ms = time_eager(sets, eager_steps, min(warmup, 200), dev) * steps / eager_steps
    graph_ms = ms if buckets is None and not args.eager else None
    # a whole call is run either way: report the faster of the graph replays
    # and the direct calls (both measured; direct calls over exactly the
    # same step count when they are the reported figure)
    use_eager = graph_ms is not None and eager_ms < graph_ms
    if use_eager and eager_steps != steps:
        eager_ms = time_eager(sets, steps, min(warmup, 200), dev)
        use_eager = eager_ms < graph_ms
    if use_eager:
        ms = eager_ms
    ms_per_step = ms / steps
    value = w.T * steps / (ms / 1e3)
    log(f"{cfg['name']}: {ms_per_step * 1e3:.2f} us/step, {value:.4g} tokens/s "
        f"(eager {eager_ms / steps * 1e3:.2f} us/step"
        + (f", graph {graph_ms / steps * 1e3:.2f} us/step)" if graph_ms is not None else ")"))
    path = mla.mla_kv_prolog_selected_path(w.T, sets.dims)
    call_roof = roofline(w, ms_per_step / 1e3, alg_bytes, alg_flops)
    traffic = (load_traffic(cfg["name"]) if cache_mode is None and buckets is None else None)
    call_roof["traffic"] = traffic["call"] if traffic else None
    call_roof["traffic_source"] = (f"profiles/traffic_{cfg['name']}.json: rocprofv3 FETCH_SIZE / "
                                   "WRITE_SIZE of the same kernel sources from a separate profiling "
                                   "run, not measured in this run" if traffic else None)
    call_roof["kernel"] = kernel_names(w, path, cache_mode)
    # the dominant kernel, timed live per kernel (eager calls)
    kus = (kernel_times(sets, max(10, min(200, int(2e4 / max(ms_per_step * 1e3, 1.0)))), dev)
           if cache_mode is None and buckets is None else [])
    parts = kernel_parts(w, path, len(kus))
    kernels = []
    for k, ((name, (kb, kf)), us) in enumerate(zip(parts, kus)):
        r = roofline(w, us * 1e-6, kb, max(kf, 1))
        kernels.append({"kernel": name, "avg_us": us, "algorithmic_bytes": kb,
                        "algorithmic_ops": kf, "hbm_frac": r["hbm_frac"],
                        "mfma_frac": r["mfma_frac"] if kf else 0.0})
    dom = max(range(len(kus)), key=lambda k: kus[k]) if kus else None
    if dom is not None:
        name, (kb, kf) = parts[dom]
        roof = roofline(w, kus[dom] * 1e-6, kb, max(kf, 1))
        roof["kernel"] = f"{name}: the call's longest kernel ({kus[dom]:.2f} us of " \
                         f"{sum(kus):.2f} us of kernel time; HIP events at its dispatch start and end, eager calls)"
        per_k = traffic.get("kernels") if traffic else None
        roof["traffic"] = per_k[dom] if per_k and dom < len(per_k) else None
        roof["traffic_source"] = call_roof["traffic_source"] if roof["traffic"] else None
        roof["call"] = call_roof
    else:
        roof = call_roof
    timing = ("one mla_prolog_graphs_launch per step (buckets "
              f"{list(buckets.buckets)})" if buckets is not None
              else "eager calls" if args.eager
              else "direct calls, stream-ordered (faster than HIP graph replays of the same calls "
                   "here)" if use_eager
              else "HIP graph replays of the calls (faster than direct calls here)")
    res = {"workload": cfg["name"] + ("" if cache_mode is None and buckets is None
                                      else "_" + args.op),
           "T": w.T, "H": d.H, "kv_lora_rank": d.r, "rope_dim": d.dr, "heads": d.nh,
           "dn": d.dn, "dv": d.dv, "dtype": {"fp": w.dtype, "w8a8": "i8"}[w.kind],
           "kernel_family": ["decode", "prefill"][path], "timing": timing,
           "rotated_sets": n_sets, "steps": steps, "us_per_step": ms_per_step * 1e3,
           "tokens_per_s": value, "eager_us_per_step": eager_ms / steps * 1e3,
           "graph_us_per_step": graph_ms / steps * 1e3 if graph_ms is not None else None,
           "algorithmic_bytes_per_step": alg_bytes, "algorithmic_flops_per_step": alg_flops,
           "kernels": kernels, "roofline": roof}
    del sets, buckets
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, w


# time per call of the workloads that ride along with the headline, steps
# sized to ~20-50 ms of GPU time each
SIDE_STEPS = {0: 4000, 1: 3000, 2: 600, 3: 1000, 4: 100}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=None,
                    help="measure only workload N (default: the R1 W8A8 prefill as the "
                         "headline, the other four under 'configs')")
    ap.add_argument("--eager", action="store_true", help="time direct calls, not graph replays")
    ap.add_argument("--path", type=int, default=-1, help="force kernel family 0/1 (A/B runs)")
    ap.add_argument("--prefill-fusion", type=int, default=-1,
                    help="fp16/bf16 tiled path: finish and kv_b_proj in one launch (1), in two "
                         "(0), or the dispatcher's choice (-1; A/B runs)")
    ap.add_argument("--op", default="prolog",
                    choices=["prolog", "prolog_cached", "prolog_then_append", "cache_append",
                             "cache_append_int8", "rms_norm", "rope", "graph_buckets",
                             "graph_layers", "vendor_gemm"],
                    help="what one step is (default: the prolog)")
    ap.add_argument("--layers", type=int, default=27,
                    help="--op graph_layers: layers per step (default 27, V2-Lite's count)")
    ap.add_argument("--tokens", type=int, default=None,
                    help="with --config: that configuration's model and distributions at this "
                         "token count (a side measurement, not a headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the KV prolog needs no communication and "
              f"one MI355X runs a whole batch (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import mla_attention_kv_amd as mla
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mla.lib()
    if args.path in (0, 1):
        mla.mla_kv_prolog_force_path(args.path)
    if args.prefill_fusion in (0, 1):
        mla.mla_debug_set_prefill_fusion(args.prefill_fusion)

    headline = 4 if args.config is None else args.config
    cfg = workloads.CONFIGS[headline]
    if args.op == "vendor_gemm":
        vendor_gemm_reference(dev, args.steps)
        return
    if args.tokens is not None and (args.config is None or args.tokens < 1):
        print("--tokens needs --config and a positive count", file=sys.stderr)
        sys.exit(2)
    if args.op == "graph_layers":
        main_layers(args, 1 if args.config is None else args.config, dev)
        return
    if args.op in ("rms_norm", "rope"):
        w = workloads.make_config(headline)
        if w.kind != "fp":  # the W8A8 workload's activations are bf16
            w.dtype = "bf16"
        main_elem(args, cfg, w, dev)
        return
    if args.op.startswith("cache_append") and cfg["kind"] != "fp":
        print(f"--op {args.op} needs an fp16 / bf16 workload", file=sys.stderr)
        sys.exit(2)
    if args.op.startswith("cache_append"):
        w = workloads.make_config(headline)
        main_cache(args, cfg, w, dev)
        return
    cache_mode = {"prolog_cached": "fused", "prolog_then_append": "separate"}.get(args.op)
    res, w = measure_prolog(headline, args.steps, args.warmup, dev, args, cache_mode,
                            graph_buckets=args.op == "graph_buckets")
    side = {}
    if args.config is None and args.op == "prolog":
        for idx in (0, 1, 2, 3):
            r, _ = measure_prolog(idx, SIDE_STEPS[idx], max(20, SIDE_STEPS[idx] // 10), dev,
                                  args)
            side[r["workload"]] = {k: r[k] for k in (
                "T", "dtype", "kernel_family", "timing", "us_per_step", "tokens_per_s", "steps",
                "rotated_sets", "eager_us_per_step", "graph_us_per_step",
                "algorithmic_bytes_per_step", "algorithmic_flops_per_step", "kernels",
                "roofline")}

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        cpu = cpu_baseline(w, args.cpu_seconds)
        log(f"oracle: {cpu['value']:.4g} tokens/s on {cpu['cores']} threads")

    config = {k: res[k] for k in ("workload", "T", "H", "kv_lora_rank", "rope_dim", "heads",
                                  "dn", "dv", "kernel_family", "timing", "rotated_sets",
                                  "eager_us_per_step", "graph_us_per_step",
                                  "algorithmic_bytes_per_step",
                                  "algorithmic_flops_per_step", "kernels")}
    if side:
        config["configs"] = side
    out = {
        "metric": "MLA KV prolog tokens/s + % HBM (decode) / % MFMA (prefill) roofline",
        "value": res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["us_per_step"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": res["dtype"],
        "data": "synthetic (seeded; no public dataset exists for this path)",
        "config": config,
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
