"""The benchmark's host-side bookkeeping, on the CPU: which roof binds each
workload, the per-kernel algorithmic bytes and operations that the live
roofline divides by the kernel durations, the committed traffic files and
their source check, and the one-GPU guard of the command line."""
import glob
import json
import os
import subprocess
import sys
import types

import pytest

import bench
import workloads
from workloads import R1, V2LITE

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# the five benchmark workloads: (dims, T, kind, dtype)
WORKLOADS = [(V2LITE, 1, "fp", "f16"), (V2LITE, 64, "fp", "f16"), (V2LITE, 4096, "fp", "f16"),
             (R1, 256, "fp", "bf16"), (R1, 12874, "w8a8", "bf16")]


def _w(dims, T, kind, dtype):
    return types.SimpleNamespace(dims=dims, T=T, kind=kind, dtype=dtype)


def test_workload_table_matches_configs():
    import numpy as np

    for i, (dims, T, kind, dtype) in enumerate(WORKLOADS):
        c = workloads.CONFIGS[i]
        pos, _ = workloads._positions_for(i, np.random.default_rng(1000 + i))
        assert (len(pos), c["dims"], c["kind"], c["dtype"]) == (T, dims, kind, dtype), c


@pytest.mark.parametrize("i,bound", [(0, "hbm"), (1, "hbm"), (2, "mfma"), (3, "hbm"), (4, "hbm")])
def test_roofline_picks_the_binding_roof(i, bound):
    # the bound follows the arithmetic intensity against the ridge point of
    # the workload's MFMA dtype: the W8A8 prefill (~500 int8 operations per
    # byte) sits below the int8 ridge (625) and is HBM-bound, the V2-Lite
    # fp16 prefill (~436 per byte) above the fp16 ridge (312.5)
    dims, T, kind, dtype = WORKLOADS[i]
    w = _w(dims, T, kind, dtype)
    b = workloads.algorithmic_bytes(dims, T, kind, dtype)
    f = workloads.algorithmic_flops(dims, T)
    step = 1e-4
    r = bench.roofline(w, step, b, f)
    assert r["bound"] == bound
    peak = bench.MFMA_PEAK_TFLOPS["i8" if kind == "w8a8" else dtype]
    assert r["ridge"] == pytest.approx(peak * 1e12 / (bench.HBM_PEAK_GBS * 1e9))
    assert r["hbm_frac"] == pytest.approx(b / step / 1e9 / bench.HBM_PEAK_GBS)
    assert r["mfma_frac"] == pytest.approx(f / step / 1e12 / peak)
    assert r["frac"] == pytest.approx(r["hbm_frac"] if bound == "hbm" else r["mfma_frac"])


# (workload index, kernel family, kernels per call) for every split the
# library launches: fp decode (2 kernels, 3 for a separate finish), the
# prefill family (3; 2 with the finish and kv_b_proj in one launch), W8A8
# prefill (4) and W8A8 decode (3: finish fused into kv_b_proj; 2: the
# quantiser folded into kv_a_proj as well)
SPLITS = [(0, 0, 2), (1, 0, 2), (1, 0, 3), (2, 1, 3), (2, 1, 2), (3, 1, 3), (4, 1, 4), (4, 0, 3),
          (4, 0, 2)]


@pytest.mark.parametrize("i,path,nk", SPLITS)
def test_kernel_parts_cover_the_call(i, path, nk):
    # each kernel's operations add up to the call's (every multiply-add is in
    # exactly one kernel), and its bytes at least to the call's (a kernel
    # reads back what an earlier one wrote, never less than the call moves)
    dims, T, kind, dtype = WORKLOADS[i]
    if nk == 2 and kind == "w8a8":
        T = 8
    w = _w(dims, T, kind, dtype)
    parts = bench.kernel_parts(w, path, nk)
    assert len(parts) == nk
    assert all(isinstance(n, str) and n for n, _ in parts)
    total_b = sum(b for _, (b, _) in parts)
    total_f = sum(f for _, (_, f) in parts)
    assert total_f == workloads.algorithmic_flops(dims, T)
    assert total_b >= workloads.algorithmic_bytes(dims, T, kind, dtype)
    # the extra bytes are the intermediates' round trips only: at most the
    # kv_a_proj result in fp32 twice, the latent twice and the quantised
    # activations twice, plus the row scales
    slack = T * (2 * dims.N1 * 4 + 2 * dims.r * 2 + 2 * dims.H + 64)
    assert total_b - workloads.algorithmic_bytes(dims, T, kind, dtype) <= slack


def test_traffic_files_are_consistent():
    files = sorted(f for f in os.listdir(os.path.join(ROOT, "profiles")) if f.startswith("traffic_"))
    assert len(files) == 5
    for f in files:
        with open(os.path.join(ROOT, "profiles", f)) as fh:
            t = json.load(fh)
        assert f == f"traffic_{t['workload']}.json"
        k = t["kernel_hbm_bytes"]
        assert len(k) == len(t["kernel_names"]) == len(t["kernel_avg_us"]) >= 2
        assert sum(k) == pytest.approx(t["hbm_bytes_per_launch"], rel=1e-9)
        assert t["read_bytes"] + t["write_bytes"] == pytest.approx(t["hbm_bytes_per_launch"])
        assert all(os.path.exists(os.path.join(ROOT, s)) for s in t["sources"])
        assert os.path.exists(os.path.join(ROOT, "profiles", t["profile"]))


def test_traffic_is_dropped_when_sources_change(monkeypatch):
    name = "r1_w8a8_ragged_prefill_8seq"
    with open(os.path.join(ROOT, "profiles", f"traffic_{name}.json")) as fh:
        t = json.load(fh)
    monkeypatch.setattr(bench, "kernel_source_hash", lambda files=None: t["src_hash"])
    got = bench.load_traffic(name)
    assert got is not None and got["kernels"] == t["kernel_hbm_bytes"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda files=None: "0" * 16)
    assert bench.load_traffic(name) is None
    assert bench.load_traffic("no_such_workload") is None


def test_source_hash_covers_every_kernel_source():
    srcs = sorted(os.path.relpath(p, ROOT)
                  for p in glob.glob(os.path.join(ROOT, "mla_attention_kv_amd", "csrc", "*")))
    assert bench.kernel_source_hash() == bench.kernel_source_hash(srcs)


@pytest.mark.parametrize("argv", [["--gpus", "2"], ["--gpus", "8", "--steps", "3"]])
def test_more_than_one_gpu_is_refused(argv):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                       capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, WORLD_SIZE="1"))
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
