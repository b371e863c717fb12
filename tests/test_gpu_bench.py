"""bench.py on the GPU: one short run of the smallest workload, in a child
process as the driver runs it, and the JSON line it prints checked field by
field against the benchmark contract (metric, value, timing, roofline with
its live dominant-kernel measurement, the CPU oracle baseline)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench_line():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--config", "0", "--steps", "50",
           "--warmup", "5", "--cpu-seconds", "1"]
    print("[bench test] " + " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT,
                       env=dict(os.environ, WORLD_SIZE="1"))
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


def test_contract_fields(bench_line):
    d = bench_line
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 50 and d["warmup"] == 5
    assert d["unit"] == "tokens/s" and d["higher_is_better"] is True
    assert d["dtype"] == "f16" and d["vs_baseline"] is None
    c = d["config"]
    assert c["workload"] == "v2lite_fp16_decode_T1" and c["T"] == 1
    # value is tokens per second of the reported timing
    assert d["value"] == pytest.approx(c["T"] / (d["ms_per_step"] / 1e3), rel=1e-6)
    assert c["timing"].startswith(("HIP graph replays", "direct calls"))
    assert c["eager_us_per_step"] > 0 and c["graph_us_per_step"] > 0
    assert d["ms_per_step"] * 1e3 == pytest.approx(
        min(c["eager_us_per_step"], c["graph_us_per_step"]), rel=0.05)


def test_roofline_is_live_and_consistent(bench_line):
    r = bench_line["roofline"]
    assert r["bound"] in ("hbm", "mfma") and r["unit"] in ("GB/s", "TFLOP/s")
    assert 0 < r["frac"] < 1 and r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-9)
    ks = bench_line["config"]["kernels"]
    assert len(ks) == 2 and all(k["avg_us"] > 0 for k in ks)
    dom = max(ks, key=lambda k: k["avg_us"])
    assert dom["kernel"] in r["kernel"]
    # achieved = the dominant kernel's algorithmic bytes / its live duration
    assert r["achieved"] == pytest.approx(dom["algorithmic_bytes"] / (dom["avg_us"] * 1e-6) / 1e9,
                                          rel=1e-6)
    # the call's own roofline rides along, and its traffic is either the
    # committed counters of these sources or null
    call = r["call"]
    assert call["bound"] == "hbm" and 0 < call["frac"] < 1
    assert call["traffic"] is None or call["traffic"] > 0


def test_cpu_baseline_is_the_oracle(bench_line):
    cb = bench_line["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s"
    assert cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
