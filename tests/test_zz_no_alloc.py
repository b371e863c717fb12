"""The fp16 / bf16 prolog entry point that allocates nothing
(mla_kv_prolog_noalloc: its workspace is a device array inside the
library) against the workspace entry point mla_kv_prolog, through the C
ABI: two calls in a row on the same array, the second with a smaller input,
each bit for bit equal to mla_kv_prolog's output on the same inputs and
within the oracle's tolerance.  (Its argument checks, including the
rejection of token counts whose workspace exceeds the array, are host logic
and are tested on the CPU.)"""
import ctypes

import numpy as np
import pytest

import workloads
from workloads import V2LITE, R1

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from parity import compare, gpu_rows, run_oracle, upload  # noqa: E402


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_attention_kv_amd as mla

    mla.lib()
    return torch.device("cuda:0")


def outputs(w, dev):
    odt = torch.float16 if w.dtype == "f16" else torch.bfloat16
    d = w.dims
    return (torch.full((w.T, d.nh, d.dn), 7.0, dtype=odt, device=dev),
            torch.full((w.T, d.nh, d.dv), 7.0, dtype=odt, device=dev),
            torch.full((w.T, d.dr), 7.0, dtype=odt, device=dev),
            torch.full((w.T, d.r), 7.0, dtype=odt, device=dev))


def call_noalloc(w, t, outs):
    import mla_attention_kv_amd as mla

    d = mla.Dims(H=w.dims.H, nh=w.dims.nh)
    code = mla.MLA_F16 if w.dtype == "f16" else mla.MLA_BF16
    sp = torch.cuda.current_stream().cuda_stream
    return mla.lib().mla_kv_prolog_noalloc(
        t["X"].data_ptr(), t["Wa"].data_ptr(), t["gamma"].data_ptr(), t["Wb"].data_ptr(),
        t["pos"].data_ptr(), w.T, d.c(), code, w.eps, w.theta, outs[0].data_ptr(),
        outs[1].data_ptr(), outs[2].data_ptr(), outs[3].data_ptr(), ctypes.c_void_p(sp))


def call_workspace(w, t, outs):
    import mla_attention_kv_amd as mla

    d = mla.Dims(H=w.dims.H, nh=w.dims.nh)
    code = mla.MLA_F16 if w.dtype == "f16" else mla.MLA_BF16
    ws = torch.full((mla.mla_kv_prolog_workspace_size(w.T, d, code),), 0x5A, dtype=torch.uint8,
                    device=t["X"].device)
    sp = torch.cuda.current_stream().cuda_stream
    st = mla.lib().mla_kv_prolog(
        t["X"].data_ptr(), t["Wa"].data_ptr(), t["gamma"].data_ptr(), t["Wb"].data_ptr(),
        t["pos"].data_ptr(), w.T, d.c(), code, w.eps, w.theta, outs[0].data_ptr(),
        outs[1].data_ptr(), outs[2].data_ptr(), outs[3].data_ptr(), ws.data_ptr(), ws.numel(),
        ctypes.c_void_p(sp))
    torch.cuda.synchronize()
    return st


@pytest.mark.parametrize("dims,dtype,T1,T2", [
    (V2LITE, "f16", 64, 17),      # decode family, then a smaller decode batch
    (V2LITE, "f16", 4096, 300),   # prefill family, then a smaller prefill
    (R1, "bf16", 256, 40),        # R1 decode share, then a decode batch
])
def test_noalloc_two_calls_match_workspace_entry_point(dev, dims, dtype, T1, T2):
    import mla_attention_kv_amd as mla

    for i, T in enumerate((T1, T2)):
        print(f"[noalloc] {dtype} H={dims.H} T={T} call {i}", flush=True)
        w = workloads.make_custom(dims, T, dtype=dtype, seed=700 + T,
                                  wstd=0.02 if dims is V2LITE else 0.01, max_pos=32768)
        t = upload(w, dev)
        outs = outputs(w, dev)
        st = call_noalloc(w, t, outs)
        assert st == mla.MLA_OK, mla.mla_status_string(st)
        torch.cuda.synchronize()
        ref = outputs(w, dev)
        assert call_workspace(w, t, ref) == mla.MLA_OK
        for a, b in zip(outs, ref):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        compare(gpu_rows(outs), run_oracle(w), f"noalloc T={T}")
