"""Python binding of libmlaprolog, the MLA KV prolog for MI355X (gfx950).

Argument marshalling only: every step of the prolog runs in the library's
HIP kernels.  PyTorch provides device memory and the current stream; the
functions below check tensor dtypes / shapes / devices, allocate outputs and
workspace when they are not given, and call the C entry points of the same
names (declared in include/libmlaprolog.h).

If the shared library has not been built, importing works but every call
raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import sys
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmlaprolog.so")

MLA_OK = 0
MLA_ERR_INVALID_ARG = -1
MLA_ERR_UNSUPPORTED = -2
MLA_ERR_MISALIGNED = -3
MLA_ERR_WORKSPACE = -4
MLA_ERR_HIP = -5
MLA_F16 = 1
MLA_BF16 = 2
MLA_MAX_TOKENS = 1 << 22
MLA_NOALLOC_SCRATCH_BYTES = 64 << 20

# entry points declared in include/libmlaprolog.h
EXPORTS = (
    "mla_kv_prolog_workspace_size",
    "mla_kv_prolog",
    "mla_kv_prolog_w8a8_workspace_size",
    "mla_kv_prolog_w8a8",
    "mla_kv_cache_append",
    "mla_kv_cache_append_int8",
    "mla_kv_prolog_cached",
    "mla_kv_prolog_w8a8_cached",
    "mla_rms_norm",
    "mla_rope",
    "mla_kv_prolog_noalloc",
    "mla_debug_set_launch_events",
    "mla_debug_set_handoff_spin",
    "mla_debug_handoff_fallbacks",
    "mla_debug_set_prefill_fusion",
    "mla_prolog_graphs_create",
    "mla_prolog_graphs_create_layers",
    "mla_prolog_graphs_update_layers",
    "mla_prolog_graphs_layers",
    "mla_prolog_graphs_launch",
    "mla_prolog_graphs_bucket",
    "mla_prolog_graphs_update",
    "mla_prolog_graphs_destroy",
    "mla_kv_prolog_selected_path",
    "mla_kv_prolog_force_path",
    "mla_status_string",
)


class mla_dims_t(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("r", ctypes.c_int32), ("dr", ctypes.c_int32),
                ("nh", ctypes.c_int32), ("dn", ctypes.c_int32), ("dv", ctypes.c_int32)]


class mla_prolog_graph_desc_t(ctypes.Structure):
    _fields_ = [("w8a8", ctypes.c_int32), ("d", mla_dims_t), ("dt", ctypes.c_int),
                ("eps", ctypes.c_float), ("theta", ctypes.c_float),
                ("W_kv_a", ctypes.c_void_p), ("s_kv_a", ctypes.c_void_p),
                ("gamma", ctypes.c_void_p), ("W_kv_b", ctypes.c_void_p),
                ("s_kv_b", ctypes.c_void_p), ("hidden", ctypes.c_void_p),
                ("positions", ctypes.c_void_p), ("k_nope", ctypes.c_void_p),
                ("value", ctypes.c_void_p), ("k_pe", ctypes.c_void_p),
                ("compressed_kv", ctypes.c_void_p), ("slot_mapping", ctypes.c_void_p),
                ("kv_cache", ctypes.c_void_p), ("kv_cache_q", ctypes.c_void_p),
                ("kv_scale", ctypes.c_void_p), ("num_slots", ctypes.c_int64),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


@dataclass(frozen=True)
class Dims:
    H: int
    nh: int
    r: int = 512
    dr: int = 64
    dn: int = 128
    dv: int = 128

    def c(self) -> mla_dims_t:
        return mla_dims_t(self.H, self.r, self.dr, self.nh, self.dn, self.dv)


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {mla_status_string(status)} ({status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded shared library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -m mla_attention_kv_amd.build_lib "
            "or __graft_entry__.build()); there is no fallback implementation")
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, f32, vp, sz = (ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                             ctypes.c_size_t)
    L.mla_kv_prolog_workspace_size.argtypes = [i64, mla_dims_t, i32]
    L.mla_kv_prolog_workspace_size.restype = sz
    L.mla_kv_prolog_w8a8_workspace_size.argtypes = [i64, mla_dims_t]
    L.mla_kv_prolog_w8a8_workspace_size.restype = sz
    L.mla_kv_prolog.argtypes = [vp, vp, vp, vp, vp, i64, mla_dims_t, i32, f32, f32,
                                vp, vp, vp, vp, vp, sz, vp]
    L.mla_kv_prolog.restype = i32
    L.mla_kv_prolog_w8a8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, mla_dims_t, f32, f32,
                                     vp, vp, vp, vp, vp, vp, i64, i64, vp, sz, vp]
    L.mla_kv_prolog_w8a8.restype = i32
    L.mla_kv_cache_append.argtypes = [vp, vp, vp, i64, mla_dims_t, i32, vp, i64, vp]
    L.mla_kv_cache_append.restype = i32
    L.mla_kv_cache_append_int8.argtypes = [vp, vp, vp, i64, mla_dims_t, i32, vp, vp, i64, vp]
    L.mla_kv_cache_append_int8.restype = i32
    L.mla_kv_prolog_cached.argtypes = [vp, vp, vp, vp, vp, i64, mla_dims_t, i32, f32, f32,
                                       vp, vp, vp, vp, vp, vp, i64, vp, sz, vp]
    L.mla_kv_prolog_cached.restype = i32
    L.mla_kv_prolog_w8a8_cached.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, mla_dims_t, f32,
                                            f32, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, sz,
                                            vp]
    L.mla_kv_prolog_w8a8_cached.restype = i32
    L.mla_rms_norm.argtypes = [vp, vp, i64, i64, i32, f32, vp, vp]
    L.mla_rms_norm.restype = i32
    L.mla_rope.argtypes = [vp, vp, i64, i64, i64, i32, f32, vp, vp]
    L.mla_rope.restype = i32
    gp = ctypes.c_void_p
    L.mla_prolog_graphs_create.argtypes = [ctypes.POINTER(mla_prolog_graph_desc_t),
                                           ctypes.POINTER(ctypes.c_int64), ctypes.c_int32,
                                           ctypes.POINTER(gp)]
    L.mla_prolog_graphs_create.restype = i32
    L.mla_prolog_graphs_create_layers.argtypes = [ctypes.POINTER(mla_prolog_graph_desc_t), i32,
                                                  ctypes.POINTER(ctypes.c_int64), i32,
                                                  ctypes.POINTER(gp)]
    L.mla_prolog_graphs_create_layers.restype = i32
    L.mla_prolog_graphs_update_layers.argtypes = [gp, ctypes.POINTER(mla_prolog_graph_desc_t),
                                                  i32]
    L.mla_prolog_graphs_update_layers.restype = i32
    L.mla_prolog_graphs_layers.argtypes = [gp]
    L.mla_prolog_graphs_layers.restype = i32
    L.mla_prolog_graphs_launch.argtypes = [gp, i64, vp, ctypes.POINTER(ctypes.c_int64)]
    L.mla_prolog_graphs_launch.restype = i32
    L.mla_prolog_graphs_bucket.argtypes = [gp, i64]
    L.mla_prolog_graphs_bucket.restype = i64
    L.mla_prolog_graphs_update.argtypes = [gp, ctypes.POINTER(mla_prolog_graph_desc_t)]
    L.mla_prolog_graphs_update.restype = i32
    L.mla_prolog_graphs_destroy.argtypes = [gp]
    L.mla_prolog_graphs_destroy.restype = None
    L.mla_kv_prolog_selected_path.argtypes = [i64, mla_dims_t]
    L.mla_kv_prolog_selected_path.restype = i32
    L.mla_kv_prolog_force_path.argtypes = [i32]
    L.mla_kv_prolog_force_path.restype = i32
    L.mla_status_string.argtypes = [i32]
    L.mla_status_string.restype = ctypes.c_char_p
    L.mla_kv_prolog_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, mla_dims_t, i32, f32, f32,
                                        vp, vp, vp, vp, vp]
    L.mla_kv_prolog_noalloc.restype = i32
    L.mla_debug_set_launch_events.argtypes = [vp, i32]
    L.mla_debug_set_launch_events.restype = i32
    L.mla_debug_set_handoff_spin.argtypes = [i64]
    L.mla_debug_set_handoff_spin.restype = i64
    L.mla_debug_handoff_fallbacks.argtypes = [i32]
    L.mla_debug_handoff_fallbacks.restype = i64
    L.mla_debug_set_prefill_fusion.argtypes = [i32]
    L.mla_debug_set_prefill_fusion.restype = i32
    _lib = L
    return L


def mla_status_string(status: int) -> str:
    return lib().mla_status_string(int(status)).decode()


def mla_kv_prolog_workspace_size(T: int, dims: Dims, dtype: int = MLA_F16) -> int:
    return int(lib().mla_kv_prolog_workspace_size(int(T), dims.c(), int(dtype)))


def mla_kv_prolog_w8a8_workspace_size(T: int, dims: Dims) -> int:
    return int(lib().mla_kv_prolog_w8a8_workspace_size(int(T), dims.c()))


def mla_kv_prolog_selected_path(T: int, dims: Dims) -> int:
    return int(lib().mla_kv_prolog_selected_path(int(T), dims.c()))


def mla_kv_prolog_force_path(path: int) -> int:
    return int(lib().mla_kv_prolog_force_path(int(path)))


def mla_debug_set_handoff_spin(limit: int) -> int:
    """Test hook: bound on the decode hand-off's polls (0: every workgroup
    rebuilds its rows itself; negative: the default); returns the previous
    setting."""
    return int(lib().mla_debug_set_handoff_spin(int(limit)))


def mla_debug_handoff_fallbacks(reset: bool = False) -> int:
    """Test hook: the current device's count of decode hand-off fallbacks
    since the last reset (synchronises; clears it when reset)."""
    return int(lib().mla_debug_handoff_fallbacks(1 if reset else 0))


def mla_debug_set_prefill_fusion(mode: int) -> int:
    """Test hook: the fp16/bf16 prefill's finish and kv_b_proj as one launch
    with the latent staged in LDS (1), as two launches (0), or the
    dispatcher's choice (-1); returns the previous setting."""
    return int(lib().mla_debug_set_prefill_fusion(int(mode)))


# ---------------------------------------------------------------------------
# torch-tensor front ends
# ---------------------------------------------------------------------------

def _torch():
    import torch

    return torch


def _check(t, name, dtype, shape, device):
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _stream_ptr(device, stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _dims_from(hidden, W_kv_b, gamma, W_kv_a, dn=128, dv=128) -> Dims:
    H = hidden.shape[1]
    r = gamma.shape[0]
    dr = W_kv_a.shape[1] - r
    N2 = W_kv_b.shape[1]
    if N2 % (dn + dv):
        raise ValueError(f"W_kv_b has {N2} columns, not a multiple of dn+dv={dn + dv}")
    return Dims(H=H, nh=N2 // (dn + dv), r=r, dr=dr, dn=dn, dv=dv)


def _outputs(T, d, dtype, device, k_nope, value, k_pe, compressed_kv):
    torch = _torch()
    if k_nope is None:
        k_nope = torch.empty((T, d.nh, d.dn), dtype=dtype, device=device)
    if value is None:
        value = torch.empty((T, d.nh, d.dv), dtype=dtype, device=device)
    if k_pe is None:
        k_pe = torch.empty((T, d.dr), dtype=dtype, device=device)
    if compressed_kv is None:
        compressed_kv = torch.empty((T, d.r), dtype=dtype, device=device)
    _check(k_nope, "k_nope", dtype, (T, d.nh, d.dn), device)
    _check(value, "value", dtype, (T, d.nh, d.dv), device)
    _check(k_pe, "k_pe", dtype, (T, d.dr), device)
    _check(compressed_kv, "compressed_kv", dtype, (T, d.r), device)
    return k_nope, value, k_pe, compressed_kv


def _workspace(nbytes, device, workspace):
    torch = _torch()
    if workspace is None:
        # the library writes everything it reads from its workspace
        workspace = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace: contiguous uint8 tensor expected")
    if workspace.numel() < nbytes:
        raise ValueError(f"workspace: {workspace.numel()} bytes, need {nbytes}")
    return workspace


def mla_kv_prolog(hidden, W_kv_a, gamma, W_kv_b, positions, eps: float = 1e-6,
                  theta: float = 10000.0, *, k_nope=None, value=None, k_pe=None,
                  compressed_kv=None, workspace=None, stream=None, dn: int = 128,
                  dv: int = 128):
    """fp16 / bf16 KV prolog on torch tensors (all on one GPU).

    hidden [T,H], W_kv_a [H,r+dr], gamma [r], W_kv_b [r,nh*(dn+dv)] of one
    dtype (float16 or bfloat16); positions [T] int32.  Returns
    (k_nope [T,nh,dn], value [T,nh,dv], k_pe [T,dr], compressed_kv [T,r])."""
    return _prolog_fp(hidden, W_kv_a, gamma, W_kv_b, positions, eps, theta, k_nope, value,
                      k_pe, compressed_kv, workspace, stream, dn, dv, None, None)


def mla_kv_prolog_cached(hidden, W_kv_a, gamma, W_kv_b, positions, slot_mapping, kv_cache,
                         eps: float = 1e-6, theta: float = 10000.0, *, k_nope=None,
                         value=None, k_pe=None, compressed_kv=None, workspace=None,
                         stream=None, dn: int = 128, dv: int = 128):
    """mla_kv_prolog that also writes each token's [compressed_kv | k_pe] row
    into slot slot_mapping[t] ([T] int64) of kv_cache ([num_slots, r+dr] or
    [blocks, block_size, r+dr], the hidden dtype, contiguous); slots outside
    [0, num_slots) skip the token.  Returns the prolog's four outputs."""
    return _prolog_fp(hidden, W_kv_a, gamma, W_kv_b, positions, eps, theta, k_nope, value,
                      k_pe, compressed_kv, workspace, stream, dn, dv, slot_mapping, kv_cache)


def _prolog_fp(hidden, W_kv_a, gamma, W_kv_b, positions, eps, theta, k_nope, value, k_pe,
               compressed_kv, workspace, stream, dn, dv, slot_mapping, kv_cache):
    torch = _torch()
    dtype = hidden.dtype
    code = {torch.float16: MLA_F16, torch.bfloat16: MLA_BF16}.get(dtype)
    if code is None:
        raise ValueError(f"hidden: dtype {dtype}, expected float16 or bfloat16")
    dev = hidden.device
    if hidden.dim() != 2:
        raise ValueError("hidden must be [T, H]")
    T = hidden.shape[0]
    d = _dims_from(hidden, W_kv_b, gamma, W_kv_a, dn, dv)
    _check(hidden, "hidden", dtype, (T, d.H), dev)
    _check(W_kv_a, "W_kv_a", dtype, (d.H, d.r + d.dr), dev)
    _check(gamma, "gamma", dtype, (d.r,), dev)
    _check(W_kv_b, "W_kv_b", dtype, (d.r, d.nh * (d.dn + d.dv)), dev)
    _check(positions, "positions", torch.int32, (T,), dev)
    outs = _outputs(T, d, dtype, dev, k_nope, value, k_pe, compressed_kv)
    nbytes = mla_kv_prolog_workspace_size(T, d, code)
    if T > 0 and nbytes == 0:
        raise MlaError(MLA_ERR_UNSUPPORTED, "mla_kv_prolog_workspace_size")
    ws = _workspace(nbytes, dev, workspace)
    if kv_cache is None:
        st = lib().mla_kv_prolog(
            hidden.data_ptr(), W_kv_a.data_ptr(), gamma.data_ptr(), W_kv_b.data_ptr(),
            positions.data_ptr(), T, d.c(), code, float(eps), float(theta),
            outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(), outs[3].data_ptr(),
            ws.data_ptr(), ws.numel(), _stream_ptr(dev, stream))
        if st != MLA_OK:
            raise MlaError(st, "mla_kv_prolog")
        return outs
    W = d.r + d.dr
    _check(slot_mapping, "slot_mapping", torch.int64, (T,), dev)
    if kv_cache.dtype != dtype or kv_cache.device != dev or kv_cache.shape[-1] != W \
            or not kv_cache.is_contiguous():
        raise ValueError(f"kv_cache: contiguous {dtype} [..., {W}] on {dev} expected")
    st = lib().mla_kv_prolog_cached(
        hidden.data_ptr(), W_kv_a.data_ptr(), gamma.data_ptr(), W_kv_b.data_ptr(),
        positions.data_ptr(), T, d.c(), code, float(eps), float(theta),
        outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(), outs[3].data_ptr(),
        slot_mapping.data_ptr(), kv_cache.data_ptr(), kv_cache.numel() // W,
        ws.data_ptr(), ws.numel(), _stream_ptr(dev, stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_kv_prolog_cached")
    return outs


def mla_kv_prolog_w8a8(hidden, Wq_kv_a, s_kv_a, gamma, Wq_kv_b, s_kv_b, positions,
                       eps: float = 1e-6, theta: float = 10000.0, *, k_nope=None,
                       value=None, k_pe=None, compressed_kv=None, dbg_acc1=None,
                       dbg_acc2=None, dbg_row_begin: int = 0, dbg_rows: int = 0,
                       workspace=None, stream=None, dn: int = 128, dv: int = 128):
    """W8A8 KV prolog on torch tensors: hidden/gamma bfloat16, int8 weights
    with float32 per-output-column scales, bfloat16 outputs.  dbg_acc1
    [dbg_rows, r+dr] / dbg_acc2 [dbg_rows, nh*(dn+dv)] int32 (optional)
    receive the exact accumulators of rows [dbg_row_begin, +dbg_rows)."""
    return _prolog_w8(hidden, Wq_kv_a, s_kv_a, gamma, Wq_kv_b, s_kv_b, positions, eps, theta,
                      k_nope, value, k_pe, compressed_kv, dbg_acc1, dbg_acc2, dbg_row_begin,
                      dbg_rows, workspace, stream, dn, dv, None)


def mla_kv_prolog_w8a8_cached(hidden, Wq_kv_a, s_kv_a, gamma, Wq_kv_b, s_kv_b, positions,
                              slot_mapping, eps: float = 1e-6, theta: float = 10000.0, *,
                              kv_cache=None, kv_cache_q=None, kv_scale=None, k_nope=None,
                              value=None, k_pe=None, compressed_kv=None, workspace=None,
                              stream=None, dn: int = 128, dv: int = 128):
    """mla_kv_prolog_w8a8 that also writes each token's [compressed_kv |
    k_pe] row into slot slot_mapping[t] ([T] int64) of exactly one cache:
    kv_cache ([..., r+dr] bfloat16) or the int8 cache kv_cache_q ([...,
    r+dr] int8) with kv_scale ([num_slots] float32).  Returns the four
    outputs."""
    return _prolog_w8(hidden, Wq_kv_a, s_kv_a, gamma, Wq_kv_b, s_kv_b, positions, eps, theta,
                      k_nope, value, k_pe, compressed_kv, None, None, 0, 0, workspace, stream,
                      dn, dv, (slot_mapping, kv_cache, kv_cache_q, kv_scale))


def _prolog_w8(hidden, Wq_kv_a, s_kv_a, gamma, Wq_kv_b, s_kv_b, positions, eps, theta, k_nope,
               value, k_pe, compressed_kv, dbg_acc1, dbg_acc2, dbg_row_begin, dbg_rows,
               workspace, stream, dn, dv, cache):
    torch = _torch()
    dev = hidden.device
    if hidden.dim() != 2:
        raise ValueError("hidden must be [T, H]")
    T = hidden.shape[0]
    d = _dims_from(hidden, Wq_kv_b, gamma, Wq_kv_a, dn, dv)
    N1, N2 = d.r + d.dr, d.nh * (d.dn + d.dv)
    _check(hidden, "hidden", torch.bfloat16, (T, d.H), dev)
    _check(Wq_kv_a, "Wq_kv_a", torch.int8, (d.H, N1), dev)
    _check(s_kv_a, "s_kv_a", torch.float32, (N1,), dev)
    _check(gamma, "gamma", torch.bfloat16, (d.r,), dev)
    _check(Wq_kv_b, "Wq_kv_b", torch.int8, (d.r, N2), dev)
    _check(s_kv_b, "s_kv_b", torch.float32, (N2,), dev)
    _check(positions, "positions", torch.int32, (T,), dev)
    if dbg_acc1 is not None:
        _check(dbg_acc1, "dbg_acc1", torch.int32, (dbg_rows, N1), dev)
    if dbg_acc2 is not None:
        _check(dbg_acc2, "dbg_acc2", torch.int32, (dbg_rows, N2), dev)
    outs = _outputs(T, d, torch.bfloat16, dev, k_nope, value, k_pe, compressed_kv)
    nbytes = mla_kv_prolog_w8a8_workspace_size(T, d)
    if T > 0 and nbytes == 0:
        raise MlaError(MLA_ERR_UNSUPPORTED, "mla_kv_prolog_w8a8_workspace_size")
    ws = _workspace(nbytes, dev, workspace)
    if cache is not None:
        slot_mapping, kv_cache, kv_cache_q, kv_scale = cache
        W = d.r + d.dr
        _check(slot_mapping, "slot_mapping", torch.int64, (T,), dev)
        if (kv_cache is None) == (kv_cache_q is None):
            raise ValueError("give exactly one of kv_cache (bfloat16) and kv_cache_q (int8)")
        if kv_cache is not None:
            if kv_cache.dtype != torch.bfloat16 or kv_cache.device != dev \
                    or kv_cache.shape[-1] != W or not kv_cache.is_contiguous():
                raise ValueError(f"kv_cache: contiguous bfloat16 [..., {W}] on {dev} expected")
            ptrs = (kv_cache.data_ptr(), None, None)
            nslots = kv_cache.numel() // W
        else:
            if kv_cache_q.dtype != torch.int8 or kv_cache_q.device != dev \
                    or kv_cache_q.shape[-1] != W or not kv_cache_q.is_contiguous():
                raise ValueError(f"kv_cache_q: contiguous int8 [..., {W}] on {dev} expected")
            nslots = kv_cache_q.numel() // W
            if kv_scale is None:
                raise ValueError("kv_scale is needed with kv_cache_q")
            _check(kv_scale, "kv_scale", torch.float32, (nslots,), dev)
            ptrs = (None, kv_cache_q.data_ptr(), kv_scale.data_ptr())
        st = lib().mla_kv_prolog_w8a8_cached(
            hidden.data_ptr(), Wq_kv_a.data_ptr(), s_kv_a.data_ptr(), gamma.data_ptr(),
            Wq_kv_b.data_ptr(), s_kv_b.data_ptr(), positions.data_ptr(), T, d.c(), float(eps),
            float(theta), outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(),
            outs[3].data_ptr(), slot_mapping.data_ptr(), ptrs[0], ptrs[1], ptrs[2], nslots,
            ws.data_ptr(), ws.numel(), _stream_ptr(dev, stream))
        if st != MLA_OK:
            raise MlaError(st, "mla_kv_prolog_w8a8_cached")
        return outs
    st = lib().mla_kv_prolog_w8a8(
        hidden.data_ptr(), Wq_kv_a.data_ptr(), s_kv_a.data_ptr(), gamma.data_ptr(),
        Wq_kv_b.data_ptr(), s_kv_b.data_ptr(), positions.data_ptr(), T, d.c(), float(eps),
        float(theta), outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(),
        outs[3].data_ptr(), dbg_acc1.data_ptr() if dbg_acc1 is not None else None,
        dbg_acc2.data_ptr() if dbg_acc2 is not None else None, int(dbg_row_begin),
        int(dbg_rows), ws.data_ptr(), ws.numel(), _stream_ptr(dev, stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_kv_prolog_w8a8")
    return outs


def _cache_inputs(compressed_kv, k_pe, slot_mapping, r=512, dr=64):
    torch = _torch()
    code = {torch.float16: MLA_F16, torch.bfloat16: MLA_BF16}.get(compressed_kv.dtype)
    if code is None:
        raise ValueError(f"compressed_kv: dtype {compressed_kv.dtype}, expected float16/bfloat16")
    T = compressed_kv.shape[0]
    dev = compressed_kv.device
    _check(compressed_kv, "compressed_kv", compressed_kv.dtype, (T, r), dev)
    _check(k_pe, "k_pe", compressed_kv.dtype, (T, dr), dev)
    _check(slot_mapping, "slot_mapping", torch.int64, (T,), dev)
    return code, T, dev


def mla_kv_cache_append(compressed_kv, k_pe, slot_mapping, kv_cache, *, stream=None):
    """Write each token's [compressed_kv row | k_pe row] into slot
    slot_mapping[t] of kv_cache ([num_slots, 576] or [blocks, block_size,
    576], same dtype, contiguous); slots outside [0, num_slots) skip the
    token.  Returns kv_cache."""
    code, T, dev = _cache_inputs(compressed_kv, k_pe, slot_mapping)
    W = compressed_kv.shape[1] + k_pe.shape[1]
    if kv_cache.dtype != compressed_kv.dtype or kv_cache.device != dev or kv_cache.shape[-1] != W \
            or not kv_cache.is_contiguous():
        raise ValueError(f"kv_cache: contiguous {compressed_kv.dtype} [..., {W}] on {dev} expected")
    rc = lib().mla_kv_cache_append(compressed_kv.data_ptr(), k_pe.data_ptr(), slot_mapping.data_ptr(),
                                   T, Dims(H=64, nh=1).c(), code, kv_cache.data_ptr(),
                                   kv_cache.numel() // W, _stream_ptr(dev, stream))
    if rc != MLA_OK:
        raise MlaError(rc, "mla_kv_cache_append")
    return kv_cache


def mla_kv_cache_append_int8(compressed_kv, k_pe, slot_mapping, kv_cache_q, kv_scale, *,
                             stream=None):
    """The same into an int8 cache (kv_cache_q [..., 576] int8) with one fp32
    scale per slot (kv_scale [num_slots]).  Returns (kv_cache_q, kv_scale)."""
    torch = _torch()
    code, T, dev = _cache_inputs(compressed_kv, k_pe, slot_mapping)
    W = compressed_kv.shape[1] + k_pe.shape[1]
    if kv_cache_q.dtype != torch.int8 or kv_cache_q.device != dev or kv_cache_q.shape[-1] != W \
            or not kv_cache_q.is_contiguous():
        raise ValueError(f"kv_cache_q: contiguous int8 [..., {W}] on {dev} expected")
    S = kv_cache_q.numel() // W
    _check(kv_scale, "kv_scale", torch.float32, (S,), dev)
    rc = lib().mla_kv_cache_append_int8(compressed_kv.data_ptr(), k_pe.data_ptr(),
                                        slot_mapping.data_ptr(), T, Dims(H=64, nh=1).c(), code,
                                        kv_cache_q.data_ptr(), kv_scale.data_ptr(), S,
                                        _stream_ptr(dev, stream))
    if rc != MLA_OK:
        raise MlaError(rc, "mla_kv_cache_append_int8")
    return kv_cache_q, kv_scale


def _dt_code(t, name):
    torch = _torch()
    code = {torch.float16: MLA_F16, torch.bfloat16: MLA_BF16}.get(t.dtype)
    if code is None:
        raise ValueError(f"{name}: dtype {t.dtype}, expected float16 or bfloat16")
    return code


def mla_rms_norm(x, gamma, eps: float = 1e-6, *, out=None, stream=None):
    """RMSNorm over the last dimension of x ([..., n], float16 / bfloat16,
    contiguous) with weight gamma [n]; out may be x (in place).  Returns out."""
    code = _dt_code(x, "x")
    n = x.shape[-1]
    rows = x.numel() // n if n else 0
    dev = x.device
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    _check(gamma, "gamma", x.dtype, (n,), dev)
    if out is None:
        out = _torch().empty_like(x)
    _check(out, "out", x.dtype, tuple(x.shape), dev)
    st = lib().mla_rms_norm(x.data_ptr(), gamma.data_ptr(), rows, n, code, float(eps),
                            out.data_ptr(), _stream_ptr(dev, stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_rms_norm")
    return out


def mla_rope(x, positions, theta: float = 10000.0, *, out=None, stream=None):
    """Rotate-half RoPE of x ([T, heads, dr] or [T, dr], float16 / bfloat16,
    contiguous), every head of token t rotated by positions[t] ([T] int32);
    out may be x (in place).  Returns out."""
    torch = _torch()
    code = _dt_code(x, "x")
    if x.dim() not in (2, 3):
        raise ValueError("x must be [T, dr] or [T, heads, dr]")
    T, dr = x.shape[0], x.shape[-1]
    heads = x.shape[1] if x.dim() == 3 else 1
    dev = x.device
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    _check(positions, "positions", torch.int32, (T,), dev)
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", x.dtype, tuple(x.shape), dev)
    st = lib().mla_rope(x.data_ptr(), positions.data_ptr(), T, heads, dr, code, float(theta),
                        out.data_ptr(), _stream_ptr(dev, stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_rope")
    return out


# ---------------------------------------------------------------------------
# captured decode buckets
# ---------------------------------------------------------------------------

class PrologGraphs:
    """A set of captured prolog graphs, one per token-count bucket, over
    static buffers this object allocates (zero-filled; slot_mapping -1).

    weights: fp16/bf16 (W_kv_a, gamma, W_kv_b) or, with w8a8=True,
    (Wq_kv_a, s_kv_a, gamma, Wq_kv_b, s_kv_b).  cache: None, an fp cache
    tensor ([..., r+dr], the model dtype), or for W8A8 a bfloat16 cache or a
    (kv_cache_q int8, kv_scale float32) pair.  A step: write the first T rows
    of .hidden / .positions (/ .slot_mapping), call run(T), read the first T
    rows of .k_nope / .value / .k_pe / .compressed_kv.  Steps and the static
    buffers belong to one device; keep them on one stream.

    Several layers: weights is a list of per-layer weight tuples (and cache,
    if given, a list of per-layer caches).  Each graph then replays every
    layer's prolog in order with one launch; the layers read the same static
    .hidden / .positions / .slot_mapping rows and write their own outputs,
    .k_nope[l] / .value[l] / .k_pe[l] / .compressed_kv[l]."""

    def __init__(self, weights, buckets, eps: float = 1e-6, theta: float = 10000.0, *,
                 w8a8: bool = False, cache=None, dn: int = 128, dv: int = 128,
                 device=None):
        torch = _torch()
        self.buckets = tuple(int(b) for b in buckets)
        if not self.buckets or list(self.buckets) != sorted(set(self.buckets)):
            raise ValueError("buckets: ascending distinct token counts expected")
        self.w8a8 = bool(w8a8)
        self.multi = isinstance(weights, list)
        self.n_layers = len(weights) if self.multi else 1
        if self.n_layers < 1:
            raise ValueError("weights: at least one layer expected")
        first = weights[0] if self.multi else weights
        self.device = first[0].device if device is None else torch.device(device)
        self._handle = ctypes.c_void_p(None)
        self._bind(weights, eps, theta, cache, dn, dv, create=True)

    def _layer_dims(self, weights, dn, dv):
        """Dims, dtype, dtype code and the five weight pointers' tensors of
        one layer, after checking its weights."""
        torch = _torch()
        dev = self.device
        if self.w8a8:
            Wqa, swa, gamma, Wqb, swb = weights
            dtype, code = torch.bfloat16, MLA_BF16
            H = Wqa.shape[0]
            d = Dims(H=H, nh=Wqb.shape[1] // (dn + dv), r=gamma.shape[0],
                     dr=Wqa.shape[1] - gamma.shape[0], dn=dn, dv=dv)
            N1, N2 = d.r + d.dr, d.nh * (d.dn + d.dv)
            _check(Wqa, "Wq_kv_a", torch.int8, (H, N1), dev)
            _check(swa, "s_kv_a", torch.float32, (N1,), dev)
            _check(gamma, "gamma", torch.bfloat16, (d.r,), dev)
            _check(Wqb, "Wq_kv_b", torch.int8, (d.r, N2), dev)
            _check(swb, "s_kv_b", torch.float32, (N2,), dev)
            return d, dtype, code, (Wqa, swa, gamma, Wqb, swb)
        Wa, gamma, Wb = weights
        dtype = Wa.dtype
        code = {torch.float16: MLA_F16, torch.bfloat16: MLA_BF16}.get(dtype)
        if code is None:
            raise ValueError(f"W_kv_a: dtype {dtype}, expected float16 or bfloat16")
        H = Wa.shape[0]
        d = Dims(H=H, nh=Wb.shape[1] // (dn + dv), r=gamma.shape[0],
                 dr=Wa.shape[1] - gamma.shape[0], dn=dn, dv=dv)
        _check(Wa, "W_kv_a", dtype, (H, d.r + d.dr), dev)
        _check(gamma, "gamma", dtype, (d.r,), dev)
        _check(Wb, "W_kv_b", dtype, (d.r, d.nh * (d.dn + d.dv)), dev)
        return d, dtype, code, (Wa, None, gamma, Wb, None)

    def _cache_ptrs(self, cache, dtype, W):
        torch = _torch()
        dev = self.device
        kv_cache = kv_cache_q = kv_scale = None
        nslots = 0
        if cache is not None:
            if isinstance(cache, tuple):
                if not self.w8a8:
                    raise ValueError("an int8 cache needs w8a8=True")
                kv_cache_q, kv_scale = cache
                if kv_cache_q.dtype != torch.int8 or kv_cache_q.shape[-1] != W \
                        or not kv_cache_q.is_contiguous() or kv_cache_q.device != dev:
                    raise ValueError(f"kv_cache_q: contiguous int8 [..., {W}] on {dev} expected")
                nslots = kv_cache_q.numel() // W
                _check(kv_scale, "kv_scale", torch.float32, (nslots,), dev)
            else:
                kv_cache = cache
                if kv_cache.dtype != dtype or kv_cache.shape[-1] != W \
                        or not kv_cache.is_contiguous() or kv_cache.device != dev:
                    raise ValueError(f"kv_cache: contiguous {dtype} [..., {W}] on {dev} expected")
                nslots = kv_cache.numel() // W
        return kv_cache, kv_cache_q, kv_scale, nslots

    def _bind(self, weights, eps, theta, cache, dn, dv, create):
        torch = _torch()
        dev = self.device
        L = self.n_layers
        wl = weights if self.multi else [weights]
        if len(wl) != L:
            raise ValueError(f"weights: {L} layers expected")
        if cache is None:
            cl = [None] * L
        elif self.multi:
            if not isinstance(cache, list) or len(cache) != L:
                raise ValueError(f"cache: a list of {L} per-layer caches expected")
            cl = cache
        else:
            cl = [tuple(cache) if isinstance(cache, list) else cache]
        kinds = [self._layer_dims(w, dn, dv) for w in wl]
        d, dtype, code, _ = kinds[0]
        for dl, tl, _c, _p in kinds[1:]:
            if dl != d or tl != dtype:
                raise ValueError("every layer must have the same dims and dtype")
        if not create and (d != self.dims or dtype != self.dtype):
            raise ValueError("update: dims and dtype must stay those of the set")
        Tm = self.buckets[-1]
        if create:
            self.dims, self.dtype = d, dtype
            lead = (L,) if self.multi else ()
            self.hidden = torch.zeros((Tm, d.H), dtype=dtype, device=dev)
            self.positions = torch.zeros(Tm, dtype=torch.int32, device=dev)
            self.slot_mapping = torch.full((Tm,), -1, dtype=torch.int64, device=dev)
            self.k_nope = torch.empty(lead + (Tm, d.nh, d.dn), dtype=dtype, device=dev)
            self.value = torch.empty(lead + (Tm, d.nh, d.dv), dtype=dtype, device=dev)
            self.k_pe = torch.empty(lead + (Tm, d.dr), dtype=dtype, device=dev)
            self.compressed_kv = torch.empty(lead + (Tm, d.r), dtype=dtype, device=dev)
            if self.w8a8:
                nb = max(mla_kv_prolog_w8a8_workspace_size(b, d) for b in self.buckets)
            else:
                nb = max(mla_kv_prolog_workspace_size(b, d, code) for b in self.buckets)
            if nb == 0:
                raise MlaError(MLA_ERR_UNSUPPORTED, "workspace size")
            # one workspace for every layer: a graph's replays are ordered
            self.workspace = torch.empty(nb, dtype=torch.uint8, device=dev)
        W = d.r + d.dr

        def p(t):
            return t.data_ptr() if t is not None else None

        descs = (mla_prolog_graph_desc_t * L)()
        for l, ((_d, _t, _c, ptrs), c) in enumerate(zip(kinds, cl)):
            kv_cache, kv_cache_q, kv_scale, nslots = self._cache_ptrs(c, dtype, W)
            outs = ((self.k_nope[l], self.value[l], self.k_pe[l], self.compressed_kv[l])
                    if self.multi else (self.k_nope, self.value, self.k_pe, self.compressed_kv))
            descs[l] = mla_prolog_graph_desc_t(
                1 if self.w8a8 else 0, d.c(), code, float(eps), float(theta),
                p(ptrs[0]), p(ptrs[1]), p(ptrs[2]), p(ptrs[3]), p(ptrs[4]),
                self.hidden.data_ptr(), self.positions.data_ptr(), outs[0].data_ptr(),
                outs[1].data_ptr(), outs[2].data_ptr(), outs[3].data_ptr(),
                self.slot_mapping.data_ptr() if nslots else None, p(kv_cache), p(kv_cache_q),
                p(kv_scale), nslots, self.workspace.data_ptr(), self.workspace.numel())
        arr = (ctypes.c_int64 * len(self.buckets))(*self.buckets)
        with torch.cuda.device(dev):
            if create:
                st = lib().mla_prolog_graphs_create_layers(descs, L, arr, len(self.buckets),
                                                           ctypes.byref(self._handle))
            else:
                st = lib().mla_prolog_graphs_update_layers(self._handle, descs, L)
        if st != MLA_OK:
            raise MlaError(st, "mla_prolog_graphs_create_layers" if create
                           else "mla_prolog_graphs_update_layers")
        # keep the bound tensors alive as long as the graphs refer to them
        self._bound = (weights, cache)

    def update(self, weights, eps: float = 1e-6, theta: float = 10000.0, *, cache=None,
               dn: int = 128, dv: int = 128):
        """Rebind the graphs to other weights (say the next layer's, or for a
        multi-layer set another list of layers) and caches; the static
        buffers stay."""
        self._bind(weights, eps, theta, cache, dn, dv, create=False)

    @property
    def handle(self) -> ctypes.c_void_p:
        """The C handle (mla_prolog_graphs *), for direct library calls."""
        return self._handle

    def bucket(self, T: int) -> int:
        return int(lib().mla_prolog_graphs_bucket(self._handle, int(T)))

    def run(self, T: int, *, stream=None) -> int:
        """One step over the first T rows; returns the bucket it ran."""
        used = ctypes.c_int64(0)
        st = lib().mla_prolog_graphs_launch(self._handle, int(T), _stream_ptr(self.device, stream),
                                            ctypes.byref(used))
        if st != MLA_OK:
            raise MlaError(st, "mla_prolog_graphs_launch")
        return int(used.value)

    def close(self):
        if self._handle:
            lib().mla_prolog_graphs_destroy(self._handle)
            self._handle = ctypes.c_void_p(None)

    def __del__(self):
        # at interpreter exit the runtime may already be torn down: leave the
        # graphs to the process end then
        if sys.is_finalizing():
            return
        try:
            self.close()
        except Exception:
            pass
