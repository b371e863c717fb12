"""Seeded synthetic inputs for the MLA KV prolog.

This module only draws random numbers and stores them in the formats the
prolog consumes (fp16 / bf16 / int8 with per-column scales).  It holds none
of the prolog's arithmetic; both the CPU oracle and the HIP library are fed
from it.

The shapes are those of the DeepSeek-V2-Lite case printed in the migration
guide's "Precision verification" section (hidden 2048, kv_lora_rank 512,
rope dim 64, 16 heads of 128 + 128) and of a DeepSeek-R1-sized attention
block (hidden 7168, 128 heads), as used by the R1 inference recipe page.
There is no public dataset for this path: every tensor is synthetic.

Draw order for every workload (numpy ``default_rng(seed)``): sequence
lengths / positions, hidden, W_kv_a, gamma, W_kv_b.  Values are drawn in
float32 and rounded to the storage dtype with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Dims:
    H: int
    nh: int
    r: int = 512
    dr: int = 64
    dn: int = 128
    dv: int = 128

    @property
    def N1(self) -> int:
        return self.r + self.dr

    @property
    def N2(self) -> int:
        return self.nh * (self.dn + self.dv)


V2LITE = Dims(H=2048, nh=16)
R1 = Dims(H=7168, nh=128)

EPS = 1e-6
THETA = 10000.0


# --------------------------------------------------------------------------
# storage-format helpers (format conversion only)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the
    16-bit patterns as uint16."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32, exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_storage(a32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> stored array: np.float16 for 'f16', uint16 bit patterns for
    'bf16'."""
    if dtype == "f16":
        return np.ascontiguousarray(a32, dtype=np.float32).astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    raise ValueError(dtype)


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored array -> float32 values (exact)."""
    if dtype == "f16":
        return a.astype(np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(a)
    raise ValueError(dtype)


def quantize_weight_per_column(W: np.ndarray):
    """Offline weight preparation for the W8A8 workload: symmetric int8 per
    output column, scale = max_k |W[k,n]| / 127, code = clamp(rint(W/scale),
    -127, 127).  Returns (int8 codes, float32 scales)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    amax = np.max(np.abs(W), axis=0)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = np.clip(np.rint(W / safe[None, :]), -127, 127).astype(np.int8)
    q[:, scale == 0] = 0
    return q, scale


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    dims: Dims
    kind: str            # 'fp' or 'w8a8'
    dtype: str           # storage dtype of activations / outputs: 'f16' | 'bf16'
    T: int
    positions: np.ndarray            # int32 [T]
    X: np.ndarray                    # [T,H]   stored dtype
    gamma: np.ndarray                # [r]     stored dtype
    Wa: Optional[np.ndarray] = None  # [H,N1]  stored dtype (fp path)
    Wb: Optional[np.ndarray] = None  # [r,N2]  stored dtype (fp path)
    Wqa: Optional[np.ndarray] = None  # int8 [H,N1] (w8a8)
    swa: Optional[np.ndarray] = None  # f32 [N1]
    Wqb: Optional[np.ndarray] = None  # int8 [r,N2]
    swb: Optional[np.ndarray] = None  # f32 [N2]
    seq_lens: Optional[np.ndarray] = None
    eps: float = EPS
    theta: float = THETA
    meta: dict = field(default_factory=dict)

    def rows(self, idx) -> "Workload":
        """The same workload restricted to a subset of tokens (every output
        row depends only on its own token)."""
        idx = np.asarray(idx)
        return dataclasses.replace(self, T=len(idx), X=self.X[idx],
                                   positions=self.positions[idx])


CONFIGS = [
    dict(idx=0, name="v2lite_fp16_decode_T1", dims=V2LITE, kind="fp", dtype="f16",
         wstd=0.02, desc="DeepSeek-V2-Lite KV prolog, one decode token"),
    dict(idx=1, name="v2lite_fp16_decode_b32x2_T64", dims=V2LITE, kind="fp", dtype="f16",
         wstd=0.02, desc="DeepSeek-V2-Lite decode, 32 sequences x 2 query tokens"),
    dict(idx=2, name="v2lite_fp16_prefill_T4096", dims=V2LITE, kind="fp", dtype="f16",
         wstd=0.02, desc="DeepSeek-V2-Lite prefill of one 4096-token sequence"),
    dict(idx=3, name="r1_bf16_decode_b128x2_T256", dims=R1, kind="fp", dtype="bf16",
         wstd=0.01, desc="DeepSeek-R1-sized decode, 128 sequences x 2 tokens"),
    dict(idx=4, name="r1_w8a8_ragged_prefill_8seq", dims=R1, kind="w8a8", dtype="bf16",
         wstd=0.01, desc="DeepSeek-R1-sized W8A8 packed prefill of 8 sequences"),
]


def _positions_for(idx: int, rng: np.random.Generator):
    """Token count, positions and sequence lengths of a configuration."""
    if idx == 0:
        return np.array([rng.integers(0, 4096)], np.int32), np.array([1], np.int64)
    if idx == 1:
        lens = rng.integers(16, 4096, 32)
        pos = np.stack([lens, lens + 1], axis=1).reshape(-1)
        return pos.astype(np.int32), np.full(32, 2, np.int64)
    if idx == 2:
        return np.arange(4096, dtype=np.int32), np.array([4096], np.int64)
    if idx == 3:
        base = rng.integers(0, 32767, 128)
        pos = np.stack([base, base + 1], axis=1).reshape(-1)
        return pos.astype(np.int32), np.full(128, 2, np.int64)
    if idx == 4:
        lens = rng.integers(512, 4097, 8)
        pos = np.concatenate([np.arange(L) for L in lens])
        return pos.astype(np.int32), lens.astype(np.int64)
    raise ValueError(idx)


def _draw_tensors(rng, dims: Dims, T: int, kind: str, dtype: str, wstd: float):
    X32 = rng.standard_normal((T, dims.H), dtype=np.float32)
    Wa32 = (rng.standard_normal((dims.H, dims.N1), dtype=np.float32) * np.float32(wstd))
    g32 = rng.uniform(0.5, 1.5, dims.r).astype(np.float32)
    Wb32 = (rng.standard_normal((dims.r, dims.N2), dtype=np.float32) * np.float32(wstd))
    out = dict(X=to_storage(X32, dtype), gamma=to_storage(g32, dtype))
    del X32
    if kind == "fp":
        out["Wa"] = to_storage(Wa32, dtype)
        out["Wb"] = to_storage(Wb32, dtype)
    else:
        out["Wqa"], out["swa"] = quantize_weight_per_column(Wa32)
        out["Wqb"], out["swb"] = quantize_weight_per_column(Wb32)
    return out


def make_config(idx: int, seed: Optional[int] = None) -> Workload:
    """The workload of configuration ``idx`` (seed defaults to 1000 + idx)."""
    c = CONFIGS[idx]
    rng = np.random.default_rng(1000 + idx if seed is None else seed)
    pos, lens = _positions_for(idx, rng)
    T = len(pos)
    tens = _draw_tensors(rng, c["dims"], T, c["kind"], c["dtype"], c["wstd"])
    return Workload(name=c["name"], dims=c["dims"], kind=c["kind"], dtype=c["dtype"],
                    T=T, positions=pos, seq_lens=lens, meta=dict(config=idx), **tens)


def make_custom(dims: Dims, T: int, *, kind: str = "fp", dtype: str = "f16",
                seed: int = 0, wstd: float = 0.02, max_pos: int = 4096,
                positions: Optional[np.ndarray] = None) -> Workload:
    """A workload of arbitrary shape with config-0 value distributions;
    positions ~ U[0, max_pos) unless given."""
    rng = np.random.default_rng(seed)
    if positions is None:
        positions = rng.integers(0, max_pos, T)
    positions = np.asarray(positions, np.int32)
    assert positions.shape == (T,)
    tens = _draw_tensors(rng, dims, T, kind, dtype, wstd)
    return Workload(name=f"custom_T{T}_H{dims.H}_nh{dims.nh}_{kind}_{dtype}", dims=dims,
                    kind=kind, dtype=dtype, T=T, positions=positions, **tens)


def paged_slot_mapping(w: Workload, block_size: int = 64, seed: int = 0,
                       spare_blocks: float = 1.0):
    """A paged-cache slot mapping for the workload's tokens: every sequence
    owns blocks of ``block_size`` slots drawn at random (without replacement)
    from one pool, one block per ``block_size`` positions it touches, and
    token t of sequence q goes to slot block(q, pos // B) * B + pos % B.
    Returns (int64 slots [T], number of slots in the pool); the pool holds
    ``1 + spare_blocks`` times the blocks in use, so most slots stay empty.
    In a workload without sequence lengths every token is a sequence of its
    own (its positions are independent draws)."""
    rng = np.random.default_rng(seed)
    lens = w.seq_lens if w.seq_lens is not None else np.ones(w.T, np.int64)
    seq = np.repeat(np.arange(len(lens)), lens)
    assert len(seq) == w.T
    keys = seq.astype(np.int64) * (1 << 32) + (w.positions.astype(np.int64) // block_size)
    uniq, inv = np.unique(keys, return_inverse=True)
    nblocks = int(np.ceil(len(uniq) * (1.0 + spare_blocks)))
    blocks = rng.permutation(nblocks)[:len(uniq)].astype(np.int64)
    slots = blocks[inv] * block_size + w.positions.astype(np.int64) % block_size
    return slots, nblocks * block_size


def algorithmic_bytes(dims: Dims, T: int, kind: str, dtype: str = "f16") -> int:
    """Bytes a call must move at least once: the weights (and scales), gamma,
    the hidden rows and positions it reads, and the four outputs it writes."""
    D = 2
    if kind == "fp":
        w = (dims.H * dims.N1 + dims.r * dims.N2) * D + dims.r * D
    else:
        w = dims.H * dims.N1 + dims.r * dims.N2 + 4 * (dims.N1 + dims.N2) + dims.r * D
    per_tok_in = dims.H * D + 4
    per_tok_out = (dims.nh * (dims.dn + dims.dv) + dims.dr + dims.r) * D
    return w + T * (per_tok_in + per_tok_out)


def algorithmic_flops(dims: Dims, T: int) -> int:
    """Multiply-adds of the two projections, counted as 2 operations each."""
    return 2 * T * (dims.H * dims.N1 + dims.r * dims.N2)
