"""Seeded inputs for LongT5 Transient-Global attention.

Shapes follow the LongT5 guide's defaults: d_model 512, 8 heads of d_kv 64, local radius 127,
global blocks of 16 tokens, 32 relative-position buckets with max distance 128, RMS-norm epsilon
1e-6, inputs up to 16,384 tokens.  The learned parameters (RMS-norm weight, key and value
projections, the two bias tables) are random stand-ins: gamma ~ 1 + 0.1 N(0, 1), W ~ N(0, 1) /
sqrt(d_model), bias tables ~ N(0, 1).  x, q, k, v are N(0, 1) draws rounded once to bf16 (bf16
dtype); the projections are rounded to bf16 as well, gamma and the bias tables stay fp32.
Draw order: x, q, k, v, gamma, wk, wv, bias_local, bias_side, then the padding.

Input preparation only; no attention arithmetic.
"""

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .gen import bf16_bits_to_f32, round_to_bf16_bits


@dataclass(frozen=True)
class TGWorkload:
    name: str
    batch: int
    heads: int
    n: int
    d: int
    d_model: int
    radius: int
    block: int
    seed: int
    pad_tail: tuple = ()
    note: str = ""


TG_WORKLOADS = {
    "tglobal_16k": TGWorkload(
        name="tglobal_16k", batch=1, heads=8, n=16384, d=64, d_model=512, radius=127, block=16,
        seed=61,
        note="B1 H8 n16384 d64 bf16, LongT5 Transient-Global: radius 127, 1024 global tokens of "
             "16-token blocks, 32 buckets / max distance 128, d_model 512",
    ),
}


@dataclass
class TGInputs:
    batch: int
    heads: int
    n: int
    d: int
    d_model: int
    radius: int
    block: int
    dtype: str
    x: np.ndarray       # [B, n, dm]
    q: np.ndarray       # [B, H, n, d]
    k: np.ndarray
    v: np.ndarray
    gamma: np.ndarray   # float32 [dm]
    wk: np.ndarray      # [dm, H*d]
    wv: np.ndarray
    bias_local: np.ndarray  # float32 [num_buckets, H]
    bias_side: np.ndarray
    key_pad: Optional[np.ndarray] = None  # uint8 [B, n]
    scale: float = 0.125
    eps: float = 1e-6
    num_buckets: int = 32
    max_distance: int = 128

    def f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if self.dtype == "bf16":
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)


def make_tglobal_inputs(seed: int, *, batch: int, heads: int, n: int, d: int, d_model: int,
                        radius: int, block: int, dtype: str = "bf16", pad_tail=(),
                        num_buckets: int = 32, max_distance: int = 128,
                        scale: Optional[float] = None) -> TGInputs:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((batch, n, d_model), dtype=np.float32)
    q = rng.standard_normal((batch, heads, n, d), dtype=np.float32)
    k = rng.standard_normal((batch, heads, n, d), dtype=np.float32)
    v = rng.standard_normal((batch, heads, n, d), dtype=np.float32)
    gamma = (1.0 + 0.1 * rng.standard_normal(d_model)).astype(np.float32)
    wk = (rng.standard_normal((d_model, heads * d)) / np.sqrt(d_model)).astype(np.float32)
    wv = (rng.standard_normal((d_model, heads * d)) / np.sqrt(d_model)).astype(np.float32)
    bl = rng.standard_normal((num_buckets, heads)).astype(np.float32)
    bs = rng.standard_normal((num_buckets, heads)).astype(np.float32)
    if dtype == "bf16":
        x, q, k, v, wk, wv = (round_to_bf16_bits(a) for a in (x, q, k, v, wk, wv))
    kp = None
    if any(pad_tail):
        kp = np.zeros((batch, n), dtype=np.uint8)
        for b, c in enumerate(pad_tail):
            if c:
                kp[b, n - c:] = 1
    return TGInputs(batch=batch, heads=heads, n=n, d=d, d_model=d_model, radius=radius,
                    block=block, dtype=dtype, x=x, q=q, k=k, v=v, gamma=gamma, wk=wk, wv=wv,
                    bias_local=bl, bias_side=bs, key_pad=kp,
                    scale=(1.0 / d ** 0.5) if scale is None else float(scale),
                    num_buckets=num_buckets, max_distance=max_distance)


def tglobal_workload_inputs(wl: TGWorkload) -> TGInputs:
    return make_tglobal_inputs(wl.seed, batch=wl.batch, heads=wl.heads, n=wl.n, d=wl.d,
                               d_model=wl.d_model, radius=wl.radius, block=wl.block,
                               pad_tail=wl.pad_tail)


def tglobal_to_torch(inp: TGInputs, device):
    """Every array of ``inp`` as a device tensor (bf16 or fp32; fp32 gamma and bias tables;
    uint8 padding)."""
    import torch

    def mat(a):
        if inp.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    return dict(x=mat(inp.x), q=mat(inp.q), k=mat(inp.k), v=mat(inp.v), wk=mat(inp.wk),
                wv=mat(inp.wv), gamma=f32(inp.gamma), bias_local=f32(inp.bias_local),
                bias_side=f32(inp.bias_side),
                key_pad=None if inp.key_pad is None else torch.from_numpy(inp.key_pad).to(device))
