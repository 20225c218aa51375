"""Seeded input generators.

Everything is drawn with numpy's PCG64 ``default_rng`` so both sides of a parity test see the
same bytes.  Q, K, V are standard normal float32 draws in the order q, k, v, multiplied by the
workload's scale, optionally pre-rotated (rotary encoding on the leading dims, applied in
float32), then rounded once to bf16 with round-to-nearest-even.  fp32 workloads skip the
rounding.  The fp64 copies handed to the oracle are exact widenings of those values.
"""

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import Workload


# ----------------------------------------------------------------------------- bf16 helpers
def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Inputs must be finite; the workloads never produce anything else.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the exactly equal float32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32
    )


# ----------------------------------------------------------------------------- container
@dataclass
class Inputs:
    """One problem instance.  Arrays are host numpy arrays, layout [B, H, n, d] (BHND)."""

    batch: int
    heads: int
    n: int
    d: int
    dtype: str  # "bf16": q/k/v are uint16 bf16 bit patterns; "f32": float32
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    scale: float
    win_left: int
    win_right: int
    dilation: Optional[np.ndarray] = None  # int32 [H]
    global_idx: Optional[np.ndarray] = None  # int32 [B, g], ascending, distinct
    key_pad: Optional[np.ndarray] = None  # uint8 [B, n], nonzero = padded key
    layout: Optional[np.ndarray] = None  # int32 [H, n/block, max_kb], -1 = unused slot
    block: int = 0
    max_kb: int = 0

    @property
    def n_global(self) -> int:
        return 0 if self.global_idx is None else int(self.global_idx.shape[1])

    def f64(self, name: str) -> np.ndarray:
        """Exact float64 copy of q, k or v."""
        a = getattr(self, name)
        if self.dtype == "bf16":
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)

    def f32(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if self.dtype == "bf16":
            return bf16_bits_to_f32(a)
        return a.astype(np.float32)

    def select_heads(self, heads) -> "Inputs":
        """The same problem restricted to the listed heads (dilation and layout follow)."""
        hs = list(heads)
        return Inputs(
            batch=self.batch, heads=len(hs), n=self.n, d=self.d, dtype=self.dtype,
            q=np.ascontiguousarray(self.q[:, hs]),
            k=np.ascontiguousarray(self.k[:, hs]),
            v=np.ascontiguousarray(self.v[:, hs]),
            scale=self.scale, win_left=self.win_left, win_right=self.win_right,
            dilation=None if self.dilation is None else self.dilation[hs].copy(),
            global_idx=self.global_idx, key_pad=self.key_pad,
            layout=None if self.layout is None else np.ascontiguousarray(self.layout[hs]),
            block=self.block, max_kb=self.max_kb,
        )


# ----------------------------------------------------------------------------- pieces
def draw_qkv(rng: np.random.Generator, shape, scale: float):
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        s = np.float32(scale)
        q *= s
        k *= s
        v *= s
    return q, k, v


def rotary_prerotate(x: np.ndarray, dims: int, base: float) -> np.ndarray:
    """Rotate interleaved pairs (x[2i], x[2i+1]), i < dims/2, by angle t * base**(-2i/dims)
    at row position t, in float32; dims >= ``dims`` are left position-free.

    This is input preparation for the causal sliding-window workload (rotary encoding on part
    of the dims, the rest content-only); the attention itself never sees positions.
    """
    n = x.shape[-2]
    half = dims // 2
    inv = base ** (-2.0 * np.arange(half, dtype=np.float64) / dims)
    ang = np.arange(n, dtype=np.float64)[:, None] * inv[None, :]
    c = np.cos(ang).astype(np.float32)
    s = np.sin(ang).astype(np.float32)
    out = x.copy()
    ev = x[..., 0:dims:2]
    od = x[..., 1:dims:2]
    out[..., 0:dims:2] = ev * c - od * s
    out[..., 1:dims:2] = ev * s + od * c
    return out


def bigbird_layout(heads: int, n: int, block: int, rng: np.random.Generator,
                   n_random: int = 3) -> np.ndarray:
    """Block layout of the ITC pattern with the first and last block global.

    Query block q (not first or last) lists its sliding blocks {q-1, q, q+1} minus the two
    global blocks, plus ``n_random`` distinct random blocks drawn without replacement from the
    blocks that are neither sliding nor global.  The global blocks' columns are supplied as
    global tokens instead of layout entries, and the rows of the global blocks are global rows,
    so their layout rows are empty.  Drawn per (head, query block), shared across the batch.
    """
    nb = n // block
    max_kb = 3 + n_random
    lay = np.full((heads, nb, max_kb), -1, dtype=np.int32)
    for h in range(heads):
        for q in range(1, nb - 1):
            sliding = [b for b in (q - 1, q, q + 1) if b not in (0, nb - 1)]
            excluded = {q - 1, q, q + 1, 0, nb - 1}
            cand = np.array([b for b in range(nb) if b not in excluded], dtype=np.int64)
            pick = rng.choice(cand, size=n_random, replace=False)
            row = sorted(sliding) + sorted(int(b) for b in pick)
            lay[h, q, : len(row)] = row
    return lay


def _globals(w: Workload) -> Optional[np.ndarray]:
    if w.globals_kind == "none" or w.n_global == 0:
        return None
    if w.globals_kind == "first":
        row = np.arange(w.n_global, dtype=np.int32)
    elif w.globals_kind == "seeded":
        pos = np.random.default_rng(w.globals_seed).choice(w.n, w.n_global, replace=False)
        row = np.sort(pos).astype(np.int32)
    elif w.globals_kind == "bigbird_ends":
        nb = w.n // w.block
        row = np.concatenate(
            [np.arange(0, w.block), np.arange((nb - 1) * w.block, nb * w.block)]
        ).astype(np.int32)
        assert row.size == w.n_global
    else:
        raise ValueError(f"unknown globals_kind {w.globals_kind!r}")
    return np.ascontiguousarray(np.broadcast_to(row, (w.batch, row.size)), dtype=np.int32)


def _pad(w: Workload) -> Optional[np.ndarray]:
    if not any(w.pad_tail):
        return None
    m = np.zeros((w.batch, w.n), dtype=np.uint8)
    for b, cnt in enumerate(w.pad_tail):
        if cnt:
            m[b, w.n - cnt:] = 1
    return m


def make_inputs(w: Workload) -> Inputs:
    """Build the seeded inputs of a named workload."""
    shape = (w.batch, w.heads, w.n, w.d)
    q, k, v = draw_qkv(np.random.default_rng(w.seed), shape, w.qkv_scale)
    if w.rope_dims:
        q = rotary_prerotate(q, w.rope_dims, w.rope_base)
        k = rotary_prerotate(k, w.rope_dims, w.rope_base)
    if w.dtype == "bf16":
        q, k, v = (round_to_bf16_bits(a) for a in (q, k, v))
    layout = None
    if w.block:
        layout = bigbird_layout(w.heads, w.n, w.block, np.random.default_rng(w.layout_seed),
                                n_random=w.max_kb - 3)
    return Inputs(
        batch=w.batch, heads=w.heads, n=w.n, d=w.d, dtype=w.dtype, q=q, k=k, v=v,
        scale=w.scale, win_left=w.win_left, win_right=w.win_right,
        dilation=None if w.dilation is None else np.array(w.dilation, dtype=np.int32),
        global_idx=_globals(w), key_pad=_pad(w), layout=layout,
        block=w.block, max_kb=w.max_kb,
    )


def random_case(seed: int, *, batch: int, heads: int, n: int, d: int, dtype: str = "bf16",
                win_left: int = -1, win_right: int = -1, dilations=None, n_global: int = 0,
                pad: str = "none", pad_count: int = 0, block: int = 0, max_kb: int = 0,
                layout_fill: float = 0.5, qkv_scale: float = 1.0,
                scale: Optional[float] = None) -> Inputs:
    """A seeded instance with explicit shape and randomly drawn structure.

    ``dilations``: None, an int (every head), or a sequence of per-head values.
    ``pad``: "none", "tail" (the last ``pad_count`` keys of each sample but the first) or
    "random" (``pad_count`` random keys per sample).
    ``block``/``max_kb``: a random layout whose rows list up to ``max_kb`` distinct blocks
    (each slot filled with probability ``layout_fill``), unused slots -1 at the end.
    """
    rng = np.random.default_rng(seed)
    shape = (batch, heads, n, d)
    q, k, v = draw_qkv(rng, shape, qkv_scale)
    if dtype == "bf16":
        q, k, v = (round_to_bf16_bits(a) for a in (q, k, v))
    dil = None
    if dilations is not None:
        if isinstance(dilations, int):
            dil = np.full(heads, dilations, dtype=np.int32)
        else:
            dil = np.array(dilations, dtype=np.int32)
            assert dil.shape == (heads,)
    gidx = None
    if n_global:
        gidx = np.stack(
            [np.sort(rng.choice(n, n_global, replace=False)) for _ in range(batch)]
        ).astype(np.int32)
    kp = None
    if pad == "tail" and pad_count:
        kp = np.zeros((batch, n), dtype=np.uint8)
        kp[1:, n - pad_count:] = 1
    elif pad == "random" and pad_count:
        kp = np.zeros((batch, n), dtype=np.uint8)
        for b in range(batch):
            kp[b, rng.choice(n, pad_count, replace=False)] = 1
    lay = None
    if block:
        assert n % block == 0
        nb = n // block
        lay = np.full((heads, nb, max_kb), -1, dtype=np.int32)
        for h in range(heads):
            for qb in range(nb):
                cnt = int((rng.random(max_kb) < layout_fill).sum())
                cnt = min(cnt, nb)
                if cnt:
                    lay[h, qb, :cnt] = rng.choice(nb, cnt, replace=False)
    return Inputs(
        batch=batch, heads=heads, n=n, d=d, dtype=dtype, q=q, k=k, v=v,
        scale=(1.0 / d ** 0.5) if scale is None else scale,
        win_left=win_left, win_right=win_right, dilation=dil, global_idx=gidx,
        key_pad=kp, layout=lay, block=block, max_kb=max_kb,
    )


def draw_dout(inp: Inputs, seed: int, scale: float = 1.0) -> np.ndarray:
    """A seeded output gradient dO of q's shape: N(0, 1) * scale draws, rounded once to bf16 for
    bf16 inputs (uint16 bit patterns), float32 otherwise."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal(inp.q.shape, dtype=np.float32)
    if scale != 1.0:
        g *= np.float32(scale)
    return round_to_bf16_bits(g) if inp.dtype == "bf16" else g


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 copy of a bf16 (uint16 bits) or float32 array."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)
