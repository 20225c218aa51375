"""Seeded inputs for sliding-window decode over a key/value cache.

A decode step brings m new query rows per sample at positions t0_b .. t0_b + m - 1; the keys
and values of every position up to the last new row are already in the cache.  Position p sits
in slot p (linear cache) or p mod cache_len (rolling buffer).  Slots that hold no position the
step may read (a rolling buffer not yet full, a linear cache past the last new row) are filled
with NaN, so any read of them shows in the output.

This module holds input preparation only (draws, bf16 rounding, the slot map); no attention
arithmetic.
"""

from dataclasses import dataclass
from typing import Sequence

import numpy as np

from .gen import bf16_bits_to_f32, draw_qkv, round_to_bf16_bits

BF16_NAN = np.uint16(0x7FC0)


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    batch: int
    heads: int
    d: int
    dtype: str
    window: int
    m: int
    cache_len: int
    ring: bool
    seed: int
    context: int  # positions are drawn in [context - window, context): a cache at that depth
    note: str = ""


DECODE_WORKLOADS = {
    # One decode step of the 512-key causal sliding-window layers (SWAN-GPT summary, section 3.3;
    # SWA/Hybrid-RoPE blog, section 3) at 32K context: 32 sequences, 16 heads of dim 128, one
    # new token each, a rolling buffer of exactly the window.
    "swa512_decode_32k": DecodeWorkload(
        name="swa512_decode_32k", batch=32, heads=16, d=128, dtype="bf16", window=512, m=1,
        cache_len=512, ring=True, seed=41, context=32768,
        note="B32 H16 d128 bf16, 1 new row per sequence at ~32K context, causal window 512, "
             "rolling cache of 512 slots",
    ),
}


@dataclass
class DecodeInputs:
    batch: int
    heads: int
    d: int
    dtype: str          # "bf16" (uint16 bit patterns) or "f32"
    window: int
    m: int
    cache_len: int
    ring: bool
    scale: float
    q: np.ndarray       # [B, H, m, d]
    k_cache: np.ndarray  # [B, H, cache_len, d]
    v_cache: np.ndarray
    positions: np.ndarray  # int32 [B]

    def slot_positions(self, b: int) -> np.ndarray:
        """Position held by each slot of sample b's cache (-1: none the step may read)."""
        last = int(self.positions[b]) + self.m - 1
        s = np.arange(self.cache_len, dtype=np.int64)
        if self.ring:
            # the newest position p <= last with p = s (mod cache_len)
            p = last - ((last - s) % self.cache_len)
        else:
            p = np.where(s <= last, s, -1)
        return np.where(p >= 0, p, -1)

    def f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if self.dtype == "bf16":
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)

    def gathered(self, b: int):
        """Keys and values of positions p0 .. last of sample b in position order (fp64,
        [H, last - p0 + 1, d]) and p0, where p0 = max(0, t0_b - window + 1)."""
        t0 = int(self.positions[b])
        last = t0 + self.m - 1
        p0 = max(0, t0 - self.window + 1)
        pos = self.slot_positions(b)
        slot_of = {int(p): s for s, p in enumerate(pos) if p >= 0}
        slots = [slot_of[p] for p in range(p0, last + 1)]
        k = self.f64("k_cache")[b][:, slots]
        v = self.f64("v_cache")[b][:, slots]
        return p0, k, v


def make_decode_inputs(seed: int, *, batch: int, heads: int, d: int, dtype: str, window: int,
                       m: int, cache_len: int, ring: bool, positions: Sequence[int],
                       scale=None) -> DecodeInputs:
    """Q [B, H, m, d], caches [B, H, cache_len, d] drawn N(0, 1) (order: caches' k and v, then q),
    rounded once to bf16 for bf16; unused slots NaN."""
    rng = np.random.default_rng(seed)
    _, k, v = draw_qkv(rng, (batch, heads, cache_len, d), 1.0)
    q = rng.standard_normal((batch, heads, m, d), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = (round_to_bf16_bits(a) for a in (q, k, v))
    pos = np.asarray(positions, dtype=np.int32)
    assert pos.shape == (batch,) and np.all(pos >= 0)
    if ring:
        assert window + m - 1 <= cache_len
    else:
        assert np.all(pos.astype(np.int64) + m - 1 < cache_len)
    inp = DecodeInputs(batch=batch, heads=heads, d=d, dtype=dtype, window=window, m=m,
                       cache_len=cache_len, ring=ring,
                       scale=(1.0 / d ** 0.5) if scale is None else float(scale),
                       q=q, k_cache=k, v_cache=v, positions=pos)
    nan = BF16_NAN if dtype == "bf16" else np.float32(np.nan)
    for b in range(batch):
        unused = inp.slot_positions(b) < 0
        k[b][:, unused] = nan
        v[b][:, unused] = nan
    return inp


def decode_workload_inputs(wl: DecodeWorkload) -> DecodeInputs:
    rng = np.random.default_rng(wl.seed + 1000)
    positions = rng.integers(wl.context - wl.window, wl.context, size=wl.batch)
    return make_decode_inputs(wl.seed, batch=wl.batch, heads=wl.heads, d=wl.d, dtype=wl.dtype,
                              window=wl.window, m=wl.m, cache_len=wl.cache_len, ring=wl.ring,
                              positions=positions)


def decode_to_torch(inp: DecodeInputs, device):
    """q, k_cache, v_cache (bfloat16 or float32) and positions (int32) on ``device``."""
    import torch

    def mat(a):
        if inp.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    return dict(q=mat(inp.q), k_cache=mat(inp.k_cache), v_cache=mat(inp.v_cache),
                positions=torch.from_numpy(inp.positions.copy()).to(device))
