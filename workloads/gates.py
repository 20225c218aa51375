"""Seeded inputs for the output gates of gated attention: elementwise gate logits and the
low-rank gate's weights (random stand-ins for learned parameters).  Input preparation only."""

import numpy as np

from .gen import round_to_bf16_bits


def gate_logits(shape, seed: int, dtype: str = "bf16", scale: float = 2.0) -> np.ndarray:
    """N(0, 1) * scale logits, bf16 bits (bf16) or float32."""
    g = (np.random.default_rng(seed).standard_normal(shape, dtype=np.float32) *
         np.float32(scale))
    return round_to_bf16_bits(g) if dtype == "bf16" else g


def lowrank_inputs(seed: int, *, batch: int, heads: int, n: int, d: int, rank: int):
    """(out [B, H, n, d], w_down [r, H*d], w_up [H*d, r]) as bf16 bits: the outputs N(0, 1),
    the weights N(0, 1) scaled by 1/sqrt(fan-in)."""
    rng = np.random.default_rng(seed)
    hd = heads * d
    out = rng.standard_normal((batch, heads, n, d), dtype=np.float32)
    wd = rng.standard_normal((rank, hd), dtype=np.float32) / np.float32(np.sqrt(hd))
    wu = rng.standard_normal((hd, rank), dtype=np.float32) / np.float32(np.sqrt(rank))
    return tuple(round_to_bf16_bits(a) for a in (out, wd, wu))
