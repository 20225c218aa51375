"""The five named workloads of banded sparse attention forward, as plain data.

Window extents are one-sided and inclusive, counted in dilated steps: query i sees keys
i + dil*t for t in [-win_left, win_right].  Shapes follow the pages' workloads:

* tiny_f32: a small symmetric window with one global token (the Longformer hub page,
  section 2: sliding window plus global tokens), kept in fp32.
* longformer_base: 4096 tokens, 12 heads, 512-token window (256 each side), a 32-token
  question span made global, and the tail of the second sample padded (Longformer hub page,
  sections 2 and 5: window around 512, question tokens global, mask value 0 = pad).
* dilated_16k: 16384 tokens with dilation 2 on four heads (Longformer hub page, section 2:
  dilated windows, inference at 16K) and 64 global tokens at seeded positions.
* swa512_causal_32k: causal 512-key window at head dim 128 (SWAN-GPT summary, section 3.3:
  512-token SWA-RoPE layers; SWA/Hybrid-RoPE blog, section 3: w = 512, rotary encoding on part
  of the dims only).
* bigbird_itc: 64-token blocks with three sliding blocks, first and last block global and
  three random blocks per query block (Big Bird reading notes, sections 3.2.2, 3.2.3, 3.3).
"""

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    n: int
    d: int
    dtype: str  # "bf16" or "f32": the dtype of Q, K, V and the output
    win_left: int  # -1 together with win_right = -1 means "no band"
    win_right: int
    seed: int  # seed of the Q, K, V draws (drawn in the order q, k, v)
    qkv_scale: float = 1.0  # N(0,1) draws are multiplied by this before rounding
    dilation: Optional[Tuple[int, ...]] = None  # per head; None = 1 everywhere
    globals_kind: str = "none"  # none | first | seeded | bigbird_ends
    n_global: int = 0
    globals_seed: int = 0
    pad_tail: Tuple[int, ...] = ()  # per sample: number of padded keys at the end
    block: int = 0  # block-sparse layout block size; 0 = no layout
    max_kb: int = 0
    layout_seed: int = 0
    rope_dims: int = 0  # rotary pre-rotation of Q and K on dims [0, rope_dims)
    rope_base: float = 10000.0
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / float(self.d) ** 0.5


WORKLOADS = {
    "tiny_f32": Workload(
        name="tiny_f32", batch=1, heads=1, n=256, d=64, dtype="f32",
        win_left=32, win_right=32, seed=1, globals_kind="first", n_global=1,
        note="B1 H1 n256 d64 fp32, window 32 each side, token 0 global",
    ),
    "longformer_base": Workload(
        name="longformer_base", batch=2, heads=12, n=4096, d=64, dtype="bf16",
        win_left=256, win_right=256, seed=2, qkv_scale=0.5,
        globals_kind="first", n_global=32, pad_tail=(0, 137),
        note="B2 H12 n4096 d64 bf16, window 256 each side, tokens 0..31 global, "
             "last 137 keys of sample 2 padded, N(0,1)*0.5",
    ),
    "dilated_16k": Workload(
        name="dilated_16k", batch=1, heads=16, n=16384, d=64, dtype="bf16",
        win_left=256, win_right=256, seed=3,
        dilation=(2, 2, 2, 2) + (1,) * 12,
        globals_kind="seeded", n_global=64, globals_seed=103,
        note="B1 H16 n16384 d64 bf16, window 256 each side, dilation 2 on heads 0-3, "
             "64 seeded global tokens",
    ),
    "swa512_causal_32k": Workload(
        name="swa512_causal_32k", batch=1, heads=16, n=32768, d=128, dtype="bf16",
        win_left=511, win_right=0, seed=4, rope_dims=64, rope_base=10000.0,
        note="B1 H16 n32768 d128 bf16, causal window 512 (keys i-511..i), rotary on dims 0-63",
    ),
    "bigbird_itc": Workload(
        name="bigbird_itc", batch=2, heads=12, n=4096, d=64, dtype="bf16",
        win_left=-1, win_right=-1, seed=5, globals_kind="bigbird_ends",
        n_global=128, block=64, max_kb=6, layout_seed=105,
        note="B2 H12 n4096 d64 bf16, block 64: 3 sliding + 3 random blocks per query block, "
             "first and last block global",
    ),
}

# The order in which the workloads are listed (smallest, parity-only case first).
ORDER = ["tiny_f32", "longformer_base", "dilated_16k", "swa512_causal_32k", "bigbird_itc"]


def workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {', '.join(ORDER)}") from None
