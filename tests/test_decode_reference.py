"""The oracle's decode result (its forward pass on the gathered window) against a direct
brute force over the cache slots (CPU only)."""

import numpy as np
import pytest

from oracle import decode_inputs as decode_expected
from workloads.decode import make_decode_inputs


def _brute(inp):
    """Softmax over the window of each new row, reading the cache slots directly."""
    q, K, V = inp.f64("q"), inp.f64("k_cache"), inp.f64("v_cache")
    out = np.zeros(q.shape)
    lse = np.zeros(q.shape[:3])
    for b in range(inp.batch):
        pos = inp.slot_positions(b)
        for j in range(inp.m):
            t = int(inp.positions[b]) + j
            slots = [s for s in range(inp.cache_len) if pos[s] >= 0 and t - inp.window < pos[s] <= t]
            assert len(slots) == min(inp.window, t + 1)
            for h in range(inp.heads):
                s = inp.scale * K[b, h, slots] @ q[b, h, j]
                mx = s.max()
                w = np.exp(s - mx)
                out[b, h, j] = w @ V[b, h, slots] / w.sum()
                lse[b, h, j] = mx + np.log(w.sum())
    return out, lse


@pytest.mark.parametrize("ring,positions,cache_len", [
    (False, [0, 7, 40], 48),
    (True, [0, 5, 90], 13),
    (True, [2, 3, 4], 20),
])
def test_gathered_oracle_matches_brute_force(ring, positions, cache_len):
    inp = make_decode_inputs(3, batch=3, heads=2, d=8, dtype="f32", window=10, m=4,
                             cache_len=cache_len, ring=ring, positions=positions)
    ref_o, ref_l = decode_expected(inp)
    bo, bl = _brute(inp)
    assert np.allclose(ref_o, bo, rtol=0, atol=1e-12)
    assert np.allclose(ref_l, bl, rtol=0, atol=1e-12)


def test_unused_slots_are_poisoned():
    inp = make_decode_inputs(4, batch=1, heads=1, d=8, dtype="bf16", window=6, m=2,
                             cache_len=9, ring=True, positions=[3])
    pos = inp.slot_positions(0)
    assert list(pos) == [0, 1, 2, 3, 4, -1, -1, -1, -1]
    assert np.all(np.isnan(inp.f64("k_cache")[0, 0, 5:]))
    assert np.all(np.isfinite(inp.f64("k_cache")[0, 0, :5]))
    lin = make_decode_inputs(4, batch=1, heads=1, d=8, dtype="f32", window=6, m=2,
                             cache_len=9, ring=False, positions=[3])
    assert list(lin.slot_positions(0)) == [0, 1, 2, 3, 4, -1, -1, -1, -1]
    wrap = make_decode_inputs(4, batch=1, heads=1, d=8, dtype="f32", window=6, m=2,
                              cache_len=7, ring=True, positions=[11])
    # last = 12: slots hold 7, 8, 9, 10, 11, 12, 6
    assert list(wrap.slot_positions(0)) == [7, 8, 9, 10, 11, 12, 6]
