"""GPU parity of the sliding-window decode entry point against the fp64 oracle.

The expected rows come from the oracle's forward pass on each sample's gathered window
(``oracle.decode_inputs``).  Slots that the step must not read hold NaN.
"""

import sys

import numpy as np
import pytest

import sparse_long_sequence_banded_amd as la
from oracle import decode_inputs as decode_expected
from tests.gpu_helpers import compare
from workloads.decode import (DECODE_WORKLOADS, decode_to_torch, decode_workload_inputs,
                              make_decode_inputs)

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.load()
    yield


def run_decode(inp, samples=None):
    import torch

    t = decode_to_torch(inp, "cuda:0")
    out, lse = la.decode(t["q"], t["k_cache"], t["v_cache"], t["positions"], window=inp.window,
                         scale=inp.scale, ring=inp.ring)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    if samples is not None:
        o, l = o[samples], l[samples]
    return o, l, out


def check(inp, label, samples=None):
    ref_o, ref_l = decode_expected(inp, samples)
    o, l, _ = run_decode(inp, samples)
    max_abs = compare(inp, o, l, ref_o, ref_l, label)
    _note(f"[decode] {label}: max-abs {max_abs:.3e}")


CASES = [
    # (label, kwargs)
    ("linear bf16 m1", dict(batch=3, heads=2, d=128, dtype="bf16", window=512, m=1,
                            cache_len=2000, ring=False, positions=[0, 511, 1700])),
    ("ring bf16 m4 tight", dict(batch=3, heads=2, d=128, dtype="bf16", window=512, m=4,
                                cache_len=515, ring=True, positions=[3, 600, 2049])),
    ("ring f32 m16", dict(batch=3, heads=2, d=64, dtype="f32", window=100, m=16,
                          cache_len=200, ring=True, positions=[0, 150, 999])),
    ("linear f32 d8", dict(batch=2, heads=3, d=8, dtype="f32", window=37, m=3,
                           cache_len=300, ring=False, positions=[1, 250])),
    ("ring bf16 d24", dict(batch=2, heads=1, d=24, dtype="bf16", window=300, m=2,
                           cache_len=333, ring=True, positions=[299, 5000])),
    ("linear bf16 d256 long window", dict(batch=1, heads=2, d=256, dtype="bf16", window=3000,
                                          m=2, cache_len=4100, ring=False,
                                          positions=[4000])),
    ("ring bf16 d64 m7 ragged", dict(batch=4, heads=3, d=64, dtype="bf16", window=257, m=7,
                                     cache_len=300, ring=True, positions=[0, 256, 257, 1023])),
]


@pytest.mark.parametrize("label,kw", CASES, ids=[c[0] for c in CASES])
def test_decode_parity(label, kw):
    _note(f"[decode] {label}: {kw}")
    inp = make_decode_inputs(11 + len(label), **kw)
    check(inp, label)


# Shapes that give 8-wave workgroups (one chunk per window, or several chunks merged); the
# oracle checks a sample of the batch.
LARGE = [
    ("bf16 d64 one chunk", dict(batch=64, heads=8, d=64, dtype="bf16", window=1000, m=1,
                                cache_len=1000, ring=True,
                                positions=[(977 * i) % 5000 for i in range(64)]),
     [0, 1, 17, 40, 63]),
    ("f32 d128 three chunks", dict(batch=32, heads=16, d=128, dtype="f32", window=512, m=2,
                                   cache_len=600, ring=True,
                                   positions=[(331 * i) % 2000 for i in range(32)]),
     [0, 5, 31]),
    ("f32 d256 linear", dict(batch=2, heads=2, d=256, dtype="f32", window=300, m=3,
                             cache_len=700, ring=False, positions=[250, 600]),
     None),
]


@pytest.mark.parametrize("label,kw,samples", LARGE, ids=[c[0] for c in LARGE])
def test_decode_parity_wide_launches(label, kw, samples):
    _note(f"[decode] {label}")
    inp = make_decode_inputs(21 + len(label), **kw)
    check(inp, label, samples)


def test_window_one_returns_the_new_value_rows():
    inp = make_decode_inputs(12, batch=2, heads=2, d=64, dtype="bf16", window=1, m=3,
                             cache_len=64, ring=True, positions=[0, 100])
    _, _, out = run_decode(inp)
    bits = out.cpu().view(__import__("torch").int16).numpy().view(np.uint16)
    for b in range(2):
        slots = [int(np.nonzero(inp.slot_positions(b) == int(inp.positions[b]) + j)[0][0])
                 for j in range(3)]
        assert np.array_equal(bits[b], inp.v_cache[b][:, slots])


def test_decode_agrees_with_the_forward_pass():
    """The decode rows equal the corresponding rows of the library's own causal forward on the
    whole sequence (within the bf16 tolerance: the two paths round differently; the forward's lse
    is the log of its bf16-rounded weights' sum, within ln(1 + 2^-8) of the exact one)."""
    import torch

    n, window, m, d = 1100, 256, 4, 64
    inp = make_decode_inputs(13, batch=1, heads=2, d=d, dtype="bf16", window=window, m=m,
                             cache_len=n, ring=False, positions=[n - m])
    t = decode_to_torch(inp, "cuda:0")
    out_d, lse_d = la.decode(t["q"], t["k_cache"], t["v_cache"], t["positions"], window=window)
    q_full = torch.zeros_like(t["k_cache"])
    q_full[:, :, n - m:] = t["q"]
    out_f, lse_f = la.forward(q_full, t["k_cache"], t["v_cache"], win_left=window - 1,
                              win_right=0)
    torch.cuda.synchronize()
    assert (out_d.float() - out_f[:, :, n - m:].float()).abs().max().item() <= 2e-2
    assert (lse_d - lse_f[:, :, n - m:]).abs().max().item() <= 4e-3


def test_decode_full_size_sampled():
    wl = DECODE_WORKLOADS["swa512_decode_32k"]
    _note(f"[decode] {wl.name} full launch, oracle on 4 samples")
    inp = decode_workload_inputs(wl)
    o, l, _ = run_decode(inp)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    samples = [0, 9, 22, 31]
    ref_o, ref_l = decode_expected(inp, samples)
    compare(inp, o[samples], l[samples], ref_o, ref_l, wl.name)


def test_decode_is_deterministic_and_lse_optional():
    import torch

    inp = make_decode_inputs(14, batch=2, heads=2, d=128, dtype="bf16", window=700, m=2,
                             cache_len=800, ring=True, positions=[10, 3000])
    t = decode_to_torch(inp, "cuda:0")
    a, _ = la.decode(t["q"], t["k_cache"], t["v_cache"], t["positions"], window=700, ring=True)
    b, l = la.decode(t["q"], t["k_cache"], t["v_cache"], t["positions"], window=700, ring=True,
                     want_lse=False)
    torch.cuda.synchronize()
    assert l is None
    assert (a.view(torch.int16) == b.view(torch.int16)).all()
