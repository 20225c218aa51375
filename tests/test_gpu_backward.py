"""GPU parity of the backward pass (dQ, dK, dV) against the fp64 oracle.

The GPU backward takes the forward's own out and lse (as in training); the oracle recomputes
everything in fp64 from q, k, v.  Tolerance, elementwise |gpu - oracle| <= atol + rtol * |oracle|:
  bf16: atol 2e-2 (the stated bf16 bar), rtol 1e-2.  The gradients are stored in bf16 (relative
        2^-9), and the forward's bf16 output enters Drow = dO . O; gradients of global keys sum
        over every row and reach magnitudes of several units, so a relative term is needed.
  fp32: atol 1e-4 (the stated fp32 bar), rtol 1e-4 (fp32 sums over up to a few thousand terms).
"""

import sys

import numpy as np
import pytest

import oracle
import sparse_long_sequence_banded_amd as la
from workloads import draw_dout, make_inputs, random_case, widen, workload
from workloads.torch_io import to_torch

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}


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


def _mat(a, dtype, device):
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def run_gpu_backward(inp, dout_np):
    import torch

    t = to_torch(inp, "cuda:0")
    kw = dict(scale=inp.scale, win_left=inp.win_left, win_right=inp.win_right,
              dilation=inp.dilation, global_idx=t["global_idx"], key_pad=t["key_pad"],
              block_layout=t["layout"], block=inp.block)
    out, lse = la.forward(t["q"], t["k"], t["v"], **kw)
    dout = _mat(dout_np, inp.dtype, "cuda:0")
    dq, dk, dv = la.backward(t["q"], t["k"], t["v"], out, lse, dout, **kw)
    torch.cuda.synchronize()
    return tuple(x.float().cpu().numpy().astype(np.float64) for x in (dq, dk, dv))


def compare_grads(inp, got, ref, label):
    atol, rtol = TOL[inp.dtype]
    worst = 0.0
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert a.shape == b.shape
        err = np.abs(a - b)
        bound = atol + rtol * np.abs(b)
        bad = err > bound
        assert not bad.any(), (f"{label} {name}: {int(bad.sum())} elements out of tolerance, "
                               f"worst excess {float((err - bound).max()):.3e}, "
                               f"max-abs {float(err.max()):.3e}")
        if inp.dtype == "bf16" and b.size:
            denom = float(np.sqrt(np.mean(b ** 2)))
            if denom > 0:
                assert float(np.sqrt(np.mean(err ** 2))) / denom <= 1e-2, f"{label} {name}: rel-RMS"
        worst = max(worst, float(err.max()) if err.size else 0.0)
    return worst


def check(inp, seed, label, heads=None):
    dout_np = draw_dout(inp, seed)
    got = run_gpu_backward(inp, dout_np)
    sub, d_sub = inp, dout_np
    if heads is not None:
        sub = inp.select_heads(heads)
        d_sub = np.ascontiguousarray(dout_np[:, heads])
        got = tuple(np.ascontiguousarray(x[:, heads]) for x in got)
    ref = oracle.backward_inputs(sub, widen(d_sub, inp.dtype))
    worst = compare_grads(sub, got, ref, label)
    _note(f"[backward] {label}: max-abs {worst:.3e}")


# ------------------------------------------------------------------------------ named workloads
@pytest.mark.parametrize("name", ["tiny_f32", "longformer_base", "bigbird_itc"])
def test_workload_backward_parity(name):
    _note(f"[backward] {name}")
    check(make_inputs(workload(name)), 70, name)


@pytest.mark.parametrize("name", ["dilated_16k", "swa512_causal_32k"])
def test_workload_backward_full_size_every_head(name):
    """Full-size launch; dQ, dK and dV of every head compared with the oracle element by element
    (the 32K causal window at head dim 128 is the long-context fine-tuning shape)."""
    _note(f"[backward] {name} full launch, oracle on every head")
    check(make_inputs(workload(name)), 71, name)


@pytest.mark.parametrize("wl,wr", [(150, 77), (333, 1)])
def test_backward_rotated_window_walk_with_global_keys_inside(wl, wr):
    """Head dim 64 walks each workgroup's window tiles from a rotated start; the per-tile bits of
    the global keys inside the windows are indexed by the rotated tile, the tile count varies at
    the sequence ends and with the dilation, and the key ranges start off the 64-key grid."""
    inp = random_case(79, batch=2, heads=3, n=2000, d=64, win_left=wl, win_right=wr,
                      dilations=[1, 2, 3], n_global=60, pad="random", pad_count=97)
    check(inp, 79, f"rotated walk wl={wl} wr={wr}")


def test_causal_512_window_backward():
    """The causal 512-key window at head dim 128 on 4096 positions with two heads."""
    inp = random_case(72, batch=1, heads=2, n=4096, d=128, win_left=511, win_right=0)
    check(inp, 72, "causal 512, d128")


# ------------------------------------------------------------------------------ random sweep
def _sweep():
    rng = np.random.default_rng(4242)
    cases = []
    for t in range(24):
        dtype = "bf16" if t % 3 else "f32"
        d = int(rng.choice([64, 128])) if dtype == "bf16" else int(rng.choice([8, 40, 64, 128]))
        # the bf16 forward (which provides out and lse) takes a layout of 64- or 128-blocks
        # without a window; the fp32 forward takes every combination
        layout = rng.random() < 0.25
        block = (64 if dtype == "bf16" else int(rng.choice([16, 64]))) if layout else 0
        n = int(rng.choice([1, 2, 63, 65, 127, 200, 257, 384, 641]))
        if layout:
            n = block * int(rng.integers(1, 6))
        H = int(rng.integers(1, 4))
        band = (not layout) or (dtype == "f32" and rng.random() < 0.5)
        wl = int(rng.choice([0, 1, 5, 31, 64, 100, 300])) if band else -1
        wr = int(rng.choice([0, 0, 3, 33, 63, 128])) if band else -1
        dil = [int(x) for x in rng.integers(1, 4, size=H)] if band and rng.random() < 0.5 else None
        g = int(rng.integers(0, min(n, 40) + 1)) if rng.random() < 0.6 else 0
        pad = str(rng.choice(["none", "tail", "random"]))
        cases.append(dict(seed=7000 + t, batch=int(rng.integers(1, 3)), heads=H, n=n, d=d,
                          dtype=dtype, win_left=wl, win_right=wr, dilations=dil, n_global=g,
                          pad=pad, pad_count=int(rng.integers(0, n + 1)), block=block,
                          max_kb=int(rng.integers(1, 4)) if layout else 0))
    return cases


SWEEP = _sweep()


@pytest.mark.parametrize("case", SWEEP, ids=[f"s{i}" for i in range(len(SWEEP))])
def test_random_shapes_backward_parity(case):
    _note(f"[backward sweep] {case}")
    check(random_case(**case), case["seed"], str(case["seed"]))


@pytest.mark.parametrize("block,d", [(64, 128), (128, 64), (128, 128)])
def test_layout_backward_with_globals_and_padding(block, d):
    """Block layouts on the matrix-core path: listed blocks, global tokens inside and outside
    the listed blocks, key padding."""
    inp = random_case(78 + block + d, batch=2, heads=2, n=block * 9, d=d, block=block, max_kb=3,
                      n_global=21, pad="random", pad_count=40)
    check(inp, 78, f"layout block {block} d{d}")


# ------------------------------------------------------------------------------ edge cases
@pytest.mark.parametrize("d,block", [(64, 0), (128, 0), (64, 64)])
def test_global_owners_ordered_by_xcd(d, block):
    # eight (batch, head) pairs with equal main work: the global-owner workgroups take the heads
    # whose main work their XCD ran, in reverse order; 150 global tokens give two (window) or
    # three (64-row blocks) owner groups per head over three chunks
    if block:
        inp = random_case(58, batch=2, heads=4, n=1280, d=d, block=block, max_kb=3,
                          n_global=150, pad="random", pad_count=40)
    else:
        inp = random_case(57 + d, batch=2, heads=4, n=1300, d=d, win_left=100, win_right=60,
                          n_global=150, pad="random", pad_count=40)
    check(inp, 59, f"global owners by XCD d={d} block={block}")


def test_window_zero_sends_the_gradient_to_v():
    inp = random_case(75, batch=2, heads=2, n=300, d=64, win_left=0, win_right=0,
                      dilations=[1, 2])
    dout_np = draw_dout(inp, 75)
    dq, dk, dv = run_gpu_backward(inp, dout_np)
    # one key per row: dS = P (dO.v - dO.O) with O = v, zero up to fp32 rounding
    assert np.all(np.abs(dq) <= 1e-4) and np.all(np.abs(dk) <= 1e-4)
    np.testing.assert_allclose(dv, widen(dout_np, "bf16"), rtol=2 ** -8, atol=0)


def test_padded_keys_and_empty_rows_get_zero_gradients():
    inp = random_case(76, batch=2, heads=2, n=256, d=64, win_left=5, win_right=5, n_global=2)
    kp = np.zeros((2, 256), np.uint8)
    kp[1, :] = 1             # sample 2: every key padded, every row empty
    kp[0, 100:140] = 1       # sample 1: a padded stretch
    inp.key_pad = kp
    dout_np = draw_dout(inp, 76)
    dq, dk, dv = run_gpu_backward(inp, dout_np)
    assert np.all(dq[1] == 0) and np.all(dk[1] == 0) and np.all(dv[1] == 0)
    assert np.all(dk[0][:, 100:140] == 0) and np.all(dv[0][:, 100:140] == 0)
    ref = oracle.backward_inputs(inp, widen(dout_np, "bf16"))
    compare_grads(inp, (dq, dk, dv), ref, "padded")


def test_backward_is_deterministic():
    inp = make_inputs(workload("longformer_base"))
    dout_np = draw_dout(inp, 77)
    a = run_gpu_backward(inp, dout_np)
    b = run_gpu_backward(inp, dout_np)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
