"""Pins for the oracle's backward pass (CPU only).

The gradients are tied to things other than the oracle's own formula: central finite
differences of the oracle's forward pass (which the forward pins tie to the pages), torch
autograd through a dense masked softmax attention, and two closed forms that follow from the
softmax (the key gradients of a head sum to zero; the value gradients sum to the output
gradients of the non-empty rows).
"""

import numpy as np
import pytest
import torch

import oracle
from tests.dense_ref import dense_mask
from workloads import random_case

SMALL = [
    dict(seed=900, batch=1, heads=2, n=11, d=3, win_left=2, win_right=1, dilations=[1, 2]),
    dict(seed=901, batch=2, heads=1, n=9, d=4, win_left=1, win_right=3, n_global=2,
         pad="tail", pad_count=3),
    dict(seed=902, batch=1, heads=2, n=12, d=2, win_left=3, win_right=0, dilations=[3, 1],
         n_global=1, pad="random", pad_count=4),
    dict(seed=903, batch=1, heads=1, n=12, d=3, block=4, max_kb=2, n_global=1),
    dict(seed=904, batch=2, heads=1, n=8, d=2, win_left=0, win_right=0, pad="random",
         pad_count=8),  # sample 2: every key padded, all its rows empty
]


def _loss_grad_fd(inp, dout, eps=1e-6):
    """Central differences of L = sum(dout * out) over every coordinate of q, k and v."""
    base = dict(q=inp.f64("q"), k=inp.f64("k"), v=inp.f64("v"))
    kw = dict(scale=inp.scale, win_left=inp.win_left, win_right=inp.win_right,
              dilation=inp.dilation, global_idx=inp.global_idx, key_pad=inp.key_pad,
              layout=inp.layout, block=inp.block, max_kb=inp.max_kb, nthreads=1)

    def L(arrs):
        out, _, _ = oracle.forward(arrs["q"], arrs["k"], arrs["v"], **kw)
        return float((dout * out).sum())

    grads = {}
    for name in ("q", "k", "v"):
        g = np.zeros_like(base[name])
        flat = g.reshape(-1)
        for idx in range(flat.size):
            arrs = {kk: vv.copy() for kk, vv in base.items()}
            arrs[name].reshape(-1)[idx] += eps
            up = L(arrs)
            arrs[name].reshape(-1)[idx] -= 2 * eps
            dn = L(arrs)
            flat[idx] = (up - dn) / (2 * eps)
        grads[name] = g
    return grads["q"], grads["k"], grads["v"]


def _dout(inp, seed):
    return np.random.default_rng(seed).standard_normal(inp.q.shape)


@pytest.mark.parametrize("case", SMALL, ids=[f"s{i}" for i in range(len(SMALL))])
def test_backward_matches_finite_differences_of_the_forward(case):
    inp = random_case(dtype="f32", **case)
    dout = _dout(inp, case["seed"])
    dq, dk, dv = oracle.backward_inputs(inp, dout)
    fq, fk, fv = _loss_grad_fd(inp, dout)
    for a, b in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-7)


BRUTE = []
_rng = np.random.default_rng(77)
for _t in range(16):
    n = int(_rng.choice([1, 5, 16, 33, 64]))
    H = int(_rng.integers(1, 3))
    band = _rng.random() < 0.85
    blk = 0
    if n % 8 == 0 and n >= 16 and _rng.random() < 0.3:
        blk = 8
    BRUTE.append(dict(
        seed=950 + _t, batch=int(_rng.integers(1, 3)), heads=H, n=n,
        d=int(_rng.choice([1, 4, 8])),
        win_left=int(_rng.integers(0, n + 1)) if band else -1,
        win_right=int(_rng.integers(0, n + 1)) if band else -1,
        dilations=[int(x) for x in _rng.integers(1, 4, size=H)] if _rng.random() < 0.5 else None,
        n_global=int(_rng.integers(0, min(n, 4) + 1)) if _rng.random() < 0.6 else 0,
        pad=str(_rng.choice(["none", "tail", "random"])), pad_count=int(_rng.integers(0, n + 1)),
        block=blk, max_kb=2 if blk else 0))


@pytest.mark.parametrize("case", BRUTE, ids=[f"b{i}" for i in range(len(BRUTE))])
def test_backward_matches_autograd_of_dense_masked_attention(case):
    inp = random_case(dtype="f32", **case)
    dout = _dout(inp, case["seed"])
    M = torch.from_numpy(dense_mask(inp.batch, inp.heads, inp.n, win_left=inp.win_left,
                                    win_right=inp.win_right, dilation=inp.dilation,
                                    global_idx=inp.global_idx, key_pad=inp.key_pad,
                                    layout=inp.layout, block=inp.block))
    q, k, v = (torch.tensor(inp.f64(x), requires_grad=True) for x in ("q", "k", "v"))
    S = torch.matmul(q, k.transpose(-1, -2).contiguous()) * inp.scale
    S = S.masked_fill(~M, float("-inf"))
    empty = ~M.any(dim=-1, keepdim=True)
    P = torch.softmax(S.masked_fill(empty, 0.0), dim=-1).masked_fill(empty, 0.0)
    out = torch.matmul(P, v)
    (out * torch.from_numpy(dout)).sum().backward()
    dq, dk, dv = oracle.backward_inputs(inp, dout)
    for a, b in ((dq, q.grad), (dk, k.grad), (dv, v.grad)):
        np.testing.assert_allclose(a, b.numpy(), rtol=1e-10, atol=1e-12)


def test_key_gradients_sum_to_zero_and_value_gradients_to_the_output_gradients():
    inp = random_case(960, batch=2, heads=3, n=300, d=16, win_left=20, win_right=7,
                      dilations=[1, 2, 5], n_global=4, pad="random", pad_count=30)
    dout = _dout(inp, 960)
    dq, dk, dv = oracle.backward_inputs(inp, dout)
    # every row's softmax weights sum to 1 and its dS sum to 0 (no row is empty here)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-10)
    np.testing.assert_allclose(dv.sum(axis=2), dout.sum(axis=2), rtol=1e-12, atol=1e-10)
    assert np.abs(dq).max() > 1e-3 and np.abs(dk).max() > 1e-3


def test_window_zero_passes_the_gradient_to_v_only():
    inp = random_case(961, batch=1, heads=2, n=50, d=8, win_left=0, win_right=0,
                      dilations=[1, 3])
    dout = _dout(inp, 961)
    dq, dk, dv = oracle.backward_inputs(inp, dout)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_array_equal(dv, dout)


def test_backward_thread_count_does_not_change_result():
    inp = random_case(962, batch=2, heads=3, n=200, d=8, win_left=9, win_right=9, n_global=3)
    dout = _dout(inp, 962)
    a = oracle.backward_inputs(inp, dout, nthreads=1)
    b = oracle.backward_inputs(inp, dout, nthreads=5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
