"""Pins for the oracle's output gates (CPU only): sigmoid closed forms, torch's sigmoid and
matrix products on the token-major layout, and special weights whose effect is known."""

import numpy as np
import pytest
import torch

import oracle


def test_elementwise_gate_closed_forms_and_torch():
    rng = np.random.default_rng(1)
    o = rng.standard_normal((2, 3, 17, 8))
    assert np.allclose(oracle.gate_elementwise(o, np.zeros_like(o)), o / 2, rtol=0, atol=0)
    big = np.full_like(o, 800.0)
    assert np.array_equal(oracle.gate_elementwise(o, big), o)           # sigmoid(800) = 1
    assert np.all(oracle.gate_elementwise(o, -big) == 0)                # sigmoid(-800) = 0
    g = rng.standard_normal(o.shape) * 3
    ref = torch.from_numpy(o) * torch.sigmoid(torch.from_numpy(g))
    np.testing.assert_allclose(oracle.gate_elementwise(o, g), ref.numpy(), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("B,H,n,d,r", [(1, 2, 5, 4, 3), (2, 3, 9, 8, 16), (1, 1, 1, 64, 128)])
def test_lowrank_gate_matches_token_major_products(B, H, n, d, r):
    rng = np.random.default_rng(B * 100 + r)
    o = rng.standard_normal((B, H, n, d))
    wd = rng.standard_normal((r, H * d)) / np.sqrt(H * d)
    wu = rng.standard_normal((H * d, r)) / np.sqrt(r)
    tok = torch.from_numpy(o).permute(0, 2, 1, 3).reshape(B, n, H * d)  # head-major per token
    g = torch.sigmoid(tok @ torch.from_numpy(wd).T @ torch.from_numpy(wu).T)
    ref = (tok * g).reshape(B, n, H, d).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(oracle.gate_lowrank(o, wd, wu), ref, rtol=1e-12, atol=1e-13)


def test_lowrank_gate_special_weights():
    rng = np.random.default_rng(3)
    o = rng.standard_normal((1, 2, 6, 4))
    hd = 8
    # zero down-projection: every gate is sigmoid(0) = 1/2
    np.testing.assert_array_equal(oracle.gate_lowrank(o, np.zeros((5, hd)), rng.standard_normal((hd, 5))), o / 2)
    # identity through a full-rank bottleneck: gate = sigmoid(o) itself
    eye = np.eye(hd)
    tok = o.transpose(0, 2, 1, 3).reshape(1, 6, hd)
    ref = (tok / (1 + np.exp(-tok))).reshape(1, 6, 2, 4).transpose(0, 2, 1, 3)
    np.testing.assert_allclose(oracle.gate_lowrank(o, eye, eye), ref, rtol=1e-14, atol=1e-15)
