"""Pins for the fp64 oracle (CPU only).

Each test ties the oracle to something other than itself: the independent dense brute force,
the library's dense attention, the worked example the Big Bird notes print, closed-form counts
and exact special cases.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from tests.dense_ref import dense_attention, dense_mask
from workloads import bigbird_layout, random_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _oracle(inp, **kw):
    return oracle.forward_inputs(inp, **kw)


def _dense(inp):
    M = dense_mask(inp.batch, inp.heads, inp.n, win_left=inp.win_left, win_right=inp.win_right,
                   dilation=inp.dilation, global_idx=inp.global_idx, key_pad=inp.key_pad,
                   layout=inp.layout, block=inp.block)
    out, lse = dense_attention(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.scale, M)
    return out, lse, int(M.sum())


def _close(a, b, rtol=1e-12, atol=1e-12):
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin)
    assert np.array_equal(a[~fin], b[~fin])
    np.testing.assert_allclose(a[fin], b[fin], rtol=rtol, atol=atol)


# ------------------------------------------------------------------------------ p1 brute force
CASES = []
_rng = np.random.default_rng(1234)
for _t in range(40):
    n = int(_rng.choice([1, 2, 3, 7, 16, 33, 64, 130]))
    d = int(_rng.choice([1, 3, 8, 16]))
    band = _rng.random() < 0.85
    wl = int(_rng.integers(0, n + 2)) if band else -1
    wr = int(_rng.integers(0, n + 2)) if band else -1
    if band and _rng.random() < 0.2:
        wr = 0
    H = int(_rng.integers(1, 4))
    dil = [int(x) for x in _rng.integers(1, 4, size=H)] if _rng.random() < 0.5 else None
    g = int(_rng.integers(0, min(n, 5) + 1)) if _rng.random() < 0.6 else 0
    pad = str(_rng.choice(["none", "tail", "random"]))
    pc = int(_rng.integers(0, n + 1))
    blk = 0
    mkb = 0
    if n % 4 == 0 and n >= 8 and _rng.random() < 0.4:
        blk = int(_rng.choice([b for b in (4, 8, 16) if n % b == 0]))
        mkb = int(_rng.integers(1, 4))
    CASES.append(dict(seed=100 + _t, batch=int(_rng.integers(1, 3)), heads=H, n=n, d=d,
                      win_left=wl, win_right=wr, dilations=dil, n_global=g, pad=pad,
                      pad_count=pc, block=blk, max_kb=mkb, dtype="f32"))


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_oracle_matches_dense_brute_force(case):
    inp = random_case(**case)
    out, lse, E = _oracle(inp)
    dout, dlse, dE = _dense(inp)
    assert E == dE
    _close(out, dout)
    _close(lse, dlse)


def test_oracle_thread_count_does_not_change_result():
    inp = random_case(7, batch=2, heads=3, n=130, d=8, win_left=5, win_right=9, dilations=[1, 2, 3],
                      n_global=4, pad="random", pad_count=10)
    a = _oracle(inp, nthreads=1)
    b = _oracle(inp, nthreads=7)
    assert a[2] == b[2]
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------------------------ p2 library
@pytest.mark.parametrize("n,d", [(1, 4), (37, 8), (128, 16)])
def test_window_covering_sequence_is_full_attention(n, d):
    inp = random_case(11, batch=2, heads=2, n=n, d=d, dtype="f32", win_left=n, win_right=n + 5)
    out, lse, E = _oracle(inp)
    q, k, v = (torch.from_numpy(inp.f64(x)) for x in "qkv")
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=inp.scale)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)
    S = torch.einsum("bhid,bhjd->bhij", q, k) * inp.scale
    np.testing.assert_allclose(lse, torch.logsumexp(S, dim=-1).numpy(), rtol=1e-12, atol=1e-12)
    assert E == 2 * 2 * n * n


@pytest.mark.parametrize("n", [1, 50, 129])
def test_causal_window_covering_sequence_is_causal_attention(n):
    inp = random_case(12, batch=1, heads=3, n=n, d=8, dtype="f32", win_left=n - 1, win_right=0)
    out, _, E = _oracle(inp)
    q, k, v = (torch.from_numpy(inp.f64(x)) for x in "qkv")
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=inp.scale,
                                                           is_causal=True)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)
    assert E == 3 * n * (n + 1) // 2


def test_layout_listing_every_block_is_full_attention():
    n, blk = 64, 8
    nb = n // blk
    inp = random_case(13, batch=1, heads=2, n=n, d=8, dtype="f32")
    inp.layout = np.broadcast_to(np.arange(nb, dtype=np.int32), (2, nb, nb)).copy()
    inp.block, inp.max_kb = blk, nb
    out, _, E = _oracle(inp)
    q, k, v = (torch.from_numpy(inp.f64(x)) for x in "qkv")
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=inp.scale)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)
    assert E == 2 * n * n


# ------------------------------------------------------------------------------ p3 rows sum to 1
def test_softmax_rows_sum_to_one():
    inp = random_case(14, batch=2, heads=2, n=96, d=16, dtype="f32", win_left=7, win_right=3,
                      dilations=[1, 3], n_global=3, pad="random", pad_count=9)
    _, lse, _ = _oracle(inp)
    q, k = inp.f64("q"), inp.f64("k")
    for b in range(2):
        for h in range(2):
            for i in range(0, 96, 5):
                S = oracle.row_set(2, 2, 96, b, h, i, win_left=7, win_right=3,
                                   dilation=inp.dilation, global_idx=inp.global_idx,
                                   key_pad=inp.key_pad)
                s = inp.scale * (k[b, h, S] @ q[b, h, i])
                assert abs(np.exp(s - lse[b, h, i]).sum() - 1.0) < 1e-12


# ------------------------------------------------------------------------------ p4 masked keys
def test_keys_outside_the_set_contribute_exactly_zero():
    n = 80
    inp = random_case(15, batch=1, heads=2, n=n, d=8, dtype="f32", win_left=4, win_right=6,
                      dilations=[1, 2], n_global=2, pad="random", pad_count=12, block=8,
                      max_kb=2, layout_fill=0.7)
    out, lse, _ = _oracle(inp)
    for poison in (1e30, np.nan):
        for h in range(2):
            for i in (0, 17, 40, 79):
                S = oracle.row_set(1, 2, n, 0, h, i, win_left=4, win_right=6,
                                   dilation=inp.dilation, global_idx=inp.global_idx,
                                   key_pad=inp.key_pad, layout=inp.layout, block=8, max_kb=2)
                outside = np.setdiff1d(np.arange(n), S)
                k = inp.f64("k").copy()
                v = inp.f64("v").copy()
                k[0, h, outside] = poison
                v[0, h, outside] = poison
                o2, l2, _ = oracle.forward(inp.f64("q"), k, v, scale=inp.scale, win_left=4,
                                           win_right=6, dilation=inp.dilation,
                                           global_idx=inp.global_idx, key_pad=inp.key_pad,
                                           layout=inp.layout, block=8, max_kb=2)
                assert np.array_equal(o2[0, h, i], out[0, h, i])
                assert l2[0, h, i] == lse[0, h, i]


# ------------------------------------------------------------------------------ p5 worked example
def test_bigbird_worked_window_example():
    fx = json.load(open(os.path.join(GOLDEN, "bigbird_window_w6.json")))
    n, w = fx["sequence_length"], fx["w"]
    S = oracle.row_set(1, 1, n, 0, 0, fx["query_1based"] - 1, win_left=w // 2, win_right=w // 2)
    assert [int(j) + 1 for j in S] == fx["keys_1based"]


# ------------------------------------------------------------------------------ p6 3-block context
def test_longt5_radius_fits_three_blocks():
    fx = json.load(open(os.path.join(GOLDEN, "longt5_three_block.json")))
    r, bl = fx["local_radius"], fx["block_len"]
    assert bl == r + 1
    n = 5 * bl + 17
    for i in range(0, n, 7):
        S = oracle.row_set(1, 1, n, 0, 0, i, win_left=r, win_right=r)
        blocks = set((S // bl).tolist())
        allowed = {i // bl + o for o in fx["context_blocks"]}
        assert blocks <= allowed
        ctx = np.array([j for j in range(n) if j // bl in allowed])
        assert np.array_equal(S, ctx[np.abs(ctx - i) <= r])


# ------------------------------------------------------------------------------ p7 window 0
def test_window_zero_returns_v_exactly():
    inp = random_case(16, batch=2, heads=3, n=77, d=8, dtype="f32", win_left=0, win_right=0,
                      dilations=[1, 2, 5])
    out, lse, E = _oracle(inp)
    assert np.array_equal(out, inp.f64("v"))
    s_ii = np.einsum("bhid,bhid->bhi", inp.f64("q"), inp.f64("k")) * inp.scale
    np.testing.assert_allclose(lse, s_ii, rtol=0, atol=1e-15)
    assert E == 2 * 3 * 77


# ------------------------------------------------------------------------------ p8 K = 0
def test_zero_keys_give_the_mean_of_values():
    inp = random_case(17, batch=1, heads=2, n=60, d=8, dtype="f32", win_left=3, win_right=5,
                      dilations=[1, 4], n_global=2, pad="random", pad_count=7)
    k0 = np.zeros_like(inp.f64("k"))
    out, lse, _ = oracle.forward(inp.f64("q"), k0, inp.f64("v"), scale=inp.scale, win_left=3,
                                 win_right=5, dilation=inp.dilation, global_idx=inp.global_idx,
                                 key_pad=inp.key_pad)
    v = inp.f64("v")
    for h in range(2):
        for i in range(60):
            S = oracle.row_set(1, 2, 60, 0, h, i, win_left=3, win_right=5, dilation=inp.dilation,
                               global_idx=inp.global_idx, key_pad=inp.key_pad)
            np.testing.assert_allclose(out[0, h, i], v[0, h, S].mean(axis=0), rtol=1e-13,
                                       atol=1e-15)
            assert abs(lse[0, h, i] - np.log(len(S))) < 1e-13


# ------------------------------------------------------------------------------ p9 closed forms
@pytest.mark.parametrize("n,wl,wr", [(1, 0, 0), (10, 3, 3), (100, 7, 2), (513, 256, 256),
                                     (4096, 256, 256), (4096, 0, 17), (1000, 999, 0)])
def test_band_count_closed_form(n, wl, wr):
    E = oracle.count(1, 1, n, win_left=wl, win_right=wr)
    assert n > max(wl, wr)
    assert E == n * (wl + wr + 1) - wl * (wl + 1) // 2 - wr * (wr + 1) // 2


@pytest.mark.parametrize("n,W", [(32768, 512), (1000, 1), (600, 512)])
def test_causal_window_count_is_n_times_w(n, W):
    """A causal window of W keys (keys i-W+1 .. i): E = n W - W (W - 1) / 2, i.e. O(n w)."""
    E = oracle.count(1, 1, n, win_left=W - 1, win_right=0)
    assert E == n * W - W * (W - 1) // 2


@pytest.mark.parametrize("n,dil,wl,wr", [(100, 2, 5, 5), (101, 3, 4, 9), (17, 5, 2, 1),
                                         (64, 2, 40, 0)])
def test_dilated_row_counts(n, dil, wl, wr):
    for i in range(n):
        S = oracle.row_set(1, 1, n, 0, 0, i, win_left=wl, win_right=wr,
                           dilation=np.array([dil], np.int32))
        assert len(S) == min(wl, i // dil) + min(wr, (n - 1 - i) // dil) + 1
        assert np.all((S - i) % dil == 0)
        assert S.min() >= i - dil * wl and S.max() <= i + dil * wr


def test_counts_match_dense_mask_sums():
    rng = np.random.default_rng(99)
    for t in range(300):
        n = int(rng.integers(1, 40))
        H = int(rng.integers(1, 3))
        wl, wr = (int(rng.integers(0, n + 1)), int(rng.integers(0, n + 1)))
        if rng.random() < 0.15:
            wl = wr = -1
        inp = random_case(1000 + t, batch=2, heads=H, n=n, d=1, dtype="f32", win_left=wl,
                          win_right=wr, dilations=[int(x) for x in rng.integers(1, 4, size=H)],
                          n_global=int(rng.integers(0, min(n, 4) + 1)), pad="random",
                          pad_count=int(rng.integers(0, n + 1)))
        M = dense_mask(2, H, n, win_left=wl, win_right=wr, dilation=inp.dilation,
                       global_idx=inp.global_idx, key_pad=inp.key_pad)
        assert oracle.count_inputs(inp) == int(M.sum())


def test_transient_global_cost_law():
    """Band of radius r plus n/k evenly spaced global tokens costs Theta(n (r + n/k))."""
    r, k = 127, 16
    ratios = []
    for n in (1024, 4096, 16384):
        g = n // k
        gi = (np.arange(g, dtype=np.int32) * k)[None]
        E = oracle.count(1, 1, n, win_left=r, win_right=r, global_idx=gi)
        ratios.append(E / (n * (2 * r + 1) + 2 * n * n / k))
    assert all(0.85 < x <= 1.0 for x in ratios)
    assert ratios == sorted(ratios)


def test_page_full_attention_count():
    fx = json.load(open(os.path.join(GOLDEN, "longformer_full_count.json")))
    n = fx["n"]
    E = oracle.count(1, 1, n, win_left=n - 1, win_right=n - 1)
    assert E == n * n
    assert abs(E - fx["printed_value"]) / E < fx["relative_tolerance"]


# ------------------------------------------------------------------------------ p10 residues
def test_dilated_band_is_independent_bands_on_residue_classes():
    n, dil, wl, wr = 103, 3, 4, 6
    inp = random_case(18, batch=1, heads=1, n=n, d=8, dtype="f32", win_left=wl, win_right=wr,
                      dilations=[dil])
    out, lse, _ = _oracle(inp)
    for p in range(dil):
        sub = [inp.f64(x)[:, :, p::dil] for x in "qkv"]
        o2, l2, _ = oracle.forward(*sub, scale=inp.scale, win_left=wl, win_right=wr)
        assert np.array_equal(o2, out[:, :, p::dil])
        assert np.array_equal(l2, lse[:, :, p::dil])


# ------------------------------------------------------------------------------ p11 translation
def test_interior_rows_are_translation_invariant():
    n, s, wl, wr = 120, 9, 5, 7
    inp = random_case(19, batch=1, heads=1, n=n + s, d=8, dtype="f32", win_left=wl, win_right=wr)
    q, k, v = (inp.f64(x) for x in "qkv")
    a, la, _ = oracle.forward(q[:, :, :n], k[:, :, :n], v[:, :, :n], scale=inp.scale,
                              win_left=wl, win_right=wr)
    b, lb, _ = oracle.forward(q[:, :, s:], k[:, :, s:], v[:, :, s:], scale=inp.scale,
                              win_left=wl, win_right=wr)
    # rows whose window is inside both sequences
    for i in range(s + wl, n - wr):
        assert np.array_equal(a[0, 0, i], b[0, 0, i - s])
        assert la[0, 0, i] == lb[0, 0, i - s]


# ------------------------------------------------------------------------------ p12 dual forms
def test_bigbird_global_blocks_as_layout_or_as_global_tokens():
    n, blk, H = 512, 32, 2
    nb = n // blk
    lay = bigbird_layout(H, n, blk, np.random.default_rng(5))
    inp = random_case(20, batch=2, heads=H, n=n, d=8, dtype="f32")
    gtok = np.concatenate([np.arange(blk), np.arange(n - blk, n)]).astype(np.int32)
    gi = np.stack([gtok, gtok])
    a, la, Ea = oracle.forward(inp.f64("q"), inp.f64("k"), inp.f64("v"), scale=inp.scale,
                               win_left=-1, win_right=-1, global_idx=gi, layout=lay, block=blk,
                               max_kb=lay.shape[2])
    # same pattern written only as a layout: global block rows list every block, every other
    # row also lists the two global blocks
    lay2 = np.full((H, nb, nb), -1, dtype=np.int32)
    for h in range(H):
        lay2[h, 0] = np.arange(nb)
        lay2[h, nb - 1] = np.arange(nb)
        for qb in range(1, nb - 1):
            row = sorted(set(int(x) for x in lay[h, qb] if x >= 0) | {0, nb - 1})
            lay2[h, qb, : len(row)] = row
    b, lb, Eb = oracle.forward(inp.f64("q"), inp.f64("k"), inp.f64("v"), scale=inp.scale,
                               win_left=-1, win_right=-1, layout=lay2, block=blk, max_kb=nb)
    assert Ea == Eb
    assert np.array_equal(a, b) and np.array_equal(la, lb)


# ------------------------------------------------------------------------------ semantics edges
def test_global_rows_attend_every_unpadded_key_and_padding_wins():
    n = 40
    inp = random_case(21, batch=1, heads=1, n=n, d=4, dtype="f32", win_left=2, win_right=2)
    gi = np.array([[3, 20]], np.int32)
    kp = np.zeros((1, n), np.uint8)
    kp[0, [20, 30, 31]] = 1  # a padded global position: not a key, still a global row
    S_g = oracle.row_set(1, 1, n, 0, 0, 20, win_left=2, win_right=2, global_idx=gi, key_pad=kp)
    assert np.array_equal(S_g, np.setdiff1d(np.arange(n), [20, 30, 31]))
    S_i = oracle.row_set(1, 1, n, 0, 0, 29, win_left=2, win_right=2, global_idx=gi, key_pad=kp)
    assert S_i.tolist() == [3, 27, 28, 29]
    S_b = oracle.row_set(1, 1, n, 0, 0, 4, win_left=2, win_right=2, global_idx=gi, key_pad=kp)
    assert S_b.tolist() == [2, 3, 4, 5, 6]  # global key 3 inside the band is counted once


def test_empty_rows_give_zero_output_and_minus_infinity_lse():
    n = 16
    inp = random_case(22, batch=1, heads=1, n=n, d=4, dtype="f32", win_left=1, win_right=1)
    kp = np.zeros((1, n), np.uint8)
    kp[0, 4:9] = 1
    out, lse, E = oracle.forward(inp.f64("q"), inp.f64("k"), inp.f64("v"), scale=inp.scale,
                                 win_left=1, win_right=1, key_pad=kp)
    for i in (5, 6, 7):
        assert np.all(out[0, 0, i] == 0.0) and lse[0, 0, i] == -np.inf
    assert np.all(np.isfinite(lse[0, 0, [0, 1, 2, 3, 10, 15]]))
    assert E == (n * 3 - 2) - 5 * 3  # each padded key drops out of the 3 rows that see it


def test_empty_problem():
    z = np.zeros((1, 1, 0, 4))
    out, lse, E = oracle.forward(z, z, z, scale=1.0, win_left=3, win_right=3)
    assert out.shape == (1, 1, 0, 4) and E == 0


@pytest.mark.parametrize("kw", [
    dict(win_left=-1, win_right=3),
    dict(win_left=2, win_right=-5),
    dict(win_left=1, win_right=1, dilation=np.array([0], np.int32)),
    dict(win_left=1, win_right=1, global_idx=np.array([[9]], np.int32)),
    dict(win_left=1, win_right=1, layout=np.array([[[0], [5]]], np.int32), block=4, max_kb=1),
])
def test_bad_arguments_are_rejected(kw):
    z = np.zeros((1, 1, 8, 2))
    with pytest.raises(ValueError):
        oracle.forward(z, z, z, scale=1.0, **kw)
