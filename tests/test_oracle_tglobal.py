"""Pins for the oracle's LongT5 Transient-Global attention (CPU only).

Each test ties the oracle to something other than its own code: an exact integer statement of
the bucket rule, numpy brute force of the aggregation / RMS norm / projections and of the
attention with explicit bias matrices, torch attention over concatenated keys, softmax shift
invariance, and the entry count's closed form.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads.tglobal import make_tglobal_inputs


def bucket_exact(rel, nb, md):
    """The bucket rule with integers only: beyond the exact range, the offset is the largest m
    with (a / e)^(h - e) >= (md / e)^m, i.e. a^(h-e) * e^m >= e^(h-e) * md^m."""
    h = nb // 2
    base = h if rel > 0 else 0
    a = abs(rel)
    e = h // 2
    if a < e:
        return base + a
    m = 0
    while m + 1 <= h - e - 1 and a ** (h - e) * e ** (m + 1) >= e ** (h - e) * md ** (m + 1):
        m += 1
    return base + e + m


@pytest.mark.parametrize("nb,md", [(32, 128), (16, 64), (64, 256), (32, 32)])
def test_bucket_matches_integer_statement(nb, md):
    for rel in range(-3 * md, 3 * md + 1):
        assert oracle.t5_bucket(rel, nb, md) == bucket_exact(rel, nb, md), rel


def test_bucket_shape_of_the_rule():
    # exact buckets near zero, one half per direction, saturation at max_distance
    assert [oracle.t5_bucket(-r) for r in range(0, 8)] == list(range(0, 8))  # key at/before
    assert [oracle.t5_bucket(r) for r in range(1, 8)] == list(range(17, 24))
    assert oracle.t5_bucket(128) == oracle.t5_bucket(10 ** 6) == 31
    assert oracle.t5_bucket(-128) == oracle.t5_bucket(-10 ** 6) == 15
    vals = [oracle.t5_bucket(r) for r in range(1, 200)]
    assert all(x <= y for x, y in zip(vals, vals[1:]))  # monotone in the distance
    neg = [oracle.t5_bucket(-r) for r in range(0, 200)]
    assert all(x <= y for x, y in zip(neg, neg[1:]))


def _case(seed, **kw):
    base = dict(batch=2, heads=2, n=70, d=8, d_model=12, radius=5, block=8, dtype="f32",
                pad_tail=(0, 13))
    base.update(kw)
    return make_tglobal_inputs(seed, **base)


def _side_brute(inp):
    B, n, dm = inp.x.shape
    x = inp.f64("x")
    G = max(1, n // inp.block)
    blk = np.minimum(np.arange(n) // inp.block, G - 1)
    pad = np.zeros((B, n), bool) if inp.key_pad is None else inp.key_pad.astype(bool)
    S = np.zeros((B, G, dm))
    valid = np.zeros((B, G), np.uint8)
    for b in range(B):
        for g in range(G):
            sel = (blk == g) & ~pad[b]
            S[b, g] = x[b, sel].sum(axis=0)
            valid[b, g] = sel.any()
    y = S / np.sqrt((S ** 2).mean(axis=-1, keepdims=True) + inp.eps) * inp.gamma.astype(np.float64)
    wk, wv = inp.f64("wk"), inp.f64("wv")
    sk = (y @ wk).reshape(B, G, inp.heads, inp.d).transpose(0, 2, 1, 3)
    sv = (y @ wv).reshape(B, G, inp.heads, inp.d).transpose(0, 2, 1, 3)
    return sk, sv, valid


@pytest.mark.parametrize("n,block", [(70, 8), (64, 16), (5, 16), (33, 16)])
def test_side_tokens_match_brute_force(n, block):
    inp = _case(3, n=n, block=block, pad_tail=(0, min(13, n - 1)))
    sk, sv, valid = oracle.tglobal_side(inp.f64("x"), inp.gamma, inp.f64("wk"), inp.f64("wv"),
                                        heads=inp.heads, d=inp.d, block=inp.block, eps=inp.eps,
                                        key_pad=inp.key_pad)
    bk, bv, bval = _side_brute(inp)
    np.testing.assert_allclose(sk, bk, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sv, bv, rtol=1e-12, atol=1e-12)
    assert np.array_equal(valid, bval)


def test_rms_norm_gives_unit_rms_and_the_tail_block_merges():
    inp = _case(4, n=45, block=16, pad_tail=(), d_model=16, heads=1, d=16)
    inp.gamma[:] = 1.0
    inp.wk[:] = 0
    # identity projection: side keys are the normalised aggregates themselves
    ident = np.eye(16, dtype=np.float32)
    sk, _, valid = oracle.tglobal_side(inp.f64("x"), inp.gamma, ident, ident, heads=1, d=16,
                                       block=16, eps=0.0)
    assert sk.shape[2] == 2  # 45 tokens: blocks 0..15, 16..44 (the 13-token tail merges)
    np.testing.assert_allclose(np.sqrt((sk ** 2).mean(axis=-1)), 1.0, rtol=1e-12)
    x = inp.f64("x")
    s1 = x[:, 16:45].sum(axis=1)
    np.testing.assert_allclose(sk[:, 0, 1], s1 / np.sqrt((s1 ** 2).mean(-1, keepdims=True)),
                               rtol=1e-12)
    assert valid.all()


def _forward_brute(inp, sk, sv, valid):
    """Dense scores over [local keys ; global tokens] with explicit bias matrices."""
    B, H, n, d = inp.q.shape
    q, k, v = inp.f64("q"), inp.f64("k"), inp.f64("v")
    G = sk.shape[2]
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    rel_l = j - i
    blk = np.minimum(np.arange(n) // inp.block, G - 1)
    rel_s = np.arange(G)[None, :] - blk[:, None]
    bfun = np.vectorize(lambda r: bucket_exact(int(r), inp.num_buckets, inp.max_distance))
    bl_idx, bs_idx = bfun(rel_l), bfun(rel_s)
    pad = np.zeros((B, n), bool) if inp.key_pad is None else inp.key_pad.astype(bool)
    out = np.zeros((B, H, n, d))
    lse = np.zeros((B, H, n))
    for b in range(B):
        for h in range(H):
            Sl = inp.scale * q[b, h] @ k[b, h].T + inp.bias_local.astype(np.float64)[bl_idx, h]
            Ss = inp.scale * q[b, h] @ sk[b, h].T + inp.bias_side.astype(np.float64)[bs_idx, h]
            Ml = (np.abs(rel_l) <= inp.radius) & ~pad[b][None, :]
            Ms = np.broadcast_to(valid[b].astype(bool)[None, :], Ss.shape)
            S = np.concatenate([np.where(Ml, Sl, -np.inf), np.where(Ms, Ss, -np.inf)], axis=1)
            Vc = np.concatenate([v[b, h], sv[b, h]], axis=0)
            m = S.max(axis=1, keepdims=True)
            P = np.exp(S - m)
            out[b, h] = P @ Vc / P.sum(axis=1, keepdims=True)
            lse[b, h] = m[:, 0] + np.log(P.sum(axis=1))
    return out, lse


@pytest.mark.parametrize("kw", [dict(), dict(radius=0), dict(radius=100), dict(n=33, block=16),
                                dict(pad_tail=(5, 40)), dict(n=64, block=4, radius=9)])
def test_forward_matches_dense_brute_force(kw):
    inp = _case(5, **kw)
    out, lse, E, sk, sv, valid = oracle.tglobal_inputs(inp)
    bo, bl = _forward_brute(inp, sk, sv, valid)
    np.testing.assert_allclose(out, bo, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-12)


def test_without_bias_and_with_a_full_window_it_is_attention_over_concatenated_keys():
    inp = _case(6, n=40, radius=40, pad_tail=())
    inp.bias_local[:] = 0
    inp.bias_side[:] = 0
    out, lse, _, sk, sv, _ = oracle.tglobal_inputs(inp)
    q = torch.from_numpy(inp.f64("q"))
    kc = torch.cat([torch.from_numpy(inp.f64("k")), torch.from_numpy(sk)], dim=2)
    vc = torch.cat([torch.from_numpy(inp.f64("v")), torch.from_numpy(sv)], dim=2)
    ref = torch.nn.functional.scaled_dot_product_attention(q, kc, vc, scale=inp.scale)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-10, atol=1e-12)
    S = torch.matmul(q, kc.transpose(-1, -2)) * inp.scale
    np.testing.assert_allclose(lse, torch.logsumexp(S, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


def test_equal_constant_bias_tables_change_nothing_but_lse():
    inp = _case(7)
    out0, lse0, *_ = oracle.tglobal_inputs(inp)
    inp.bias_local[:] = 0.75
    inp.bias_side[:] = 0.75
    out1, lse1, *_ = oracle.tglobal_inputs(inp)
    inp.bias_local[:] = 0.0
    inp.bias_side[:] = 0.0
    out2, lse2, *_ = oracle.tglobal_inputs(inp)
    np.testing.assert_allclose(out1, out2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse1, lse2 + 0.75, rtol=1e-12, atol=1e-12)
    assert np.abs(out0 - out2).max() > 1e-3  # the random tables do matter


@pytest.mark.parametrize("n,r,k", [(16384, 127, 16), (1000, 127, 16), (300, 5, 8), (50, 60, 16)])
def test_entry_count_closed_form(n, r, k):
    """Without padding: each row sees min(n-1, i+r) - max(0, i-r) + 1 local keys and every one
    of the G = max(1, n // k) global tokens; the sum is n(2r+1) - r(r+1) + nG for r < n, the
    guide's O(l (r + l/k))."""
    inp = make_tglobal_inputs(8, batch=1, heads=1, n=n, d=4, d_model=4, radius=r, block=k,
                              dtype="f32")
    G = max(1, n // k)
    sk = np.zeros((1, 1, G, 4))
    _, _, E = oracle.tglobal_forward(inp.f64("q"), inp.f64("k"), inp.f64("v"), sk, sk,
                                     np.ones((1, G), np.uint8), radius=r, block=k,
                                     num_buckets=32, max_distance=128, scale=0.5,
                                     bias_local=inp.bias_local, bias_side=inp.bias_side)
    rr = min(r, n - 1)
    assert E == n * (2 * rr + 1) - rr * (rr + 1) + n * G
