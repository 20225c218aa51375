"""The tensor-level helpers on a side stream.

forward, backward, count_entries and decode launch on the stream the caller names.  Their
temporaries (workspace, zeroed counters, contiguous index copies) and outputs are allocated on
the current stream, so the helpers order the side stream after the current one and mark every
such tensor as used on the side stream.  Each call here is made on a side stream, the current
stream then allocates and fills memory of the same sizes while the side stream may still be
running, and the results must equal those of the same calls on the current stream bit for bit.
"""

import numpy as np
import pytest

import sparse_long_sequence_banded_amd as la
from workloads import draw_dout, random_case
from workloads.decode import decode_to_torch, make_decode_inputs
from workloads.torch_io import to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.load()
    yield


def _bits(t):
    import torch

    x = t.cpu()
    return x.view(torch.int16).numpy() if x.dtype == torch.bfloat16 else x.numpy()


def _churn(nbytes):
    """Allocate and overwrite memory on the current stream (reuse bait for freed blocks)."""
    import torch

    junk = [torch.full((max(nbytes // 4, 1),), 1e30, device="cuda:0") for _ in range(4)]
    return junk


def test_forward_backward_count_on_a_side_stream():
    import torch

    inp = random_case(61, batch=2, heads=3, n=3000, d=64, win_left=200, win_right=100,
                      dilations=[1, 2, 3], n_global=40, pad="random", pad_count=100)
    t = to_torch(inp, "cuda:0")
    # index tensors passed as non-contiguous views, so the helpers make contiguous copies
    gidx = torch.stack([t["global_idx"], t["global_idx"]], dim=2)[:, :, 0]
    assert not gidx.is_contiguous()
    kw = dict(scale=inp.scale, win_left=inp.win_left, win_right=inp.win_right,
              dilation=inp.dilation, global_idx=gidx, key_pad=t["key_pad"])
    dout = torch.from_numpy(draw_dout(inp, 62).view(np.int16)).view(torch.bfloat16).to("cuda:0")

    out0, lse0 = la.forward(t["q"], t["k"], t["v"], **kw)
    g0 = la.backward(t["q"], t["k"], t["v"], out0, lse0, dout, **kw)
    e0 = la.count_entries(t["q"], **{k: v for k, v in kw.items() if k != "scale"})
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    out1, lse1 = la.forward(t["q"], t["k"], t["v"], stream=side, **kw)
    junk = _churn(out1.numel() * 2)
    g1 = la.backward(t["q"], t["k"], t["v"], out1, lse1, dout, stream=side, **kw)
    junk += _churn(out1.numel() * 6)
    e1 = la.count_entries(t["q"], stream=side, **{k: v for k, v in kw.items() if k != "scale"})
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    assert e1 == e0
    assert np.array_equal(_bits(out1), _bits(out0))
    assert np.array_equal(_bits(lse1), _bits(lse0))
    for a, b in zip(g1, g0):
        assert np.array_equal(_bits(a), _bits(b))


def test_decode_on_a_side_stream():
    import torch

    inp = make_decode_inputs(63, batch=3, heads=2, d=128, dtype="bf16", window=512, m=2,
                             cache_len=1500, ring=False, positions=[10, 600, 1400])
    t = decode_to_torch(inp, "cuda:0")
    kw = dict(window=inp.window, scale=inp.scale, ring=inp.ring)
    o0, l0 = la.decode(t["q"], t["k_cache"], t["v_cache"], t["positions"], **kw)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    o1, l1 = la.decode(t["q"], t["k_cache"], t["v_cache"], t["positions"], stream=side, **kw)
    junk = _churn(1 << 20)
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    assert np.array_equal(_bits(o1), _bits(o0))
    assert np.array_equal(_bits(l1), _bits(l0))
