"""GPU parity of the output gates of gated attention against the fp64 oracle: the elementwise
gate fused into the forward pass (oracle: forward, then gate) and the low-rank gate on given
outputs.  Tolerance |gpu - oracle| <= 2e-2 + 1e-2 |oracle| (bf16 outputs), 1e-4 + 1e-4 |oracle|
(fp32); the gate multiplies by a value in (0, 1), so the attention's own bar carries over."""

import sys

import numpy as np
import pytest

import oracle
import sparse_long_sequence_banded_amd as la
from workloads import make_inputs, random_case, widen, workload
from workloads.gates import gate_logits, lowrank_inputs
from workloads.torch_io import to_torch

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


def _dev(a, dtype):
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")


def _close(got, ref, dtype, label):
    atol, rtol = (2e-2, 1e-2) if dtype == "bf16" else (1e-4, 1e-4)
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    assert not bad.any(), f"{label}: {int(bad.sum())} out of tolerance, max-abs {err.max():.3e}"
    return float(err.max())


@pytest.mark.parametrize("name", ["tiny_f32", "longformer_base", "bigbird_itc"])
def test_forward_with_elementwise_gate(name):
    import torch

    inp = make_inputs(workload(name))
    g = gate_logits(inp.q.shape, 500, inp.dtype)
    t = to_torch(inp, "cuda:0")
    out, _ = la.forward(t["q"], t["k"], t["v"], scale=inp.scale, win_left=inp.win_left,
                        win_right=inp.win_right, dilation=inp.dilation,
                        global_idx=t["global_idx"], key_pad=t["key_pad"],
                        block_layout=t["layout"], block=inp.block, gate=_dev(g, inp.dtype))
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref_o, _, _ = oracle.forward_inputs(inp)
    ref = oracle.gate_elementwise(ref_o, widen(g, inp.dtype))
    e = _close(got, ref, inp.dtype, name)
    _note(f"[gate] {name}: max-abs {e:.3e}")


def test_gated_forward_equals_gate_of_plain_forward_bits():
    """With logits of +40 every gate is 1 in fp32: the gated output equals the plain one."""
    import torch

    inp = make_inputs(workload("longformer_base"))
    t = to_torch(inp, "cuda:0")
    kw = dict(scale=inp.scale, win_left=inp.win_left, win_right=inp.win_right,
              global_idx=t["global_idx"], key_pad=t["key_pad"])
    plain, _ = la.forward(t["q"], t["k"], t["v"], **kw)
    ones = torch.full_like(t["q"], 40.0)
    gated, _ = la.forward(t["q"], t["k"], t["v"], gate=ones, **kw)
    torch.cuda.synchronize()
    assert (plain.view(torch.int16) == gated.view(torch.int16)).all()


# H*d a multiple of 128 up to 1024 with r <= 128 takes the split kernel (one wave per 128
# outputs: 1, 2, 3, 4, 6 and 8 waves below), the rest the general one (r = 256; H*d = 32, 480,
# 1280 or 2048)
@pytest.mark.parametrize("B,H,n,d,r", [(2, 12, 300, 64, 128), (1, 16, 1000, 64, 128),
                                       (1, 8, 50, 128, 32), (1, 4, 77, 64, 256),
                                       (2, 2, 33, 16, 64), (1, 2, 65, 128, 64),
                                       (1, 8, 257, 64, 64), (2, 20, 40, 64, 32),
                                       (1, 16, 300, 128, 128), (1, 6, 70, 80, 128),
                                       (2, 2, 90, 64, 32), (1, 6, 100, 64, 64),
                                       (1, 16, 16384, 64, 128)])
def test_lowrank_gate(B, H, n, d, r):
    import torch

    o, wd, wu = lowrank_inputs(600 + r + n, batch=B, heads=H, n=n, d=d, rank=r)
    out = _dev(o, "bf16")
    la.gate_lowrank(out, _dev(wd, "bf16"), _dev(wu, "bf16"))
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref = oracle.gate_lowrank(widen(o, "bf16"), widen(wd, "bf16"), widen(wu, "bf16"))
    e = _close(got, ref, "bf16", f"lowrank {B, H, n, d, r}")
    _note(f"[gate] lowrank {B, H, n, d, r}: max-abs {e:.3e}")
