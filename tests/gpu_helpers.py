"""Shared helpers of the GPU parity tests: run the HIP path on seeded inputs and compare it
with the fp64 oracle."""

import numpy as np

import oracle
import sparse_long_sequence_banded_amd as la
from workloads.torch_io import to_torch

# Tolerances.  max-abs 2e-2 (bf16 I/O, fp32 accumulate) and 1e-4 (fp32) are the stated bars.
# The tighter internal gates follow from the arithmetic: the bf16 kernels multiply the value rows
# by softmax weights rounded to bf16 (round to nearest: relative error at most 2^-8 each) and
# divide by the sum of those rounded weights, then round the output to bf16, so the relative RMS
# error of a bf16 output stays well under 1e-2.  lse = ref + log2 of that same sum: its error is
# at most ln(1 + 2^-8) = 3.9e-3 (reached when one key dominates a row), hence 4e-3.
BF16_MAX_ABS = 2e-2
BF16_REL_RMS = 1e-2
F32_MAX_ABS = 1e-4
LSE_ABS = {"bf16": 4e-3, "f32": 1e-4}


def run_gpu(inp, device="cuda:0", want_lse=True):
    import torch

    t = to_torch(inp, device)
    out, lse = la.forward(t["q"], t["k"], t["v"], scale=inp.scale, win_left=inp.win_left,
                          win_right=inp.win_right, dilation=inp.dilation,
                          global_idx=t["global_idx"], key_pad=t["key_pad"],
                          block_layout=t["layout"], block=inp.block, want_lse=want_lse)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    l = None if lse is None else lse.cpu().numpy().astype(np.float64)
    return o, l, out


def gpu_count(inp, device="cuda:0"):
    t = to_torch(inp, device)
    E, _ = la.count_entries(t["q"], win_left=inp.win_left, win_right=inp.win_right,
                            dilation=inp.dilation, global_idx=t["global_idx"],
                            key_pad=t["key_pad"], block_layout=t["layout"], block=inp.block)
    return E


def heads_subset(inp, heads):
    return inp.select_heads(heads)


def compare(inp, o, l, ref_o, ref_l, label=""):
    """Element-by-element comparison with the oracle at the dtype's tolerance."""
    assert o.shape == ref_o.shape, (o.shape, ref_o.shape)
    err = np.abs(o - ref_o)
    max_abs = float(err.max()) if err.size else 0.0
    if inp.dtype == "bf16":
        assert max_abs <= BF16_MAX_ABS, f"{label}: max-abs {max_abs:.3e}"
        denom = float(np.sqrt(np.mean(ref_o ** 2))) if ref_o.size else 0.0
        if denom > 0:
            rel_rms = float(np.sqrt(np.mean(err ** 2))) / denom
            assert rel_rms <= BF16_REL_RMS, f"{label}: rel-RMS {rel_rms:.3e}"
    else:
        assert max_abs <= F32_MAX_ABS, f"{label}: max-abs {max_abs:.3e}"
    if l is not None:
        fin = np.isfinite(ref_l)
        assert np.array_equal(np.isfinite(l), fin), f"{label}: lse finiteness differs"
        assert np.all(l[~fin] == ref_l[~fin]), f"{label}: empty rows must have lse = -inf"
        if fin.any():
            lerr = float(np.abs(l[fin] - ref_l[fin]).max())
            assert lerr <= LSE_ABS[inp.dtype], f"{label}: lse error {lerr:.3e}"
    return max_abs


def parity(inp, label="", nthreads=0):
    ref_o, ref_l, E = oracle.forward_inputs(inp, nthreads=nthreads)
    o, l, _ = run_gpu(inp)
    return compare(inp, o, l, ref_o, ref_l, label), E
