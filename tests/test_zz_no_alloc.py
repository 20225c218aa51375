"""The allocation-free forward entry point against the workspace one, through the C ABI.

longattn_forward_noalloc keeps the global rows' partials in the library's own device array and
otherwise runs the same kernels as longattn_forward, so its results must equal that entry
point's bit for bit (and therefore the oracle, which the other parity tests compare the
workspace entry point with).  Two calls in a row, the second with a smaller problem, so that the
second call runs over the first call's leftover partials.
"""

import ctypes
import sys

import numpy as np
import pytest

import oracle
import sparse_long_sequence_banded_amd as la
from tests.gpu_helpers import compare
from workloads import random_case
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


def _both(inp):
    """(workspace entry point, allocation-free entry point) outputs and lse of one problem."""
    import torch

    t = to_torch(inp, "cuda:0")
    desc, keep = la.make_desc(t["q"], scale=inp.scale, win_left=inp.win_left,
                              win_right=inp.win_right, dilation=inp.dilation,
                              global_idx=t["global_idx"], key_pad=t["key_pad"],
                              block_layout=t["layout"], block=inp.block)
    st, ws_bytes = la.longattn_workspace_size(desc)
    assert st == la.LONGATTN_OK and 0 < ws_bytes <= la.LONGATTN_NOALLOC_SCRATCH_BYTES
    stream = torch.cuda.current_stream().cuda_stream
    res = []
    for noalloc in (False, True):
        out = torch.empty_like(t["q"])
        lse = torch.empty(t["q"].shape[:3], dtype=torch.float32, device="cuda:0")
        if noalloc:
            st = la.longattn_forward_noalloc(desc, t["q"].data_ptr(), t["k"].data_ptr(),
                                             t["v"].data_ptr(), out.data_ptr(), lse.data_ptr(),
                                             stream)
        else:
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda:0")
            st = la.longattn_forward(desc, t["q"].data_ptr(), t["k"].data_ptr(),
                                     t["v"].data_ptr(), out.data_ptr(), lse.data_ptr(),
                                     ws.data_ptr(), ws_bytes, stream)
        assert st == la.LONGATTN_OK, la.longattn_status_string(st)
        torch.cuda.synchronize()
        res.append((out.cpu().view(torch.int16).numpy(), lse.cpu().numpy()))
    del keep
    return res, ws_bytes


def test_noalloc_matches_the_workspace_entry_point_twice_in_a_row():
    big = random_case(91, batch=2, heads=4, n=5000, d=64, win_left=256, win_right=256,
                      dilations=[1, 2, 1, 3], n_global=64, pad="tail", pad_count=300)
    small = random_case(92, batch=1, heads=2, n=900, d=128, win_left=100, win_right=0,
                        n_global=7)
    for label, inp in (("first, larger", big), ("second, smaller", small)):
        _note(f"[noalloc] {label}: B{inp.batch} H{inp.heads} n{inp.n} d{inp.d} g{inp.n_global}")
        ((o_ws, l_ws), (o_na, l_na)), ws_bytes = _both(inp)
        assert np.array_equal(o_ws, o_na), label
        assert np.array_equal(l_ws, l_na), label
        _note(f"[noalloc] {label}: bit-identical ({ws_bytes} bytes of scratch)")
    # the smaller call against the oracle as well
    ref_o, ref_l, _ = oracle.forward_inputs(small)
    o = (o_na.astype(np.int32) << 16).view(np.float32).astype(np.float64)
    compare(small, o, l_na.astype(np.float64), ref_o, ref_l, "noalloc")


def test_noalloc_rejects_problems_beyond_its_scratch():
    # 64 heads x 256 global rows x 32 chunks (of 512 keys) x 66 floats = 138 MB of partials,
    # beyond the 32 MiB scratch
    desc = la.longattn_desc(batch=1, heads=64, n=16384, d=64, dtype=la.LONGATTN_BF16,
                            scale=0.125, win_left=256, win_right=256, dilation=None,
                            global_idx=ctypes.c_void_p(256).value, n_global=256, key_pad=None,
                            block_layout=None, block=0, max_kb=0)
    st, ws = la.longattn_workspace_size(desc)
    assert st == la.LONGATTN_OK and ws > la.LONGATTN_NOALLOC_SCRATCH_BYTES
    assert la.longattn_forward_noalloc(desc, 256, 256, 256, 256, None, None) == \
        la.LONGATTN_ERR_WORKSPACE
