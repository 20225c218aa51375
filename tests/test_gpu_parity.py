"""GPU parity: the HIP library against the fp64 oracle on the same seeded inputs.

Every test here calls the C-ABI library through the Python binding and needs an MI355X.
"""

import os
import sys

import numpy as np
import pytest

import oracle
import sparse_long_sequence_banded_amd as la
from tests.gpu_helpers import compare, gpu_count, heads_subset, parity, run_gpu
from workloads import make_inputs, random_case, round_to_bf16_bits, workload
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


# ------------------------------------------------------------------------------ named workloads
@pytest.mark.parametrize("name", ["tiny_f32", "longformer_base", "bigbird_itc"])
def test_workload_full_parity(name):
    _note(f"[parity] {name} (all rows)")
    inp = make_inputs(workload(name))
    max_abs, E = parity(inp, name)
    _note(f"[parity] {name}: max-abs {max_abs:.3e}, E {E}")


@pytest.mark.parametrize("name", ["dilated_16k", "swa512_causal_32k"])
def test_workload_full_size_parity_every_head(name):
    """Full-size launch; every row of every head is compared with the oracle element by
    element (the oracle runs all heads at once, a few seconds on the host cores)."""
    _note(f"[parity] {name} full launch, oracle on every head")
    inp = make_inputs(workload(name))
    o, l, _ = run_gpu(inp)
    ref_o, ref_l, E = oracle.forward_inputs(inp)
    max_abs = compare(inp, o, l, ref_o, ref_l, name)
    _note(f"[parity] {name}: max-abs {max_abs:.3e} over {inp.heads} heads, E {E}")


@pytest.mark.parametrize("name", ["tiny_f32", "longformer_base", "dilated_16k",
                                  "swa512_causal_32k", "bigbird_itc"])
def test_workload_entry_count_is_exact(name):
    inp = make_inputs(workload(name))
    assert gpu_count(inp) == oracle.count_inputs(inp)


# ------------------------------------------------------------------------------ random sweep
def _sweep_cases():
    rng = np.random.default_rng(2024)
    cases = []
    for t in range(36):
        dtype = "bf16" if t % 4 else "f32"
        d = int(rng.choice([64, 128])) if dtype == "bf16" else int(rng.choice([8, 64, 100, 128]))
        layout = dtype == "f32" and rng.random() < 0.3 or (dtype == "bf16" and t % 6 == 5)
        block = int(rng.choice([64, 128])) if layout else 0
        n = int(rng.choice([1, 2, 63, 65, 127, 129, 200, 257, 384, 641, 1000]))
        if layout:
            n = block * int(rng.integers(1, 7))
        H = int(rng.integers(1, 4))
        band = (not layout) or dtype == "f32" and rng.random() < 0.5
        wl = int(rng.choice([0, 1, 5, 31, 64, 100, 300, 5000])) if band else -1
        wr = int(rng.choice([0, 0, 3, 33, 63, 128, 200])) if band else -1
        dil = [int(x) for x in rng.integers(1, 4, size=H)] if band and rng.random() < 0.5 else None
        g = int(rng.integers(0, min(n, 70) + 1)) if rng.random() < 0.6 else 0
        pad = str(rng.choice(["none", "tail", "random"]))
        pc = int(rng.integers(0, n + 1))
        cases.append(dict(seed=5000 + t, batch=int(rng.integers(1, 3)), heads=H, n=n, d=d,
                          dtype=dtype, win_left=wl, win_right=wr, dilations=dil, n_global=g,
                          pad=pad, pad_count=pc, block=block,
                          max_kb=int(rng.integers(1, 5)) if layout else 0))
    return cases


SWEEP = _sweep_cases()


@pytest.mark.parametrize("case", SWEEP, ids=[f"s{i}" for i in range(len(SWEEP))])
def test_random_shapes_parity(case):
    _note(f"[sweep] {case}")
    inp = random_case(**case)
    parity(inp, str(case))
    assert gpu_count(inp) == oracle.count_inputs(inp)


# ------------------------------------------------------------------------------ edge cases
def test_window_zero_returns_v_bits_exactly():
    inp = random_case(31, batch=2, heads=3, n=300, d=64, win_left=0, win_right=0,
                      dilations=[1, 2, 3])
    _, _, out = run_gpu(inp)
    bits = out.cpu().view(__import__("torch").int16).numpy().view(np.uint16)
    assert np.array_equal(bits, inp.v)


def test_window_covering_sequence_is_full_attention():
    n = 333
    inp = random_case(32, batch=1, heads=2, n=n, d=128, win_left=n, win_right=n)
    parity(inp, "full")


def test_rows_whose_keys_are_all_padded_are_empty():
    inp = random_case(33, batch=2, heads=2, n=256, d=64, win_left=3, win_right=3, n_global=2)
    kp = np.zeros((2, 256), np.uint8)
    kp[1, :] = 1  # sample 2: every key padded, so every row (global rows too) is empty
    kp[0, 100:140] = 1  # sample 1: rows 104..135 see only padded window keys (plus globals)
    inp.key_pad = kp
    ref_o, ref_l, _ = oracle.forward_inputs(inp)
    o, l, _ = run_gpu(inp)
    compare(inp, o, l, ref_o, ref_l, "padded")
    assert np.all(o[1] == 0.0) and np.all(l[1] == -np.inf)


BIG = {"bf16": round_to_bf16_bits(np.array([1e30], np.float32))[0], "f32": np.float32(1e30)}


def _poison(inp, keys_of_sample):
    """A copy of inp whose K and V rows at the listed positions (per sample) hold 1e30."""
    import copy

    p = copy.deepcopy(inp)
    big = BIG[inp.dtype]
    for b, idx in enumerate(keys_of_sample):
        idx = np.asarray(sorted(idx), dtype=np.int64)
        if idx.size:
            p.k[b][:, idx] = big
            p.v[b][:, idx] = big
    return p


def _clean_rows(inp, poisoned):
    """Rows (b, h, i) whose key set (the oracle's) holds none of the poisoned positions."""
    clean = np.zeros((inp.batch, inp.heads, inp.n), bool)
    for b in range(inp.batch):
        bad = np.zeros(inp.n, bool)
        bad[np.asarray(sorted(poisoned[b]), dtype=np.int64)] = True
        for h in range(inp.heads):
            for i in range(inp.n):
                keys = oracle.row_set(inp.batch, inp.heads, inp.n, b, h, i,
                                      win_left=inp.win_left, win_right=inp.win_right,
                                      dilation=inp.dilation, global_idx=inp.global_idx,
                                      key_pad=inp.key_pad, layout=inp.layout, block=inp.block,
                                      max_kb=inp.max_kb)
                clean[b, h, i] = not bad[keys].any()
    return clean


def _bits(out):
    import torch

    x = out.cpu()
    return (x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)).numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_masked_keys_contribute_exactly_zero(dtype):
    """Padded keys poisoned with a huge finite value leave the output bit-identical; among them
    are global tokens inside the windows (padding wins over global: such a key is attended
    neither through its window tile nor through its global column)."""
    inp = random_case(34, batch=2, heads=2, n=520, d=64, dtype=dtype, win_left=40, win_right=7,
                      dilations=[1, 2], n_global=9, pad="random", pad_count=60)
    for b in range(2):  # three of each sample's global tokens are padded too
        inp.key_pad[b, inp.global_idx[b, [1, 4, 7]]] = 1
    _, _, out_a = run_gpu(inp)
    poisoned = _poison(inp, [np.nonzero(inp.key_pad[b])[0] for b in range(2)])
    _, _, out_b = run_gpu(poisoned)
    assert np.array_equal(_bits(out_a), _bits(out_b))


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_out_of_band_keys_in_edge_tiles_contribute_exactly_zero(dtype, d):
    """Every 61st position poisoned: the key tiles at each window's edges load them while they lie
    outside the window of many rows.  Rows whose key set holds no poisoned key keep their output
    bits (scores small enough that the poisoned rows of a wave change no other row's softmax
    decisions: N(0, 1) * 0.5 draws)."""
    inp = random_case(40 + d, batch=2, heads=3, n=700, d=d, dtype=dtype, win_left=23,
                      win_right=9, dilations=[1, 2, 3], qkv_scale=0.5)
    bad = [set(range(5, inp.n, 61)) for _ in range(2)]
    clean = _clean_rows(inp, bad)
    assert clean.sum() > 0.3 * clean.size and (~clean).sum() > 0.1 * clean.size
    _, _, out_a = run_gpu(inp)
    _, _, out_b = run_gpu(_poison(inp, bad))
    a, b = _bits(out_a), _bits(out_b)
    assert np.array_equal(a[clean], b[clean])


@pytest.mark.parametrize("block,d", [(64, 64), (128, 128)])
def test_unlisted_layout_blocks_contribute_exactly_zero(block, d):
    """Keys of blocks that a query block's layout row does not list (and that hold no global
    token) are poisoned; every row of the query blocks that list none of them keeps its bits."""
    inp = random_case(44 + block, batch=2, heads=2, n=block * 12, d=d, block=block, max_kb=3,
                      n_global=2, qkv_scale=0.5)
    nb = inp.n // block
    gblocks = set(int(x) // block for x in inp.global_idx.ravel())
    rng = np.random.default_rng(46)
    cand = [x for x in range(nb) if x not in gblocks]
    pick = set(int(x) for x in rng.choice(cand, size=min(3, len(cand)), replace=False))
    bad = [set(j for j in range(inp.n) if j // block in pick) for _ in range(2)]
    clean = _clean_rows(inp, bad)
    assert clean.sum() > 0.2 * clean.size and (~clean).sum() > 0
    _, _, out_a = run_gpu(inp)
    _, _, out_b = run_gpu(_poison(inp, bad))
    a, b = _bits(out_a), _bits(out_b)
    assert np.array_equal(a[clean], b[clean])


def test_results_are_deterministic():
    inp = make_inputs(workload("longformer_base"))
    _, _, a = run_gpu(inp)
    _, _, b = run_gpu(inp)
    assert (a.cpu().view(__import__("torch").int16) == b.cpu().view(__import__("torch").int16)).all()


def test_causal_window_with_global_tokens():
    inp = random_case(35, batch=1, heads=2, n=1500, d=128, win_left=200, win_right=0,
                      n_global=9)
    parity(inp, "causal+globals")


def test_global_tokens_only():
    inp = random_case(36, batch=2, heads=2, n=700, d=64, n_global=40, pad="tail", pad_count=50)
    parity(inp, "globals only")


@pytest.mark.parametrize("wl,wr", [(150, 77), (64, 64), (333, 1)])
def test_window_tiles_in_rotated_order_with_global_keys_inside(wl, wr):
    # head dim 64 walks each workgroup's window tiles starting at a rotated tile; many global
    # keys fall inside the windows (their per-tile bits are indexed by the rotated tile), the
    # per-workgroup tile count varies at the sequence ends and with the dilation, and the key
    # range starts off the 64-key grid
    inp = random_case(39, batch=2, heads=3, n=2000, d=64, win_left=wl, win_right=wr,
                      dilations=[1, 2, 3], n_global=60, pad="random", pad_count=97)
    parity(inp, f"rotated walk wl={wl} wr={wr}")
    assert gpu_count(inp) == oracle.count_inputs(inp)


@pytest.mark.parametrize("d,block", [(64, 0), (128, 0), (64, 64)])
def test_global_rows_ordered_by_xcd(d, block):
    # eight (batch, head) pairs that take equal main work, so the global-row workgroups take the
    # heads whose main work their XCD ran, most recent first and chunks from the last keys down;
    # 150 global rows make two (window) or three (64-row blocks) row groups per head, over three
    # key chunks; any order of that work must give the oracle's result
    if block:
        inp = random_case(48, batch=2, heads=4, n=1280, d=d, block=block, max_kb=3,
                          n_global=150, pad="random", pad_count=40)
    else:
        inp = random_case(47 + d, batch=2, heads=4, n=1300, d=d, win_left=100, win_right=60,
                          n_global=150, pad="random", pad_count=40)
    parity(inp, f"global rows by XCD d={d} block={block}")
    assert gpu_count(inp) == oracle.count_inputs(inp)


def test_uniform_and_per_head_dilation_tables():
    for dil in (3, [1, 2, 3, 4, 5]):
        inp = random_case(37, batch=1, heads=5, n=900, d=64, win_left=17, win_right=9,
                          dilations=dil, n_global=3)
        parity(inp, f"dilation {dil}")


def test_debug_mode_rejects_unsorted_global_tokens():
    import torch

    inp = random_case(38, batch=1, heads=1, n=128, d=64, win_left=4, win_right=4, n_global=3)
    t = to_torch(inp, "cuda:0")
    bad = t["global_idx"].flip(1).contiguous()
    os.environ["LONGATTN_DEBUG"] = "1"
    try:
        with pytest.raises(la.LongAttnError) as ei:
            la.forward(t["q"], t["k"], t["v"], win_left=4, win_right=4, global_idx=bad)
        assert ei.value.status == la.LONGATTN_ERR_INVALID_ARG
        la.forward(t["q"], t["k"], t["v"], win_left=4, win_right=4, global_idx=t["global_idx"])
    finally:
        del os.environ["LONGATTN_DEBUG"]
    torch.cuda.synchronize()


def test_marks_time_each_phase():
    import ctypes

    import torch

    inp = make_inputs(workload("longformer_base"))
    t = to_torch(inp, "cuda:0")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(la.LONGATTN_N_MARKS)]
    for e in ev:  # make sure the underlying events exist before handing them to the library
        e.record()
    torch.cuda.synchronize()
    handles = [ctypes.c_void_p(e.cuda_event).value for e in ev]
    la.forward(t["q"], t["k"], t["v"], scale=inp.scale, win_left=256, win_right=256,
               global_idx=t["global_idx"], key_pad=t["key_pad"], marks=handles)
    torch.cuda.synchronize()
    spans = [ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(ev[3])]  # attention, combine
    assert all(s > 0 for s in spans) and ev[1].elapsed_time(ev[2]) >= 0
