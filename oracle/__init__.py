"""fp64 CPU oracle for banded sparse self-attention forward (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg import this package.  It shares no code with the HIP library
(``sparse_long_sequence_banded_amd``) and neither imports the other; the only code both sides
use is the seeded input generator package ``workloads``.

The arithmetic lives in ``longattn_oracle.c`` (plain C, fp64, OpenMP); what it computes and
which passage each step follows is written at the top of that file.  ``decode_inputs`` states a
decode step over a key/value cache as that same forward pass on the gathered window;
``backward`` gives the exact gradients of the forward pass; ``tglobal_side`` and
``tglobal_forward`` state LongT5's Transient-Global attention; ``gate_elementwise`` and
``gate_lowrank`` the output gates of gated attention.  Every function is pinned
by the CPU tests (dense brute force, library full/causal attention, the Big Bird worked window
example, closed-form counts and invariants); none is left "parity unpinned".
"""

import contextlib
import ctypes
import os
import subprocess
import threading
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "longattn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblongattn_oracle.so")
_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (IEEE fp64: no fast-math) into ``liblongattn_oracle.so``."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + f".tmp{os.getpid()}"
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(lib):
    lib.longattn_oracle_forward.restype = ctypes.c_int
    lib.longattn_oracle_forward.argtypes = [
        _I64, _I64, _I64, _I64, ctypes.c_double, _I64, _I64, _P, _P, _I64, _P, _P,
        _I64, _I64, _P, _P, _P, _P, _P, _P, ctypes.c_int,
    ]
    lib.longattn_oracle_count.restype = ctypes.c_int
    lib.longattn_oracle_count.argtypes = [
        _I64, _I64, _I64, _I64, _I64, _P, _P, _I64, _P, _P, _I64, _I64, _P, ctypes.c_int,
    ]
    lib.longattn_oracle_backward.restype = ctypes.c_int
    lib.longattn_oracle_backward.argtypes = [
        _I64, _I64, _I64, _I64, ctypes.c_double, _I64, _I64, _P, _P, _I64, _P, _P,
        _I64, _I64, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int,
    ]
    lib.longattn_oracle_t5_bucket.restype = ctypes.c_int64
    lib.longattn_oracle_t5_bucket.argtypes = [_I64, _I64, _I64]
    lib.longattn_oracle_tglobal_side.restype = ctypes.c_int
    lib.longattn_oracle_tglobal_side.argtypes = [
        _I64, _I64, _I64, _I64, _I64, _I64, ctypes.c_double, _P, _P, _P, _P, _P, _P, _P, _P,
    ]
    lib.longattn_oracle_tglobal_forward.restype = ctypes.c_int
    lib.longattn_oracle_tglobal_forward.argtypes = [
        _I64, _I64, _I64, _I64, _I64, _I64, _I64, _I64, ctypes.c_double, _P, _P, _P, _P, _P, _P,
        _P, _P, _P, _P, _P, _P, ctypes.c_int,
    ]
    lib.longattn_oracle_gate_elementwise.restype = ctypes.c_int
    lib.longattn_oracle_gate_elementwise.argtypes = [_I64, _P, _P, _P]
    lib.longattn_oracle_gate_lowrank.restype = ctypes.c_int
    lib.longattn_oracle_gate_lowrank.argtypes = [_I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P]
    lib.longattn_oracle_row_set.restype = ctypes.c_int64
    lib.longattn_oracle_row_set.argtypes = [
        _I64, _I64, _I64, _I64, _I64, _P, _P, _I64, _P, _P, _I64, _I64, _I64, _I64,
        _I64, _P,
    ]
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


@contextlib.contextmanager
def substituted_library(path: str):
    """Temporarily route every oracle call to another build of the oracle source.

    Used only by the test that plants deliberate mistakes in a copy of the C source and checks
    that the pins catch each one.
    """
    global _lib
    _load()
    saved = _lib
    _lib = _bind(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _struct_args(B, H, n, win_left, win_right, dilation, global_idx, key_pad, layout, block,
                 max_kb):
    dil = _c(dilation, np.int32)
    gi = _c(global_idx, np.int32)
    kp = _c(key_pad, np.uint8)
    lay = _c(layout, np.int32)
    g = 0 if gi is None else int(gi.shape[-1])
    if gi is not None:
        assert gi.shape == (B, g), gi.shape
    if dil is not None:
        assert dil.shape == (H,), dil.shape
    if kp is not None:
        assert kp.shape == (B, n), kp.shape
    if lay is not None:
        assert block > 0 and n % block == 0
        assert lay.shape == (H, n // block, max_kb), lay.shape
    keep = (dil, gi, kp, lay)
    return keep, (win_left, win_right, _ptr(dil), _ptr(gi), g, _ptr(kp), _ptr(lay), block, max_kb)


def forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, scale: float, win_left: int,
            win_right: int, dilation=None, global_idx=None, key_pad=None, layout=None,
            block: int = 0, max_kb: int = 0, nthreads: int = 0
            ) -> Tuple[np.ndarray, np.ndarray, int]:
    """Returns (out [B,H,n,d] fp64, lse [B,H,n] fp64, E)."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    B, H, n, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    keep, sargs = _struct_args(B, H, n, win_left, win_right, dilation, global_idx, key_pad,
                               layout, block, max_kb)
    out = np.empty_like(q)
    lse = np.empty((B, H, n), dtype=np.float64)
    E = ctypes.c_int64(0)
    w_l, w_r, dil, gi, g, kp, lay, blk, mkb = sargs
    rc = _load().longattn_oracle_forward(
        B, H, n, d, float(scale), w_l, w_r, dil, gi, g, kp, lay, blk, mkb,
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), ctypes.byref(E), int(nthreads))
    del keep
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return out, lse, int(E.value)


def backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, *, scale: float,
             win_left: int, win_right: int, dilation=None, global_idx=None, key_pad=None,
             layout=None, block: int = 0, max_kb: int = 0, nthreads: int = 0
             ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients (dq, dk, dv) [B,H,n,d] fp64 of sum(dout * out) for the forward pass above."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    dout = np.ascontiguousarray(dout, dtype=np.float64)
    B, H, n, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape and dout.shape == q.shape
    keep, sargs = _struct_args(B, H, n, win_left, win_right, dilation, global_idx, key_pad,
                               layout, block, max_kb)
    dq = np.empty_like(q)
    dk = np.empty_like(q)
    dv = np.empty_like(q)
    w_l, w_r, dil, gi, g, kp, lay, blk, mkb = sargs
    rc = _load().longattn_oracle_backward(
        B, H, n, d, float(scale), w_l, w_r, dil, gi, g, kp, lay, blk, mkb,
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), int(nthreads))
    del keep
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return dq, dk, dv


def backward_inputs(inp, dout: np.ndarray, nthreads: int = 0):
    """Oracle backward on a ``workloads.Inputs`` instance and an output gradient ``dout``."""
    return backward(inp.f64("q"), inp.f64("k"), inp.f64("v"), dout, scale=inp.scale,
                    win_left=inp.win_left, win_right=inp.win_right, dilation=inp.dilation,
                    global_idx=inp.global_idx, key_pad=inp.key_pad, layout=inp.layout,
                    block=inp.block, max_kb=inp.max_kb, nthreads=nthreads)


def count(B: int, H: int, n: int, *, win_left: int, win_right: int, dilation=None,
          global_idx=None, key_pad=None, layout=None, block: int = 0, max_kb: int = 0,
          nthreads: int = 0) -> int:
    """E: the number of useful (query, key) score entries."""
    keep, sargs = _struct_args(B, H, n, win_left, win_right, dilation, global_idx, key_pad,
                               layout, block, max_kb)
    E = ctypes.c_int64(0)
    w_l, w_r, dil, gi, g, kp, lay, blk, mkb = sargs
    rc = _load().longattn_oracle_count(B, H, n, w_l, w_r, dil, gi, g, kp, lay, blk, mkb,
                                       ctypes.byref(E), int(nthreads))
    del keep
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return int(E.value)


def row_set(B: int, H: int, n: int, b: int, h: int, i: int, *, win_left: int, win_right: int,
            dilation=None, global_idx=None, key_pad=None, layout=None, block: int = 0,
            max_kb: int = 0) -> np.ndarray:
    """The ascending allowed key set S(b, h, i)."""
    keep, sargs = _struct_args(B, H, n, win_left, win_right, dilation, global_idx, key_pad,
                               layout, block, max_kb)
    buf = np.empty(max(n, 1), dtype=np.int32)
    w_l, w_r, dil, gi, g, kp, lay, blk, mkb = sargs
    cnt = _load().longattn_oracle_row_set(B, H, n, w_l, w_r, dil, gi, g, kp, lay, blk, mkb,
                                          b, h, i, _ptr(buf))
    del keep
    if cnt < 0:
        raise ValueError(f"oracle rejected the arguments (code {cnt})")
    return buf[:cnt].copy()


def forward_inputs(inp, nthreads: int = 0):
    """Oracle forward on a ``workloads.Inputs`` instance (exact fp64 widening of its values)."""
    return forward(inp.f64("q"), inp.f64("k"), inp.f64("v"), scale=inp.scale,
                   win_left=inp.win_left, win_right=inp.win_right, dilation=inp.dilation,
                   global_idx=inp.global_idx, key_pad=inp.key_pad, layout=inp.layout,
                   block=inp.block, max_kb=inp.max_kb, nthreads=nthreads)


def count_inputs(inp, nthreads: int = 0) -> int:
    return count(inp.batch, inp.heads, inp.n, win_left=inp.win_left, win_right=inp.win_right,
                 dilation=inp.dilation, global_idx=inp.global_idx, key_pad=inp.key_pad,
                 layout=inp.layout, block=inp.block, max_kb=inp.max_kb, nthreads=nthreads)


def decode_inputs(inp, samples=None, nthreads: int = 0):
    """Expected result of a sliding-window decode step on a ``workloads.decode.DecodeInputs``.

    A decode step is the causal sliding-window forward pass (win_left = window - 1,
    win_right = 0) restricted to the new rows.  For sample b the positions p0 .. last
    (p0 = max(0, t0 - window + 1), last = t0 + m - 1) are taken from the cache in position order,
    the new query rows go at the end of that sequence, and ``forward`` runs on it; its last m
    rows are the step's result.  The window depends only on position differences (and the start
    of the sequence stays at index 0 whenever p0 = 0), so each new row sees exactly the keys it
    sees in the full sequence.  Returns (out [B', H, m, d], lse [B', H, m]) in fp64 for the listed
    samples (all by default).
    """
    samples = range(inp.batch) if samples is None else list(samples)
    outs, lses = [], []
    q = inp.f64("q")
    for b in samples:
        _, k, v = inp.gathered(b)
        L = k.shape[1]
        qs = np.zeros_like(k)
        qs[:, L - inp.m:] = q[b]
        o, l, _ = forward(qs[None], k[None], v[None], scale=inp.scale,
                          win_left=inp.window - 1, win_right=0, nthreads=nthreads)
        outs.append(o[0, :, L - inp.m:])
        lses.append(l[0, :, L - inp.m:])
    return np.stack(outs), np.stack(lses)


# ---------------------------------------------------------------------- Transient-Global attention
def t5_bucket(rel: int, num_buckets: int = 32, max_distance: int = 128) -> int:
    """T5 bidirectional relative-position bucket of key position - query position."""
    return int(_load().longattn_oracle_t5_bucket(int(rel), int(num_buckets), int(max_distance)))


def num_global(n: int, block: int) -> int:
    """Global tokens of a sequence of n tokens with blocks of ``block`` (the tail merges)."""
    return max(1, n // block)


def tglobal_side(x: np.ndarray, gamma: np.ndarray, wk: np.ndarray, wv: np.ndarray, *,
                 heads: int, d: int, block: int, eps: float, key_pad=None):
    """Global tokens' keys and values.  x [B, n, dm]; gamma [dm]; wk, wv [dm, heads*d].
    Returns (side_k, side_v [B, heads, G, d] fp64, side_valid [B, G] uint8)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    B, n, dm = x.shape
    gamma = np.ascontiguousarray(gamma, dtype=np.float64)
    wk = np.ascontiguousarray(wk, dtype=np.float64)
    wv = np.ascontiguousarray(wv, dtype=np.float64)
    assert gamma.shape == (dm,) and wk.shape == (dm, heads * d) and wv.shape == wk.shape
    G = num_global(n, block)
    sk = np.empty((B, heads, G, d))
    sv = np.empty((B, heads, G, d))
    valid = np.empty((B, G), dtype=np.uint8)
    kp = None if key_pad is None else np.ascontiguousarray(key_pad, dtype=np.uint8)
    rc = _load().longattn_oracle_tglobal_side(B, n, dm, heads, d, block, float(eps), _ptr(x),
                                              _ptr(gamma), _ptr(wk), _ptr(wv), _ptr(kp),
                                              _ptr(sk), _ptr(sv), _ptr(valid))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return sk, sv, valid


def tglobal_forward(q, k, v, side_k, side_v, side_valid, *, radius: int, block: int,
                    num_buckets: int, max_distance: int, scale: float, bias_local, bias_side,
                    key_pad=None, nthreads: int = 0):
    """Transient-Global attention.  Returns (out [B,H,n,d], lse [B,H,n], E)."""
    q, k, v = (np.ascontiguousarray(a, dtype=np.float64) for a in (q, k, v))
    side_k = np.ascontiguousarray(side_k, dtype=np.float64)
    side_v = np.ascontiguousarray(side_v, dtype=np.float64)
    sval = np.ascontiguousarray(side_valid, dtype=np.uint8)
    bl = np.ascontiguousarray(bias_local, dtype=np.float64)
    bs = np.ascontiguousarray(bias_side, dtype=np.float64)
    B, H, n, d = q.shape
    G = num_global(n, block)
    assert side_k.shape == (B, H, G, d) and side_v.shape == side_k.shape
    assert sval.shape == (B, G) and bl.shape == (num_buckets, H) and bs.shape == bl.shape
    kp = None if key_pad is None else np.ascontiguousarray(key_pad, dtype=np.uint8)
    out = np.empty_like(q)
    lse = np.empty((B, H, n))
    E = ctypes.c_int64(0)
    rc = _load().longattn_oracle_tglobal_forward(
        B, H, n, d, int(radius), int(block), int(num_buckets), int(max_distance), float(scale),
        _ptr(q), _ptr(k), _ptr(v), _ptr(side_k), _ptr(side_v), _ptr(sval), _ptr(kp), _ptr(bl),
        _ptr(bs), _ptr(out), _ptr(lse), ctypes.byref(E), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return out, lse, int(E.value)


def tglobal_inputs(inp, nthreads: int = 0):
    """Both oracle steps on a ``workloads.tglobal.TGInputs``: (out, lse, E, side_k, side_v,
    side_valid)."""
    sk, sv, valid = tglobal_side(inp.f64("x"), inp.gamma, inp.f64("wk"), inp.f64("wv"),
                                 heads=inp.heads, d=inp.d, block=inp.block, eps=inp.eps,
                                 key_pad=inp.key_pad)
    out, lse, E = tglobal_forward(inp.f64("q"), inp.f64("k"), inp.f64("v"), sk, sv, valid,
                                  radius=inp.radius, block=inp.block,
                                  num_buckets=inp.num_buckets, max_distance=inp.max_distance,
                                  scale=inp.scale, bias_local=inp.bias_local,
                                  bias_side=inp.bias_side, key_pad=inp.key_pad,
                                  nthreads=nthreads)
    return out, lse, E, sk, sv, valid


# ---------------------------------------------------------------------- output gates
def gate_elementwise(out: np.ndarray, gate: np.ndarray) -> np.ndarray:
    """out * sigmoid(gate), elementwise (any matching shapes), fp64."""
    o = np.ascontiguousarray(out, dtype=np.float64)
    g = np.ascontiguousarray(gate, dtype=np.float64)
    assert o.shape == g.shape
    res = np.empty_like(o)
    rc = _load().longattn_oracle_gate_elementwise(o.size, _ptr(o), _ptr(g), _ptr(res))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return res


def gate_lowrank(out: np.ndarray, w_down: np.ndarray, w_up: np.ndarray) -> np.ndarray:
    """out [B, H, n, d] gated by sigmoid(W_up (W_down o)) over each token's H*d outputs;
    w_down [r, H*d], w_up [H*d, r]."""
    o = np.ascontiguousarray(out, dtype=np.float64)
    B, H, n, d = o.shape
    wd = np.ascontiguousarray(w_down, dtype=np.float64)
    wu = np.ascontiguousarray(w_up, dtype=np.float64)
    r = wd.shape[0]
    assert wd.shape == (r, H * d) and wu.shape == (H * d, r)
    res = np.empty_like(o)
    rc = _load().longattn_oracle_gate_lowrank(B, H, n, d, r, _ptr(o), _ptr(wd), _ptr(wu),
                                              _ptr(res))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return res
