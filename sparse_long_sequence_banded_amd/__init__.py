"""Banded sparse self-attention forward for AMD MI355X (gfx950): Python binding.

This module only marshals arguments for ``liblongattn.so`` (built from ``csrc/`` by
``python -m sparse_long_sequence_banded_amd.build``); every step of the attention runs in the
library's HIP kernels.  PyTorch supplies device memory and the current HIP stream.  If the
library has not been built, every call raises ``LongAttnNotBuilt``; there is no fallback.

The C entry points keep their names here (``longattn_forward``, ``longattn_workspace_size``,
``longattn_forward_marked``, ``longattn_count_entries``, ``longattn_backward``,
``longattn_backward_workspace_size``, ``longattn_decode``, ``longattn_decode_workspace_size``,
``longattn_status_string``); the ``forward`` / ``backward`` / ``count_entries`` / ``decode``
helpers wrap them for torch tensors.
"""

import ctypes
import os
import threading
from typing import Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblongattn.so")

LONGATTN_OK = 0
LONGATTN_ERR_INVALID_ARG = 1
LONGATTN_ERR_UNSUPPORTED = 2
LONGATTN_ERR_ALIGNMENT = 3
LONGATTN_ERR_WORKSPACE = 4
LONGATTN_ERR_HIP = 5
LONGATTN_BF16 = 0
LONGATTN_F32 = 1
LONGATTN_N_MARKS = 4
LONGATTN_BWD_N_MARKS = 6

EXPORTED = (
    "longattn_workspace_size",
    "longattn_forward",
    "longattn_forward_marked",
    "longattn_forward_noalloc",
    "longattn_count_entries",
    "longattn_forward_gated",
    "longattn_backward_workspace_size",
    "longattn_backward",
    "longattn_backward_marked",
    "longattn_gate_lowrank",
    "longattn_tglobal_workspace_size",
    "longattn_tglobal_side",
    "longattn_tglobal_forward",
    "longattn_decode_workspace_size",
    "longattn_decode",
    "longattn_status_string",
)


class longattn_desc(ctypes.Structure):
    """Mirror of ``struct longattn_desc`` in include/longattn.h."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("n", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("win_left", ctypes.c_int32),
        ("win_right", ctypes.c_int32),
        ("dilation", ctypes.c_void_p),
        ("global_idx", ctypes.c_void_p),
        ("n_global", ctypes.c_int32),
        ("key_pad", ctypes.c_void_p),
        ("block_layout", ctypes.c_void_p),
        ("block", ctypes.c_int32),
        ("max_kb", ctypes.c_int32),
    ]


class longattn_decode_desc(ctypes.Structure):
    """Mirror of ``struct longattn_decode_desc`` in include/longattn.h."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("window", ctypes.c_int32),
        ("n_queries", ctypes.c_int32),
        ("cache_len", ctypes.c_int32),
        ("ring", ctypes.c_int32),
        ("positions", ctypes.c_void_p),
    ]


class longattn_tglobal_desc(ctypes.Structure):
    """Mirror of ``longattn_tglobal_desc`` in include/longattn.h."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("n", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("d_model", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("radius", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("num_buckets", ctypes.c_int32),
        ("max_distance", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("key_pad", ctypes.c_void_p),
    ]


class longattn_gate_desc(ctypes.Structure):
    """Mirror of ``longattn_gate_desc`` in include/longattn.h."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("n", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("rank", ctypes.c_int32),
    ]


class LongAttnNotBuilt(RuntimeError):
    pass


class LongAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {longattn_status_string(status)} (status {status})")


_lock = threading.Lock()
_lib = None


def load():
    """Load liblongattn.so (raises LongAttnNotBuilt if it is missing)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise LongAttnNotBuilt(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m sparse_long_sequence_banded_amd.build`")
            lib = ctypes.CDLL(LIB_PATH)
            P = ctypes.c_void_p
            D = ctypes.POINTER(longattn_desc)
            lib.longattn_workspace_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
            lib.longattn_workspace_size.restype = ctypes.c_int
            lib.longattn_forward.argtypes = [D, P, P, P, P, P, P, ctypes.c_size_t, P]
            lib.longattn_forward.restype = ctypes.c_int
            lib.longattn_forward_marked.argtypes = [D, P, P, P, P, P, P, ctypes.c_size_t, P,
                                                    ctypes.POINTER(P), ctypes.c_int32]
            lib.longattn_forward_marked.restype = ctypes.c_int
            lib.longattn_forward_noalloc.argtypes = [D, P, P, P, P, P, P]
            lib.longattn_forward_noalloc.restype = ctypes.c_int
            lib.longattn_count_entries.argtypes = [D, P, P]
            lib.longattn_count_entries.restype = ctypes.c_int
            lib.longattn_forward_gated.argtypes = [D, P, P, P, P, P, P, P, ctypes.c_size_t, P]
            lib.longattn_forward_gated.restype = ctypes.c_int
            lib.longattn_backward_workspace_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
            lib.longattn_backward_workspace_size.restype = ctypes.c_int
            lib.longattn_backward.argtypes = [D, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
            lib.longattn_backward.restype = ctypes.c_int
            lib.longattn_backward_marked.argtypes = [D, P, P, P, P, P, P, P, P, P, P,
                                                     ctypes.c_size_t, P,
                                                     ctypes.POINTER(ctypes.c_void_p),
                                                     ctypes.c_int32]
            lib.longattn_backward_marked.restype = ctypes.c_int
            lib.longattn_gate_lowrank.argtypes = [ctypes.POINTER(longattn_gate_desc), P, P, P, P]
            lib.longattn_gate_lowrank.restype = ctypes.c_int
            TD = ctypes.POINTER(longattn_tglobal_desc)
            lib.longattn_tglobal_workspace_size.argtypes = [TD, ctypes.POINTER(ctypes.c_size_t)]
            lib.longattn_tglobal_workspace_size.restype = ctypes.c_int
            lib.longattn_tglobal_side.argtypes = [TD, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
            lib.longattn_tglobal_side.restype = ctypes.c_int
            lib.longattn_tglobal_forward.argtypes = [TD, P, P, P, P, P, P, P, P, P, P, P,
                                                     ctypes.c_size_t, P]
            lib.longattn_tglobal_forward.restype = ctypes.c_int
            DD = ctypes.POINTER(longattn_decode_desc)
            lib.longattn_decode_workspace_size.argtypes = [DD, ctypes.POINTER(ctypes.c_size_t)]
            lib.longattn_decode_workspace_size.restype = ctypes.c_int
            lib.longattn_decode.argtypes = [DD, P, P, P, P, P, P, ctypes.c_size_t, P]
            lib.longattn_decode.restype = ctypes.c_int
            lib.longattn_status_string.argtypes = [ctypes.c_int]
            lib.longattn_status_string.restype = ctypes.c_char_p
            _lib = lib
    return _lib


# ----------------------------------------------------------------------------- raw C calls
def longattn_status_string(status: int) -> str:
    return load().longattn_status_string(int(status)).decode()


def longattn_workspace_size(desc: longattn_desc) -> Tuple[int, int]:
    """Returns (status, bytes)."""
    nbytes = ctypes.c_size_t(0)
    st = load().longattn_workspace_size(ctypes.byref(desc), ctypes.byref(nbytes))
    return st, int(nbytes.value)


def longattn_forward(desc, q, k, v, out, lse, workspace, workspace_bytes, stream) -> int:
    """Raw call; pointer arguments are integers (device addresses) or None."""
    return load().longattn_forward(ctypes.byref(desc), q, k, v, out, lse, workspace,
                                   int(workspace_bytes), stream)


def longattn_forward_marked(desc, q, k, v, out, lse, workspace, workspace_bytes, stream,
                            marks: Optional[Sequence[int]]) -> int:
    arr = None
    n = 0
    if marks is not None:
        n = len(marks)
        arr = (ctypes.c_void_p * n)(*marks)
    return load().longattn_forward_marked(ctypes.byref(desc), q, k, v, out, lse, workspace,
                                          int(workspace_bytes), stream, arr, n)


def longattn_forward_noalloc(desc, q, k, v, out, lse, stream) -> int:
    """Raw call of the allocation-free forward pass (scratch in the library's own device array
    of LONGATTN_NOALLOC_SCRATCH_BYTES per GPU; calls that overlap on one GPU race)."""
    return load().longattn_forward_noalloc(ctypes.byref(desc), q, k, v, out, lse, stream)


LONGATTN_NOALLOC_SCRATCH_BYTES = 32 << 20


def longattn_count_entries(desc, entries_out, stream) -> int:
    return load().longattn_count_entries(ctypes.byref(desc), entries_out, stream)


def longattn_forward_gated(desc, q, k, v, gate, out, lse, workspace, workspace_bytes,
                           stream) -> int:
    """Raw call of the forward pass with an elementwise output gate."""
    return load().longattn_forward_gated(ctypes.byref(desc), q, k, v, gate, out, lse, workspace,
                                         int(workspace_bytes), stream)


def longattn_backward_workspace_size(desc: longattn_desc) -> Tuple[int, int]:
    """Returns (status, bytes)."""
    nbytes = ctypes.c_size_t(0)
    st = load().longattn_backward_workspace_size(ctypes.byref(desc), ctypes.byref(nbytes))
    return st, int(nbytes.value)


def longattn_backward(desc, q, k, v, out, lse, dout, dq, dk, dv, workspace, workspace_bytes,
                      stream) -> int:
    """Raw call; pointer arguments are integers (device addresses) or None."""
    return load().longattn_backward(ctypes.byref(desc), q, k, v, out, lse, dout, dq, dk, dv,
                                    workspace, int(workspace_bytes), stream)


def longattn_backward_marked(desc, q, k, v, out, lse, dout, dq, dk, dv, workspace,
                             workspace_bytes, stream, marks) -> int:
    """Raw call with LONGATTN_BWD_N_MARKS event handles (integers) in ``marks``."""
    arr = (ctypes.c_void_p * len(marks))(*marks)
    return load().longattn_backward_marked(ctypes.byref(desc), q, k, v, out, lse, dout, dq, dk,
                                           dv, workspace, int(workspace_bytes), stream, arr,
                                           len(marks))


def longattn_decode_workspace_size(desc: longattn_decode_desc) -> Tuple[int, int]:
    """Returns (status, bytes)."""
    nbytes = ctypes.c_size_t(0)
    st = load().longattn_decode_workspace_size(ctypes.byref(desc), ctypes.byref(nbytes))
    return st, int(nbytes.value)


def longattn_decode(desc, q, k_cache, v_cache, out, lse, workspace, workspace_bytes,
                    stream) -> int:
    """Raw call; pointer arguments are integers (device addresses) or None."""
    return load().longattn_decode(ctypes.byref(desc), q, k_cache, v_cache, out, lse, workspace,
                                  int(workspace_bytes), stream)


# ----------------------------------------------------------------------------- torch helpers
def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream_handle(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _launch_on(stream):
    """Handle of the stream a helper launches on.  A stream other than the current one first
    waits for the current one, which holds the helper's own preparation (zeroed counters,
    contiguous copies of index tensors) and the caller's preceding work."""
    import torch

    cur = torch.cuda.current_stream()
    if stream is not None and stream != cur:
        stream.wait_stream(cur)
    return _stream_handle(stream)


def _used_on(stream, *tensors):
    """Tensors allocated on the current stream and used by a launch on another ``stream``: tell
    the caching allocator, so that their memory is not handed out again before that stream has
    finished with it."""
    import torch

    if stream is None or stream == torch.cuda.current_stream():
        return
    for t in tensors:
        if isinstance(t, torch.Tensor):
            t.record_stream(stream)


def make_desc(q, *, scale: Optional[float] = None, win_left: int = -1, win_right: int = -1,
              dilation=None, global_idx=None, key_pad=None, block_layout=None, block: int = 0):
    """Build the descriptor for q of shape [B, H, n, d].  Returns (desc, keepalive)."""
    import torch

    B, H, n, d = q.shape
    if q.dtype == torch.bfloat16:
        dt = LONGATTN_BF16
    elif q.dtype == torch.float32:
        dt = LONGATTN_F32
    else:
        raise TypeError(f"unsupported dtype {q.dtype} (bfloat16 or float32)")
    keep = []
    dil_ptr = None
    if dilation is not None:
        vals = [int(x) for x in dilation]
        if len(vals) != H:
            raise ValueError("dilation needs one entry per head")
        dil = (ctypes.c_int32 * H)(*vals)
        keep.append(dil)
        dil_ptr = ctypes.cast(dil, ctypes.c_void_p).value
    g = 0
    if global_idx is not None:
        if global_idx.dtype != torch.int32 or global_idx.device != q.device:
            raise TypeError("global_idx must be an int32 tensor on q's device")
        global_idx = global_idx.contiguous()
        if global_idx.shape[0] != B:
            raise ValueError("global_idx must be [batch, n_global]")
        g = int(global_idx.shape[1])
        keep.append(global_idx)
    if key_pad is not None:
        if key_pad.dtype not in (torch.uint8, torch.bool) or key_pad.device != q.device:
            raise TypeError("key_pad must be a uint8/bool tensor on q's device")
        key_pad = key_pad.contiguous().view(torch.uint8)
        if tuple(key_pad.shape) != (B, n):
            raise ValueError("key_pad must be [batch, n]")
        keep.append(key_pad)
    max_kb = 0
    if block_layout is not None:
        if block_layout.dtype != torch.int32 or block_layout.device != q.device:
            raise TypeError("block_layout must be an int32 tensor on q's device")
        block_layout = block_layout.contiguous()
        max_kb = int(block_layout.shape[-1])
        keep.append(block_layout)
    desc = longattn_desc(
        batch=B, heads=H, n=n, d=d, dtype=dt,
        scale=float(scale) if scale is not None else 1.0 / float(d) ** 0.5,
        win_left=int(win_left), win_right=int(win_right), dilation=dil_ptr,
        global_idx=_ptr(global_idx), n_global=g, key_pad=_ptr(key_pad),
        block_layout=_ptr(block_layout), block=int(block), max_kb=max_kb,
    )
    return desc, keep


def forward(q, k, v, *, scale: Optional[float] = None, win_left: int = -1,
            win_right: int = -1, dilation=None, global_idx=None, key_pad=None,
            block_layout=None, block: int = 0, out=None, lse=None, want_lse: bool = True,
            workspace=None, stream=None, marks=None, gate=None):
    """Banded / global / block-sparse attention forward on torch device tensors [B, H, n, d].

    ``gate``: optional [B, H, n, d] logits of an elementwise output gate (out *= sigmoid(gate)).
    Returns (out, lse); lse is None when ``want_lse`` is False and no ``lse`` is given.
    """
    import torch

    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous device tensors")
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    desc, keep = make_desc(q, scale=scale, win_left=win_left, win_right=win_right,
                           dilation=dilation, global_idx=global_idx, key_pad=key_pad,
                           block_layout=block_layout, block=block)
    st, ws_bytes = longattn_workspace_size(desc)
    if st != LONGATTN_OK:
        raise LongAttnError(st, "longattn_workspace_size")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    sh = _launch_on(stream)
    if gate is not None:
        if gate.shape != q.shape or gate.dtype != q.dtype or not gate.is_contiguous():
            raise ValueError("gate must be a contiguous tensor of q's shape and dtype")
        if marks is not None:
            raise ValueError("marks are not available with a gate")
        st = longattn_forward_gated(desc, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                    gate.data_ptr(), out.data_ptr(), _ptr(lse),
                                    _ptr(workspace) if ws_bytes else None, ws_bytes, sh)
    elif marks is None:
        st = longattn_forward(desc, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              _ptr(lse), _ptr(workspace) if ws_bytes else None, ws_bytes, sh)
    else:
        st = longattn_forward_marked(desc, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                     out.data_ptr(), _ptr(lse),
                                     _ptr(workspace) if ws_bytes else None, ws_bytes, sh, marks)
    _used_on(stream, out, lse, workspace, gate, *keep)
    del keep
    if st != LONGATTN_OK:
        raise LongAttnError(st, "longattn_forward")
    return out, lse


def backward(q, k, v, out, lse, dout, *, scale: Optional[float] = None, win_left: int = -1,
             win_right: int = -1, dilation=None, global_idx=None, key_pad=None,
             block_layout=None, block: int = 0, dq=None, dk=None, dv=None, workspace=None,
             stream=None):
    """Gradients (dq, dk, dv) of a loss through ``forward``, given out and lse of that forward
    pass and dout = dLoss/dout (torch device tensors [B, H, n, d], lse [B, H, n] fp32)."""
    import torch

    for t in (q, k, v, out, dout, lse):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v, out, lse, dout must be contiguous device tensors")
    for t in (k, v, out, dout):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("k, v, out, dout must share q's shape and dtype")
    if lse.dtype != torch.float32 or lse.shape != q.shape[:3]:
        raise ValueError("lse must be float32 [B, H, n]")
    desc, keep = make_desc(q, scale=scale, win_left=win_left, win_right=win_right,
                           dilation=dilation, global_idx=global_idx, key_pad=key_pad,
                           block_layout=block_layout, block=block)
    st, ws_bytes = longattn_backward_workspace_size(desc)
    if st != LONGATTN_OK:
        raise LongAttnError(st, "longattn_backward_workspace_size")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    st = longattn_backward(desc, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                           dv.data_ptr(), _ptr(workspace) if ws_bytes else None, ws_bytes,
                           _launch_on(stream))
    _used_on(stream, dq, dk, dv, workspace, *keep)
    del keep
    if st != LONGATTN_OK:
        raise LongAttnError(st, "longattn_backward")
    return dq, dk, dv


def count_entries(q, *, win_left: int = -1, win_right: int = -1, dilation=None,
                  global_idx=None, key_pad=None, block_layout=None, block: int = 0,
                  stream=None) -> Tuple[int, int]:
    """(E, E in global rows): useful score entries counted on the GPU (synchronises)."""
    import torch

    desc, keep = make_desc(q, win_left=win_left, win_right=win_right, dilation=dilation,
                           global_idx=global_idx, key_pad=key_pad, block_layout=block_layout,
                           block=block)
    e = torch.zeros(2, dtype=torch.int64, device=q.device)
    st = longattn_count_entries(desc, e.data_ptr(), _launch_on(stream))
    _used_on(stream, e, *keep)
    del keep
    if st != LONGATTN_OK:
        raise LongAttnError(st, "longattn_count_entries")
    if stream is not None:
        stream.synchronize()  # the counts were written on that stream
    vals = e.cpu().tolist()
    return int(vals[0]), int(vals[1])


def from_hf_mask(mask):
    """HF-style attention mask [B, n] with 0 = padding, 1 = local, 2 = global tokens
    (Longformer hub page, section 5) -> (global_idx int32 [B, g], key_pad uint8 [B, n]).

    Every sample must have the same number g of global tokens.
    """
    import torch

    if mask.dim() != 2:
        raise ValueError("mask must be [batch, n]")
    is_g = mask == 2
    counts = is_g.sum(dim=1)
    if counts.numel() and not bool((counts == counts[0]).all()):
        raise ValueError("every sample needs the same number of global tokens")
    B = mask.shape[0]
    g = int(counts[0]) if B else 0
    idx = torch.nonzero(is_g, as_tuple=False)[:, 1].to(torch.int32).reshape(B, g)
    key_pad = (mask == 0).to(torch.uint8)
    return idx.contiguous(), key_pad.contiguous()


def make_decode_desc(q, k_cache, positions, *, window: int, scale: Optional[float] = None,
                     ring: bool = False) -> longattn_decode_desc:
    """Descriptor for q [B, H, m, d], caches [B, H, cache_len, d] and int32 positions [B]."""
    import torch

    B, H, m, d = q.shape
    if q.dtype == torch.bfloat16:
        dt = LONGATTN_BF16
    elif q.dtype == torch.float32:
        dt = LONGATTN_F32
    else:
        raise TypeError(f"unsupported dtype {q.dtype} (bfloat16 or float32)")
    if positions.dtype != torch.int32 or positions.device != q.device or positions.numel() != B:
        raise TypeError("positions must be an int32 tensor of [batch] on q's device")
    return longattn_decode_desc(
        batch=B, heads=H, d=d, dtype=dt,
        scale=float(scale) if scale is not None else 1.0 / float(d) ** 0.5,
        window=int(window), n_queries=m, cache_len=int(k_cache.shape[2]), ring=int(bool(ring)),
        positions=positions.data_ptr(),
    )


def decode(q, k_cache, v_cache, positions, *, window: int, scale: Optional[float] = None,
           ring: bool = False, out=None, lse=None, want_lse: bool = True, workspace=None,
           stream=None):
    """Sliding-window decode: q [B, H, m, d] rows at positions positions[b] + j attend the last
    ``window`` keys (up to their own position) held in k_cache / v_cache [B, H, cache_len, d]
    (slot = position, or position % cache_len when ``ring``).  Returns (out, lse)."""
    import torch

    for t in (q, k_cache, v_cache):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k_cache, v_cache must be contiguous device tensors")
    if k_cache.shape != v_cache.shape or k_cache.shape[:2] != q.shape[:2] or \
            k_cache.shape[3] != q.shape[3] or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("k_cache, v_cache must be [B, H, cache_len, d] of q's dtype")
    positions = positions.contiguous()
    desc = make_decode_desc(q, k_cache, positions, window=window, scale=scale, ring=ring)
    st, ws_bytes = longattn_decode_workspace_size(desc)
    if st != LONGATTN_OK:
        raise LongAttnError(st, "longattn_decode_workspace_size")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    st = longattn_decode(desc, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                         out.data_ptr(), _ptr(lse), _ptr(workspace) if ws_bytes else None,
                         ws_bytes, _launch_on(stream))
    _used_on(stream, out, lse, workspace, positions)
    if st != LONGATTN_OK:
        raise LongAttnError(st, "longattn_decode")
    return out, lse


# ---------------------------------------------------------------------- Transient-Global attention
def longattn_tglobal_workspace_size(desc: longattn_tglobal_desc) -> Tuple[int, int]:
    nbytes = ctypes.c_size_t(0)
    st = load().longattn_tglobal_workspace_size(ctypes.byref(desc), ctypes.byref(nbytes))
    return st, int(nbytes.value)


def longattn_tglobal_side(desc, x, gamma, wk, wv, side_k, side_v, side_valid, workspace,
                          workspace_bytes, stream) -> int:
    return load().longattn_tglobal_side(ctypes.byref(desc), x, gamma, wk, wv, side_k, side_v,
                                        side_valid, workspace, int(workspace_bytes), stream)


def longattn_tglobal_forward(desc, q, k, v, side_k, side_v, side_valid, bias_local, bias_side,
                             out, lse, workspace, workspace_bytes, stream) -> int:
    return load().longattn_tglobal_forward(ctypes.byref(desc), q, k, v, side_k, side_v,
                                           side_valid, bias_local, bias_side, out, lse,
                                           workspace, int(workspace_bytes), stream)


def make_tglobal_desc(q, *, d_model: int, radius: int, block: int, scale: Optional[float] = None,
                      num_buckets: int = 32, max_distance: int = 128, eps: float = 1e-6,
                      key_pad=None) -> longattn_tglobal_desc:
    B, H, n, d = q.shape
    return longattn_tglobal_desc(
        batch=B, heads=H, n=n, d=d, d_model=int(d_model),
        scale=float(scale) if scale is not None else 1.0 / float(d) ** 0.5,
        radius=int(radius), block=int(block), num_buckets=int(num_buckets),
        max_distance=int(max_distance), eps=float(eps),
        key_pad=None if key_pad is None else key_pad.data_ptr())


def tglobal(x, gamma, wk, wv, q, k, v, bias_local, bias_side, *, radius: int = 127,
            block: int = 16, scale: Optional[float] = None, num_buckets: int = 32,
            max_distance: int = 128, eps: float = 1e-6, key_pad=None, want_lse: bool = True,
            stream=None):
    """LongT5 Transient-Global attention on device tensors: x [B, n, d_model] bf16, gamma fp32,
    wk, wv [d_model, H*d] bf16, q, k, v [B, H, n, d] bf16, bias tables fp32 [num_buckets, H].
    Returns (out, lse, side_k, side_v, side_valid)."""
    import torch

    B, H, n, d = q.shape
    for t in (x, wk, wv, q, k, v, gamma, bias_local, bias_side):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("every tensor must be a contiguous device tensor")
    if key_pad is not None and (key_pad.dtype != torch.uint8 or key_pad.shape != (B, n)):
        raise ValueError("key_pad must be uint8 [B, n]")
    desc = make_tglobal_desc(q, d_model=x.shape[-1], radius=radius, block=block, scale=scale,
                             num_buckets=num_buckets, max_distance=max_distance, eps=eps,
                             key_pad=key_pad)
    st, ws_bytes = longattn_tglobal_workspace_size(desc)
    if st != LONGATTN_OK:
        raise LongAttnError(st, "longattn_tglobal_workspace_size")
    G = max(1, n // block)
    side_k = torch.empty((B, H, G, d), dtype=q.dtype, device=q.device)
    side_v = torch.empty_like(side_k)
    side_valid = torch.empty((B, G), dtype=torch.uint8, device=q.device)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    sh = _launch_on(stream)
    st = longattn_tglobal_side(desc, x.data_ptr(), gamma.data_ptr(), wk.data_ptr(),
                               wv.data_ptr(), side_k.data_ptr(), side_v.data_ptr(),
                               side_valid.data_ptr(), ws.data_ptr(), ws_bytes, sh)
    if st != LONGATTN_OK:
        raise LongAttnError(st, "longattn_tglobal_side")
    out = torch.empty_like(q)
    lse = torch.empty((B, H, n), dtype=torch.float32, device=q.device) if want_lse else None
    st = longattn_tglobal_forward(desc, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  side_k.data_ptr(), side_v.data_ptr(), side_valid.data_ptr(),
                                  bias_local.data_ptr(), bias_side.data_ptr(), out.data_ptr(),
                                  _ptr(lse), ws.data_ptr(), ws_bytes, sh)
    _used_on(stream, out, lse, ws, side_k, side_v, side_valid)
    if st != LONGATTN_OK:
        raise LongAttnError(st, "longattn_tglobal_forward")
    return out, lse, side_k, side_v, side_valid


def longattn_gate_lowrank(desc: longattn_gate_desc, out, w_down, w_up, stream) -> int:
    return load().longattn_gate_lowrank(ctypes.byref(desc), out, w_down, w_up, stream)


def gate_lowrank(out, w_down, w_up, stream=None):
    """Gate ``out`` [B, H, n, d] (bf16, in place) by sigmoid(w_up (w_down o)) over each token's
    H*d outputs; w_down [r, H*d], w_up [H*d, r] bf16.  Returns ``out``."""
    for t in (out, w_down, w_up):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("out, w_down, w_up must be contiguous device tensors")
    B, H, n, d = out.shape
    r = w_down.shape[0]
    if w_down.shape != (r, H * d) or w_up.shape != (H * d, r):
        raise ValueError("w_down must be [r, H*d] and w_up [H*d, r]")
    desc = longattn_gate_desc(batch=B, heads=H, n=n, d=d, rank=r)
    st = longattn_gate_lowrank(desc, out.data_ptr(), w_down.data_ptr(), w_up.data_ptr(),
                               _launch_on(stream))
    if st != LONGATTN_OK:
        raise LongAttnError(st, "longattn_gate_lowrank")
    return out
