"""The C-ABI library: it loads, exports every declared entry point, agrees with the header's
struct layout, and rejects bad arguments before touching the GPU (CPU only)."""

import ctypes
import os
import re
import subprocess

import pytest

import sparse_long_sequence_banded_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "longattn.h")


@pytest.fixture(scope="module", autouse=True)
def _library_built():
    """These tests load the library without a GPU; build it (hipcc cross-compiles for gfx950)
    when no built copy is in the tree."""
    if not os.path.exists(la.LIB_PATH):
        from sparse_long_sequence_banded_amd import build

        build.build()
    yield


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(longattn_[a-z_]+)\s*\(", txt)))


def test_header_declares_the_binding_entry_points():
    assert _declared() == sorted(la.EXPORTED)


def test_library_loads_and_exports_every_declared_symbol():
    lib = ctypes.CDLL(la.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", la.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\b(longattn_\w+)\b", out))
    assert set(_declared()) <= exported


def test_descriptor_layout_matches_the_header(tmp_path):
    fields = [f for f, _ in la.longattn_desc._fields_]
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "longattn.h"\nint main(void){\n'
        + 'printf("%zu\\n", sizeof(longattn_desc));\n'
        + "".join(f'printf("%zu\\n", offsetof(longattn_desc, {f}));\n' for f in fields)
        + "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(la.longattn_desc)
    assert vals[1:] == [getattr(la.longattn_desc, f).offset for f in fields]


def _desc(**kw):
    base = dict(batch=1, heads=2, n=256, d=64, dtype=la.LONGATTN_BF16, scale=0.125, win_left=8,
                win_right=8, dilation=None, global_idx=None, n_global=0, key_pad=None,
                block_layout=None, block=0, max_kb=0)
    base.update(kw)
    return la.longattn_desc(**base)


FAKE = 0x10000  # 16-byte aligned, never dereferenced: these calls fail validation first


@pytest.mark.parametrize("kw,status", [
    (dict(d=0), la.LONGATTN_ERR_INVALID_ARG),
    (dict(n=-1), la.LONGATTN_ERR_INVALID_ARG),
    (dict(dtype=7), la.LONGATTN_ERR_INVALID_ARG),
    (dict(scale=0.0), la.LONGATTN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), la.LONGATTN_ERR_INVALID_ARG),
    (dict(win_left=-1, win_right=4), la.LONGATTN_ERR_INVALID_ARG),
    (dict(win_left=3, win_right=-2), la.LONGATTN_ERR_INVALID_ARG),
    (dict(n_global=3), la.LONGATTN_ERR_INVALID_ARG),            # no global_idx pointer
    (dict(n_global=300, global_idx=FAKE), la.LONGATTN_ERR_INVALID_ARG),  # more than n
    (dict(block_layout=FAKE, block=48, max_kb=2), la.LONGATTN_ERR_INVALID_ARG),  # n % block
    (dict(d=96), la.LONGATTN_ERR_UNSUPPORTED),
    (dict(d=300, dtype=la.LONGATTN_F32), la.LONGATTN_ERR_UNSUPPORTED),
    (dict(block_layout=FAKE, block=64, max_kb=2), la.LONGATTN_ERR_UNSUPPORTED),  # + window
    (dict(block_layout=FAKE, block=32, max_kb=2, win_left=-1, win_right=-1),
     la.LONGATTN_ERR_UNSUPPORTED),
    (dict(n=(1 << 28) + 64), la.LONGATTN_ERR_UNSUPPORTED),
    # bf16 limits: a head's K or V must stay under 2 GiB (32-bit buffer offsets) ...
    (dict(n=1 << 23, d=128), la.LONGATTN_ERR_UNSUPPORTED),
    (dict(n=1 << 24, d=64), la.LONGATTN_ERR_UNSUPPORTED),
    # ... and at most 256 global tokens are staged per workgroup
    (dict(n=4096, n_global=257, global_idx=FAKE), la.LONGATTN_ERR_UNSUPPORTED),
])
def test_bad_descriptors_are_rejected(kw, status):
    d = _desc(**kw)
    st, _ = la.longattn_workspace_size(d)
    assert st == status
    assert la.longattn_forward(d, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == status


def test_largest_supported_sizes_are_accepted():
    # just under the bf16 limits: n*d*2 = 2^31 - 256 bytes per head, 256 global tokens
    assert la.longattn_workspace_size(_desc(n=(1 << 23) - 1, d=128))[0] == la.LONGATTN_OK
    st, nbytes = la.longattn_workspace_size(_desc(n=8192, n_global=256, global_idx=FAKE))
    assert st == la.LONGATTN_OK and nbytes > 0


def test_bad_dilations_are_rejected():
    dil = (ctypes.c_int32 * 2)(1, 0)
    d = _desc(dilation=ctypes.cast(dil, ctypes.c_void_p).value)
    assert la.longattn_workspace_size(d)[0] == la.LONGATTN_ERR_INVALID_ARG
    big = (ctypes.c_int32 * 2)(1, 300)
    d = _desc(dilation=ctypes.cast(big, ctypes.c_void_p).value)
    assert la.longattn_workspace_size(d)[0] == la.LONGATTN_ERR_UNSUPPORTED
    same = (ctypes.c_int32 * 2)(300, 300)  # one dilation for every head: any value
    d = _desc(dilation=ctypes.cast(same, ctypes.c_void_p).value)
    assert la.longattn_workspace_size(d)[0] == la.LONGATTN_OK


def test_pointer_alignment_and_workspace_checks():
    d = _desc()
    assert la.longattn_forward(d, None, FAKE, FAKE, FAKE, None, None, 0, None) == \
        la.LONGATTN_ERR_INVALID_ARG
    assert la.longattn_forward(d, FAKE + 2, FAKE, FAKE, FAKE, None, None, 0, None) == \
        la.LONGATTN_ERR_ALIGNMENT
    dg = _desc(n_global=4, global_idx=FAKE)
    st, nbytes = la.longattn_workspace_size(dg)
    assert st == la.LONGATTN_OK and nbytes > 0
    assert la.longattn_forward(dg, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == \
        la.LONGATTN_ERR_WORKSPACE
    assert la.longattn_forward(dg, FAKE, FAKE, FAKE, FAKE, None, FAKE, nbytes - 1, None) == \
        la.LONGATTN_ERR_WORKSPACE
    assert la.longattn_forward_marked(d, FAKE, FAKE, FAKE, FAKE, None, None, 0, None,
                                      [FAKE, FAKE]) == la.LONGATTN_ERR_INVALID_ARG


def test_workspace_size_formula():
    # global-row partials: B*H*g*chunks*(d+2) floats (the partial output row, its reference and
    # its weight sum; the forward takes chunks of 512 keys: 500 keys -> 1, 1000 -> 2, 3000 -> 6)
    dg = _desc(batch=2, heads=3, n=500, d=128, n_global=5, global_idx=FAKE)
    assert la.longattn_workspace_size(dg) == (la.LONGATTN_OK, 2 * 3 * 5 * 1 * 130 * 4)
    dg = _desc(batch=2, heads=3, n=1000, d=128, n_global=5, global_idx=FAKE)
    assert la.longattn_workspace_size(dg) == (la.LONGATTN_OK, 2 * 3 * 5 * 2 * 130 * 4)
    dg = _desc(batch=2, heads=3, n=3000, d=64, n_global=5, global_idx=FAKE)
    assert la.longattn_workspace_size(dg) == (la.LONGATTN_OK, 2 * 3 * 5 * 6 * 66 * 4)
    # the same with a block layout: 1536 keys -> 3
    dl = _desc(batch=1, heads=2, n=1536, d=64, win_left=-1, win_right=-1, n_global=3,
               global_idx=FAKE, block_layout=FAKE, block=64, max_kb=3)
    assert la.longattn_workspace_size(dl) == (la.LONGATTN_OK, 1 * 2 * 3 * 3 * 66 * 4)
    assert la.longattn_workspace_size(_desc()) == (la.LONGATTN_OK, 0)
    f32 = _desc(dtype=la.LONGATTN_F32, n_global=5, global_idx=FAKE)
    assert la.longattn_workspace_size(f32) == (la.LONGATTN_OK, 0)


def test_empty_problems_launch_nothing():
    for kw in (dict(n=0), dict(batch=0), dict(heads=0)):
        d = _desc(**kw)
        assert la.longattn_workspace_size(d) == (la.LONGATTN_OK, 0)
        assert la.longattn_forward(d, None, None, None, None, None, None, 0, None) == la.LONGATTN_OK


def test_status_strings():
    for s in range(6):
        assert la.longattn_status_string(s) != "unknown status"
    assert la.longattn_status_string(42) == "unknown status"


# ------------------------------------------------------------------------------ decode
def test_decode_descriptor_layout_matches_the_header(tmp_path):
    fields = [f for f, _ in la.longattn_decode_desc._fields_]
    src = tmp_path / "dlayout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "longattn.h"\nint main(void){\n'
        + 'printf("%zu\\n", sizeof(longattn_decode_desc));\n'
        + "".join(f'printf("%zu\\n", offsetof(longattn_decode_desc, {f}));\n' for f in fields)
        + "return 0;}\n")
    exe = tmp_path / "dlayout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(la.longattn_decode_desc)
    assert vals[1:] == [getattr(la.longattn_decode_desc, f).offset for f in fields]


def _ddesc(**kw):
    base = dict(batch=2, heads=3, d=128, dtype=la.LONGATTN_BF16, scale=0.0884, window=512,
                n_queries=1, cache_len=4096, ring=0, positions=FAKE)
    base.update(kw)
    return la.longattn_decode_desc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(d=0), la.LONGATTN_ERR_INVALID_ARG),
    (dict(batch=-1), la.LONGATTN_ERR_INVALID_ARG),
    (dict(dtype=5), la.LONGATTN_ERR_INVALID_ARG),
    (dict(scale=-1.0), la.LONGATTN_ERR_INVALID_ARG),
    (dict(scale=float("inf")), la.LONGATTN_ERR_INVALID_ARG),
    (dict(window=0), la.LONGATTN_ERR_INVALID_ARG),
    (dict(n_queries=0), la.LONGATTN_ERR_INVALID_ARG),
    (dict(cache_len=0), la.LONGATTN_ERR_INVALID_ARG),
    (dict(ring=2), la.LONGATTN_ERR_INVALID_ARG),
    (dict(positions=None), la.LONGATTN_ERR_INVALID_ARG),
    # a rolling buffer shorter than window + m - 1 would overwrite positions still needed
    (dict(ring=1, cache_len=512, n_queries=2), la.LONGATTN_ERR_INVALID_ARG),
    (dict(d=100), la.LONGATTN_ERR_UNSUPPORTED),
    (dict(d=264), la.LONGATTN_ERR_UNSUPPORTED),
    (dict(n_queries=17), la.LONGATTN_ERR_UNSUPPORTED),
    (dict(cache_len=1 << 23), la.LONGATTN_ERR_UNSUPPORTED),  # 2 GiB per (b, h) cache
])
def test_bad_decode_descriptors_are_rejected(kw, status):
    d = _ddesc(**kw)
    st, _ = la.longattn_decode_workspace_size(d)
    assert st == status
    assert la.longattn_decode(d, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == status


def test_decode_workspace_formula_and_checks():
    # partials: B*H*m rows x chunks x (d + 2) floats; a chunk is 4 or 8 waves of 16 loads of
    # 16 bytes per lane (positions per wave: 64 for bf16 d=128, 64 for fp32 d=64), 4 waves when
    # 8-wave chunks would give fewer than 512 workgroups; no workspace when one chunk covers
    # the window
    d = _ddesc()
    assert la.longattn_decode_workspace_size(d) == (la.LONGATTN_OK, 2 * 3 * 1 * 2 * 130 * 4)
    d = _ddesc(window=4000, n_queries=5, d=64, dtype=la.LONGATTN_F32)
    assert la.longattn_decode_workspace_size(d) == (la.LONGATTN_OK, 2 * 3 * 5 * 16 * 66 * 4)
    d = _ddesc(batch=32, heads=16)  # 512 workgroups of 8 waves, one per window
    assert la.longattn_decode_workspace_size(d) == (la.LONGATTN_OK, 0)
    d = _ddesc(batch=32, heads=16, window=200)  # a 4-wave chunk covers the window
    assert la.longattn_decode_workspace_size(d) == (la.LONGATTN_OK, 0)
    d = _ddesc(d=24, window=300, n_queries=2)  # other head dims: 256-position chunks, always
    assert la.longattn_decode_workspace_size(d) == (la.LONGATTN_OK, 2 * 3 * 2 * 2 * 26 * 4)
    d = _ddesc(ring=1, cache_len=512)  # exactly window + m - 1 slots
    st, nbytes = la.longattn_decode_workspace_size(d)
    assert st == la.LONGATTN_OK
    assert la.longattn_decode(d, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == \
        la.LONGATTN_ERR_WORKSPACE
    assert la.longattn_decode(d, FAKE, FAKE, FAKE, FAKE, None, FAKE, nbytes - 1, None) == \
        la.LONGATTN_ERR_WORKSPACE
    assert la.longattn_decode(d, FAKE + 8, FAKE, FAKE, FAKE, None, FAKE, nbytes, None) == \
        la.LONGATTN_ERR_ALIGNMENT
    assert la.longattn_decode(d, FAKE, None, FAKE, FAKE, None, FAKE, nbytes, None) == \
        la.LONGATTN_ERR_INVALID_ARG


def test_empty_decode_launches_nothing():
    for kw in (dict(batch=0, positions=None), dict(heads=0, positions=None)):
        d = _ddesc(**kw)
        assert la.longattn_decode_workspace_size(d) == (la.LONGATTN_OK, 0)
        assert la.longattn_decode(d, None, None, None, None, None, None, 0, None) == \
            la.LONGATTN_OK


# ------------------------------------------------------------------------------ backward
@pytest.mark.parametrize("kw,status", [
    (dict(d=0), la.LONGATTN_ERR_INVALID_ARG),
    (dict(scale=0.0), la.LONGATTN_ERR_INVALID_ARG),
    (dict(win_left=-1, win_right=4), la.LONGATTN_ERR_INVALID_ARG),
    (dict(n_global=3), la.LONGATTN_ERR_INVALID_ARG),
    (dict(d=300), la.LONGATTN_ERR_UNSUPPORTED),
])
def test_bad_backward_descriptors_are_rejected(kw, status):
    d = _desc(**kw)
    assert la.longattn_backward_workspace_size(d)[0] == status
    assert la.longattn_backward(d, *([FAKE] * 9), FAKE, 1 << 30, None) == status


def test_backward_workspace_and_pointer_checks():
    d = _desc(batch=2, heads=3, n=500, d=40, dtype=la.LONGATTN_F32)
    st, nbytes = la.longattn_backward_workspace_size(d)
    assert st == la.LONGATTN_OK and nbytes == 2 * 3 * 500 * 4  # one float per row
    # layouts combined with a window are fine for the backward in both dtypes
    dl = _desc(block_layout=FAKE, block=16, max_kb=2)
    assert la.longattn_backward_workspace_size(dl)[0] == la.LONGATTN_OK
    args = [FAKE] * 9
    assert la.longattn_backward(d, *args, None, 0, None) == la.LONGATTN_ERR_WORKSPACE
    assert la.longattn_backward(d, *args, FAKE, nbytes - 1, None) == la.LONGATTN_ERR_WORKSPACE
    for slot in range(9):
        bad = list(args)
        bad[slot] = None
        assert la.longattn_backward(d, *bad, FAKE, nbytes, None) == la.LONGATTN_ERR_INVALID_ARG
        bad[slot] = FAKE + (2 if slot == 4 else 8)  # lse needs 4-byte alignment, tensors 16
        assert la.longattn_backward(d, *bad, FAKE, nbytes, None) == la.LONGATTN_ERR_ALIGNMENT
    assert la.longattn_backward_workspace_size(_desc(n=0)) == (la.LONGATTN_OK, 0)
    assert la.longattn_backward(_desc(n=0), *([None] * 9), None, 0, None) == la.LONGATTN_OK


def test_backward_matrix_core_workspace_formula():
    # bf16, d in {64, 128}, no layout: Drow and lse2 per row (padded to 4 floats each) plus the
    # global rows' partials: 3 * B*H*g*chunks*d floats (chunks of 512 rows: 1001 rows -> 2)
    d = _desc(batch=2, heads=3, n=1001, d=64, n_global=5, global_idx=FAKE)
    rows_pad = (2 * 3 * 1001 + 3) // 4 * 4
    assert la.longattn_backward_workspace_size(d) == (la.LONGATTN_OK,
                                                      (2 * rows_pad + 3 * 2 * 3 * 5 * 2 * 64) * 4)
    d = _desc(batch=1, heads=2, n=3000, d=128)
    assert la.longattn_backward_workspace_size(d) == (la.LONGATTN_OK, 2 * 6000 * 4)
    # a layout of 64- or 128-blocks alone also runs on matrix cores ...
    dl = _desc(block_layout=FAKE, block=64, max_kb=2, win_left=-1, win_right=-1)
    assert la.longattn_backward_workspace_size(dl) == (la.LONGATTN_OK, 2 * 512 * 4)
    # ... a layout together with a window, other head dims or fp32 take the per-row kernels:
    # one float per row
    dw = _desc(block_layout=FAKE, block=64, max_kb=2)
    assert la.longattn_backward_workspace_size(dw) == (la.LONGATTN_OK, 2 * 256 * 4)
    assert la.longattn_backward_workspace_size(_desc(d=96)) == (la.LONGATTN_OK, 2 * 256 * 4)
    assert la.longattn_backward_marked(_desc(), *([FAKE] * 9), FAKE, 1 << 30, None,
                                       [FAKE] * 3) == la.LONGATTN_ERR_INVALID_ARG


# ------------------------------------------------------------------------------ TGlobal
def test_tglobal_descriptor_layout_matches_the_header(tmp_path):
    fields = [f for f, _ in la.longattn_tglobal_desc._fields_]
    src = tmp_path / "tlayout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "longattn.h"\nint main(void){\n'
        + 'printf("%zu\\n", sizeof(longattn_tglobal_desc));\n'
        + "".join(f'printf("%zu\\n", offsetof(longattn_tglobal_desc, {f}));\n' for f in fields)
        + "return 0;}\n")
    exe = tmp_path / "tlayout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(la.longattn_tglobal_desc)
    assert vals[1:] == [getattr(la.longattn_tglobal_desc, f).offset for f in fields]


def _tdesc(**kw):
    base = dict(batch=1, heads=8, n=16384, d=64, d_model=512, scale=0.125, radius=127, block=16,
                num_buckets=32, max_distance=128, eps=1e-6, key_pad=None)
    base.update(kw)
    return la.longattn_tglobal_desc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(heads=0), la.LONGATTN_ERR_INVALID_ARG),
    (dict(scale=0.0), la.LONGATTN_ERR_INVALID_ARG),
    (dict(eps=-1.0), la.LONGATTN_ERR_INVALID_ARG),
    (dict(radius=-1), la.LONGATTN_ERR_INVALID_ARG),
    (dict(block=0), la.LONGATTN_ERR_INVALID_ARG),
    (dict(num_buckets=31), la.LONGATTN_ERR_INVALID_ARG),
    (dict(num_buckets=2), la.LONGATTN_ERR_INVALID_ARG),
    (dict(d=96), la.LONGATTN_ERR_UNSUPPORTED),
    (dict(radius=513), la.LONGATTN_ERR_UNSUPPORTED),
    (dict(max_distance=600), la.LONGATTN_ERR_UNSUPPORTED),
    # W [d_model][heads * d] must stay under 2^31 bytes
    (dict(heads=1 << 16, d=128, d_model=128), la.LONGATTN_ERR_UNSUPPORTED),
])
def test_bad_tglobal_descriptors_are_rejected(kw, status):
    d = _tdesc(**kw)
    assert la.longattn_tglobal_workspace_size(d)[0] == status
    assert la.longattn_tglobal_side(d, *([FAKE] * 7), FAKE, 1 << 30, None) == status
    assert la.longattn_tglobal_forward(d, *([FAKE] * 10), FAKE, 1 << 30, None) == status


def test_tglobal_workspace_covers_both_calls():
    # max(B*G*d_model aggregates, H*(2*(r+191)+1 + 2*md+1) bias entries) floats
    st, nbytes = la.longattn_tglobal_workspace_size(_tdesc())
    assert st == la.LONGATTN_OK and nbytes == max(1024 * 512, 8 * (2 * 318 + 1 + 257)) * 4
    st, nbytes = la.longattn_tglobal_workspace_size(_tdesc(n=100, d_model=64))
    assert nbytes == max(6 * 64, 8 * (2 * (99 + 191) + 1 + 257)) * 4  # radius clamps to n - 1
    assert la.longattn_tglobal_workspace_size(_tdesc(d_model=96))[0] == la.LONGATTN_ERR_UNSUPPORTED
    d = _tdesc()
    assert la.longattn_tglobal_side(d, *([FAKE] * 7), None, 0, None) == la.LONGATTN_ERR_WORKSPACE
    assert la.longattn_tglobal_forward(d, *([FAKE] * 10), FAKE, nbytes - 1, None) == \
        la.LONGATTN_ERR_WORKSPACE
    assert la.longattn_tglobal_forward(d, FAKE + 2, *([FAKE] * 9), FAKE, 1 << 30, None) == \
        la.LONGATTN_ERR_ALIGNMENT
    # the workspace itself must be 16-byte aligned
    assert la.longattn_tglobal_side(d, *([FAKE] * 7), FAKE + 4, 1 << 30, None) == \
        la.LONGATTN_ERR_ALIGNMENT
    assert la.longattn_tglobal_forward(d, *([FAKE] * 10), FAKE + 8, 1 << 30, None) == \
        la.LONGATTN_ERR_ALIGNMENT
    assert la.longattn_tglobal_side(_tdesc(batch=0), *([None] * 7), None, 0, None) == \
        la.LONGATTN_OK


# ------------------------------------------------------------------------------ output gates
def test_gate_descriptor_layout_matches_the_header(tmp_path):
    fields = [f for f, _ in la.longattn_gate_desc._fields_]
    src = tmp_path / "glayout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "longattn.h"\nint main(void){\n'
        + 'printf("%zu\\n", sizeof(longattn_gate_desc));\n'
        + "".join(f'printf("%zu\\n", offsetof(longattn_gate_desc, {f}));\n' for f in fields)
        + "return 0;}\n")
    exe = tmp_path / "glayout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(la.longattn_gate_desc)
    assert vals[1:] == [getattr(la.longattn_gate_desc, f).offset for f in fields]


@pytest.mark.parametrize("kw,status", [
    (dict(heads=0), la.LONGATTN_ERR_INVALID_ARG),
    (dict(rank=0), la.LONGATTN_ERR_INVALID_ARG),
    (dict(rank=100), la.LONGATTN_ERR_UNSUPPORTED),
    (dict(d=24), la.LONGATTN_ERR_UNSUPPORTED),
    (dict(heads=3, d=16), la.LONGATTN_ERR_UNSUPPORTED),  # H*d not a multiple of 32
])
def test_bad_gate_descriptors_are_rejected(kw, status):
    base = dict(batch=1, heads=16, n=100, d=64, rank=128)
    base.update(kw)
    d = la.longattn_gate_desc(**base)
    assert la.longattn_gate_lowrank(d, FAKE, FAKE, FAKE, None) == status


def test_gate_pointer_checks():
    d = la.longattn_gate_desc(batch=1, heads=16, n=100, d=64, rank=128)
    assert la.longattn_gate_lowrank(d, None, FAKE, FAKE, None) == la.LONGATTN_ERR_INVALID_ARG
    assert la.longattn_gate_lowrank(d, FAKE + 8, FAKE, FAKE, None) == la.LONGATTN_ERR_ALIGNMENT
    e = la.longattn_gate_desc(batch=0, heads=16, n=100, d=64, rank=128)
    assert la.longattn_gate_lowrank(e, None, None, None, None) == la.LONGATTN_OK
    f = _desc()
    assert la.longattn_forward_gated(f, FAKE, FAKE, FAKE, None, FAKE, None, None, 0, None) == \
        la.LONGATTN_ERR_INVALID_ARG
    assert la.longattn_forward_gated(f, FAKE, FAKE, FAKE, FAKE + 4, FAKE, None, None, 0, None) == \
        la.LONGATTN_ERR_ALIGNMENT
