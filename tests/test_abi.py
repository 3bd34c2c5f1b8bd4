"""The C ABI library loads, exports every declared symbol and validates arguments on the host.

Nothing here launches a kernel: every call below is rejected (or is a no-op)
before the library makes any HIP call, so it runs on a CPU-only machine.
"""
import ctypes
import os
import re

import pytest

from scaled_dot_product_08_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(attn_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_header_declares_expected_entry_points():
    assert set(_declared_functions()) == set(binding.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_strerror(lib):
    assert binding.attn_version() >= 10000
    for code, name in binding.STATUS.items():
        assert binding.attn_strerror(code)
    assert binding.attn_strerror(12345) == "unknown status"


P = 1 << 20   # a 16-byte-aligned fake device address (never dereferenced)


def call(q=P, k=P, v=P, o=P, lse=None, B=1, H=2, S=128, D=64, causal=0, scale=0.125,
         dtype=binding.ATTN_DTYPE_FP16, cu=None):
    return binding.attn_fwd_raw(q, k, v, o, lse, B, H, S, D, causal, scale, dtype, cu, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1),
    (dict(dtype=2), -3), (dict(dtype=-1), -3),
    (dict(D=96), -5), (dict(D=256), -5), (dict(D=0), -5),
    (dict(scale=float("nan")), -4), (dict(scale=float("inf")), -4), (dict(scale=-float("inf")), -4),
    (dict(H=0), -2), (dict(H=70000), -2), (dict(B=0), -2), (dict(S=-1), -2), (dict(B=-1, cu=P), -2),
    (dict(q=P + 8), -8), (dict(o=P + 2), -8), (dict(lse=P + 2), -8),
    (dict(B=4096, H=4096, S=1 << 30), -2),
])
def test_argument_errors(kw, code):
    assert call(**kw) == code


@pytest.mark.parametrize("kw", [dict(S=0), dict(B=0, S=0, cu=P), dict(B=0, S=100, cu=P)])
def test_empty_problems_are_noops(kw):
    # Returns before any HIP call: nothing to compute.
    assert call(**kw) == 0


def call_tuned(tile_rows=0, head_group=0, key_split=0, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, H=2, S=128, D=64, causal=0, scale=0.125,
             dtype=binding.ATTN_DTYPE_FP16, cu=None)
    a.update(kw)
    return binding.attn_fwd_tuned_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                      a["S"], a["D"], a["causal"], a["scale"], a["dtype"], a["cu"],
                                      tile_rows, key_split, head_group, None)


@pytest.mark.parametrize("kw,code", [
    (dict(tile_rows=64), -5), (dict(tile_rows=-128), -5), (dict(tile_rows=512), -5),
    (dict(head_group=-1), -2), (dict(tile_rows=128, D=96), -5), (dict(head_group=3, q=None), -1),
    (dict(tile_rows=256, scale=float("nan")), -4), (dict(tile_rows=256, H=0), -2),
    (dict(key_split=3), -5), (dict(key_split=-1), -5), (dict(tile_rows=256, key_split=2), -5),
])
def test_tuned_argument_errors(kw, code):
    assert call_tuned(**kw) == code


@pytest.mark.parametrize("kw", [dict(tile_rows=128, S=0), dict(tile_rows=256, head_group=9, S=0),
                                dict(tile_rows=256, B=0, S=10, cu=P)])
def test_tuned_empty_problems_are_noops(kw):
    assert call_tuned(**kw) == 0


def call_ext(window=0, n_global=0, alibi=None, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, H=2, S=128, D=64, causal=0, scale=0.125,
             dtype=binding.ATTN_DTYPE_FP16, cu=None)
    a.update(kw)
    return binding.attn_fwd_ext_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["S"],
                                    a["D"], a["causal"], a["scale"], a["dtype"], a["cu"], window,
                                    n_global, alibi, None)


@pytest.mark.parametrize("kw,code", [
    (dict(window=-1), -2), (dict(n_global=-5), -2), (dict(alibi=P + 2), -8),
    (dict(D=80, window=8), -5), (dict(q=None, window=8), -1), (dict(scale=float("nan"), n_global=2), -4),
])
def test_ext_argument_errors(kw, code):
    assert call_ext(**kw) == code


def test_ext_empty_problem_is_noop():
    assert call_ext(window=16, S=0) == 0


def call_ext_tuned(window=0, n_global=0, alibi=P, tile_rows=256, head_group=0, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, H=2, S=128, D=128, causal=1, scale=0.125,
             dtype=binding.ATTN_DTYPE_BF16, cu=None)
    a.update(kw)
    return binding.attn_fwd_ext_tuned_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                          a["S"], a["D"], a["causal"], a["scale"], a["dtype"],
                                          a["cu"], window, n_global, alibi, tile_rows, head_group,
                                          None)


@pytest.mark.parametrize("kw,code", [
    (dict(tile_rows=64), -5), (dict(tile_rows=512), -5), (dict(window=8), -5), (dict(n_global=1), -5),
    (dict(alibi=None), -5), (dict(D=64), -5), (dict(head_group=-1), -2), (dict(alibi=P + 2), -8),
    (dict(tile_rows=128, window=-1), -2), (dict(q=None), -1), (dict(scale=float("nan")), -4),
])
def test_ext_tuned_argument_errors(kw, code):
    assert call_ext_tuned(**kw) == code


@pytest.mark.parametrize("kw", [dict(S=0), dict(tile_rows=128, window=4, S=0), dict(B=0, S=7, cu=P)])
def test_ext_tuned_empty_problems_are_noops(kw):
    assert call_ext_tuned(**kw) == 0


def call_dec(**kw):
    a = dict(q=P, k=P, v=P, sl=None, o=P, lse=None, B=2, H=4, Sq=1, S_max=4096, D=128, causal=0,
             scale=0.1, dtype=binding.ATTN_DTYPE_BF16, ns=0, ws=None, wsb=0)
    a.update(kw)
    return binding.attn_decode_raw(a["q"], a["k"], a["v"], a["sl"], a["o"], a["lse"], a["B"],
                                   a["H"], a["Sq"], a["S_max"], a["D"], a["causal"], a["scale"],
                                   a["dtype"], a["ns"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1),
    (dict(dtype=5), -3), (dict(D=80), -5), (dict(scale=float("inf")), -4),
    (dict(H=0), -2), (dict(B=-1), -2), (dict(Sq=-1), -2), (dict(S_max=-1), -2), (dict(ns=-2), -2),
    (dict(S_max=1 << 24), -2),
    (dict(q=P + 4), -8), (dict(lse=P + 1), -8), (dict(ns=1, sl=P + 2), -8),
    (dict(ns=4), -9), (dict(ns=4, ws=P, wsb=100), -9),
])
def test_decode_argument_errors(kw, code):
    assert call_dec(**kw) == code


def test_decode_workspace_size_rules(lib):
    ws = binding.decode_workspace_size
    assert ws(2, 4, 1, 4096, 128, 1) == 0                    # one split: no workspace
    n = ws(2, 4, 1, 4096, 128, 4)
    assert n == 2 * 4 * 1 * 4 * 129 * 4                      # rows x splits x (D + 1) floats
    assert ws(4, 32, 1, 65536, 128, 0) > 0                   # automatic split count
    assert ws(4, 32, 1, 65536, 128, 100000) <= 4 * 32 * 256 * 129 * 4   # capped at 256 splits
    assert ws(1, 1, 1, 0, 64, 0) == 0
    # a too-small workspace is refused before anything is enqueued
    assert call_dec(ns=4, ws=P, wsb=n // 2 - 1, B=2, H=4) == -9


def test_decode_empty_problem_is_noop():
    assert call_dec(B=0) == 0
    assert call_dec(Sq=0) == 0


def call_bwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, H=2, S=128, D=128, causal=0,
             scale=0.1, dtype=binding.ATTN_DTYPE_BF16, cu=None, ws=None, wsb=0)
    a.update(kw)
    return binding.attn_bwd_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                                a["dv"], a["B"], a["H"], a["S"], a["D"], a["causal"], a["scale"],
                                a["dtype"], a["cu"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(lse=None), -1), (dict(do=None), -1),
    (dict(dq=None), -1), (dict(dk=None), -1), (dict(dv=None), -1),
    (dict(dtype=7), -3), (dict(D=32), -5), (dict(scale=float("nan")), -4), (dict(H=0), -2),
    (dict(do=P + 8), -8), (dict(dv=P + 2), -8), (dict(lse=P + 1), -8),
    (dict(), -9), (dict(ws=P, wsb=2 * 2 * 128 * 4 - 1), -9), (dict(ws=P + 4, wsb=1 << 20), -8),
])
def test_bwd_argument_errors(kw, code):
    assert call_bwd(**kw) == code


def test_bwd_workspace_and_empty(lib):
    assert binding.bwd_workspace_size(2, 3, 100, False) == 2 * 2 * 3 * 100 * 4
    assert binding.bwd_workspace_size(5, 3, 100, True) == 2 * 3 * 100 * 4
    assert call_bwd(S=0) == 0
    assert call_bwd(B=0, cu=P, S=10) == 0


def call_fp8(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, H=2, S=128, D=128, causal=0, scale=0.1, dq=1.0,
             dk=1.0, dv=1.0, od=binding.ATTN_DTYPE_BF16, cu=None)
    a.update(kw)
    return binding.attn_fwd_fp8_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["S"],
                                    a["D"], a["causal"], a["scale"], a["dq"], a["dk"], a["dv"],
                                    a["od"], a["cu"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(od=3), -3), (dict(D=64), -5), (dict(D=96), -5),
    (dict(dq=float("inf")), -4), (dict(dv=float("nan")), -4), (dict(scale=1e30, dq=1e30), -4),
    (dict(k=P + 8), -8), (dict(H=0), -2),
])
def test_fp8_argument_errors(kw, code):
    assert call_fp8(**kw) == code


def test_fp8_empty_problem_is_noop():
    assert call_fp8(S=0) == 0


def test_binding_rejects_mismatched_tensors():
    """The Python binding checks shapes, dtypes and devices before any library call."""
    import torch
    q = torch.zeros(1, 8, 2, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        binding.attn_fwd(q, q, q, q, causal=False)
    with pytest.raises(ValueError):
        binding.fwd_fp8(q, q, q, causal=False)
    with pytest.raises(ValueError):
        binding.attn_decode(q, q, q, q)


def call_dec_noalloc(**kw):
    a = dict(q=P, k=P, v=P, sl=None, o=P, lse=None, B=2, H=4, Sq=1, S_max=4096, D=128, causal=0,
             scale=0.1, dtype=binding.ATTN_DTYPE_BF16, ns=0)
    a.update(kw)
    return binding.attn_decode_noalloc_raw(a["q"], a["k"], a["v"], a["sl"], a["o"], a["lse"],
                                           a["B"], a["H"], a["Sq"], a["S_max"], a["D"],
                                           a["causal"], a["scale"], a["dtype"], a["ns"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(D=96), -5), (dict(dtype=7), -3), (dict(scale=float("nan")), -4),
    (dict(H=0), -2), (dict(ns=-1), -2), (dict(sl=P + 2), -8), (dict(o=P + 4), -8),
    # 8192 query rows x 64 explicit splits x 129 floats: 270 MB of partials > 16 MiB
    (dict(B=64, H=32, Sq=4, S_max=8192, ns=64), -10),
])
def test_decode_noalloc_argument_errors(kw, code):
    assert call_dec_noalloc(**kw) == code


def test_decode_noalloc_empty_problem_is_noop():
    assert call_dec_noalloc(B=0) == 0
    assert call_dec_noalloc(Sq=0, ns=3) == 0


def test_one_hip_runtime_in_the_process(lib):
    """Loading the library through the binding leaves exactly one HIP runtime in the process
    (torch's, which the library's dependency then resolves to)."""
    maps = open("/proc/self/maps").read()
    hips = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(hips) == 1, hips


def test_clock_sample_argument_errors(lib):
    assert lib.attn_clock_sample(None, None) == -1
    assert lib.attn_clock_sample(P + 4, None) == -8
