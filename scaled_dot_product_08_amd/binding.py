"""ctypes binding of the C ABI in include/attn.h (argument marshalling only).

Every step of the attention forward runs in the HIP library; this module
only turns torch tensors into device pointers, sizes and a stream handle.
There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import math
import os

ATTN_DTYPE_FP16 = 0
ATTN_DTYPE_BF16 = 1

STATUS = {
    0: "ATTN_OK", -1: "ATTN_ERR_NULL", -2: "ATTN_ERR_SHAPE", -3: "ATTN_ERR_DTYPE",
    -4: "ATTN_ERR_SCALE", -5: "ATTN_ERR_UNSUPPORTED", -6: "ATTN_ERR_LAUNCH",
    -7: "ATTN_ERR_SEQLENS", -8: "ATTN_ERR_ALIGN", -9: "ATTN_ERR_WORKSPACE",
    -10: "ATTN_ERR_SCRATCH",
}
EXPORTS = ("attn_fwd", "attn_fwd_tuned", "attn_fwd_ext", "attn_fwd_ext_tuned", "attn_fwd_fp8", "attn_bwd", "attn_bwd_workspace_size", "attn_decode",
           "attn_decode_noalloc", "attn_decode_workspace_size", "attn_strerror", "attn_check_cu_seqlens", "attn_version",
           "attn_last_hip_error", "attn_clock_sample")

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libsdpa08.so")
_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, text: str):
        hip = None
        if status == -6 and _lib is not None:
            hip = int(_lib.attn_last_hip_error())
            text = f"{text} (hipError_t {hip})"
        super().__init__(f"{STATUS.get(status, status)}: {text}")
        self.status = status
        self.hip_error = hip


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load the built HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"HIP attention library not built: {p} "
                           "(run python -m scaled_dot_product_08_amd.build)")
    # One HIP runtime per process. torch bundles its own libamdhip64 under the same soname;
    # loaded first, it also serves this library. Loading this library first would bring the
    # system runtime in beside torch's, and of two runtimes in one process one sees no device
    # (its launches fail with hipErrorNoDevice).
    import torch  # noqa: F401
    lib = ctypes.CDLL(p)
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + \
        [ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.attn_fwd_tuned.restype = ctypes.c_int
    lib.attn_fwd_tuned.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + \
        [ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
         ctypes.c_void_p]
    lib.attn_fwd_ext.restype = ctypes.c_int
    lib.attn_fwd_ext.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + \
        [ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
         ctypes.c_void_p]
    lib.attn_fwd_ext_tuned.restype = ctypes.c_int
    lib.attn_fwd_ext_tuned.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + \
        [ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
         ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.attn_fwd_fp8.restype = ctypes.c_int
    lib.attn_fwd_fp8.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + [ctypes.c_float] * 4 + \
        [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int] * 5 + \
        [ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
         ctypes.c_void_p]
    lib.attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.attn_bwd_workspace_size.argtypes = [ctypes.c_int] * 4
    lib.attn_decode.restype = ctypes.c_int
    lib.attn_decode.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int] * 6 + \
        [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
         ctypes.c_void_p]
    lib.attn_decode_noalloc.restype = ctypes.c_int
    lib.attn_decode_noalloc.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int] * 6 + \
        [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.attn_decode_workspace_size.restype = ctypes.c_size_t
    lib.attn_decode_workspace_size.argtypes = [ctypes.c_int] * 6
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_strerror.argtypes = [ctypes.c_int]
    lib.attn_check_cu_seqlens.restype = ctypes.c_int
    lib.attn_check_cu_seqlens.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.attn_version.restype = ctypes.c_int
    lib.attn_version.argtypes = []
    lib.attn_last_hip_error.restype = ctypes.c_int
    lib.attn_last_hip_error.argtypes = []
    lib.attn_clock_sample.restype = ctypes.c_int
    lib.attn_clock_sample.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    if path is None:
        _lib = lib
    return lib


def attn_strerror(status: int) -> str:
    return load_library().attn_strerror(int(status)).decode()


CLOCK_SLOTS = 1024      # CU slots of attn_clock_sample (8 XCDs x 128)


def clock_sample(dst, stream=None) -> None:
    """Enqueue attn_clock_sample into ``dst`` (a device int64 tensor of 2048 elements: per CU
    slot, its shader-clock counter and the 100 MHz real-time counter)."""
    if dst.numel() < 2 * CLOCK_SLOTS or not dst.is_cuda or dst.element_size() != 8:
        raise ValueError("clock_sample takes a device tensor of 2048 int64")
    st = load_library().attn_clock_sample(dst.data_ptr(), _stream_ptr(stream))
    if st != 0:
        raise AttnError(st, attn_strerror(st))


def clock_mhz(before, after) -> list:
    """Average shader clock (MHz) of every CU slot that both samples (host lists of 2048 ints,
    taken from zero-filled buffers) recorded and whose counter advanced."""
    out = []
    for s in range(CLOCK_SLOTS):
        t0, r0, t1, r1 = before[2 * s], before[2 * s + 1], after[2 * s], after[2 * s + 1]
        if t0 and t1 and r1 > r0 and t1 > t0:
            out.append((t1 - t0) / (r1 - r0) * 100.0)
    return out


def attn_version() -> int:
    return load_library().attn_version()


def attn_fwd_raw(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, B, H, S, D, causal, scale, dtype,
                 cu_ptr, stream_ptr) -> int:
    """Direct call with integer pointers; returns the status code."""
    return load_library().attn_fwd(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, int(B), int(H), int(S),
                                   int(D), int(causal), float(scale), int(dtype), cu_ptr, stream_ptr)


def attn_fwd_tuned_raw(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, B, H, S, D, causal, scale, dtype,
                       cu_ptr, tile_rows, key_split, head_group, stream_ptr) -> int:
    """Direct call of attn_fwd_tuned with integer pointers; returns the status code."""
    return load_library().attn_fwd_tuned(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, int(B), int(H),
                                         int(S), int(D), int(causal), float(scale), int(dtype),
                                         cu_ptr, int(tile_rows), int(key_split), int(head_group),
                                         stream_ptr)


def attn_fwd_ext_raw(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, B, H, S, D, causal, scale, dtype,
                     cu_ptr, window, n_global, alibi_ptr, stream_ptr) -> int:
    """Direct call of attn_fwd_ext with integer pointers; returns the status code."""
    return load_library().attn_fwd_ext(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, int(B), int(H), int(S),
                                       int(D), int(causal), float(scale), int(dtype), cu_ptr,
                                       int(window), int(n_global), alibi_ptr, stream_ptr)


def attn_fwd_ext_tuned_raw(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, B, H, S, D, causal, scale, dtype,
                           cu_ptr, window, n_global, alibi_ptr, tile_rows, head_group, stream_ptr) -> int:
    """Direct call of attn_fwd_ext_tuned with integer pointers; returns the status code."""
    return load_library().attn_fwd_ext_tuned(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, int(B), int(H),
                                             int(S), int(D), int(causal), float(scale), int(dtype),
                                             cu_ptr, int(window), int(n_global), alibi_ptr,
                                             int(tile_rows), int(head_group), stream_ptr)


def attn_decode_raw(q_ptr, k_ptr, v_ptr, seqlens_ptr, out_ptr, lse_ptr, B, H, Sq, S_max, D, causal,
                    scale, dtype, num_splits, ws_ptr, ws_bytes, stream_ptr) -> int:
    """Direct call of attn_decode with integer pointers; returns the status code."""
    return load_library().attn_decode(q_ptr, k_ptr, v_ptr, seqlens_ptr, out_ptr, lse_ptr, int(B),
                                      int(H), int(Sq), int(S_max), int(D), int(causal),
                                      float(scale), int(dtype), int(num_splits), ws_ptr,
                                      int(ws_bytes), stream_ptr)


def attn_decode_noalloc_raw(q_ptr, k_ptr, v_ptr, seqlens_ptr, out_ptr, lse_ptr, B, H, Sq, S_max, D,
                            causal, scale, dtype, num_splits, stream_ptr) -> int:
    """Direct call of attn_decode_noalloc with integer pointers; returns the status code."""
    return load_library().attn_decode_noalloc(q_ptr, k_ptr, v_ptr, seqlens_ptr, out_ptr, lse_ptr,
                                              int(B), int(H), int(Sq), int(S_max), int(D),
                                              int(causal), float(scale), int(dtype),
                                              int(num_splits), stream_ptr)


def attn_fwd_fp8_raw(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, B, H, S, D, causal, scale, dq, dk, dv,
                     out_dtype, cu_ptr, stream_ptr) -> int:
    """Direct call of attn_fwd_fp8 with integer pointers; returns the status code."""
    return load_library().attn_fwd_fp8(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, int(B), int(H), int(S),
                                       int(D), int(causal), float(scale), float(dq), float(dk),
                                       float(dv), int(out_dtype), cu_ptr, stream_ptr)


def attn_bwd_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr, dv_ptr, B, H, S, D,
                 causal, scale, dtype, cu_ptr, ws_ptr, ws_bytes, stream_ptr) -> int:
    """Direct call of attn_bwd with integer pointers; returns the status code."""
    return load_library().attn_bwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr,
                                   dv_ptr, int(B), int(H), int(S), int(D), int(causal),
                                   float(scale), int(dtype), cu_ptr, ws_ptr, int(ws_bytes),
                                   stream_ptr)


def bwd_workspace_size(B, H, S, packed=False) -> int:
    return int(load_library().attn_bwd_workspace_size(int(B), int(H), int(S), int(bool(packed))))


def decode_workspace_size(B, H, Sq, S_max, D, num_splits=0) -> int:
    return int(load_library().attn_decode_workspace_size(int(B), int(H), int(Sq), int(S_max),
                                                          int(D), int(num_splits)))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return ATTN_DTYPE_FP16
    if t.dtype == torch.bfloat16:
        return ATTN_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def torch_float32():
    import torch
    return torch.float32


def _check_tensors(names, tensors, shape=None, dtype=None):
    """Same shape, dtype and GPU device, contiguous (the library reads raw pointers)."""
    first = tensors[0]
    shape = tuple(first.shape) if shape is None else tuple(shape)
    dtype = first.dtype if dtype is None else dtype
    for n, t in zip(names, tensors):
        if not t.is_cuda:
            raise ValueError(f"{n} must be a GPU tensor")
        if t.device != first.device:
            raise ValueError(f"{n} is on {t.device}, expected {first.device}")
        if tuple(t.shape) != shape:
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {shape}")
        if t.dtype != dtype:
            raise ValueError(f"{n} has dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")


def _check_aux(lse, lse_shape, cu_seqlens, device):
    import torch
    if lse is not None:
        if (lse.dtype != torch.float32 or tuple(lse.shape) != tuple(lse_shape)
                or lse.device != device or not lse.is_contiguous()):
            raise ValueError(f"lse must be a contiguous float32 tensor of shape {tuple(lse_shape)} "
                             f"on {device}")
    if cu_seqlens is not None:
        if (cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1
                or cu_seqlens.device != device):
            raise ValueError(f"cu_seqlens must be a 1-D int32 tensor on {device}")


def _stream_ptr(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def attn_fwd(q, k, v, out, lse=None, *, causal: bool, scale: float | None = None,
             cu_seqlens=None, stream=None, window: int = 0, n_global: int = 0,
             alibi_slopes=None, tile_rows: int = 0, key_split: int = 0,
             head_group: int = 0) -> None:
    """Call attn_fwd on torch device tensors.

    Padded: q,k,v,out (B,S,H,D), lse (B,H,S) fp32 or None.
    Packed: q,k,v,out (T,H,D), cu_seqlens int32 (nseq+1,), lse (H,T) or None.
    ``scale=None`` means 1/sqrt(D) rounded to float32. ``window``, ``n_global`` and
    ``alibi_slopes`` (float32 device tensor of H slopes) call attn_fwd_ext;
    ``tile_rows`` / ``key_split`` / ``head_group`` (launch shape, 0 = automatic) call
    attn_fwd_tuned.
    """
    _check_tensors(("q", "k", "v", "out"), (q, k, v, out))
    if cu_seqlens is None:
        if q.dim() != 4:
            raise ValueError("padded mode takes (B, S, H, D) tensors")
        B, S, H, D = q.shape
        cu_ptr = None
        _check_aux(lse, (B, H, S), None, q.device)
    else:
        if q.dim() != 3:
            raise ValueError("packed mode takes (T, H, D) tensors")
        T, H, D = q.shape
        B, S = cu_seqlens.numel() - 1, T
        _check_aux(lse, (H, T), cu_seqlens, q.device)
        cu_ptr = cu_seqlens.data_ptr()
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    lse_ptr = None if lse is None else lse.data_ptr()
    masks = bool(window or n_global or alibi_slopes is not None)
    tuned = bool(tile_rows or key_split or head_group)
    if masks and key_split:
        raise ValueError("the mask/bias variants take no key_split argument")
    if tuned and not masks:
        st = attn_fwd_tuned_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr,
                                B, H, S, D, int(bool(causal)), scale, _dtype_code(q), cu_ptr,
                                tile_rows, key_split, head_group, _stream_ptr(stream))
    elif masks:
        al = None
        if alibi_slopes is not None:
            if (alibi_slopes.dtype != torch_float32() or alibi_slopes.numel() != H
                    or alibi_slopes.device != q.device or not alibi_slopes.is_contiguous()):
                raise ValueError("alibi_slopes must be a contiguous float32 tensor of H slopes "
                                 "on q's device")
            al = alibi_slopes.data_ptr()
        if tuned:
            st = attn_fwd_ext_tuned_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                        lse_ptr, B, H, S, D, int(bool(causal)), scale,
                                        _dtype_code(q), cu_ptr, window, n_global, al, tile_rows,
                                        head_group, _stream_ptr(stream))
        else:
            st = attn_fwd_ext_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr,
                                  B, H, S, D, int(bool(causal)), scale, _dtype_code(q), cu_ptr,
                                  window, n_global, al, _stream_ptr(stream))
    else:
        st = attn_fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr,
                          B, H, S, D, int(bool(causal)), scale, _dtype_code(q), cu_ptr,
                          _stream_ptr(stream))
    if st != 0:
        raise AttnError(st, attn_strerror(st))


def fwd(q, k, v, *, causal: bool, scale: float | None = None, cu_seqlens=None,
        with_lse: bool = True, stream=None, window: int = 0, n_global: int = 0,
        alibi_slopes=None, tile_rows: int = 0, key_split: int = 0, head_group: int = 0):
    """Allocate O (and LSE) with torch and run attn_fwd. Returns (O, LSE or None)."""
    import torch
    out = torch.empty_like(q)
    lse = None
    if with_lse:
        if cu_seqlens is None:
            B, S, H, _ = q.shape
            lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
        else:
            T, H, _ = q.shape
            lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    attn_fwd(q, k, v, out, lse, causal=causal, scale=scale, cu_seqlens=cu_seqlens, stream=stream,
             window=window, n_global=n_global, alibi_slopes=alibi_slopes, tile_rows=tile_rows,
             key_split=key_split, head_group=head_group)
    return out, lse


def check_cu_seqlens(cu_seqlens, T: int, stream=None) -> int:
    return load_library().attn_check_cu_seqlens(cu_seqlens.data_ptr(), cu_seqlens.numel() - 1,
                                                int(T), _stream_ptr(stream))


def attn_decode(q, k_cache, v_cache, out, lse=None, *, seqlens_k=None, causal: bool = False,
                scale: float | None = None, num_splits: int = 0, workspace=None,
                stream=None, noalloc: bool = False) -> None:
    """Call attn_decode on torch device tensors.

    q, out (B, Sq, H, D); k_cache, v_cache (B, H, S_max, D); seqlens_k int32 (B,) or None;
    lse (B, H, Sq) fp32 or None; workspace a device tensor of at least
    decode_workspace_size(...) bytes (allocated here with torch when None). With
    ``noalloc`` it calls attn_decode_noalloc instead (no workspace; nothing allocated).
    """
    import torch
    _check_tensors(("q", "out"), (q, out))
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q is (B, Sq, H, D) and the caches (B, H, S_max, D)")
    B, Sq, H, D = q.shape
    S_max = k_cache.shape[2]
    _check_tensors(("k_cache", "v_cache"), (k_cache, v_cache), shape=(B, H, S_max, D),
                   dtype=q.dtype)
    if k_cache.device != q.device:
        raise ValueError("the caches must be on q's device")
    _check_aux(lse, (B, H, Sq), None, q.device)
    if seqlens_k is not None and (seqlens_k.dtype != torch.int32 or seqlens_k.numel() != B
                                  or seqlens_k.device != q.device):
        raise ValueError("seqlens_k must be an int32 tensor of B lengths on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if noalloc:
        if workspace is not None:
            raise ValueError("attn_decode_noalloc takes no workspace")
        st = attn_decode_noalloc_raw(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                     None if seqlens_k is None else seqlens_k.data_ptr(),
                                     out.data_ptr(), None if lse is None else lse.data_ptr(), B, H,
                                     Sq, S_max, D, int(bool(causal)), scale, _dtype_code(q),
                                     num_splits, _stream_ptr(stream))
        if st != 0:
            raise AttnError(st, attn_strerror(st))
        return
    need = decode_workspace_size(B, H, Sq, S_max, D, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = attn_decode_raw(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                         None if seqlens_k is None else seqlens_k.data_ptr(), out.data_ptr(),
                         None if lse is None else lse.data_ptr(), B, H, Sq, S_max, D,
                         int(bool(causal)), scale, _dtype_code(q), num_splits, ws_ptr, ws_bytes,
                         _stream_ptr(stream))
    if st != 0:
        raise AttnError(st, attn_strerror(st))


def decode(q, k_cache, v_cache, *, seqlens_k=None, causal: bool = False, scale: float | None = None,
           num_splits: int = 0, with_lse: bool = True, stream=None):
    """Allocate O (and LSE) with torch and run attn_decode. Returns (O, LSE or None)."""
    import torch
    B, Sq, H, _ = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device) if with_lse else None
    attn_decode(q, k_cache, v_cache, out, lse, seqlens_k=seqlens_k, causal=causal, scale=scale,
                num_splits=num_splits, stream=stream)
    return out, lse


def attn_bwd(q, k, v, out, lse, dout, dq, dk, dv, *, causal: bool, scale: float | None = None,
             cu_seqlens=None, workspace=None, stream=None) -> None:
    """Call attn_bwd on torch device tensors (layouts as attn_fwd; lse required)."""
    import torch
    _check_tensors(("q", "k", "v", "out", "dout", "dq", "dk", "dv"),
                   (q, k, v, out, dout, dq, dk, dv))
    if lse is None:
        raise ValueError("attn_bwd needs the forward's lse")
    if cu_seqlens is None:
        B, S, H, D = q.shape
        cu_ptr = None
        _check_aux(lse, (B, H, S), None, q.device)
    else:
        T, H, D = q.shape
        B, S = cu_seqlens.numel() - 1, T
        _check_aux(lse, (H, T), cu_seqlens, q.device)
        cu_ptr = cu_seqlens.data_ptr()
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = bwd_workspace_size(B, H, S, cu_seqlens is not None)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = attn_bwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                      dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, S, D,
                      int(bool(causal)), scale, _dtype_code(q), cu_ptr, workspace.data_ptr(),
                      workspace.numel() * workspace.element_size(), _stream_ptr(stream))
    if st != 0:
        raise AttnError(st, attn_strerror(st))


def bwd(q, k, v, out, lse, dout, *, causal: bool, scale: float | None = None, cu_seqlens=None,
        stream=None):
    """Allocate dQ, dK, dV with torch and run attn_bwd. Returns (dq, dk, dv)."""
    import torch
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    attn_bwd(q, k, v, out, lse, dout, dq, dk, dv, causal=causal, scale=scale,
             cu_seqlens=cu_seqlens, stream=stream)
    return dq, dk, dv


def fwd_fp8(q8, k8, v8, *, causal: bool, scale: float | None = None, descale_q: float = 1.0,
            descale_k: float = 1.0, descale_v: float = 1.0, out_dtype=None, cu_seqlens=None,
            with_lse: bool = True, stream=None):
    """attn_fwd_fp8 on uint8 device tensors of E4M3 codes. Returns (O, LSE or None)."""
    import torch
    _check_tensors(("q8", "k8", "v8"), (q8, k8, v8), dtype=torch.uint8)
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    out = torch.empty(q8.shape, dtype=out_dtype, device=q8.device)
    if cu_seqlens is None:
        B, S, H, D = q8.shape
        cu_ptr = None
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q8.device) if with_lse else None
    else:
        T, H, D = q8.shape
        B, S = cu_seqlens.numel() - 1, T
        cu_ptr = cu_seqlens.data_ptr()
        lse = torch.empty((H, T), dtype=torch.float32, device=q8.device) if with_lse else None
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = attn_fwd_fp8_raw(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(),
                          None if lse is None else lse.data_ptr(), B, H, S, D, int(bool(causal)),
                          scale, descale_q, descale_k, descale_v, _dtype_code(out), cu_ptr,
                          _stream_ptr(stream))
    if st != 0:
        raise AttnError(st, attn_strerror(st))
    return out, lse

