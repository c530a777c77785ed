"""Thin ctypes binding of libkattn.so (include/kattn.h), with the same names.

Argument marshalling only: device arguments are torch tensors on the GPU
(their ``data_ptr()`` and row strides are passed through), host arguments are
numpy arrays, and every call queues work on torch's current stream.  No
arithmetic of the hot path happens here.  If the library has not been built
the first call raises; there is no fallback.

The C side sees bare pointers and cannot check what they point to, so before
each call the binding checks every tensor it passes: on the GPU, the element
type the C ABI expects (float32, binary16 for the half output, int32 for the
index tables), unit column stride, and enough rows and columns for the sizes
given.  A mismatch raises KattnError(KATTN_EINVAL) and nothing is called.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import numpy as np

LIB_PATH = Path(__file__).resolve().parent / "libkattn.so"
HEAD_DIM = 64

KATTN_OK = 0
KATTN_EINVAL = -1
KATTN_EUNSUPPORTED = -2
KATTN_EBOUNDS = -3
KATTN_EDEVICE = -4

EXPORTS = ("kattn_last_error", "kattn_rope_tables", "kattn_build_index", "kattn_rope_prologue",
           "kattn_varlen_fwd_workspace", "kattn_varlen_fwd", "kattn_varlen_fwd_rope",
           "kattn_varlen_fwd_f16", "kattn_prefill_cached_workspace", "kattn_prefill_cached",
           "kattn_decode_workspace", "kattn_decode", "kattn_decode_noalloc")


class KattnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


_lib = None


def lib():
    """The loaded library (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m transformer_attention_varlen_amd.build`")
        L = ctypes.CDLL(str(LIB_PATH))
        i32, i64, f32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
        p, sz = ctypes.c_void_p, ctypes.c_size_t
        L.kattn_last_error.restype = ctypes.c_char_p
        L.kattn_last_error.argtypes = []
        L.kattn_rope_tables.argtypes = [f64, i32, p, p]
        L.kattn_build_index.argtypes = [p, i32, i32, p, p, p]
        L.kattn_rope_prologue.argtypes = [p, i64, i32, p, i64, i32, p, i32, p, p, i32, i32, p]
        L.kattn_varlen_fwd_workspace.argtypes = [i32, i32]
        L.kattn_varlen_fwd_workspace.restype = sz
        L.kattn_varlen_fwd.argtypes = [p, i64, p, i64, p, i64, p, i64, p, i32, i32, i32, i32, i32,
                                       i32, i32, i32, f32, p, sz, p]
        fwd_tab = [p, i64, p, i64, p, i64, p, i64, p, i32, i32, i32, i32, i32, i32, i32, i32, f32,
                   p, p, i32, p, sz, p]
        L.kattn_varlen_fwd_rope.argtypes = fwd_tab
        L.kattn_varlen_fwd_f16.argtypes = fwd_tab
        L.kattn_prefill_cached_workspace.argtypes = [i32, i32]
        L.kattn_prefill_cached_workspace.restype = sz
        L.kattn_prefill_cached.argtypes = [p, i64, p, i64, p, i64, p, i64, p, p, i32, i32, i32, i32,
                                           p, p, i32, i32, i32, i32, f32, p, p, i32, p, sz, p]
        L.kattn_decode_workspace.argtypes = [i32, i32, i32]
        L.kattn_decode_workspace.restype = sz
        L.kattn_decode.argtypes = [p, p, p, p, p, p, i32, p, i32, i32, i32, i32, i32, f32, p, p,
                                   i32, p, sz, p]
        L.kattn_decode_noalloc.argtypes = [p, p, p, p, p, p, i32, p, i32, i32, i32, i32, i32, f32,
                                           p, p, i32, p]
        for name in ("kattn_rope_tables", "kattn_build_index", "kattn_rope_prologue",
                     "kattn_varlen_fwd", "kattn_varlen_fwd_rope", "kattn_varlen_fwd_f16",
                     "kattn_prefill_cached", "kattn_decode", "kattn_decode_noalloc"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int):
    if rc != KATTN_OK:
        raise KattnError(rc, lib().kattn_last_error().decode())


def _dev(t):
    """Device pointer of a tensor (None passes NULL)."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _bad(fn: str, msg: str):
    raise KattnError(KATTN_EINVAL, f"{fn}: {msg}")


def _dtype_name(t):
    return str(t.dtype).replace("torch.", "")


def _on_gpu(fn: str, name: str, t, dtype: str):
    """``t`` is a torch tensor of element type ``dtype`` on the GPU."""
    if t is None or not hasattr(t, "data_ptr") or not hasattr(t, "dtype"):
        _bad(fn, f"{name} must be a torch tensor")
    if _dtype_name(t) != dtype:
        _bad(fn, f"{name} must be {dtype} (got {_dtype_name(t)})")
    if not t.is_cuda:
        _bad(fn, f"{name} must be on the GPU")


def _rows(fn: str, name: str, t, rows: int, cols: int, dtype: str = "float32"):
    """A 2-D tensor of at least ``rows`` rows of ``cols`` contiguous elements."""
    _on_gpu(fn, name, t, dtype)
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        _bad(fn, f"{name} must be 2-D with unit column stride")
    if t.shape[0] < rows or t.shape[1] < cols:
        _bad(fn, f"{name} is {tuple(t.shape)}, needs at least ({rows}, {cols})")


def _vec(fn: str, name: str, t, n: int, dtype: str = "int32"):
    """A contiguous 1-D tensor of at least ``n`` elements."""
    _on_gpu(fn, name, t, dtype)
    if t.dim() != 1 or (t.shape[0] > 1 and t.stride(0) != 1):
        _bad(fn, f"{name} must be a contiguous 1-D tensor")
    if t.shape[0] < n:
        _bad(fn, f"{name} has {t.shape[0]} elements, needs at least {n}")


def _dense(fn: str, name: str, t, shape, dtype: str = "float32"):
    """A contiguous tensor of exactly ``shape``."""
    _on_gpu(fn, name, t, dtype)
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        _bad(fn, f"{name} must be a contiguous tensor of shape {tuple(shape)} "
                 f"(got {tuple(t.shape)})")


def _tables(fn: str, cos, sin, need: int, required: bool) -> int:
    """cos and sin: contiguous float32 [len, 32] on the GPU, len >= need; returns len."""
    if cos is None and sin is None and not required:
        return 0
    if cos is None or sin is None:
        _bad(fn, "cos and sin must both be given" + ("" if required else " or both be None"))
    for name, t in (("cos", cos), ("sin", sin)):
        _on_gpu(fn, name, t, "float32")
        if t.dim() != 2 or t.shape[1] != HEAD_DIM // 2 or not t.is_contiguous():
            _bad(fn, f"{name} must be a contiguous [len, {HEAD_DIM // 2}] table")
    if cos.shape[0] != sin.shape[0]:
        _bad(fn, "cos and sin have different lengths")
    if cos.shape[0] < need:
        _bad(fn, f"RoPE tables hold {cos.shape[0]} positions, need {need}")
    return int(cos.shape[0])


def _workspace(fn: str, ws) -> int:
    """Bytes of a contiguous device workspace tensor (any element type)."""
    if ws is None:
        _bad(fn, "a workspace tensor is required")
    if not hasattr(ws, "data_ptr") or not ws.is_cuda or not ws.is_contiguous():
        _bad(fn, "workspace must be a contiguous tensor on the GPU")
    return ws.numel() * ws.element_size()


def _host(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _stride(t):
    return 0 if t is None else int(t.stride(0))


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# ----------------------------------------------------------------------------- host calls

def kattn_rope_tables(theta: float, length: int):
    """(cos, sin) float32 host arrays [length, 32]."""
    cos = np.empty((length, HEAD_DIM // 2), np.float32)
    sin = np.empty_like(cos)
    _check(lib().kattn_rope_tables(float(theta), int(length), _host(cos), _host(sin)))
    return cos, sin


def kattn_build_index(cu):
    """(seq, pos, max_seqlen) from host offsets ``cu`` (int32 [S+1])."""
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    S = cu.shape[0] - 1
    T = int(cu[-1]) if S >= 0 else 0
    seq = np.empty(max(T, 0), np.int32)
    pos = np.empty(max(T, 0), np.int32)
    mx = ctypes.c_int32(0)
    _check(lib().kattn_build_index(_host(cu), S, T, _host(seq), _host(pos), ctypes.byref(mx)))
    return seq, pos, int(mx.value)


def kattn_varlen_fwd_workspace(S: int, T: int) -> int:
    return int(lib().kattn_varlen_fwd_workspace(int(S), int(T)))


def kattn_decode_workspace(B: int, H: int, G: int) -> int:
    return int(lib().kattn_decode_workspace(int(B), int(H), int(G)))


# ----------------------------------------------------------------------------- device calls

def _packed(fn: str, name: str, t, rows: int, width: int):
    """Rows of exactly ``width`` floats laid end to end (the decode call takes no strides)."""
    _rows(fn, name, t, rows, width)
    if t.shape[1] != width or (t.shape[0] > 1 and t.stride(0) != width):
        _bad(fn, f"{name} must hold rows of exactly {width} floats, end to end")


def _prefill_operands(fn, out, q, k, v, cu, S, T, H, G, out_dtype="float32"):
    _rows(fn, "out", out, T, H * HEAD_DIM, out_dtype)
    _rows(fn, "q", q, T, H * HEAD_DIM)
    _rows(fn, "k", k, T, G * HEAD_DIM)
    _rows(fn, "v", v, T, G * HEAD_DIM)
    _vec(fn, "cu", cu, S + 1)


def kattn_rope_prologue(q, H: int, k, G: int, pos, cos, sin, *, T: int | None = None,
                        stream=None):
    """Rotate the q heads of ``q`` and the k heads of ``k`` in place (2-D row-strided tensors)."""
    fn = "kattn_rope_prologue"
    T = int(pos.shape[0]) if T is None else T
    _vec(fn, "pos", pos, T)
    _rows(fn, "q", q, T, H * HEAD_DIM)
    if G > 0:
        _rows(fn, "k", k, T, G * HEAD_DIM)
    table_len = _tables(fn, cos, sin, 1, required=True)
    _check(lib().kattn_rope_prologue(_dev(q), _stride(q), H, _dev(k), _stride(k), G, _dev(pos), T,
                                     _dev(cos), _dev(sin), table_len, HEAD_DIM, _stream(stream)))


def kattn_varlen_fwd(out, q, k, v, cu, S: int, T: int, max_seqlen: int, H: int, G: int, *,
                     window: int = -1, causal: bool = False, scale: float = 0.125,
                     workspace=None, stream=None):
    """Varlen attention forward; ``workspace`` is a device uint8 tensor of at least
    ``kattn_varlen_fwd_workspace(S, T)`` bytes."""
    fn = "kattn_varlen_fwd"
    _prefill_operands(fn, out, q, k, v, cu, S, T, H, G)
    ws_bytes = _workspace(fn, workspace)
    _check(lib().kattn_varlen_fwd(_dev(out), _stride(out), _dev(q), _stride(q), _dev(k), _stride(k),
                                  _dev(v), _stride(v), _dev(cu), S, T, max_seqlen, H, G, HEAD_DIM,
                                  int(window), int(bool(causal)), float(scale), _dev(workspace),
                                  ws_bytes, _stream(stream)))


def kattn_varlen_fwd_rope(out, q, k, v, cu, S: int, T: int, max_seqlen: int, H: int, G: int,
                          cos, sin, *, window: int = -1, causal: bool = False,
                          scale: float = 0.125, workspace=None, stream=None):
    """Varlen attention over UNROTATED q/k, rotated inside the tile loads (q, k read-only)."""
    fn = "kattn_varlen_fwd_rope"
    _prefill_operands(fn, out, q, k, v, cu, S, T, H, G)
    table_len = _tables(fn, cos, sin, 1, required=True)
    ws_bytes = _workspace(fn, workspace)
    _check(lib().kattn_varlen_fwd_rope(_dev(out), _stride(out), _dev(q), _stride(q), _dev(k),
                                       _stride(k), _dev(v), _stride(v), _dev(cu), S, T, max_seqlen,
                                       H, G, HEAD_DIM, int(window), int(bool(causal)),
                                       float(scale), _dev(cos), _dev(sin), table_len,
                                       _dev(workspace), ws_bytes, _stream(stream)))


def kattn_varlen_fwd_f16(out, q, k, v, cu, S: int, T: int, max_seqlen: int, H: int, G: int, *,
                         cos=None, sin=None, window: int = -1, causal: bool = False,
                         scale: float = 0.125, workspace=None, stream=None):
    """Varlen attention with a float16 ``out`` tensor; ``cos``/``sin`` select fused rotation."""
    fn = "kattn_varlen_fwd_f16"
    _prefill_operands(fn, out, q, k, v, cu, S, T, H, G, out_dtype="float16")
    table_len = _tables(fn, cos, sin, 1, required=False)
    ws_bytes = _workspace(fn, workspace)
    _check(lib().kattn_varlen_fwd_f16(_dev(out), _stride(out), _dev(q), _stride(q), _dev(k),
                                      _stride(k), _dev(v), _stride(v), _dev(cu), S, T, max_seqlen,
                                      H, G, HEAD_DIM, int(window), int(bool(causal)),
                                      float(scale), _dev(cos), _dev(sin), table_len,
                                      _dev(workspace), ws_bytes, _stream(stream)))


def kattn_prefill_cached_workspace(B: int, T: int) -> int:
    return int(lib().kattn_prefill_cached_workspace(int(B), int(T)))


def kattn_prefill_cached(out, q, k_new, v_new, cu, offset, B: int, T: int, max_chunk: int,
                         max_ctx: int, k_cache, v_cache, cap: int, H: int, G: int, *,
                         scale: float = 0.125, cos=None, sin=None, workspace=None, stream=None):
    """Chunked prefill continuing from the caches; the chunk is appended at rows offset[b].."""
    fn = "kattn_prefill_cached"
    _prefill_operands(fn, out, q, k_new, v_new, cu, B, T, H, G)
    _vec(fn, "offset", offset, B)
    _dense(fn, "k_cache", k_cache, (B, G, cap, HEAD_DIM))
    _dense(fn, "v_cache", v_cache, (B, G, cap, HEAD_DIM))
    table_len = _tables(fn, cos, sin, 1, required=False)
    ws_bytes = _workspace(fn, workspace)
    _check(lib().kattn_prefill_cached(_dev(out), _stride(out), _dev(q), _stride(q), _dev(k_new),
                                      _stride(k_new), _dev(v_new), _stride(v_new), _dev(cu),
                                      _dev(offset), B, T, max_chunk, max_ctx, _dev(k_cache),
                                      _dev(v_cache), cap, H, G, HEAD_DIM, float(scale), _dev(cos),
                                      _dev(sin), table_len, _dev(workspace), ws_bytes,
                                      _stream(stream)))


def _decode_operands(fn, out, q, k_new, v_new, k_cache, v_cache, cap, used, B, H, G):
    _packed(fn, "out", out, B, H * HEAD_DIM)
    _packed(fn, "q", q, B, H * HEAD_DIM)
    _packed(fn, "k_new", k_new, B, G * HEAD_DIM)
    _packed(fn, "v_new", v_new, B, G * HEAD_DIM)
    _dense(fn, "k_cache", k_cache, (B, G, cap, HEAD_DIM))
    _dense(fn, "v_cache", v_cache, (B, G, cap, HEAD_DIM))
    _vec(fn, "used", used, B)


def kattn_decode(out, q, k_new, v_new, k_cache, v_cache, cap: int, used, max_used: int, B: int,
                 H: int, G: int, *, scale: float = 0.125, cos=None, sin=None, workspace=None,
                 stream=None):
    """One decode step; caches are updated in place at row used[b]-1."""
    fn = "kattn_decode"
    _decode_operands(fn, out, q, k_new, v_new, k_cache, v_cache, cap, used, B, H, G)
    table_len = _tables(fn, cos, sin, 1, required=False)
    ws_bytes = _workspace(fn, workspace)
    _check(lib().kattn_decode(_dev(out), _dev(q), _dev(k_new), _dev(v_new), _dev(k_cache),
                              _dev(v_cache), cap, _dev(used), max_used, B, H, G, HEAD_DIM,
                              float(scale), _dev(cos), _dev(sin), table_len, _dev(workspace),
                              ws_bytes, _stream(stream)))


def kattn_decode_noalloc(out, q, k_new, v_new, k_cache, v_cache, cap: int, used, max_used: int,
                         B: int, H: int, G: int, *, scale: float = 0.125, cos=None, sin=None,
                         stream=None):
    """kattn_decode on the library's static per-GPU scratch: no workspace, nothing allocated."""
    fn = "kattn_decode_noalloc"
    _decode_operands(fn, out, q, k_new, v_new, k_cache, v_cache, cap, used, B, H, G)
    table_len = _tables(fn, cos, sin, 1, required=False)
    _check(lib().kattn_decode_noalloc(_dev(out), _dev(q), _dev(k_new), _dev(v_new), _dev(k_cache),
                                      _dev(v_cache), cap, _dev(used), max_used, B, H, G, HEAD_DIM,
                                      float(scale), _dev(cos), _dev(sin), table_len,
                                      _stream(stream)))
