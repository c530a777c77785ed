"""Thin ctypes binding of libkattn.so (include/kattn.h), with the same names.

Argument marshalling only: device arguments are torch tensors on the GPU
(their ``data_ptr()`` and row strides are passed through), host arguments are
numpy arrays, and every call queues work on torch's current stream.  No
arithmetic of the hot path happens here.  If the library has not been built
the first call raises; there is no fallback.
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
           "kattn_decode_workspace", "kattn_decode")


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
        for name in ("kattn_rope_tables", "kattn_build_index", "kattn_rope_prologue",
                     "kattn_varlen_fwd", "kattn_varlen_fwd_rope", "kattn_varlen_fwd_f16",
                     "kattn_prefill_cached", "kattn_decode"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int):
    if rc != KATTN_OK:
        raise KattnError(rc, lib().kattn_last_error().decode())


def _dev(t):
    """Device pointer of a tensor (None passes NULL)."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


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

def kattn_rope_prologue(q, H: int, k, G: int, pos, cos, sin, *, T: int | None = None,
                        stream=None):
    """Rotate the q heads of ``q`` and the k heads of ``k`` in place (2-D row-strided tensors)."""
    T = int(pos.shape[0]) if T is None else T
    _check(lib().kattn_rope_prologue(_dev(q), _stride(q), H, _dev(k), _stride(k), G, _dev(pos), T,
                                     _dev(cos), _dev(sin), int(cos.shape[0]), HEAD_DIM,
                                     _stream(stream)))


def kattn_varlen_fwd(out, q, k, v, cu, S: int, T: int, max_seqlen: int, H: int, G: int, *,
                     window: int = -1, causal: bool = False, scale: float = 0.125,
                     workspace=None, stream=None):
    """Varlen attention forward; ``workspace`` is a device uint8 tensor of at least
    ``kattn_varlen_fwd_workspace(S, T)`` bytes."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().kattn_varlen_fwd(_dev(out), _stride(out), _dev(q), _stride(q), _dev(k), _stride(k),
                                  _dev(v), _stride(v), _dev(cu), S, T, max_seqlen, H, G, HEAD_DIM,
                                  int(window), int(bool(causal)), float(scale), _dev(workspace),
                                  ws_bytes, _stream(stream)))


def kattn_varlen_fwd_rope(out, q, k, v, cu, S: int, T: int, max_seqlen: int, H: int, G: int,
                          cos, sin, *, window: int = -1, causal: bool = False,
                          scale: float = 0.125, workspace=None, stream=None):
    """Varlen attention over UNROTATED q/k, rotated inside the tile loads (q, k read-only)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().kattn_varlen_fwd_rope(_dev(out), _stride(out), _dev(q), _stride(q), _dev(k),
                                       _stride(k), _dev(v), _stride(v), _dev(cu), S, T, max_seqlen,
                                       H, G, HEAD_DIM, int(window), int(bool(causal)),
                                       float(scale), _dev(cos), _dev(sin), int(cos.shape[0]),
                                       _dev(workspace), ws_bytes, _stream(stream)))


def kattn_varlen_fwd_f16(out, q, k, v, cu, S: int, T: int, max_seqlen: int, H: int, G: int, *,
                         cos=None, sin=None, window: int = -1, causal: bool = False,
                         scale: float = 0.125, workspace=None, stream=None):
    """Varlen attention with a float16 ``out`` tensor; ``cos``/``sin`` select fused rotation."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    table_len = 0 if cos is None else int(cos.shape[0])
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
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    table_len = 0 if cos is None else int(cos.shape[0])
    _check(lib().kattn_prefill_cached(_dev(out), _stride(out), _dev(q), _stride(q), _dev(k_new),
                                      _stride(k_new), _dev(v_new), _stride(v_new), _dev(cu),
                                      _dev(offset), B, T, max_chunk, max_ctx, _dev(k_cache),
                                      _dev(v_cache), cap, H, G, HEAD_DIM, float(scale), _dev(cos),
                                      _dev(sin), table_len, _dev(workspace), ws_bytes,
                                      _stream(stream)))


def kattn_decode(out, q, k_new, v_new, k_cache, v_cache, cap: int, used, max_used: int, B: int,
                 H: int, G: int, *, scale: float = 0.125, cos=None, sin=None, workspace=None,
                 stream=None):
    """One decode step; caches are updated in place at row used[b]-1."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    table_len = 0 if cos is None else int(cos.shape[0])
    _check(lib().kattn_decode(_dev(out), _dev(q), _dev(k_new), _dev(v_new), _dev(k_cache),
                              _dev(v_cache), cap, _dev(used), max_used, B, H, G, HEAD_DIM,
                              float(scale), _dev(cos), _dev(sin), table_len, _dev(workspace),
                              ws_bytes, _stream(stream)))
