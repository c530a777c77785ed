"""FP64 CPU oracle for packed variable-length attention -- test infrastructure.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it; the two
share no code.  The arithmetic lives in ``kattn_oracle.c`` (plain C, FP64,
OpenMP over rows); this module only builds it with the host compiler and
marshals numpy arrays into it.

Each function says which passage of the pages it follows (see the C file for
the full statement of the definition and of the readings taken).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "kattn_oracle.c"
_LIB = _HERE / "liboracle.so"

HEAD_DIM = 64


def build(verbose: bool = False) -> Path:
    """Compile ``kattn_oracle.c`` with gcc into ``liboracle.so`` (always rebuilds).

    ``-ffp-contract=off`` keeps every product and sum a separately rounded
    FP64 operation, so results do not depend on the compiler's FMA choices.
    """
    tmp = _LIB.with_suffix(".so.tmp")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", str(tmp), str(_SRC), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not _LIB.exists():
            build()
        lib = ctypes.CDLL(str(_LIB))
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        p = ctypes.c_void_p
        lib.oracle_rope_tables.argtypes = [f64, i32, p, p]
        lib.oracle_rope_apply.argtypes = [p, i64, p, i64, i32, i32, p, p, p, i32]
        lib.oracle_varlen_attention.argtypes = [p, i64, p, i64, p, i64, p, i64, p, i32, i32, i32,
                                                i32, i32, i32, f64, p, p, i32, p, i32, i32, i32]
        lib.oracle_varlen_attention64.argtypes = lib.oracle_varlen_attention.argtypes
        lib.oracle_decode.argtypes = [p, p, p, p, p, p, i32, p, i32, i32, i32, f64, p, p, i32, i32]
        lib.oracle_prefill_cached.argtypes = [p, i64, p, i64, p, i64, p, i64, p, p, i32, i32, p, p,
                                              i32, i32, i32, f64, p, p, i32, i32]
        for f in (lib.oracle_rope_tables, lib.oracle_rope_apply, lib.oracle_varlen_attention,
                  lib.oracle_varlen_attention64, lib.oracle_decode, lib.oracle_prefill_cached):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _rows_view(a, width):
    """(base array, row stride in floats) for a 2-D float32 array or column slice."""
    if not (a.dtype == np.float32 and a.ndim == 2 and a.strides[1] == 4):
        raise ValueError("expected a 2-D float32 array with unit column stride")
    if a.shape[1] < width:
        raise ValueError(f"rows of {a.shape[1]} floats are narrower than {width}")
    return a, a.strides[0] // 4


def rope_tables(theta: float, length: int):
    """cos, sin tables [length, 32] rounded as the kime-cuda `rope_tables` does."""
    cos = np.empty((max(length, 0), HEAD_DIM // 2), np.float32)
    sin = np.empty_like(cos)
    rc = _load().oracle_rope_tables(float(theta), int(length), _ptr(cos), _ptr(sin))
    if rc != 0:
        raise ValueError("oracle_rope_tables: bad arguments")
    return cos, sin


def rope_apply(x, heads: int, pos, cos, sin):
    """Rotated copy of the first ``heads`` 64-wide heads of every row of ``x`` (f32 result)."""
    x, xs = _rows_view(x, heads * HEAD_DIM)
    pos = _i32(pos)
    T = pos.shape[0]
    out = np.empty((T, heads * HEAD_DIM), np.float32)
    rc = _load().oracle_rope_apply(_ptr(out), heads * HEAD_DIM, _ptr(x), xs, T, heads, _ptr(pos),
                                   _ptr(_f32(cos)), _ptr(_f32(sin)), int(cos.shape[0]))
    if rc != 0:
        raise ValueError("oracle_rope_apply: bad arguments")
    return out


def varlen_attention(q, k, v, cu, H: int, G: int, window: int = -1, causal: bool = False,
                     scale: float = 0.125, tables=None, rows=None, mask_mode: int = 0,
                     threads: int = 0, out_dtype=np.float32):
    """Attention output (T or len(rows), H*64) from f64 arithmetic: rounded once to f32, or
    left in f64 with ``out_dtype=np.float64`` (for outputs rounded to another precision).

    ``q``, ``k``, ``v`` are 2-D float32 arrays whose last axis may be a column
    slice of a packed qkv row (strides are passed through).  ``tables`` is the
    oracle's own (cos, sin) pair, or None for inputs already rotated.
    """
    cu = _i32(cu)
    S = cu.shape[0] - 1
    T = int(cu[-1]) if S >= 0 else 0
    q, qs = _rows_view(q, H * HEAD_DIM)
    k, ks = _rows_view(k, G * HEAD_DIM)
    v, vs = _rows_view(v, G * HEAD_DIM)
    rows_a = None if rows is None else _i32(rows)
    n_out = T if rows_a is None else rows_a.shape[0]
    wide = np.dtype(out_dtype) == np.float64
    if not wide and np.dtype(out_dtype) != np.float32:
        raise ValueError("out_dtype must be float32 or float64")
    out = np.empty((n_out, H * HEAD_DIM), np.float64 if wide else np.float32)
    cos, sin = (None, None) if tables is None else (_f32(tables[0]), _f32(tables[1]))
    tl = 0 if cos is None else cos.shape[0]
    fn = _load().oracle_varlen_attention64 if wide else _load().oracle_varlen_attention
    rc = fn(
        _ptr(out), H * HEAD_DIM, _ptr(q), qs, _ptr(k), ks, _ptr(v), vs, _ptr(cu), S, T, H, G,
        int(window), int(bool(causal)), float(scale), _ptr(cos), _ptr(sin), tl, _ptr(rows_a),
        0 if rows_a is None else rows_a.shape[0], int(mask_mode), int(threads))
    if rc != 0:
        raise ValueError("oracle_varlen_attention: bad arguments")
    return out


def decode(q_new, k_new, v_new, k_cache, v_cache, used, H: int, G: int, scale: float = 0.125,
           tables=None, threads: int = 0):
    """One decode step.  Returns (out [B, H*64], k_cache', v_cache') -- the caches are copies
    with the new rows appended; the arrays passed in are left as they were."""
    q_new, k_new, v_new = _f32(q_new), _f32(k_new), _f32(v_new)
    kc = np.array(k_cache, dtype=np.float32, copy=True, order="C")
    vc = np.array(v_cache, dtype=np.float32, copy=True, order="C")
    used = _i32(used)
    B = used.shape[0]
    cap = kc.shape[2]
    out = np.empty((B, H * HEAD_DIM), np.float32)
    cos, sin = (None, None) if tables is None else (_f32(tables[0]), _f32(tables[1]))
    tl = 0 if cos is None else cos.shape[0]
    rc = _load().oracle_decode(_ptr(out), _ptr(q_new), _ptr(k_new), _ptr(v_new), _ptr(kc),
                               _ptr(vc), cap, _ptr(used), B, H, G, float(scale), _ptr(cos),
                               _ptr(sin), tl, int(threads))
    if rc != 0:
        raise ValueError("oracle_decode: bad arguments")
    return out, kc, vc


def prefill_cached(q, k_new, v_new, cu, offset, k_cache, v_cache, H: int, G: int,
                   scale: float = 0.125, tables=None, threads: int = 0):
    """Chunked prefill continuing from a KV cache (argus text.rs `KvAppend` + `CausalSoftmax`
    with an offset).  Returns (out [T, H*64], k_cache', v_cache'): the caches are copies with
    the chunk's rotated keys and values appended at rows offset[b] ..; the arrays passed in
    are left as they were."""
    cu, offset = _i32(cu), _i32(offset)
    B = cu.shape[0] - 1
    T = int(cu[-1]) if B >= 0 else 0
    q, qs = _rows_view(q, H * HEAD_DIM)
    k_new, ks = _rows_view(k_new, G * HEAD_DIM)
    v_new, vs = _rows_view(v_new, G * HEAD_DIM)
    kc = np.array(k_cache, dtype=np.float32, copy=True, order="C")
    vc = np.array(v_cache, dtype=np.float32, copy=True, order="C")
    cap = kc.shape[2]
    out = np.empty((T, H * HEAD_DIM), np.float32)
    cos, sin = (None, None) if tables is None else (_f32(tables[0]), _f32(tables[1]))
    tl = 0 if cos is None else cos.shape[0]
    rc = _load().oracle_prefill_cached(_ptr(out), H * HEAD_DIM, _ptr(q), qs, _ptr(k_new), ks,
                                       _ptr(v_new), vs, _ptr(cu), _ptr(offset), B, T, _ptr(kc),
                                       _ptr(vc), cap, H, G, float(scale), _ptr(cos), _ptr(sin), tl,
                                       int(threads))
    if rc != 0:
        raise ValueError("oracle_prefill_cached: bad arguments")
    return out, kc, vc
