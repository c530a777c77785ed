"""Algorithmic work of the hot path: visible pairs, FLOPs and HBM bytes.

These are the counts a roofline is priced on -- what the method must do, not
what a kernel happens to do (masked or padded work is not counted).  In the
spirit of the argus text.rs `crate::cost` counters (a matmul's 2mnk FLOPs,
elementwise reads and writes), with the masked pairs left out.

* A pair is one visible (query i, key j) inside one sequence for one q head.
  Each costs 2*64 FLOPs for q.k and 2*64 for p*v: 256 FLOPs.
* Prefill HBM bytes: q, k, v read once and out written once (f32).
* RoPE prologue bytes: every q and k head read and written once.
* Decode HBM bytes: every cached K and V row below the new one read once, the
  new q, k, v read, the new k and v rows written, the output written.
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 64
F32 = 4
FLOPS_PER_PAIR = 4 * HEAD_DIM


def visible_pairs_per_head(lengths, window: int = -1, causal: bool = False) -> int:
    """Visible (i, j) pairs summed over sequences, for one head (exact, integer)."""
    total = 0
    h = None if window < 0 else window // 2
    for n in np.asarray(lengths, dtype=np.int64):
        n = int(n)
        if n <= 0:
            continue
        i = np.arange(n, dtype=np.int64)
        lo = np.zeros(n, np.int64) if h is None else np.maximum(0, i - h)
        hi = np.full(n, n - 1, np.int64) if h is None else np.minimum(n - 1, i + h)
        if causal:
            hi = np.minimum(hi, i)
        total += int(np.sum(hi - lo + 1))
    return total


def prefill_flops(lengths, H: int, window: int = -1, causal: bool = False) -> int:
    return FLOPS_PER_PAIR * H * visible_pairs_per_head(lengths, window, causal)


def chunk_pairs_per_head(lengths, offsets) -> int:
    """Visible (query, key) pairs of chunks continuing from a cache: row i of a chunk whose
    sequence already holds `off` rows sees keys 0 .. off + i."""
    n = np.asarray(lengths, dtype=np.int64)
    o = np.asarray(offsets, dtype=np.int64)
    return int(np.sum(n * o + n * (n + 1) // 2))


def chunk_flops(lengths, offsets, H: int) -> int:
    return FLOPS_PER_PAIR * H * chunk_pairs_per_head(lengths, offsets)


def prefill_bytes(T: int, H: int, G: int) -> int:
    """q, k, v read and out written, f32."""
    return T * (H + 2 * G) * HEAD_DIM * F32 + T * H * HEAD_DIM * F32


def rope_bytes(T: int, H: int, G: int) -> int:
    """q and k heads read and written once (the shared table rows stay in cache)."""
    return 2 * T * (H + G) * HEAD_DIM * F32


def kv_row_bytes(G: int) -> int:
    """One cache position of one tensor (K or V) for all kv heads."""
    return G * HEAD_DIM * F32


def decode_bytes(used, H: int, G: int) -> int:
    """HBM bytes of one decode step over sequences with used lengths L_b (new token counted)."""
    used = np.asarray(used, dtype=np.int64)
    B = used.shape[0]
    cache_reads = 2 * kv_row_bytes(G) * int(np.sum(used - 1))
    per_seq = (H * HEAD_DIM * F32          # q
               + 2 * kv_row_bytes(G)       # new k, v read
               + 2 * kv_row_bytes(G)       # new k, v appended
               + H * HEAD_DIM * F32)       # out
    return cache_reads + B * per_seq


def decode_flops(used, H: int) -> int:
    used = np.asarray(used, dtype=np.int64)
    return FLOPS_PER_PAIR * H * int(np.sum(used))


def score_matrix_elements(H: int, n: int) -> int:
    """Elements of a materialised (heads, n, n) score matrix -- what the fused path never writes."""
    return H * n * n


def kv_concat_bytes_per_token(G: int, position: int, layers: int) -> int:
    """Bytes a concatenating (non-preallocated) cache copies to append at `position`:
    K and V, every kv head, position+1 rows, every layer."""
    return 2 * layers * (position + 1) * kv_row_bytes(G)
