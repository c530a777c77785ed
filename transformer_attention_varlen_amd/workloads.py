"""Seeded synthetic inputs shaped like the pages' workloads.

This module holds no attention arithmetic: it only draws lengths and values.
Both the GPU path (tests, bench) and the CPU oracle are fed from the same
arrays it returns.

Recipe (one ``numpy.random.default_rng(seed)`` PCG64 stream per case; draw
order: sequence lengths, then the activations, then -- for decode -- the
caches K, V, the new q, k, v and the used lengths; for a chunked prefill: the
chunk lengths, the filled rows (offsets), then the caches K, V, then q, k, v):

* values are ``standard_normal(dtype=float32)``, i.e. N(0, 1);
* a packed layout draws one (T, (H + 2G) * 64) array whose columns are the q
  heads, then the k heads, then the v heads (the qkv row of the kime pages);
  the SmolLM2 layout draws q (T, H*64), k (T, G*64), v (T, G*64) in that order;
* ``cu`` is the running sum of the lengths, starting at 0.

The named workloads follow the ModernBERT-base and SmolLM2-135M geometry and
the 1142-token caption prompt of the ffai-argus text.rs page.  No dataset or
checkpoint is used: the pages measure on a caption prompt that is not
available, and these synthetic inputs stand in for it.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 64


@dataclass
class PrefillCase:
    name: str
    lengths: np.ndarray        # int32 [S]
    cu: np.ndarray             # int32 [S+1]
    H: int
    G: int
    window: int                # -1: no window; else |i-j| <= window // 2
    causal: bool
    theta: float
    q: np.ndarray              # (T, H*64) float32, possibly a column view of qkv
    k: np.ndarray              # (T, G*64)
    v: np.ndarray              # (T, G*64)
    qkv: np.ndarray | None = None  # the packed parent array, when packed
    seed: int = 0

    @property
    def T(self) -> int:
        return int(self.cu[-1])

    @property
    def S(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def max_seqlen(self) -> int:
        return int(self.lengths.max()) if self.S else 0


@dataclass
class DecodeCase:
    name: str
    B: int
    H: int
    G: int
    cap: int
    theta: float
    k_cache: np.ndarray        # (B, G, cap, 64) float32
    v_cache: np.ndarray
    q_new: np.ndarray          # (B, H*64)
    k_new: np.ndarray          # (B, G*64)
    v_new: np.ndarray          # (B, G*64)
    used: np.ndarray           # int32 [B], counts the new token
    seed: int = 0

    @property
    def max_used(self) -> int:
        return int(self.used.max()) if self.B else 0


@dataclass
class ChunkCase:
    """Prefill of one chunk per sequence continuing from filled KV caches."""
    name: str
    lengths: np.ndarray        # int32 [B], rows of each chunk
    cu: np.ndarray             # int32 [B+1]
    offsets: np.ndarray        # int32 [B], cache rows filled before the chunk
    H: int
    G: int
    cap: int
    theta: float
    k_cache: np.ndarray        # (B, G, cap, 64) float32
    v_cache: np.ndarray
    q: np.ndarray              # (T, H*64)
    k: np.ndarray              # (T, G*64)
    v: np.ndarray              # (T, G*64)
    seed: int = 0

    @property
    def B(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def T(self) -> int:
        return int(self.cu[-1])

    @property
    def max_chunk(self) -> int:
        return int(self.lengths.max()) if self.B else 0

    @property
    def max_ctx(self) -> int:
        return int((self.offsets + self.lengths).max()) if self.B else 0


def _cu(lengths: np.ndarray) -> np.ndarray:
    cu = np.zeros(lengths.shape[0] + 1, np.int32)
    np.cumsum(lengths, out=cu[1:])
    return cu


def make_prefill(lengths, H: int, G: int, *, packed: bool, window: int = -1,
                 causal: bool = False, theta: float = 10000.0, seed: int = 0,
                 rng: np.random.Generator | None = None, name: str = "custom") -> PrefillCase:
    """Activations for a packed batch with the given sequence lengths."""
    rng = np.random.default_rng(seed) if rng is None else rng
    lengths = np.asarray(lengths, dtype=np.int32)
    cu = _cu(lengths)
    T = int(cu[-1])
    hq, hk = H * HEAD_DIM, G * HEAD_DIM
    if packed:
        qkv = rng.standard_normal((T, hq + 2 * hk), dtype=np.float32)
        q, k, v = qkv[:, :hq], qkv[:, hq:hq + hk], qkv[:, hq + hk:]
    else:
        qkv = None
        q = rng.standard_normal((T, hq), dtype=np.float32)
        k = rng.standard_normal((T, hk), dtype=np.float32)
        v = rng.standard_normal((T, hk), dtype=np.float32)
    return PrefillCase(name, lengths, cu, H, G, window, causal, theta, q, k, v, qkv, seed)


def make_decode(B: int, H: int, G: int, cap: int, used_lo: int, used_hi: int, *,
                theta: float = 100000.0, seed: int = 0, name: str = "custom") -> DecodeCase:
    """Caches, new token activations and used lengths drawn U[used_lo, used_hi]."""
    rng = np.random.default_rng(seed)
    k_cache = rng.standard_normal((B, G, cap, HEAD_DIM), dtype=np.float32)
    v_cache = rng.standard_normal((B, G, cap, HEAD_DIM), dtype=np.float32)
    q_new = rng.standard_normal((B, H * HEAD_DIM), dtype=np.float32)
    k_new = rng.standard_normal((B, G * HEAD_DIM), dtype=np.float32)
    v_new = rng.standard_normal((B, G * HEAD_DIM), dtype=np.float32)
    used = rng.integers(used_lo, used_hi, size=B, endpoint=True).astype(np.int32)
    return DecodeCase(name, B, H, G, cap, theta, k_cache, v_cache, q_new, k_new, v_new, used, seed)


def make_chunked(lengths, offsets, H: int, G: int, cap: int, *, theta: float = 100000.0,
                 seed: int = 0, rng: np.random.Generator | None = None,
                 name: str = "custom") -> ChunkCase:
    """Filled caches and one chunk of new rows per sequence."""
    rng = np.random.default_rng(seed) if rng is None else rng
    lengths = np.asarray(lengths, dtype=np.int32)
    offsets = np.asarray(offsets, dtype=np.int32)
    B = lengths.shape[0]
    cu = _cu(lengths)
    T = int(cu[-1])
    k_cache = rng.standard_normal((B, G, cap, HEAD_DIM), dtype=np.float32)
    v_cache = rng.standard_normal((B, G, cap, HEAD_DIM), dtype=np.float32)
    q = rng.standard_normal((T, H * HEAD_DIM), dtype=np.float32)
    k = rng.standard_normal((T, G * HEAD_DIM), dtype=np.float32)
    v = rng.standard_normal((T, G * HEAD_DIM), dtype=np.float32)
    return ChunkCase(name, lengths, cu, offsets, H, G, cap, theta, k_cache, v_cache, q, k, v,
                     seed)


# --- the named workloads -------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    key: str
    name: str
    seed: int
    kind: str                 # "prefill" | "decode" | "chunk"
    desc: str
    params: dict = field(default_factory=dict)


WORKLOADS = {
    "0": Workload("0", "tiny_packed_global", 1000, "prefill",
                  "2 sequences (37, 91), 4 heads = 4 kv heads, packed qkv width 768, global, "
                  "theta 1e4",
                  dict(lengths=[37, 91], H=4, G=4, packed=True, window=-1, causal=False,
                       theta=10000.0)),
    "1": Workload("1", "modernbert_local_w128", 1001, "prefill",
                  "64 sequences, lengths U[16,512], 12 heads, packed qkv width 2304, "
                  "bidirectional window 128 (|i-j| <= 64), theta 1e4",
                  dict(S=64, len_range=(16, 512), H=12, G=12, packed=True, window=128,
                       causal=False, theta=10000.0)),
    "2": Workload("2", "modernbert_global_long", 1002, "prefill",
                  "8 sequences, lengths U[4096,8192], 12 heads, packed qkv width 2304, global, "
                  "theta 1.6e5",
                  dict(S=8, len_range=(4096, 8192), H=12, G=12, packed=True, window=-1,
                       causal=False, theta=160000.0)),
    "3a": Workload("3a", "smollm2_causal_gqa_1142", 1003, "prefill",
                   "one 1142-token sequence, 9 q heads / 3 kv heads, q (T,576) k/v (T,192), "
                   "causal, theta 1e5",
                   dict(lengths=[1142], H=9, G=3, packed=False, window=-1, causal=True,
                        theta=100000.0)),
    "3b": Workload("3b", "smollm2_causal_gqa_16x2048", 1103, "prefill",
                   "16 sequences of 2048, 9 q heads / 3 kv heads, causal, theta 1e5",
                   dict(lengths=[2048] * 16, H=9, G=3, packed=False, window=-1, causal=True,
                        theta=100000.0)),
    # The same layer read as one call: the 1142-token sequence packed with the 16 x 2048 batch.
    "3c": Workload("3c", "smollm2_causal_gqa_1142_plus_16x2048", 1203, "prefill",
                   "one 1142-token sequence packed with 16 sequences of 2048 (33910 tokens), "
                   "9 q heads / 3 kv heads, causal, theta 1e5",
                   dict(lengths=[1142] + [2048] * 16, H=9, G=3, packed=False, window=-1,
                        causal=True, theta=100000.0)),
    "4": Workload("4", "smollm2_decode_b64", 1004, "decode",
                  "64 sequences, one new token each, 9 q heads / 3 kv heads, caches "
                  "[64][3][8192][64] f32, used U[1143,8192], theta 1e5",
                  dict(B=64, H=9, G=3, cap=8192, used_range=(1143, 8192), theta=100000.0)),
    "5": Workload("5", "smollm2_chunked_prefill_b16", 1005, "chunk",
                  "16 sequences continuing from filled caches [16][3][8192][64] f32: chunks of "
                  "U[128,1024] new rows after U[0,4096] filled rows, 9 q heads / 3 kv heads, "
                  "theta 1e5",
                  dict(B=16, H=9, G=3, cap=8192, len_range=(128, 1024), off_range=(0, 4096),
                       theta=100000.0)),
}


def build(key: str):
    """Draw the named workload (deterministic for its seed)."""
    w = WORKLOADS[key]
    p = w.params
    if w.kind == "decode":
        lo, hi = p["used_range"]
        return make_decode(p["B"], p["H"], p["G"], p["cap"], lo, hi, theta=p["theta"],
                           seed=w.seed, name=w.name)
    rng = np.random.default_rng(w.seed)
    if w.kind == "chunk":
        lengths = rng.integers(*p["len_range"], size=p["B"], endpoint=True).astype(np.int32)
        offsets = rng.integers(*p["off_range"], size=p["B"], endpoint=True).astype(np.int32)
        return make_chunked(lengths, offsets, p["H"], p["G"], p["cap"], theta=p["theta"],
                            rng=rng, name=w.name, seed=w.seed)
    if "lengths" in p:
        lengths = np.asarray(p["lengths"], np.int32)
    else:
        lo, hi = p["len_range"]
        lengths = rng.integers(lo, hi, size=p["S"], endpoint=True).astype(np.int32)
    return make_prefill(lengths, p["H"], p["G"], packed=p["packed"], window=p["window"],
                        causal=p["causal"], theta=p["theta"], rng=rng, name=w.name, seed=w.seed)
