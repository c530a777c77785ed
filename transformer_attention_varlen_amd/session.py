"""Device-side runs of the hot path for one workload: upload, index build, launches.

This is call sequencing only -- every step of the path runs in libkattn.so:

  prefill:  kattn_build_index (host) -> copy cu/pos to HBM -> kattn_rope_prologue
            (in place on q and k) -> kattn_varlen_fwd; or, fused, kattn_varlen_fwd_rope
            (q and k read-only, rotated inside the tile loads)
  decode:   kattn_decode (rotate + append + split-K + combine)
  chunk:    kattn_prefill_cached (append the chunk at the fill point, then its queries
            against the cache rows up to their positions)

Inputs are copied to HBM once when a run is created; ``step()`` then touches
only device memory, so a timed loop over ``step()`` measures the kernels with
inputs resident.  torch is used for device memory and streams only.
"""
from __future__ import annotations

import numpy as np
import torch

from . import kattn
from .workloads import ChunkCase, DecodeCase, PrefillCase

HEAD_DIM = 64


def _to_dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class PrefillRun:
    """Device buffers for a PrefillCase and the calls of one prefill step."""

    def __init__(self, case: PrefillCase, device="cuda", out_pad_rows: int = 0):
        self.case = case
        H, G = case.H, case.G
        self.seq_h, self.pos_h, self.max_seqlen = kattn.kattn_build_index(case.cu)
        self.table_len = max(self.max_seqlen, 1)
        self.cos_h, self.sin_h = kattn.kattn_rope_tables(case.theta, self.table_len)
        self.cu = _to_dev(case.cu, device)
        self.pos = _to_dev(self.pos_h, device)
        self.cos = _to_dev(self.cos_h, device)
        self.sin = _to_dev(self.sin_h, device)
        hq, hk = H * HEAD_DIM, G * HEAD_DIM
        if case.qkv is not None:
            self.qkv_host = case.qkv
            self.qkv = _to_dev(case.qkv, device)
            self.q = self.qkv[:, :hq]
            self.k = self.qkv[:, hq:hq + hk]
            self.v = self.qkv[:, hq + hk:]
        else:
            self.qkv = None
            self.q = _to_dev(case.q, device)
            self.k = _to_dev(case.k, device)
            self.v = _to_dev(case.v, device)
        T = case.T
        self.out_full = torch.empty((T + out_pad_rows, hq), dtype=torch.float32, device=device)
        self.out = self.out_full[:T]
        ws = kattn.kattn_varlen_fwd_workspace(case.S, T)
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=device)

    def reset_inputs(self):
        """Restore the unrotated q/k (the prologue rotates in place)."""
        c = self.case
        if self.qkv is not None:
            self.qkv.copy_(torch.from_numpy(c.qkv))
        else:
            self.q.copy_(torch.from_numpy(np.ascontiguousarray(c.q)))
            self.k.copy_(torch.from_numpy(np.ascontiguousarray(c.k)))

    def rope(self):
        c = self.case
        kattn.kattn_rope_prologue(self.q, c.H, self.k, c.G, self.pos, self.cos, self.sin)

    def attention(self):
        c = self.case
        kattn.kattn_varlen_fwd(self.out, self.q, self.k, self.v, self.cu, c.S, c.T,
                               self.max_seqlen, c.H, c.G, window=c.window, causal=c.causal,
                               scale=0.125, workspace=self.workspace)

    def attention_rope(self, out=None):
        """Attention with the rotation fused into the tile loads (q, k must be unrotated)."""
        c = self.case
        kattn.kattn_varlen_fwd_rope(self.out if out is None else out, self.q, self.k, self.v,
                                    self.cu, c.S, c.T, self.max_seqlen, c.H, c.G, self.cos,
                                    self.sin, window=c.window, causal=c.causal, scale=0.125,
                                    workspace=self.workspace)

    def attention_f16(self, out16, fused: bool):
        """Attention with a float16 output; ``fused`` rotates unrotated q/k in the tile loads."""
        c = self.case
        kattn.kattn_varlen_fwd_f16(out16, self.q, self.k, self.v, self.cu, c.S, c.T,
                                   self.max_seqlen, c.H, c.G, cos=self.cos if fused else None,
                                   sin=self.sin if fused else None, window=c.window,
                                   causal=c.causal, scale=0.125, workspace=self.workspace)

    def step_fused(self):
        """One pass of the prefill path with RoPE fused into attention (q, k left as they are)."""
        self.attention_rope()

    def step(self):
        """One pass of the prefill path: RoPE prologue then attention (on rotated q/k).

        The prologue rotates in place, so a second step rotates again; timed
        loops call ``reset_inputs`` first or accept rotated-twice inputs, which
        have the same cost.
        """
        self.rope()
        self.attention()


class DecodeRun:
    """Device buffers for a DecodeCase and the call of one decode step."""

    def __init__(self, case: DecodeCase, device="cuda", rotate: bool = True):
        self.case = case
        self.k_cache = _to_dev(case.k_cache, device)
        self.v_cache = _to_dev(case.v_cache, device)
        self.q = _to_dev(case.q_new, device)
        self.k_new = _to_dev(case.k_new, device)
        self.v_new = _to_dev(case.v_new, device)
        self.used = _to_dev(case.used, device)
        self.max_used = case.max_used
        self.rotate = rotate
        if rotate:
            self.cos_h, self.sin_h = kattn.kattn_rope_tables(case.theta, case.cap)
            self.cos = _to_dev(self.cos_h, device)
            self.sin = _to_dev(self.sin_h, device)
        else:
            self.cos = self.sin = None
        self.out = torch.empty((case.B, case.H * HEAD_DIM), dtype=torch.float32, device=device)
        ws = kattn.kattn_decode_workspace(case.B, case.H, case.G)
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=device)

    def step(self):
        c = self.case
        kattn.kattn_decode(self.out, self.q, self.k_new, self.v_new, self.k_cache, self.v_cache,
                           c.cap, self.used, self.max_used, c.B, c.H, c.G, scale=0.125,
                           cos=self.cos, sin=self.sin, workspace=self.workspace)


class ChunkRun:
    """Device buffers for a ChunkCase and the call of one chunked-prefill step."""

    def __init__(self, case: ChunkCase, device="cuda", rotate: bool = True, out_pad_rows: int = 0):
        self.case = case
        self.k_cache = _to_dev(case.k_cache, device)
        self.v_cache = _to_dev(case.v_cache, device)
        self.q = _to_dev(case.q, device)
        self.k = _to_dev(case.k, device)
        self.v = _to_dev(case.v, device)
        self.cu = _to_dev(case.cu, device)
        self.offsets = _to_dev(case.offsets, device)
        if rotate:
            self.cos_h, self.sin_h = kattn.kattn_rope_tables(case.theta, case.cap)
            self.cos = _to_dev(self.cos_h, device)
            self.sin = _to_dev(self.sin_h, device)
        else:
            self.cos = self.sin = None
        T = case.T
        self.out_full = torch.empty((T + out_pad_rows, case.H * HEAD_DIM), dtype=torch.float32,
                                    device=device)
        self.out = self.out_full[:T]
        ws = kattn.kattn_prefill_cached_workspace(case.B, T)
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=device)

    def step(self):
        c = self.case
        kattn.kattn_prefill_cached(self.out, self.q, self.k, self.v, self.cu, self.offsets, c.B,
                                   c.T, c.max_chunk, c.max_ctx, self.k_cache, self.v_cache, c.cap,
                                   c.H, c.G, scale=0.125, cos=self.cos, sin=self.sin,
                                   workspace=self.workspace)
