"""Fixed-shape (bucketed) launches captured in HIP graphs and replayed with new real counts.

Each call is sized for a bucket (S, T or B slots) and the real counts live in the
device tables (cu, offsets, used), so one captured graph serves every batch that
fits the bucket.  Every test replays its graph several times, with new contents
written into the device tables and inputs between replays and eager library calls
and synchronisations in between, and checks each replay:

* bit for bit against an eager call of the same bucket shape (the same kernels and
  the same order of summation), and within 2e-5 of an eager call on the exact
  (unpadded) shape, which may pick another tile kernel for its smaller launch;
* once per test against the FP64 oracle (2e-5), rows outside the real counts
  untouched.
"""
import numpy as np
import pytest
import torch

import oracle
from transformer_attention_varlen_amd import kattn, workloads as wl

pytestmark = pytest.mark.gpu

ATOL = 2e-5
D = 64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kattn.lib()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _padded_cu(lengths, S_cap):
    cu = np.zeros(S_cap + 1, np.int32)
    cu[1:len(lengths) + 1] = np.cumsum(lengths)
    cu[len(lengths) + 1:] = cu[len(lengths)]
    return cu


@pytest.mark.parametrize("S_cap", [8, 1])
@pytest.mark.parametrize("H,G,window,causal,theta", [(9, 3, -1, True, 1e5),
                                                     (12, 12, 128, False, 1e4)])
def test_fused_prefill_graph_replays_with_new_batches(H, G, window, causal, theta, S_cap):
    # S_cap = 1: a one-sequence bucket (no planning launch: the tile kernel reads its blocks'
    # bounds from cu on every replay)
    T_cap = 2048
    rng = np.random.default_rng(71)
    q = torch.zeros((T_cap, H * D), device="cuda")
    k = torch.zeros((T_cap, G * D), device="cuda")
    v = torch.zeros((T_cap, G * D), device="cuda")
    cu = torch.zeros(S_cap + 1, dtype=torch.int32, device="cuda")
    out = torch.empty((T_cap, H * D), device="cuda")
    cos_h, sin_h = kattn.kattn_rope_tables(theta, T_cap)
    cos, sin = _dev(cos_h), _dev(sin_h)
    ws = torch.empty(kattn.kattn_varlen_fwd_workspace(S_cap, T_cap), dtype=torch.uint8,
                     device="cuda")

    def call(o, S, T, max_seqlen, qq=q, kk=k, vv=v, cc=cu):
        kattn.kattn_varlen_fwd_rope(o, qq, kk, vv, cc, S, T, max_seqlen, H, G, cos, sin,
                                    window=window, causal=causal, workspace=ws)

    cu.copy_(torch.from_numpy(_padded_cu([100], S_cap)))
    call(out, S_cap, T_cap, T_cap)  # eager warm-up (fills the library's per-device caches)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, S_cap, T_cap, T_cap)
    for rep in range(4):
        S = int(rng.integers(1, S_cap + 1))
        lengths = rng.integers(70, T_cap // S_cap + 1, size=S).astype(np.int32)
        lengths[rng.integers(0, S)] = 0 if S > 1 else lengths[0]  # an empty sequence
        T = int(lengths.sum())
        qh = rng.standard_normal((T, H * D), dtype=np.float32)
        kh = rng.standard_normal((T, G * D), dtype=np.float32)
        vh = rng.standard_normal((T, G * D), dtype=np.float32)
        q[:T].copy_(torch.from_numpy(qh))
        k[:T].copy_(torch.from_numpy(kh))
        v[:T].copy_(torch.from_numpy(vh))
        cu.copy_(torch.from_numpy(_padded_cu(lengths, S_cap)))
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu()
        assert torch.all(torch.isnan(got[T:]))  # rows past the real batch are never written
        # eager, the same bucket shape: bit for bit
        same = torch.full_like(out, float("nan"))
        call(same, S_cap, T_cap, T_cap)
        torch.cuda.synchronize()
        assert torch.equal(same.cpu()[:T], got[:T])
        # eager, the exact shape (its own buffers)
        exact = torch.empty((T, H * D), device="cuda")
        call(exact, S, T, int(lengths.max()), qq=_dev(qh), kk=_dev(kh), vv=_dev(vh),
             cc=_dev(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)))
        torch.cuda.synchronize()
        assert float((exact.cpu() - got[:T]).abs().max()) <= ATOL
        if rep == 0:
            ref = oracle.varlen_attention(qh, kh, vh, np.concatenate([[0], np.cumsum(lengths)]),
                                          H, G, window, causal,
                                          tables=oracle.rope_tables(theta, T_cap), threads=16)
            assert float(np.max(np.abs(got[:T].numpy() - ref))) <= ATOL


def test_decode_graph_replays_with_new_lengths_and_tokens():
    B_cap, H, G, cap, theta = 16, 9, 3, 2048, 1e5
    rng = np.random.default_rng(72)
    kc0 = rng.standard_normal((B_cap, G, cap, D), dtype=np.float32)
    vc0 = rng.standard_normal((B_cap, G, cap, D), dtype=np.float32)
    kc, vc = _dev(kc0), _dev(vc0)           # the graph's caches
    kc_e, vc_e = _dev(kc0), _dev(vc0)       # an eager twin, same calls
    q = torch.zeros((B_cap, H * D), device="cuda")
    kn = torch.zeros((B_cap, G * D), device="cuda")
    vn = torch.zeros((B_cap, G * D), device="cuda")
    used = torch.zeros(B_cap, dtype=torch.int32, device="cuda")
    out = torch.empty((B_cap, H * D), device="cuda")
    cos_h, sin_h = kattn.kattn_rope_tables(theta, cap)
    cos, sin = _dev(cos_h), _dev(sin_h)
    ws = torch.empty(kattn.kattn_decode_workspace(B_cap, H, G), dtype=torch.uint8, device="cuda")

    def call(o, kcache, vcache):
        kattn.kattn_decode(o, q, kn, vn, kcache, vcache, cap, used, cap, B_cap, H, G, cos=cos,
                           sin=sin, workspace=ws)

    used.fill_(1)
    scratch_k, scratch_v = _dev(kc0), _dev(vc0)
    call(out, scratch_k, scratch_v)  # eager warm-up on scratch caches
    torch.cuda.synchronize()
    del scratch_k, scratch_v
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, kc, vc)
    lens = rng.integers(1, cap // 2, size=B_cap).astype(np.int32)
    for rep in range(4):
        lens = lens + 1  # one more token per step
        u = lens.copy()
        u[rng.integers(0, B_cap, size=3)] = 0  # idle slots this step
        qh = rng.standard_normal((B_cap, H * D), dtype=np.float32)
        kh = rng.standard_normal((B_cap, G * D), dtype=np.float32)
        vh = rng.standard_normal((B_cap, G * D), dtype=np.float32)
        q.copy_(torch.from_numpy(qh))
        kn.copy_(torch.from_numpy(kh))
        vn.copy_(torch.from_numpy(vh))
        used.copy_(torch.from_numpy(u))
        kc_before = kc.cpu().numpy() if rep == 0 else None
        vc_before = vc.cpu().numpy() if rep == 0 else None
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu()
        idle = u == 0
        assert torch.all(torch.isnan(got[torch.from_numpy(idle)]))  # idle slots untouched
        eager = torch.full_like(out, float("nan"))
        call(eager, kc_e, vc_e)
        torch.cuda.synchronize()
        assert torch.equal(eager.cpu()[~idle], got[~idle])
        assert torch.equal(kc_e.cpu(), kc.cpu()) and torch.equal(vc_e.cpu(), vc.cpu())
        if rep == 0:
            act = np.nonzero(~idle)[0]
            ref, _, _ = oracle.decode(qh[act], kh[act], vh[act], kc_before[act], vc_before[act],
                                      u[act], H, G, tables=oracle.rope_tables(theta, cap),
                                      threads=16)
            assert float(np.max(np.abs(got[act].numpy() - ref))) <= ATOL


def test_chunked_prefill_graph_replays_with_new_chunks():
    B_cap, T_cap, H, G, cap, theta = 4, 1024, 9, 3, 2048, 1e5
    rng = np.random.default_rng(73)
    kc0 = rng.standard_normal((B_cap, G, cap, D), dtype=np.float32)
    vc0 = rng.standard_normal((B_cap, G, cap, D), dtype=np.float32)
    kc, vc = _dev(kc0), _dev(vc0)
    kc_e, vc_e = _dev(kc0), _dev(vc0)
    q = torch.zeros((T_cap, H * D), device="cuda")
    kn = torch.zeros((T_cap, G * D), device="cuda")
    vn = torch.zeros((T_cap, G * D), device="cuda")
    cu = torch.zeros(B_cap + 1, dtype=torch.int32, device="cuda")
    off = torch.zeros(B_cap, dtype=torch.int32, device="cuda")
    out = torch.empty((T_cap, H * D), device="cuda")
    cos_h, sin_h = kattn.kattn_rope_tables(theta, cap)
    cos, sin = _dev(cos_h), _dev(sin_h)
    ws = torch.empty(kattn.kattn_prefill_cached_workspace(B_cap, T_cap), dtype=torch.uint8,
                     device="cuda")

    def call(o, kcache, vcache):
        kattn.kattn_prefill_cached(o, q, kn, vn, cu, off, B_cap, T_cap, T_cap, cap, kcache,
                                   vcache, cap, H, G, cos=cos, sin=sin, workspace=ws)

    cu.copy_(torch.from_numpy(_padded_cu([10], B_cap)))
    scratch_k, scratch_v = _dev(kc0), _dev(vc0)
    call(out, scratch_k, scratch_v)  # eager warm-up on scratch caches
    torch.cuda.synchronize()
    del scratch_k, scratch_v
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, kc, vc)
    filled = np.zeros(B_cap, np.int32)
    for rep in range(4):
        lengths = rng.integers(0, T_cap // B_cap + 1, size=B_cap).astype(np.int32)
        T = int(lengths.sum())
        qh = rng.standard_normal((T, H * D), dtype=np.float32)
        kh = rng.standard_normal((T, G * D), dtype=np.float32)
        vh = rng.standard_normal((T, G * D), dtype=np.float32)
        q[:T].copy_(torch.from_numpy(qh))
        kn[:T].copy_(torch.from_numpy(kh))
        vn[:T].copy_(torch.from_numpy(vh))
        cu.copy_(torch.from_numpy(_padded_cu(lengths, B_cap)))
        off.copy_(torch.from_numpy(filled))
        kc_before = kc.cpu().numpy() if rep == 0 else None
        vc_before = vc.cpu().numpy() if rep == 0 else None
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu()
        assert torch.all(torch.isnan(got[T:]))
        eager = torch.full_like(out, float("nan"))
        call(eager, kc_e, vc_e)
        torch.cuda.synchronize()
        assert torch.equal(eager.cpu()[:T], got[:T])
        assert torch.equal(kc_e.cpu(), kc.cpu()) and torch.equal(vc_e.cpu(), vc.cpu())
        if rep == 0:
            ref, _, _ = oracle.prefill_cached(qh, kh, vh, np.concatenate([[0], np.cumsum(lengths)]),
                                              filled, kc_before, vc_before, H, G,
                                              tables=oracle.rope_tables(theta, cap), threads=16)
            assert float(np.max(np.abs(got[:T].numpy() - ref))) <= ATOL
        filled = filled + lengths
