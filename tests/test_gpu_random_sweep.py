"""Seeded random sweep: small configurations of every entry point against the FP64 oracle.

Each case draws its sequence lengths (empty and single-token sequences included), the q/kv
head ratio, the window, the causal flag, the RoPE base and, for the cache paths, the cache
size and fill, from a generator seeded by the case number, so a failure names a case that
can be rerun alone.  Every prefill case runs with the library's own kernel choice (by launch
size, as in production) and again through each tile kernel forced with KATTN_SPLIT; the
binary16-output cases draw the kernel with the case.
"""
import numpy as np
import pytest
import torch

import oracle
from transformer_attention_varlen_amd import kattn, workloads as wl
from transformer_attention_varlen_amd.session import ChunkRun, DecodeRun, PrefillRun

pytestmark = pytest.mark.gpu

ATOL = 2e-5
ROPE_ATOL = 1e-6
RATIOS = [(1, 1), (2, 2), (4, 4), (4, 2), (6, 3), (9, 3), (8, 2), (4, 1), (5, 1), (8, 1)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kattn.lib()


def _err(a, b):
    return float(np.max(np.abs(a.astype(np.float64) - b.astype(np.float64)))) if a.size else 0.0


def _lengths(rng, max_len):
    S = int(rng.integers(1, 9))
    lengths = rng.integers(0, max_len + 1, S)
    if rng.random() < 0.3:
        lengths[rng.integers(0, S)] = 1
    if lengths.sum() == 0:
        lengths[0] = int(rng.integers(1, max_len + 1))
    return lengths.astype(np.int32)


# None: the library's own choice; the others force a tile kernel (KATTN_SPLIT): shared-tile,
# key-split with 4 and 8 waves, sliding-window (where it applies; other launches keep their own)
MODES = [None, "0", "4", "8", "band"]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("seed", range(24))
def test_random_prefill(monkeypatch, seed, mode):
    if mode is not None:
        monkeypatch.setenv("KATTN_SPLIT", mode)
    rng = np.random.default_rng(10_000 + seed)
    H, G = RATIOS[rng.integers(0, len(RATIOS))]
    lengths = _lengths(rng, 400)
    window = int(rng.choice([-1, -1, 0, 1, 7, 64, 128, 1000]))
    causal = bool(rng.random() < 0.5)
    theta = float(rng.choice([1e4, 1e5, 1.6e5]))
    fused = bool(rng.random() < 0.5)
    case = wl.make_prefill(lengths, H, G, packed=(H == G and rng.random() < 0.5), window=window,
                           causal=causal, theta=theta, seed=seed)
    run = PrefillRun(case, out_pad_rows=2)
    run.out_full.fill_(float("nan"))
    if fused:
        run.step_fused()
    else:
        run.step()
    torch.cuda.synchronize()
    got = run.out_full.cpu().numpy()
    tables = oracle.rope_tables(theta, max(case.max_seqlen, 1))
    ref = oracle.varlen_attention(case.q, case.k, case.v, case.cu, H, G, window, causal,
                                  tables=tables, threads=16)
    assert _err(got[:case.T], ref) <= ATOL, (H, G, lengths.tolist(), window, causal, fused)
    assert np.all(np.isnan(got[case.T:]))


@pytest.mark.parametrize("seed", range(12))
def test_random_prefill_f16_output(monkeypatch, seed):
    # binary16 output: within half a binary16 ulp (at the larger magnitude) plus the FP32 bar of
    # the oracle's FP64 result; the tile kernel drawn with the case
    rng = np.random.default_rng(40_000 + seed)
    mode = MODES[rng.integers(0, len(MODES))]
    if mode is not None:
        monkeypatch.setenv("KATTN_SPLIT", mode)
    H, G = RATIOS[rng.integers(0, len(RATIOS))]
    lengths = _lengths(rng, 300)
    window = int(rng.choice([-1, -1, 5, 64, 128]))
    causal = bool(rng.random() < 0.5)
    theta = float(rng.choice([1e4, 1e5]))
    fused = bool(rng.random() < 0.5)
    case = wl.make_prefill(lengths, H, G, packed=(H == G and rng.random() < 0.5), window=window,
                           causal=causal, theta=theta, seed=seed + 500)
    run = PrefillRun(case)
    out16 = torch.full((case.T + 2, H * 64), float("nan"), dtype=torch.float16, device="cuda")
    if not fused:
        run.rope()
    run.attention_f16(out16[:case.T], fused=fused)
    torch.cuda.synchronize()
    got = out16.cpu().numpy()
    tables = oracle.rope_tables(theta, max(case.max_seqlen, 1))
    ref64 = oracle.varlen_attention(case.q, case.k, case.v, case.cu, H, G, window, causal,
                                    tables=tables, threads=16, out_dtype=np.float64)
    a = np.maximum(np.abs(ref64), np.abs(got[:case.T].astype(np.float64))).astype(np.float16)
    bound = 0.5 * np.spacing(a).astype(np.float64) + ATOL
    err = np.abs(got[:case.T].astype(np.float64) - ref64)
    assert np.all(err <= bound), (mode, H, G, lengths.tolist(), window, causal, fused)
    assert np.all(np.isnan(got[case.T:]))


@pytest.mark.parametrize("seed", range(12))
def test_random_prefill_cached(seed):
    rng = np.random.default_rng(20_000 + seed)
    H, G = RATIOS[rng.integers(0, len(RATIOS))]
    B = int(rng.integers(1, 6))
    cap = int(rng.choice([64, 300, 1024]))
    lengths = rng.integers(0, min(cap, 200) + 1, B).astype(np.int32)
    offsets = np.array([rng.integers(0, cap - n + 1) for n in lengths], np.int32)
    if lengths.sum() == 0:
        lengths[0] = 1
        offsets[0] = min(offsets[0], cap - 1)
    rotate = bool(rng.random() < 0.7)
    case = wl.make_chunked(lengths, offsets, H, G, cap, theta=1e5, seed=seed)
    run = ChunkRun(case, rotate=rotate)
    run.step()
    torch.cuda.synchronize()
    tables = oracle.rope_tables(case.theta, cap) if rotate else None
    ref, kc, vc = oracle.prefill_cached(case.q, case.k, case.v, case.cu, case.offsets,
                                        case.k_cache, case.v_cache, H, G, tables=tables,
                                        threads=16)
    assert _err(run.out.cpu().numpy(), ref) <= ATOL, (H, G, lengths.tolist(), offsets.tolist())
    assert _err(run.k_cache.cpu().numpy(), kc) <= ROPE_ATOL
    assert np.array_equal(run.v_cache.cpu().numpy(), vc)


@pytest.mark.parametrize("seed", range(12))
def test_random_decode(seed):
    rng = np.random.default_rng(30_000 + seed)
    H, G = RATIOS[rng.integers(0, len(RATIOS))]
    B = int(rng.integers(1, 40))
    cap = int(rng.choice([1, 33, 500, 2048]))
    used = rng.integers(1, cap + 1, B).astype(np.int32)
    rotate = bool(rng.random() < 0.7)
    case = wl.DecodeCase("random", B, H, G, cap, 1e5,
                         rng.standard_normal((B, G, cap, 64), dtype=np.float32),
                         rng.standard_normal((B, G, cap, 64), dtype=np.float32),
                         rng.standard_normal((B, H * 64), dtype=np.float32),
                         rng.standard_normal((B, G * 64), dtype=np.float32),
                         rng.standard_normal((B, G * 64), dtype=np.float32), used)
    run = DecodeRun(case, rotate=rotate)
    run.step()
    torch.cuda.synchronize()
    tables = oracle.rope_tables(case.theta, cap) if rotate else None
    ref, kc, vc = oracle.decode(case.q_new, case.k_new, case.v_new, case.k_cache, case.v_cache,
                                used, H, G, tables=tables, threads=16)
    assert _err(run.out.cpu().numpy(), ref) <= ATOL, (H, G, B, cap, used.tolist()[:8])
    assert _err(run.k_cache.cpu().numpy(), kc) <= ROPE_ATOL
    assert np.array_equal(run.v_cache.cpu().numpy(), vc)
