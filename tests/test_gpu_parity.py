"""GPU parity: libkattn.so (through its C ABI) against the FP64 CPU oracle.

Tolerances: attention outputs max |gpu - oracle| <= 2e-5 on every element
compared (FP32 arithmetic in any order against one FP64 rounding, N(0,1)
inputs); rotated q/k and appended cache rows <= 1e-6 (one or two f32
roundings of values below 8).  Integer and index work (which rows and cache
rows are written) is checked exactly.  Full-size workloads run in the launch
configuration the bench times and are compared on every element, the global
layer one sequence per test item so that no item runs long; only the stress
cases (one 40000-token sequence, 20000 tiny sequences) compare sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
from transformer_attention_varlen_amd import kattn, workloads as wl
from transformer_attention_varlen_amd.session import DecodeRun, PrefillRun

pytestmark = pytest.mark.gpu

ATOL = 2e-5
ROPE_ATOL = 1e-6
D = 64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kattn.lib()


@pytest.fixture(params=["shared_tile_kernel", "key_split_4_waves", "key_split_8_waves",
                        "sliding_window_kernel"])
def prefill_kernel(request, monkeypatch):
    """Runs a prefill test once with each tile kernel (the library picks by launch size and
    window; KATTN_SPLIT forces the choice; the sliding-window kernel applies to packed batches
    with a half-window of at most 64, other launches keep the library's own choice)."""
    monkeypatch.setenv("KATTN_SPLIT", {"shared_tile_kernel": "0", "key_split_4_waves": "4",
                                       "key_split_8_waves": "8",
                                       "sliding_window_kernel": "band"}[request.param])
    return request.param


def oracle_prefill(case, rows=None):
    tables = oracle.rope_tables(case.theta, max(case.max_seqlen, 1))
    return oracle.varlen_attention(case.q, case.k, case.v, case.cu, case.H, case.G, case.window,
                                   case.causal, tables=tables, rows=rows, threads=16)


def gpu_prefill(case, pad_rows=0, sentinel=None):
    run = PrefillRun(case, out_pad_rows=pad_rows)
    if sentinel is not None:
        run.out_full.fill_(sentinel)
    run.step()
    torch.cuda.synchronize()
    return run


def max_err(a, b):
    return float(np.max(np.abs(a.astype(np.float64) - b.astype(np.float64)))) if a.size else 0.0


# ----------------------------------------------------------------------------- RoPE prologue

@pytest.mark.parametrize("key", ["0", "3a"])
def test_rope_prologue_matches_oracle(key):
    case = wl.build(key)
    run = PrefillRun(case)
    run.rope()
    torch.cuda.synchronize()
    tables = oracle.rope_tables(case.theta, run.table_len)
    q_ref = oracle.rope_apply(case.q, case.H, run.pos_h, *tables)
    k_ref = oracle.rope_apply(case.k, case.G, run.pos_h, *tables)
    assert max_err(run.q.cpu().numpy(), q_ref) <= ROPE_ATOL
    assert max_err(run.k.cpu().numpy(), k_ref) <= ROPE_ATOL
    assert np.array_equal(run.v.cpu().numpy(), case.v)   # v is never touched


# ----------------------------------------------------------------------------- small prefill cases

RAGGED = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200]
SMALL_CASES = [
    ([37, 91], 4, 4, -1, False),
    (RAGGED, 4, 4, -1, False),
    (RAGGED, 4, 4, -1, True),
    (RAGGED, 4, 4, 0, False),
    (RAGGED, 4, 4, 1, False),
    (RAGGED, 4, 4, 5, False),
    (RAGGED, 4, 4, 128, False),
    (RAGGED, 4, 4, 300, False),
    (RAGGED, 4, 4, 40, True),
    ([130, 7, 300, 1], 9, 3, -1, True),
    ([130, 7, 300, 1], 9, 3, 64, False),
    ([130, 7, 300], 6, 2, -1, True),
    ([130, 7, 300], 8, 2, -1, False),
    ([130, 7, 300], 5, 1, -1, True),
    ([130, 7, 300], 2, 2, 33, False),
    ([0, 45, 0, 0, 17, 0], 4, 2, -1, False),
    ([0, 45, 0, 0, 17, 0], 4, 2, 6, True),
]


@pytest.mark.parametrize("lengths,H,G,window,causal", SMALL_CASES)
def test_prefill_small_cases(prefill_kernel, lengths, H, G, window, causal):
    case = wl.make_prefill(lengths, H, G, packed=(H == G), window=window, causal=causal,
                           theta=10000.0, seed=100 + len(lengths) + H + window)
    run = gpu_prefill(case, pad_rows=5, sentinel=float("nan"))
    got = run.out_full.cpu().numpy()
    ref = oracle_prefill(case)
    assert max_err(got[:case.T], ref) <= ATOL
    assert np.all(np.isnan(got[case.T:]))  # rows past T are never written


# ----------------------------------------------------------------------------- named workloads

@pytest.mark.parametrize("key", ["0", "1", "3a"])
def test_workload_full_parity(key):
    case = wl.build(key)
    run = gpu_prefill(case)
    got = run.out.cpu().numpy()
    ref = oracle_prefill(case)
    assert max_err(got, ref) <= ATOL


def _sample_rows(case, n_random, seed):
    rng = np.random.default_rng(seed)
    rows = set()
    for s in range(case.S):
        lo, hi = int(case.cu[s]), int(case.cu[s + 1])
        if hi > lo:
            rows.update([lo, lo + 1, hi - 2, hi - 1, (lo + hi) // 2])
    rows.update(rng.integers(0, case.T, n_random).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < case.T), np.int32)


@pytest.fixture(scope="module")
def gated_outputs():
    """The GPU outputs of a large workload in both forms the bench times -- fused RoPE
    (kattn_varlen_fwd_rope on unrotated q/k) and two-pass (the in-place prologue, then
    kattn_varlen_fwd) -- computed once and kept on the host while that workload's items run."""
    held = {}

    def get(key):
        if key not in held:
            held.clear()
            case = wl.build(key)
            run = PrefillRun(case)
            run.step_fused()
            torch.cuda.synchronize()
            fused = run.out.cpu().numpy().copy()
            run.step()
            torch.cuda.synchronize()
            two_pass = run.out.cpu().numpy()
            del run
            torch.cuda.empty_cache()
            held[key] = (case, two_pass, fused)
        return held[key]

    return get


# the global layer one sequence per item (each a few tens of seconds of oracle time), the
# causal batches whole
GATED_ITEMS = [("2", s) for s in range(8)] + [("3b", None), ("3c", None)]


@pytest.mark.parametrize("key,seq", GATED_ITEMS)
def test_gated_workload_every_element(gated_outputs, key, seq):
    case, two_pass, fused = gated_outputs(key)
    if seq is None:
        rows = None
        ref = oracle_prefill(case)
        a, b = two_pass, fused
    else:
        assert case.S == 8
        rows = np.arange(case.cu[seq], case.cu[seq + 1], dtype=np.int32)
        ref = oracle_prefill(case, rows=rows)
        a, b = two_pass[rows], fused[rows]
    print(f"workload {key} rows {'all' if rows is None else f'of sequence {seq}'}: "
          f"two-pass {max_err(a, ref):.3e}, fused {max_err(b, ref):.3e}", flush=True)
    assert max_err(a, ref) <= ATOL
    assert max_err(b, ref) <= ATOL
    if seq in (None, 0):
        assert np.all(np.isfinite(two_pass)) and np.all(np.isfinite(fused))


# ----------------------------------------------------------------------------- GPU invariants

@pytest.mark.parametrize("causal", [False, True])
def test_window_of_twice_the_length_is_bit_identical_to_global(causal):
    lengths = [50, 17, 300, 129]
    a = wl.make_prefill(lengths, 4, 4, packed=True, window=-1, causal=causal, seed=5)
    b = wl.make_prefill(lengths, 4, 4, packed=True, window=2 * 300, causal=causal, seed=5)
    ga = gpu_prefill(a).out.cpu()
    gb = gpu_prefill(b).out.cpu()
    assert torch.equal(ga, gb)


@pytest.mark.parametrize("mode", [None, "4", "8"])
@pytest.mark.parametrize("n,T,max_seqlen,causal,fused", [(300, 520, 520, True, False),
                                                         (300, 520, 333, False, True),
                                                         (37, 200, 200, True, True),
                                                         (300, 520, 300, True, False)])
def test_one_sequence_in_a_larger_bucket(monkeypatch, mode, n, T, max_seqlen, causal, fused):
    # A batch of one sequence sized for a bucket: T and max_seqlen at or above the sequence's n
    # rows, cu = {0, n}.  A one-sequence launch plans nothing on the device, so its blocks come
    # from cu alone: rows past n are neither attended to nor written.
    if mode is not None:
        monkeypatch.setenv("KATTN_SPLIT", mode)
    H, G, theta = 9, 3, 1e5
    case = wl.make_prefill([n], H, G, packed=False, window=-1, causal=causal, theta=theta,
                           seed=23)
    rng = np.random.default_rng(24)

    def padded(a):
        extra = rng.standard_normal((T - n, a.shape[1]), dtype=np.float32)
        return torch.from_numpy(np.concatenate([a, extra])).cuda()

    q, k, v = padded(case.q), padded(case.k), padded(case.v)
    cu = torch.tensor([0, n], dtype=torch.int32, device="cuda")
    out = torch.full((T, H * 64), float("nan"), device="cuda")
    ws = torch.empty(max(kattn.kattn_varlen_fwd_workspace(1, T), 256), dtype=torch.uint8,
                     device="cuda")
    tables = oracle.rope_tables(theta, max_seqlen)
    if fused:
        cos_h, sin_h = kattn.kattn_rope_tables(theta, max_seqlen)
        kattn.kattn_varlen_fwd_rope(out, q, k, v, cu, 1, T, max_seqlen, H, G,
                                    torch.from_numpy(cos_h).cuda(), torch.from_numpy(sin_h).cuda(),
                                    causal=causal, workspace=ws)
        ref = oracle.varlen_attention(case.q, case.k, case.v, case.cu, H, G, -1, causal,
                                      tables=tables, threads=16)
    else:
        kattn.kattn_varlen_fwd(out, q, k, v, cu, 1, T, max_seqlen, H, G, causal=causal,
                               workspace=ws)
        ref = oracle.varlen_attention(case.q, case.k, case.v, case.cu, H, G, -1, causal,
                                      tables=None, threads=16)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isnan(got[n:]))  # rows past the sequence are never written
    assert max_err(got[:n], ref) <= ATOL


@pytest.mark.parametrize("window,causal", [(-1, False), (-1, True), (20, False)])
def test_each_sequence_alone_is_bit_identical_to_its_rows_in_the_batch(monkeypatch, window,
                                                                        causal):
    # Bitwise where the key tiles start at each sequence's first row (the shared-tile and
    # key-split kernels).  The sliding-window kernel cuts tiles at multiples of 32 packed rows,
    # so a sequence moved to another offset is summed in other groups: bitwise only for a
    # sequence starting at row 0, within the tolerance otherwise.
    lengths = [70, 0, 200, 33]
    case = wl.make_prefill(lengths, 9, 3, packed=False, window=window, causal=causal, seed=6)
    modes = ["0", "band"] if window >= 0 else [None]
    for mode in modes:
        if mode is not None:
            monkeypatch.setenv("KATTN_SPLIT", mode)
        packed = gpu_prefill(case).out.cpu()
        for s, n in enumerate(lengths):
            lo = int(case.cu[s])
            if n == 0:
                continue
            alone = wl.PrefillCase("alone", np.array([n], np.int32), np.array([0, n], np.int32),
                                   9, 3, window, causal, case.theta, case.q[lo:lo + n],
                                   case.k[lo:lo + n], case.v[lo:lo + n])
            got = gpu_prefill(alone).out.cpu()
            if mode == "band" and lo % 32 != 0:
                assert max_err(got.numpy(), packed[lo:lo + n].numpy()) <= ATOL
            else:
                assert torch.equal(got, packed[lo:lo + n])


# ----------------------------------------------------------------------------- large and shifted scores

def _attention_only(case):
    """GPU attention on q, k taken as already rotated, against the oracle without rotation."""
    run = PrefillRun(case)
    run.attention()
    torch.cuda.synchronize()
    ref = oracle.varlen_attention(case.q, case.k, case.v, case.cu, case.H, case.G, case.window,
                                  case.causal, tables=None, threads=16)
    return run.out.cpu().numpy(), ref


def _score_bar(case):
    """The output bar for scores larger than those of N(0,1) inputs: FP32 scores carry an
    absolute error that grows with their magnitude (about 2^-24 of the partial sums per
    accumulation step), so ATOL, set for scores of magnitude about 4, scales with the largest
    |q.k| / 8 over the pairs of each sequence."""
    H, G, R = case.H, case.G, case.H // case.G
    smax = 0.0
    for s in range(case.S):
        lo, hi = int(case.cu[s]), int(case.cu[s + 1])
        if hi == lo:
            continue
        q = case.q[lo:hi].reshape(hi - lo, H, D).astype(np.float64)
        k = case.k[lo:hi].reshape(hi - lo, G, D).astype(np.float64)
        for h in range(H):
            smax = max(smax, float(np.max(np.abs(q[:, h] @ k[:, h // R].T))) / 8.0)
    return ATOL * max(1.0, smax / 4.0)


def _set_score_shift(case, q_coef, k_of_pos):
    """Dim 0 of every q head is set to q_coef[row] and dim 0 of every k head to k_of_pos(p) at
    in-sequence position p, so each score gains q_coef * k_of_pos(p) / 8; the other dims stay
    N(0,1)."""
    for g in range(case.G):
        for s in range(case.S):
            lo, hi = int(case.cu[s]), int(case.cu[s + 1])
            case.k[lo:hi, g * D] = k_of_pos(np.arange(hi - lo, dtype=np.float64)).astype(np.float32)
    for h in range(case.H):
        case.q[:, h * D] = q_coef


@pytest.mark.parametrize("window,causal", [(-1, False), (-1, True), (40, False), (17, True)])
def test_score_ramps_move_the_reference(prefill_kernel, window, causal):
    # Scores that rise (or fall) by about 1/8 per key position: along a 300-key row the max
    # climbs about 54 base-2 units, so every kernel moves its exponent references up several
    # times and rescales l and O; rows with coefficient -1 start at their max; 0 adds nothing.
    lengths = [1, 37, 300, 129, 64]
    case = wl.make_prefill(lengths, 4, 2, packed=True, window=window, causal=causal, seed=41)
    rng = np.random.default_rng(41)
    coef = rng.choice(np.array([1.0, -1.0, 0.5, 0.0], np.float32), size=case.T)
    _set_score_shift(case, coef, lambda pos: pos)
    got, ref = _attention_only(case)
    assert np.all(np.isfinite(got))
    assert max_err(got, ref) <= _score_bar(case)


@pytest.mark.parametrize("shift", [75.0, 100.0])
@pytest.mark.parametrize("window,causal", [(-1, False), (-1, True), (40, False)])
def test_scores_far_from_zero_move_the_reference(prefill_kernel, window, causal, shift):
    # A constant shift of -shift (coefficient 1) or +shift (coefficient -1) per row: the
    # reference moves down below -64 base-2 units or up past +16 at the first visible tile; rows
    # with coefficient 0 keep it at 0, so one wave mixes moved and unmoved lanes.  At +100 (144
    # base-2 units) the first pass's exponentials overflow to infinity before the move.  The
    # shift is the same for every key of a row, so the softmax equals that of the unshifted
    # scores.
    lengths = [1, 37, 300, 129, 64]
    case = wl.make_prefill(lengths, 4, 2, packed=True, window=window, causal=causal, seed=43)
    rng = np.random.default_rng(43)
    coef = rng.choice(np.array([1.0, -1.0, 0.0], np.float32), size=case.T)
    _set_score_shift(case, coef, lambda pos: np.full(pos.shape, -8.0 * shift))
    got, ref = _attention_only(case)
    assert np.all(np.isfinite(got))
    assert max_err(got, ref) <= _score_bar(case)


def _norm_bar(q, k):
    """ATOL scaled as in _score_bar, with the largest score bounded by the largest norms (the
    rotation keeps each pair's norm, so the bound holds for rotated rows too)."""
    qn = float(np.max(np.linalg.norm(q.reshape(-1, D).astype(np.float64), axis=1))) if q.size else 0.0
    kn = float(np.max(np.linalg.norm(k.reshape(-1, D).astype(np.float64), axis=1))) if k.size else 0.0
    return ATOL * max(1.0, qn * kn / 8.0 / 4.0)


@pytest.mark.parametrize("window,causal", [(-1, False), (-1, True), (40, False)])
def test_large_scores_with_fused_rope(prefill_kernel, window, causal):
    # q scaled by 8: scores of standard deviation about 8, so the row maxima pass the exponent
    # references' upper bound in the fused-rotation kernels too
    lengths = [1, 37, 300, 129, 64]
    case = wl.make_prefill(lengths, 4, 2, packed=True, window=window, causal=causal, seed=47)
    case.q[:] *= 8.0
    run = PrefillRun(case)
    run.step_fused()
    torch.cuda.synchronize()
    got = run.out.cpu().numpy()
    ref = oracle_prefill(case)
    assert np.all(np.isfinite(got))
    assert max_err(got, ref) <= _norm_bar(case.q, case.k)


@pytest.mark.parametrize("rotate", [True, False])
def test_large_scores_from_a_cache(prefill_kernel, rotate):
    # the chunked prefill's tile kernels (keys from a cache) with q scaled by 8
    case = wl.make_chunked([1, 31, 32, 33, 129], [0, 0, 5, 100, 200], 9, 3, 400, seed=49)
    case.q[:] *= 8.0
    kk = np.concatenate([case.k.reshape(-1, D), case.k_cache.reshape(-1, D)], axis=0)
    _check_chunk(case, rotate, atol=_norm_bar(case.q, kk))


def test_gqa_matches_mha_with_repeated_kv():
    H, G = 9, 3
    case = wl.make_prefill([100, 257], H, G, packed=False, causal=True, seed=8)
    T = case.T
    k_rep = np.repeat(case.k.reshape(T, G, 1, D), H // G, axis=2).reshape(T, H * D)
    v_rep = np.repeat(case.v.reshape(T, G, 1, D), H // G, axis=2).reshape(T, H * D)
    mha = wl.PrefillCase("mha", case.lengths, case.cu, H, H, -1, True, case.theta, case.q, k_rep,
                         v_rep)
    a = gpu_prefill(case).out.cpu().numpy()
    b = gpu_prefill(mha).out.cpu().numpy()
    assert max_err(a, b) <= ATOL


def test_uniform_weights_recover_the_visible_range_on_gpu():
    # q = 0: every visible key has weight 1/count; v_j = [1, p_j, p_j^2] recovers the range
    lengths = [1, 37, 91, 130]
    for window, causal in [(-1, False), (-1, True), (128, False), (7, True)]:
        case = wl.make_prefill(lengths, 4, 2, packed=False, window=window, causal=causal, seed=3)
        case.q[:] = 0.0
        case.v[:] = 0.0
        for s in range(case.S):
            lo, hi = int(case.cu[s]), int(case.cu[s + 1])
            p = np.arange(hi - lo, dtype=np.float32)
            for g in range(2):
                case.v[lo:hi, g * D] = 1.0
                case.v[lo:hi, g * D + 1] = p
                case.v[lo:hi, g * D + 2] = p * p
        got = gpu_prefill(case).out.cpu().numpy()
        ref = oracle_prefill(case)
        assert max_err(got[:, 0::D], ref[:, 0::D]) <= 1e-6
        assert np.allclose(got, ref, rtol=1e-6, atol=1e-4)


# ----------------------------------------------------------------------------- decode

def _decode_case(lens, H, G, cap, seed):
    rng = np.random.default_rng(seed)
    B = len(lens)
    return wl.DecodeCase("small", B, H, G, cap, 100000.0,
                         rng.standard_normal((B, G, cap, D), dtype=np.float32),
                         rng.standard_normal((B, G, cap, D), dtype=np.float32),
                         rng.standard_normal((B, H * D), dtype=np.float32),
                         rng.standard_normal((B, G * D), dtype=np.float32),
                         rng.standard_normal((B, G * D), dtype=np.float32),
                         np.array(lens, np.int32))


def _check_decode(case, rotate):
    run = DecodeRun(case, rotate=rotate)
    run.step()
    torch.cuda.synchronize()
    tables = oracle.rope_tables(case.theta, case.cap) if rotate else None
    ref, kc, vc = oracle.decode(case.q_new, case.k_new, case.v_new, case.k_cache, case.v_cache,
                                case.used, case.H, case.G, tables=tables, threads=16)
    assert max_err(run.out.cpu().numpy(), ref) <= ATOL
    gk = run.k_cache.cpu().numpy()
    gv = run.v_cache.cpu().numpy()
    for b, L in enumerate(case.used):
        p = int(L) - 1
        assert max_err(gk[b, :, p], kc[b, :, p]) <= ROPE_ATOL
        assert np.array_equal(gv[b, :, p], vc[b, :, p])
        gk[b, :, p] = kc[b, :, p]
    # every other cache row is untouched (bit for bit, NaN contents included)
    assert np.array_equal(gk.view(np.uint32), kc.view(np.uint32))
    assert np.array_equal(gv.view(np.uint32), vc.view(np.uint32))


@pytest.mark.parametrize("rotate", [True, False])
@pytest.mark.parametrize("H,G", [(9, 3), (4, 4), (8, 1)])
def test_decode_small(rotate, H, G):
    case = _decode_case([1, 2, 255, 256, 257, 300, 513], H, G, 520, seed=H * 10 + G)
    _check_decode(case, rotate)


def test_decode_full_workload():
    _check_decode(wl.build("4"), rotate=True)


@pytest.mark.parametrize("rotate", [True, False])
def test_decode_ignores_unused_cache_rows_holding_nan(rotate):
    # The cache rows from used-1 on are write-only to a decode step: row used-1 receives the
    # new token and the rows past it are never part of the result.  Filled with NaN here (as
    # torch.empty or a reused block may leave them), they must not reach the output.  Lengths
    # put the new row at every offset inside a 32-row block and at piece boundaries.
    lens = [1, 2, 31, 32, 33, 63, 64, 65, 255, 256, 257, 300, 511, 512]
    case = _decode_case(lens, 9, 3, 520, seed=31)
    for b, L in enumerate(lens):
        case.k_cache[b, :, L - 1:] = np.nan
        case.v_cache[b, :, L - 1:] = np.nan
    _check_decode(case, rotate)


def test_decode_equals_last_causal_row_of_prefill():
    H, G, L = 9, 3, 700
    case = wl.make_prefill([L], H, G, packed=False, causal=True, theta=100000.0, seed=12)
    pre = gpu_prefill(case)
    last = pre.out.cpu().numpy()[L - 1]
    cap = 1024
    kc = np.zeros((1, G, cap, D), np.float32)
    vc = np.zeros((1, G, cap, D), np.float32)
    k_rot = pre.k.cpu().numpy()          # rotated by the prologue
    q_rot = pre.q.cpu().numpy()
    kc[0, :, :L] = k_rot.reshape(L, G, D).transpose(1, 0, 2)
    vc[0, :, :L] = case.v.reshape(L, G, D).transpose(1, 0, 2)
    dec = wl.DecodeCase("dec", 1, H, G, cap, case.theta, kc, vc, q_rot[L - 1:].copy(),
                        k_rot[L - 1:].copy(), case.v[L - 1:].copy(), np.array([L], np.int32))
    run = DecodeRun(dec, rotate=False)
    run.step()
    torch.cuda.synchronize()
    assert max_err(run.out.cpu().numpy()[0], last) <= ATOL


def test_decode_skips_sequences_with_bad_lengths():
    case = _decode_case([5, 0, 300], 9, 3, 320, seed=4)
    run = DecodeRun(case, rotate=True)
    run.max_used = 300
    run.out.fill_(7.0)
    run.step()
    torch.cuda.synchronize()
    out = run.out.cpu().numpy()
    assert np.all(out[1] == 7.0)
    assert np.array_equal(run.k_cache.cpu().numpy()[1], case.k_cache[1])


def test_many_short_sequences_plan_beyond_lds():
    # more sequences than the planner keeps in LDS: the tile prefix then lives in the workspace
    rng = np.random.default_rng(77)
    lengths = rng.integers(0, 6, 5000)
    lengths[rng.integers(0, 5000, 20)] = rng.integers(30, 140, 20)
    case = wl.make_prefill(lengths, 4, 2, packed=False, window=-1, causal=True, seed=78)
    run = gpu_prefill(case, pad_rows=3, sentinel=float("nan"))
    got = run.out_full.cpu().numpy()
    ref = oracle_prefill(case)
    assert max_err(got[:case.T], ref) <= ATOL
    assert np.all(np.isnan(got[case.T:]))


def test_decode_batch_beyond_one_launch():
    # more sequences than one launch schedules: the host cuts the batch into launches
    rng = np.random.default_rng(5)
    lens = rng.integers(1, 65, 1100).astype(np.int32)
    lens[7] = 0  # an invalid length is skipped
    case = _decode_case(lens, 4, 2, 64, seed=6)
    case.used[7] = 1
    _check_decode(case, rotate=True)


# ----------------------------------------------------------------------------- fused RoPE (read-only q/k)

def gpu_prefill_fused(case, pad_rows=0, sentinel=None):
    run = PrefillRun(case, out_pad_rows=pad_rows)
    if sentinel is not None:
        run.out_full.fill_(sentinel)
    run.step_fused()
    torch.cuda.synchronize()
    return run


@pytest.mark.parametrize("lengths,H,G,window,causal", SMALL_CASES)
def test_fused_rope_small_cases(prefill_kernel, lengths, H, G, window, causal):
    case = wl.make_prefill(lengths, H, G, packed=(H == G), window=window, causal=causal,
                           theta=10000.0, seed=200 + len(lengths) + H + window)
    run = gpu_prefill_fused(case, pad_rows=5, sentinel=float("nan"))
    got = run.out_full.cpu().numpy()
    ref = oracle_prefill(case)
    assert max_err(got[:case.T], ref) <= ATOL
    assert np.all(np.isnan(got[case.T:]))
    # q and k are read-only in the fused path
    assert np.array_equal(run.q.cpu().numpy(), case.q)
    assert np.array_equal(run.k.cpu().numpy(), case.k)


@pytest.mark.parametrize("key", ["0", "1", "3a"])
def test_fused_rope_workload_full_parity(key):
    case = wl.build(key)
    got = gpu_prefill_fused(case).out.cpu().numpy()
    assert max_err(got, oracle_prefill(case)) <= ATOL


def test_fused_rope_matches_prologue_then_attention():
    case = wl.make_prefill([300, 5, 129], 9, 3, packed=False, causal=True, theta=100000.0, seed=21)
    fused = gpu_prefill_fused(case).out.cpu().numpy()
    two_pass = gpu_prefill(case).out.cpu().numpy()
    assert max_err(fused, two_pass) <= ATOL


# ----------------------------------------------------------------------------- binary16 output

def _f16_bound(ref64, got16):
    """Per element: half a binary16 ulp (at the larger of the two magnitudes) plus the FP32 bar."""
    a = np.maximum(np.abs(ref64), np.abs(got16.astype(np.float64))).astype(np.float16)
    return 0.5 * np.spacing(a).astype(np.float64) + ATOL


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("lengths,H,G,window,causal", [SMALL_CASES[2], SMALL_CASES[8],
                                                        SMALL_CASES[9], SMALL_CASES[16]])
def test_f16_output_small_cases(prefill_kernel, fused, lengths, H, G, window, causal):
    case = wl.make_prefill(lengths, H, G, packed=(H == G), window=window, causal=causal,
                           theta=10000.0, seed=300 + len(lengths) + H)
    run = PrefillRun(case)
    out16 = torch.full((case.T + 3, H * D), float("nan"), dtype=torch.float16, device="cuda")
    if not fused:
        run.rope()
    run.attention_f16(out16[:case.T], fused=fused)
    torch.cuda.synchronize()
    got = out16.cpu().numpy()
    tables = oracle.rope_tables(case.theta, max(case.max_seqlen, 1))
    ref64 = oracle.varlen_attention(case.q, case.k, case.v, case.cu, H, G, window, causal,
                                    tables=tables, threads=16, out_dtype=np.float64)
    err = np.abs(got[:case.T].astype(np.float64) - ref64)
    assert np.all(err <= _f16_bound(ref64, got[:case.T]))
    assert np.all(np.isnan(got[case.T:]))


def test_f16_output_local_layer_workload():
    # the ModernBERT local layer (64 x U[16,512], window 128), every element
    case = wl.build("1")
    run = PrefillRun(case)
    out16 = torch.empty((case.T, case.H * D), dtype=torch.float16, device="cuda")
    run.attention_f16(out16, fused=True)
    torch.cuda.synchronize()
    got = out16.cpu().numpy()
    tables = oracle.rope_tables(case.theta, case.max_seqlen)
    ref64 = oracle.varlen_attention(case.q, case.k, case.v, case.cu, case.H, case.G, case.window,
                                    case.causal, tables=tables, threads=16, out_dtype=np.float64)
    err = np.abs(got.astype(np.float64) - ref64)
    assert np.all(err <= _f16_bound(ref64, got))


# ----------------------------------------------------------------------------- chunked prefill from a cache

from transformer_attention_varlen_amd.session import ChunkRun  # noqa: E402


def _check_chunk(case, rotate, pad_rows=3, atol=ATOL):
    run = ChunkRun(case, rotate=rotate, out_pad_rows=pad_rows)
    run.out_full.fill_(float("nan"))
    run.step()
    torch.cuda.synchronize()
    tables = oracle.rope_tables(case.theta, case.cap) if rotate else None
    ref, kc, vc = oracle.prefill_cached(case.q, case.k, case.v, case.cu, case.offsets,
                                        case.k_cache, case.v_cache, case.H, case.G, tables=tables,
                                        threads=16)
    got = run.out_full.cpu().numpy()
    assert max_err(got[:case.T], ref) <= atol
    assert np.all(np.isnan(got[case.T:]))  # rows past T are never written
    gk, gv = run.k_cache.cpu().numpy(), run.v_cache.cpu().numpy()
    for b in range(case.B):
        o, n = int(case.offsets[b]), int(case.lengths[b])
        assert max_err(gk[b, :, o:o + n], kc[b, :, o:o + n]) <= ROPE_ATOL
        assert np.array_equal(gv[b, :, o:o + n], vc[b, :, o:o + n])
        gk[b, :, o:o + n] = kc[b, :, o:o + n]
    # every other cache row is untouched (bit for bit, NaN contents included)
    assert np.array_equal(gk.view(np.uint32), kc.view(np.uint32))
    assert np.array_equal(gv.view(np.uint32), vc.view(np.uint32))
    # q, k and v are read-only
    assert np.array_equal(run.q.cpu().numpy(), case.q)
    assert np.array_equal(run.k.cpu().numpy(), case.k)
    return run


CHUNK_CASES = [
    # lengths, offsets, H, G, cap
    ([1, 31, 32, 33, 129], [0, 0, 5, 100, 200], 9, 3, 400),
    ([200, 0, 64, 1], [0, 17, 300, 399], 4, 4, 400),
    ([150, 77], [250, 323], 8, 2, 400),        # chunks that end at the last cache row
    ([300], [0], 6, 2, 300),                   # a fresh cache filled exactly
    ([65, 2, 127], [1, 63, 128], 5, 1, 256),
]


@pytest.mark.parametrize("rotate", [True, False])
@pytest.mark.parametrize("lengths,offsets,H,G,cap", CHUNK_CASES)
def test_prefill_cached_small_cases(prefill_kernel, rotate, lengths, offsets, H, G, cap):
    case = wl.make_chunked(lengths, offsets, H, G, cap, theta=1e5, seed=500 + H + cap)
    # cache rows from the chunk's first row on are write-only to the call: NaN must not leak
    for b, (n, o) in enumerate(zip(lengths, offsets)):
        case.k_cache[b, :, o:] = np.nan
        case.v_cache[b, :, o:] = np.nan
    _check_chunk(case, rotate)


def test_prefill_cached_full_workload():
    _check_chunk(wl.build("5"), rotate=True, pad_rows=0)


def test_prefill_cached_two_chunks_match_one():
    H, G, cap, n, split, off0 = 9, 3, 1024, 500, 173, 211
    one = wl.make_chunked([n], [off0], H, G, cap, seed=61)
    r1 = ChunkRun(one)
    r1.step()
    torch.cuda.synchronize()
    a = wl.ChunkCase("a", np.array([split], np.int32), np.array([0, split], np.int32),
                     np.array([off0], np.int32), H, G, cap, one.theta, one.k_cache, one.v_cache,
                     one.q[:split], one.k[:split], one.v[:split])
    ra = ChunkRun(a)
    ra.step()
    torch.cuda.synchronize()
    b = wl.ChunkCase("b", np.array([n - split], np.int32), np.array([0, n - split], np.int32),
                     np.array([off0 + split], np.int32), H, G, cap, one.theta,
                     ra.k_cache.cpu().numpy(), ra.v_cache.cpu().numpy(), one.q[split:],
                     one.k[split:], one.v[split:])
    rb = ChunkRun(b)
    rb.step()
    torch.cuda.synchronize()
    both = np.concatenate([ra.out.cpu().numpy(), rb.out.cpu().numpy()])
    assert max_err(both, r1.out.cpu().numpy()) <= ATOL
    assert torch.equal(rb.k_cache.cpu(), r1.k_cache.cpu())
    assert torch.equal(rb.v_cache.cpu(), r1.v_cache.cpu())


def test_prefill_cached_one_row_chunks_match_decode():
    H, G, cap = 9, 3, 520
    used = np.array([1, 2, 255, 256, 257, 300, 513], np.int32)
    dec = _decode_case(used, H, G, cap, seed=62)
    d = DecodeRun(dec, rotate=True)
    d.step()
    B = len(used)
    ch = wl.ChunkCase("c", np.ones(B, np.int32), np.arange(B + 1, dtype=np.int32), used - 1, H, G,
                      cap, dec.theta, dec.k_cache, dec.v_cache, dec.q_new, dec.k_new, dec.v_new)
    c = ChunkRun(ch)
    c.step()
    torch.cuda.synchronize()
    assert max_err(c.out.cpu().numpy(), d.out.cpu().numpy()) <= ATOL
    assert torch.equal(c.v_cache.cpu(), d.v_cache.cpu())
    assert max_err(c.k_cache.cpu().numpy(), d.k_cache.cpu().numpy()) <= ROPE_ATOL


@pytest.mark.parametrize("window,causal,fused", [(-1, True, False), (128, False, True),
                                                 (-1, False, True), (40, True, False)])
def test_both_tile_kernels_agree(monkeypatch, window, causal, fused):
    case = wl.make_prefill([700, 33, 260], 9, 3, packed=False, window=window, causal=causal,
                           theta=1e4, seed=90)
    outs = []
    for mode in ("0", "4", "8", "band"):
        monkeypatch.setenv("KATTN_SPLIT", mode)
        run = PrefillRun(case)
        if fused:
            run.step_fused()
        else:
            run.step()
        torch.cuda.synchronize()
        outs.append(run.out.cpu().numpy())
    assert max_err(outs[0], outs[1]) <= ATOL
    assert max_err(outs[0], outs[2]) <= ATOL
    assert max_err(outs[0], outs[3]) <= ATOL


# ----------------------------------------------------------------------------- large and boundary sizes

@pytest.mark.parametrize("window,causal", [(-1, False), (-1, True), (1024, False), (128, False),
                                           (128, True)])
def test_one_long_sequence_sampled(window, causal):
    # one 40000-token sequence: 64-bit row offsets, long key loops, both tile kernels' range;
    # window 128 runs the sliding-window kernel over runs of about 60 blocks
    n = 40000
    case = wl.make_prefill([n], 2, 1, packed=False, window=window, causal=causal, theta=1e6,
                           seed=95)
    got = gpu_prefill_fused(case).out.cpu().numpy()
    rows = np.array([0, 1, 31, 32, 33, 1023, 1024, 20000, n - 33, n - 32, n - 2, n - 1], np.int32)
    assert max_err(got[rows], oracle_prefill(case, rows=rows)) <= ATOL
    assert np.all(np.isfinite(got))


def test_decode_fills_the_cache_to_capacity():
    # used == cap: the new token lands on the last cache row
    cap = 640
    case = _decode_case([cap, 1, cap - 1, cap], 9, 3, cap, seed=96)
    _check_decode(case, rotate=True)


def test_prefill_cached_chunk_ending_on_the_last_row_of_a_large_cache():
    cap = 16384
    case = wl.make_chunked([700, 1], [cap - 700, cap - 1], 9, 3, cap, seed=97)
    _check_chunk(case, rotate=True, pad_rows=0)


def test_many_tiny_sequences_windowed():
    # 20000 sequences of 1..3 tokens, a window, GQA: the planner's workspace prefix path
    rng = np.random.default_rng(98)
    lengths = rng.integers(1, 4, 20000)
    case = wl.make_prefill(lengths, 4, 2, packed=False, window=2, causal=False, seed=99)
    run = gpu_prefill(case, pad_rows=2, sentinel=float("nan"))
    got = run.out_full.cpu().numpy()
    rows = _sample_rows(case, 64, 100)[:400]
    assert max_err(got[rows], oracle_prefill(case, rows=rows)) <= ATOL
    assert np.all(np.isnan(got[case.T:]))
    assert np.all(np.isfinite(got[:case.T]))


@pytest.mark.parametrize("S", [1023, 1024])
@pytest.mark.parametrize("fused", [False, True])
def test_sliding_window_kernel_at_its_sequence_limit(S, fused):
    # Up to 1023 sequences the sliding-window kernel holds cu in LDS; 1024 fall back to the
    # shared-tile kernel.  Lengths 0..9 (empty sequences included) put several sequence
    # boundaries inside every 32-row tile, so the staged rows' and the queries' sequence
    # cursors cross many boundaries per step; half-window 4.
    rng = np.random.default_rng(400 + S)
    lengths = rng.integers(0, 10, S)
    lengths[rng.integers(0, S, 40)] = 0
    case = wl.make_prefill(lengths, 4, 2, packed=False, window=8, causal=bool(S % 2),
                           theta=1e4, seed=401 + S)
    run = PrefillRun(case, out_pad_rows=2)
    run.out_full.fill_(float("nan"))
    if fused:
        run.step_fused()
    else:
        run.step()
    torch.cuda.synchronize()
    got = run.out_full.cpu().numpy()
    assert max_err(got[:case.T], oracle_prefill(case)) <= ATOL
    assert np.all(np.isnan(got[case.T:]))
