"""Pins for the FP64 CPU oracle, each against something other than the oracle itself.

The pages print no attention values for a worked example, so the oracle is
pinned by: a library routine the cases reduce to (torch's
``scaled_dot_product_attention`` in float64 on the CPU with an explicit
additive mask and its own GQA repeat; Hugging Face's Llama rotate-half RoPE,
the non-interleaved convention candle's ``rope`` uses), closed forms (uniform
weights over a known index range recover that range's first two moments), the
invariants the ffai-argus text.rs page argues (a skipped column equals a -inf
column bit for bit; the GQA fold equals repeat_kv; a decode step sees the
whole cache; causal rows sum to one with an exactly zero tail) and exact
values (the first RoPE frequency is exactly 1, so its table is libm's cos/sin
of the integer position).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from transformer_attention_varlen_amd import workloads as wl

D = 64


# ----------------------------------------------------------------------------- RoPE tables

@pytest.mark.parametrize("theta", [10000.0, 100000.0, 160000.0])
def test_rope_table_position_zero_is_identity(theta):
    cos, sin = oracle.rope_tables(theta, 4)
    assert np.all(cos[0] == 1.0) and np.all(sin[0] == 0.0)


def test_rope_table_first_frequency_is_exact():
    # theta^0 = 1, so the first pair's angle is the integer position itself.
    cos, sin = oracle.rope_tables(160000.0, 8192)
    for p in [0, 1, 2, 3, 7, 100, 1142, 4095, 8191]:
        assert cos[p, 0] == np.float32(math.cos(p))
        assert sin[p, 0] == np.float32(math.sin(p))


@pytest.mark.parametrize("theta", [10000.0, 100000.0, 160000.0])
def test_rope_table_within_f32_angle_rounding(theta):
    # Against the exact angle p * theta^(-i/32): the table's angle carries at most
    # three f32 roundings (theta^e, 1/x, p*inv), each <= 2^-24 relative, and the
    # stored cos/sin one more 2^-25 absolute.
    L = 8192
    cos, sin = oracle.rope_tables(theta, L)
    p = np.arange(L, dtype=np.float64)[:, None]
    i = np.arange(32, dtype=np.float64)[None, :]
    ang = p * theta ** (-i / 32.0)
    bound = 3.0 * 2.0 ** -24 * ang + 2.0 ** -24 + 1e-12
    assert np.all(np.abs(cos - np.cos(ang)) <= bound)
    assert np.all(np.abs(sin - np.sin(ang)) <= bound)
    # and a plausible mistake -- the exponent i/64 instead of 2i/64 -- is far outside it
    wrong = p * theta ** (-i / 64.0)
    assert np.max(np.abs(cos - np.cos(wrong))) > 0.1


def _angle_is_an_f32_number(cos, sin, theta, p0, p1, ulps=8):
    """Per table entry (p in [p0, p1), every pair i): is there an f32 number within `ulps` f32
    steps of the exact angle p * theta^(-i/32) whose cosine and sine, each rounded once to f32,
    are exactly the stored entries?"""
    p = np.arange(p0, p1, dtype=np.float64)[:, None]
    i = np.arange(32, dtype=np.float64)[None, :]
    exact = p * theta ** (-i / 32.0)
    up = np.float32(exact)
    down = up.copy()
    c, s = cos[p0:p1], sin[p0:p1]
    hit = (np.float32(np.cos(np.float64(up))) == c) & (np.float32(np.sin(np.float64(up))) == s)
    for _ in range(ulps):
        up = np.nextafter(up, np.float32(np.inf))
        down = np.nextafter(down, np.float32(-np.inf))
        for a in (up, down):
            a64 = np.float64(a)
            hit |= (np.float32(np.cos(a64)) == c) & (np.float32(np.sin(a64)) == s)
    return hit


@pytest.mark.parametrize("theta", [10000.0, 100000.0, 160000.0])
def test_rope_table_angle_is_rounded_to_f32_before_cos_and_sin(theta):
    # The CUDA backend page (kime-cuda plan.rs, `rope_tables`) forms the angle as the product
    # of the f32 position and an f32 inverse frequency, in f32, and only then widens it for
    # cos and sin.  So every stored pair is cos/sin of some f32 number near the exact angle.
    # Past position 4096 neighbouring f32 angles are >= 2^-12 rad apart, far more than an f32
    # rounding of cos or sin, so an angle formed in f64 (not on the f32 grid) fails this.
    L = 8192
    cos, sin = oracle.rope_tables(theta, L)
    assert np.all(_angle_is_an_f32_number(cos, sin, theta, 0, L))
    # The same check on tables whose angle is left in f64 (the mistake this pin is for): at
    # angles of 64 rad and more (f32 steps >= 2^-17 rad) almost no entry has an f32 angle that
    # reproduces it.  (At small angles the two tables agree, so those entries prove nothing.)
    e = np.float32(np.arange(32, dtype=np.float32) * np.float32(2.0 / 64.0))
    inv = np.float32(1.0) / np.float32(theta ** np.float64(e))
    a64 = np.arange(4096, L, dtype=np.float64)[:, None] * np.float64(inv)[None, :]
    mc = np.zeros((L, 32), np.float32)
    ms = np.zeros((L, 32), np.float32)
    mc[4096:], ms[4096:] = np.float32(np.cos(a64)), np.float32(np.sin(a64))
    hit = _angle_is_an_f32_number(mc, ms, theta, 4096, L)
    large = a64 >= 64.0
    assert large.sum() > 4096 and np.mean(hit[large]) < 0.1


# ----------------------------------------------------------------------------- RoPE rotation

def _hf_rope(x64, pos, cos, sin):
    """Hugging Face Llama rotate-half RoPE (library routine) on (T, heads, 64) float64."""
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb
    c = torch.from_numpy(np.concatenate([cos[pos], cos[pos]], -1).astype(np.float64))
    s = torch.from_numpy(np.concatenate([sin[pos], sin[pos]], -1).astype(np.float64))
    xt = torch.from_numpy(x64).transpose(0, 1)[None]        # (1, heads, T, 64)
    y, _ = apply_rotary_pos_emb(xt, xt, c[None], s[None], unsqueeze_dim=1)
    return y[0].transpose(0, 1).numpy()


def test_rope_matches_library_rotate_half():
    rng = np.random.default_rng(7)
    T, heads = 300, 5
    x = rng.standard_normal((T, heads * D), dtype=np.float32)
    pos = rng.integers(0, 8192, T).astype(np.int32)
    cos, sin = oracle.rope_tables(100000.0, 8192)
    ours = oracle.rope_apply(x, heads, pos, cos, sin).reshape(T, heads, D)
    ref = _hf_rope(x.astype(np.float64).reshape(T, heads, D), pos, cos, sin)
    # ours is the f64 rotation rounded once to f32: within half an f32 ulp
    assert np.all(np.abs(ours - ref) <= np.abs(ref) * 2.0 ** -24 + 1e-30)


def test_rope_preserves_pair_norms_and_keeps_zero():
    rng = np.random.default_rng(8)
    T = 64
    x = rng.standard_normal((T, D), dtype=np.float32)
    pos = np.arange(T, dtype=np.int32) * 97
    cos, sin = oracle.rope_tables(10000.0, 8192)
    y = oracle.rope_apply(x, 1, pos, cos, sin).astype(np.float64)
    n_in = x[:, :32].astype(np.float64) ** 2 + x[:, 32:].astype(np.float64) ** 2
    n_out = y[:, :32] ** 2 + y[:, 32:] ** 2
    unit = cos[pos].astype(np.float64) ** 2 + sin[pos].astype(np.float64) ** 2
    assert np.allclose(n_out, n_in * unit, rtol=1e-6, atol=1e-6)
    z = oracle.rope_apply(np.zeros((T, D), np.float32), 1, pos, cos, sin)
    assert np.all(z == 0.0)


# ----------------------------------------------------------------------------- attention vs library

def _sdpa_reference(case, tables=None):
    """torch SDPA (float64, CPU) per sequence with an explicit additive mask and its GQA repeat."""
    H, G = case.H, case.G
    out = np.zeros((case.T, H * D), np.float64)
    for s in range(case.S):
        lo, hi = int(case.cu[s]), int(case.cu[s + 1])
        n = hi - lo
        if n == 0:
            continue
        q = case.q[lo:hi].astype(np.float64).reshape(n, H, D)
        k = case.k[lo:hi].astype(np.float64).reshape(n, G, D)
        v = case.v[lo:hi].astype(np.float64).reshape(n, G, D)
        if tables is not None:
            pos = np.arange(n)
            q = _hf_rope(q, pos, *tables)
            k = _hf_rope(k, pos, *tables)
        i = np.arange(n)[:, None]
        j = np.arange(n)[None, :]
        ok = np.ones((n, n), bool)
        if case.window >= 0:
            ok &= np.abs(i - j) <= case.window // 2
        if case.causal:
            ok &= j <= i
        mask = torch.from_numpy(np.where(ok, 0.0, -np.inf))
        qt = torch.from_numpy(q).transpose(0, 1)[None]
        kt = torch.from_numpy(np.ascontiguousarray(k)).transpose(0, 1)[None].contiguous()
        vt = torch.from_numpy(np.ascontiguousarray(v)).transpose(0, 1)[None].contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(
            qt.contiguous(), kt, vt, attn_mask=mask, scale=0.125, enable_gqa=(H != G))
        out[lo:hi] = o[0].transpose(0, 1).reshape(n, H * D).numpy()
    return out


SMALL_MASKS = [(-1, False), (-1, True), (0, False), (1, False), (2, False), (3, True),
               (4, False), (7, False), (9, True), (16, False)]


@pytest.mark.parametrize("window,causal", SMALL_MASKS)
@pytest.mark.parametrize("H,G", [(4, 4), (4, 2), (6, 2), (3, 1)])
def test_attention_matches_library_on_tiny_inputs(window, causal, H, G):
    case = wl.make_prefill([1, 2, 5, 8, 0, 3], H, G, packed=(H == G), window=window,
                           causal=causal, seed=11 + H + G)
    ours = oracle.varlen_attention(case.q, case.k, case.v, case.cu, H, G, window, causal)
    ref = _sdpa_reference(case)
    assert np.all(np.abs(ours - ref) <= np.abs(ref) * 2.0 ** -23 + 1e-12)


@pytest.mark.parametrize("window,causal", [(-1, False), (-1, True), (6, False), (5, True)])
def test_attention_with_rope_matches_library(window, causal):
    case = wl.make_prefill([13, 1, 30], 6, 2, packed=False, window=window, causal=causal,
                           theta=100000.0, seed=5)
    tables = oracle.rope_tables(case.theta, 64)
    ours = oracle.varlen_attention(case.q, case.k, case.v, case.cu, case.H, case.G, window,
                                   causal, tables=tables)
    ref = _sdpa_reference(case, tables)
    assert np.all(np.abs(ours - ref) <= np.abs(ref) * 2.0 ** -23 + 1e-12)


# ----------------------------------------------------------------------------- closed forms

def _moment_case(lengths, H, G, window, causal):
    """q = 0 (uniform weights), v_j = [1, p_j, p_j^2, 0, ...] with p_j the key's position."""
    case = wl.make_prefill(lengths, H, G, packed=False, window=window, causal=causal, seed=3)
    case.q[:] = 0.0
    case.v[:] = 0.0
    for s in range(case.S):
        lo, hi = int(case.cu[s]), int(case.cu[s + 1])
        p = np.arange(hi - lo, dtype=np.float32)
        for g in range(G):
            case.v[lo:hi, g * D + 0] = 1.0
            case.v[lo:hi, g * D + 1] = p
            case.v[lo:hi, g * D + 2] = p * p
    return case


def _range_moments(a, b):
    """Mean and mean square of the integers a..b (closed forms)."""
    cnt = b - a + 1
    s1 = (a + b) * cnt / 2.0
    sq = lambda m: m * (m + 1) * (2 * m + 1) / 6.0
    s2 = sq(b) - (sq(a - 1) if a > 0 else 0.0)
    return s1 / cnt, s2 / cnt


@pytest.mark.parametrize("window,causal", [(-1, False), (-1, True), (0, False), (1, False),
                                           (128, False), (5, False), (7, True), (64, True)])
def test_uniform_weights_recover_the_visible_range(window, causal):
    lengths = [1, 37, 91, 130, 2]
    case = _moment_case(lengths, 4, 2, window, causal)
    tables = oracle.rope_tables(10000.0, 256)   # rotating q = 0 keeps it 0
    out = oracle.varlen_attention(case.q, case.k, case.v, case.cu, 4, 2, window, causal,
                                  tables=tables)
    h = window // 2 if window >= 0 else 10 ** 9
    for s in range(case.S):
        lo, hi = int(case.cu[s]), int(case.cu[s + 1])
        n = hi - lo
        for i in range(n):
            a = max(0, i - h)
            b = i if causal else min(n - 1, i + h)
            m1, m2 = _range_moments(a, b)
            for head in range(4):
                row = out[lo + i, head * D: head * D + 3].astype(np.float64)
                assert row[0] == pytest.approx(1.0, abs=1e-7)
                assert row[1] == pytest.approx(m1, rel=1e-6, abs=1e-6)
                assert row[2] == pytest.approx(m2, rel=1e-6, abs=1e-6)
            assert np.all(out[lo + i].reshape(4, D)[:, 3:] == 0.0)


@pytest.mark.parametrize("window,causal", SMALL_MASKS)
def test_rows_sum_to_one(window, causal):
    case = wl.make_prefill([33, 64, 5], 2, 2, packed=True, window=window, causal=causal, seed=4)
    case.v[:] = 1.0
    out = oracle.varlen_attention(case.q, case.k, case.v, case.cu, 2, 2, window, causal)
    assert np.all(np.abs(out - 1.0) <= 2.0 ** -23)


def test_causal_probabilities_through_identity_values():
    # V = I recovers P: each causal row sums to one and its tail past the limit is exactly 0
    # (the argus tests on s = 33 with two heads).
    n, H = 33, 2
    case = wl.make_prefill([n], H, H, packed=False, causal=True, seed=9)
    case.q[:] *= 3.0
    case.v[:] = 0.0
    for h in range(H):
        case.v[:, h * D:h * D + n] = np.eye(n, dtype=np.float32)
    P = oracle.varlen_attention(case.q, case.k, case.v, case.cu, H, H, -1, True)
    for h in range(H):
        for i in range(n):
            row = P[i, h * D:h * D + n].astype(np.float64)
            assert abs(row.sum() - 1.0) < 1e-6
            assert np.all(row[:i + 1] > 0.0)
            assert np.all(row[i + 1:] == 0.0)


# ----------------------------------------------------------------------------- invariants

ALL_MASKS = SMALL_MASKS + [(128, False), (33, True)]


@pytest.mark.parametrize("window,causal", ALL_MASKS)
def test_skipping_masked_columns_is_bit_identical_to_minus_inf(window, causal):
    case = wl.make_prefill([40, 1, 77, 12], 4, 2, packed=False, window=window, causal=causal,
                           seed=21)
    tables = oracle.rope_tables(10000.0, 128)
    a = oracle.varlen_attention(case.q, case.k, case.v, case.cu, 4, 2, window, causal,
                                tables=tables, mask_mode=0)
    b = oracle.varlen_attention(case.q, case.k, case.v, case.cu, 4, 2, window, causal,
                                tables=tables, mask_mode=1)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_window_of_twice_the_length_equals_global(causal):
    case = wl.make_prefill([50, 17, 90], 4, 4, packed=True, causal=causal, seed=22)
    tables = oracle.rope_tables(10000.0, 128)
    glob = oracle.varlen_attention(case.q, case.k, case.v, case.cu, 4, 4, -1, causal,
                                   tables=tables)
    wide = oracle.varlen_attention(case.q, case.k, case.v, case.cu, 4, 4, 180, causal,
                                   tables=tables)
    assert np.array_equal(glob, wide)


@pytest.mark.parametrize("window,causal", [(-1, False), (-1, True), (10, False)])
def test_gqa_equals_mha_with_repeated_kv(window, causal):
    H, G = 9, 3
    case = wl.make_prefill([31, 60], H, G, packed=False, window=window, causal=causal, seed=23)
    tables = oracle.rope_tables(100000.0, 64)
    gqa = oracle.varlen_attention(case.q, case.k, case.v, case.cu, H, G, window, causal,
                                  tables=tables)
    T = case.T
    k_rep = np.repeat(case.k.reshape(T, G, 1, D), H // G, axis=2).reshape(T, H * D)
    v_rep = np.repeat(case.v.reshape(T, G, 1, D), H // G, axis=2).reshape(T, H * D)
    mha = oracle.varlen_attention(case.q, k_rep, v_rep, case.cu, H, H, window, causal,
                                  tables=tables)
    assert np.array_equal(gqa, mha)


@pytest.mark.parametrize("window,causal", [(-1, False), (-1, True), (12, False)])
def test_each_sequence_alone_equals_its_rows_in_the_batch(window, causal):
    lengths = [20, 0, 45, 7]
    case = wl.make_prefill(lengths, 4, 4, packed=True, window=window, causal=causal, seed=24)
    tables = oracle.rope_tables(10000.0, 64)
    packed = oracle.varlen_attention(case.q, case.k, case.v, case.cu, 4, 4, window, causal,
                                     tables=tables)
    for s, n in enumerate(lengths):
        lo = int(case.cu[s])
        cu1 = np.array([0, n], np.int32)
        alone = oracle.varlen_attention(case.q[lo:lo + n], case.k[lo:lo + n], case.v[lo:lo + n],
                                        cu1, 4, 4, window, causal, tables=tables)
        assert np.array_equal(alone, packed[lo:lo + n])


def test_sampled_rows_equal_full_rows():
    case = wl.make_prefill([70, 3, 129], 4, 2, packed=False, window=20, causal=False, seed=25)
    tables = oracle.rope_tables(10000.0, 256)
    full = oracle.varlen_attention(case.q, case.k, case.v, case.cu, 4, 2, 20, False,
                                   tables=tables)
    rows = np.array([0, 69, 70, 72, 73, 201, 100], np.int32)
    part = oracle.varlen_attention(case.q, case.k, case.v, case.cu, 4, 2, 20, False,
                                   tables=tables, rows=rows)
    assert np.array_equal(part, full[rows])


# ----------------------------------------------------------------------------- decode

def test_decode_equals_last_causal_row_bitwise_without_rotation():
    # Unrotated inputs: the decode row over a cache holding the sequence's keys is the last
    # row of causal prefill on that sequence (argus `CausalSoftmax` with offset L-1).
    H, G, cap = 9, 3, 96
    rng = np.random.default_rng(31)
    lens = [1, 50, 96]
    B = len(lens)
    kc = rng.standard_normal((B, G, cap, D), dtype=np.float32)
    vc = rng.standard_normal((B, G, cap, D), dtype=np.float32)
    qn = rng.standard_normal((B, H * D), dtype=np.float32)
    kn = rng.standard_normal((B, G * D), dtype=np.float32)
    vn = rng.standard_normal((B, G * D), dtype=np.float32)
    used = np.array(lens, np.int32)
    out, kc2, vc2 = oracle.decode(qn, kn, vn, kc, vc, used, H, G)
    for b, L in enumerate(lens):
        k_seq = kc2[b, :, :L].transpose(1, 0, 2).reshape(L, G * D)
        v_seq = vc2[b, :, :L].transpose(1, 0, 2).reshape(L, G * D)
        q_seq = np.zeros((L, H * D), np.float32)
        q_seq[L - 1] = qn[b]
        pre = oracle.varlen_attention(q_seq, k_seq, v_seq, np.array([0, L], np.int32), H, G,
                                      -1, True)
        assert np.array_equal(pre[L - 1], out[b])
        # the append wrote row L-1 and nothing else
        assert np.array_equal(kc2[b, :, L - 1], kn[b].reshape(G, D))
        assert np.array_equal(vc2[b, :, L - 1], vn[b].reshape(G, D))
        mask = np.ones(cap, bool)
        mask[L - 1] = False
        assert np.array_equal(kc2[b][:, mask], kc[b][:, mask])
        assert np.array_equal(vc2[b][:, mask], vc[b][:, mask])


def test_decode_with_rotation_matches_causal_prefill():
    H, G, L = 6, 2, 70
    case = wl.make_prefill([L], H, G, packed=False, causal=True, theta=100000.0, seed=32)
    tables = oracle.rope_tables(case.theta, 128)
    pre = oracle.varlen_attention(case.q, case.k, case.v, case.cu, H, G, -1, True,
                                  tables=tables)
    cap = 128
    kc = np.zeros((1, G, cap, D), np.float32)
    vc = np.zeros((1, G, cap, D), np.float32)
    pos = np.arange(L - 1, dtype=np.int32)
    kc[0, :, :L - 1] = oracle.rope_apply(case.k[:L - 1], G, pos, *tables).reshape(
        L - 1, G, D).transpose(1, 0, 2)
    vc[0, :, :L - 1] = case.v[:L - 1].reshape(L - 1, G, D).transpose(1, 0, 2)
    out, kc2, _ = oracle.decode(case.q[L - 1:], case.k[L - 1:], case.v[L - 1:], kc, vc,
                                np.array([L], np.int32), H, G, tables=tables)
    # decode scores keys stored in f32; prefill keeps them in f64: a rounding apart
    assert np.max(np.abs(out[0] - pre[L - 1])) < 1e-6
    # the appended key is the rotated new key (library rotate-half, f32 rounding)
    ref = _hf_rope(case.k[L - 1:].astype(np.float64).reshape(1, G, D), np.array([L - 1]),
                   *tables)
    assert np.all(np.abs(kc2[0, :, L - 1] - ref[0]) <= np.abs(ref[0]) * 2.0 ** -24 + 1e-30)


def test_decode_attends_to_the_entire_cache():
    # q = 0, v_j = [1, j, j^2]: the output is the mean over 0..L-1, so L is recovered exactly,
    # appended row included (argus `a_decode_step_attends_to_the_entire_cache`).
    H, G, cap = 3, 1, 200
    lens = np.array([1, 2, 40, 199, 200], np.int32)
    B = len(lens)
    kc = np.random.default_rng(1).standard_normal((B, G, cap, D), dtype=np.float32)
    vc = np.zeros((B, G, cap, D), np.float32)
    j = np.arange(cap, dtype=np.float32)
    vc[:, :, :, 0] = 1.0
    vc[:, :, :, 1] = j
    vc[:, :, :, 2] = j * j
    qn = np.zeros((B, H * D), np.float32)
    kn = np.random.default_rng(2).standard_normal((B, G * D), dtype=np.float32)
    vn = np.zeros((B, G * D), np.float32)
    vn[:, 0] = 1.0
    vn[:, 1] = lens - 1
    vn[:, 2] = (lens - 1.0) ** 2
    tables = oracle.rope_tables(100000.0, 256)
    out, _, _ = oracle.decode(qn, kn, vn, kc, vc, lens, H, G, tables=tables)
    for b, L in enumerate(lens):
        m1, m2 = _range_moments(0, int(L) - 1)
        for h in range(H):
            assert out[b, h * D] == pytest.approx(1.0, abs=1e-7)
            assert out[b, h * D + 1] == pytest.approx(m1, rel=1e-6, abs=1e-6)
            assert out[b, h * D + 2] == pytest.approx(m2, rel=1e-6, abs=1e-6)


def test_decode_probabilities_all_positive_and_sum_to_one():
    H, G, cap, L = 2, 2, 40, 40
    rng = np.random.default_rng(3)
    kc = rng.standard_normal((1, G, cap, D), dtype=np.float32)
    vc = np.zeros((1, G, cap, D), np.float32)
    for g in range(G):
        vc[0, g, :, :L] = np.eye(L, dtype=np.float32)
    qn = rng.standard_normal((1, H * D), dtype=np.float32) * 2
    kn = rng.standard_normal((1, G * D), dtype=np.float32)
    vn = np.zeros((1, G * D), np.float32)
    for g in range(G):
        vn[0, g * D + L - 1] = 1.0
    out, _, _ = oracle.decode(qn, kn, vn, kc, vc, np.array([L], np.int32), H, G)
    for h in range(H):
        p = out[0, h * D:h * D + L].astype(np.float64)
        assert np.all(p > 0.0)
        assert abs(p.sum() - 1.0) < 1e-6


# ----------------------------------------------------------------------------- argument checks

def test_oracle_rejects_bad_offsets():
    q = np.zeros((4, D), np.float32)
    with pytest.raises(ValueError):
        oracle.varlen_attention(q, q, q, np.array([0, 3, 2, 4], np.int32), 1, 1)
    with pytest.raises(ValueError):
        oracle.varlen_attention(q, q, q, np.array([1, 4], np.int32), 1, 1)
    with pytest.raises(ValueError):
        oracle.varlen_attention(q, q, q, np.array([0, 4], np.int32), 3, 2)


# ----------------------------------------------------------------------------- wide output

def test_fp64_output_rounds_to_the_fp32_output_bit_for_bit():
    # the FP64-output entry is the same arithmetic with the final rounding left out
    rng = np.random.default_rng(31)
    cu = np.array([0, 5, 40, 41], np.int32)
    T, H, G = 41, 4, 2
    q = rng.standard_normal((T, H * 64), dtype=np.float32)
    k = rng.standard_normal((T, G * 64), dtype=np.float32)
    v = rng.standard_normal((T, G * 64), dtype=np.float32)
    tables = oracle.rope_tables(10000.0, 40)
    for window, causal in [(-1, False), (8, True)]:
        a = oracle.varlen_attention(q, k, v, cu, H, G, window, causal, tables=tables)
        b = oracle.varlen_attention(q, k, v, cu, H, G, window, causal, tables=tables,
                                    out_dtype=np.float64)
        assert b.dtype == np.float64
        assert np.array_equal(b.astype(np.float32), a)


def test_binary16_rounding_step_is_round_to_nearest_even():
    # the FP16-output comparison rounds the oracle's FP64 result once with numpy; pin that
    # step on values whose binary16 encodings follow from the format's definition
    cases = {1.0: 0x3C00, 1.0 / 3.0: 0x3555, 2049.0: 0x6800, 2051.0: 0x6802,
             1.0 + 2.0 ** -11: 0x3C00, 1.0 + 3 * 2.0 ** -11: 0x3C02, 65504.0: 0x7BFF,
             65520.0: 0x7C00, 2.0 ** -24: 0x0001, 2.0 ** -25: 0x0000, -0.5: 0xB800}
    with np.errstate(over="ignore"):  # 65520 rounds up to infinity, as the format says
        for x, bits in cases.items():
            assert int(np.float64(x).astype(np.float16).view(np.uint16)) == bits, x


# ----------------------------------------------------------------------------- chunked prefill from a cache

def _chunk_inputs(lengths, offsets, H, G, cap, seed):
    rng = np.random.default_rng(seed)
    B = len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    q = rng.standard_normal((T, H * D), dtype=np.float32)
    k = rng.standard_normal((T, G * D), dtype=np.float32)
    v = rng.standard_normal((T, G * D), dtype=np.float32)
    kc = rng.standard_normal((B, G, cap, D), dtype=np.float32)
    vc = rng.standard_normal((B, G, cap, D), dtype=np.float32)
    return cu, np.array(offsets, np.int32), q, k, v, kc, vc


def test_prefill_cached_one_row_chunks_are_decode_steps_bit_for_bit():
    H, G, cap = 9, 3, 300
    lengths, offsets = [1, 1, 1, 1], [0, 17, 128, 299]
    cu, off, q, k, v, kc, vc = _chunk_inputs(lengths, offsets, H, G, cap, 41)
    tables = oracle.rope_tables(1e5, cap)
    a, ka, va = oracle.prefill_cached(q, k, v, cu, off, kc, vc, H, G, tables=tables)
    b, kb, vb = oracle.decode(q, k, v, kc, vc, off + 1, H, G, tables=tables)
    assert np.array_equal(a, b) and np.array_equal(ka, kb) and np.array_equal(va, vb)


def test_prefill_cached_two_chunks_equal_one_chunk_bit_for_bit():
    H, G, cap = 4, 2, 400
    n, split, off0 = 150, 61, 37
    cu, off, q, k, v, kc, vc = _chunk_inputs([n], [off0], H, G, cap, 42)
    tables = oracle.rope_tables(1e4, cap)
    whole, kw, vw = oracle.prefill_cached(q, k, v, cu, off, kc, vc, H, G, tables=tables)
    o1, k1, v1 = oracle.prefill_cached(q[:split], k[:split], v[:split], [0, split], [off0], kc, vc,
                                       H, G, tables=tables)
    o2, k2, v2 = oracle.prefill_cached(q[split:], k[split:], v[split:], [0, n - split],
                                       [off0 + split], k1, v1, H, G, tables=tables)
    assert np.array_equal(np.concatenate([o1, o2]), whole)
    assert np.array_equal(k2, kw) and np.array_equal(v2, vw)


def test_prefill_cached_from_an_empty_cache_is_causal_attention():
    # inputs already rotated: the stored keys are the inputs themselves, and the causal
    # varlen definition (materialised -inf mask) gives the same bits
    H, G, cap = 6, 2, 256
    lengths = [70, 1, 200]
    cu, off, q, k, v, kc, vc = _chunk_inputs(lengths, [0, 0, 0], H, G, cap, 43)
    a, _, _ = oracle.prefill_cached(q, k, v, cu, off, kc, vc, H, G)
    b = oracle.varlen_attention(q, k, v, cu, H, G, -1, True)
    assert np.array_equal(a, b)
    # with rotation the cache holds f32-rounded keys: agreement to the rounding of k
    tables = oracle.rope_tables(1e5, cap)
    a, _, _ = oracle.prefill_cached(q, k, v, cu, off, kc, vc, H, G, tables=tables)
    b = oracle.varlen_attention(q, k, v, cu, H, G, -1, True, tables=tables)
    assert np.max(np.abs(a - b)) <= 1e-6


def test_prefill_cached_uniform_weights_recover_the_causal_range_with_offset():
    # q = 0: key j <= p has weight 1/(p+1); v_j = [1, j, j^2] gives [1, p/2, p(2p+1)/6]
    H, G, cap = 2, 1, 64
    lengths, offsets = [5, 9, 1], [0, 20, 63]
    cu, off, q, k, v, kc, vc = _chunk_inputs(lengths, offsets, H, G, cap, 44)
    q[:] = 0.0
    j = np.arange(cap, dtype=np.float32)
    vc[:, :, :, :] = 0.0
    vc[:, :, :, 0], vc[:, :, :, 1], vc[:, :, :, 2] = 1.0, j, j * j
    v[:] = 0.0
    for b in range(len(lengths)):
        for i in range(lengths[b]):
            p = offsets[b] + i
            v[cu[b] + i, 0:3] = [1.0, p, p * p]
    out, _, _ = oracle.prefill_cached(q, k, v, cu, off, kc, vc, H, G)
    for b in range(len(lengths)):
        for i in range(lengths[b]):
            p = offsets[b] + i
            want = np.array([1.0, p / 2.0, p * (2 * p + 1) / 6.0])
            for h in range(H):
                got = out[cu[b] + i, h * D:h * D + 3].astype(np.float64)
                assert np.allclose(got, want, rtol=1e-6, atol=0), (b, i, h)


def test_prefill_cached_writes_exactly_the_chunk_rows():
    H, G, cap = 4, 2, 128
    lengths, offsets = [10, 0, 33], [5, 7, 95]
    cu, off, q, k, v, kc, vc = _chunk_inputs(lengths, offsets, H, G, cap, 45)
    tables = oracle.rope_tables(1e4, cap)
    _, k2, v2 = oracle.prefill_cached(q, k, v, cu, off, kc, vc, H, G, tables=tables)
    for b in range(3):
        lo, n, o = int(cu[b]), lengths[b], offsets[b]
        pos = np.arange(o, o + n, dtype=np.int32)
        krot = oracle.rope_apply(k[lo:lo + n], G, pos, *tables) if n else np.zeros((0, G * D))
        for g in range(G):
            assert np.array_equal(k2[b, g, o:o + n], krot[:, g * D:(g + 1) * D])
            assert np.array_equal(v2[b, g, o:o + n], v[lo:lo + n, g * D:(g + 1) * D])
            rest = np.r_[0:o, o + n:cap]
            assert np.array_equal(k2[b, g, rest], kc[b, g, rest])
            assert np.array_equal(v2[b, g, rest], vc[b, g, rest])


def test_prefill_cached_rejects_a_chunk_past_the_capacity():
    cu, off, q, k, v, kc, vc = _chunk_inputs([10], [60], 2, 1, 64, 46)
    with pytest.raises(ValueError):
        oracle.prefill_cached(q, k, v, cu, off, kc, vc, 2, 1)
