"""kattn_decode_noalloc -- the decode step on the library's static per-GPU scratch -- against
kattn_decode with a caller workspace, through the C ABI.

Both run the same kernels with the same key split, so the outputs and the appended cache rows
agree bit for bit (the bar is the parity tolerance, 2e-5 on the output; the test asks for
equality, which is stronger).  Two calls in a row, the second with a smaller batch and shorter
caches, show that the scratch needs no clearing between calls.
"""
import numpy as np
import pytest
import torch

from transformer_attention_varlen_amd import kattn, workloads as wl

pytestmark = pytest.mark.gpu

D = 64
ATOL = 2e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kattn.lib()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _both(case, rotate=True):
    """(out, k_cache, v_cache) of kattn_decode with a workspace and of kattn_decode_noalloc,
    each on its own copies of the caches."""
    q, kn, vn, used = _dev(case.q_new), _dev(case.k_new), _dev(case.v_new), _dev(case.used)
    if rotate:
        cos_h, sin_h = kattn.kattn_rope_tables(case.theta, case.cap)
        cos, sin = _dev(cos_h), _dev(sin_h)
    else:
        cos = sin = None
    mx = int(case.used.max())
    res = []
    for noalloc in (False, True):
        kc, vc = _dev(case.k_cache), _dev(case.v_cache)
        out = torch.full((case.B, case.H * D), float("nan"), device="cuda")
        if noalloc:
            kattn.kattn_decode_noalloc(out, q, kn, vn, kc, vc, case.cap, used, mx, case.B, case.H,
                                       case.G, cos=cos, sin=sin)
        else:
            ws = torch.empty(kattn.kattn_decode_workspace(case.B, case.H, case.G),
                             dtype=torch.uint8, device="cuda")
            kattn.kattn_decode(out, q, kn, vn, kc, vc, case.cap, used, mx, case.B, case.H, case.G,
                               cos=cos, sin=sin, workspace=ws)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), kc.cpu().numpy(), vc.cpu().numpy()))
    return res


def _small_case(lens, H, G, cap, seed):
    rng = np.random.default_rng(seed)
    B = len(lens)
    return wl.DecodeCase("small", B, H, G, cap, 100000.0,
                         rng.standard_normal((B, G, cap, D), dtype=np.float32),
                         rng.standard_normal((B, G, cap, D), dtype=np.float32),
                         rng.standard_normal((B, H * D), dtype=np.float32),
                         rng.standard_normal((B, G * D), dtype=np.float32),
                         rng.standard_normal((B, G * D), dtype=np.float32),
                         np.array(lens, np.int32))


def _agree(pair):
    (o1, k1, v1), (o2, k2, v2) = pair
    assert np.all(np.isfinite(o2))
    assert float(np.max(np.abs(o1.astype(np.float64) - o2))) <= ATOL
    assert np.array_equal(o1, o2)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


def test_noalloc_matches_the_workspace_call_on_two_calls_in_a_row():
    # the SmolLM2 decode workload (64 sequences, caches [64][3][8192][64]), then a smaller batch
    print("noalloc: smollm2_decode_b64", flush=True)
    _agree(_both(wl.build("4")))
    print("noalloc: 5 sequences, cap 300", flush=True)
    _agree(_both(_small_case([1, 33, 300, 7, 129], 9, 3, 300, seed=11)))


def test_noalloc_without_rotation_and_other_head_ratios():
    for H, G in [(4, 4), (8, 1), (6, 2)]:
        print(f"noalloc: H={H} G={G}", flush=True)
        _agree(_both(_small_case([2, 255, 256, 257, 513], H, G, 520, seed=H + G), rotate=False))


def test_noalloc_rejects_a_batch_beyond_its_scratch():
    # 1024 sequences x 8 kv heads x 8 q heads each need about 19 MB of partials: above 16 MiB
    B, H, G, cap = 1024, 64, 8, 1
    out = torch.empty((B, H * D), device="cuda")
    q = torch.empty((B, H * D), device="cuda")
    kn = torch.empty((B, G * D), device="cuda")
    vn = torch.empty((B, G * D), device="cuda")
    kc = torch.empty((B, G, cap, D), device="cuda")
    vc = torch.empty((B, G, cap, D), device="cuda")
    used = torch.ones(B, dtype=torch.int32, device="cuda")
    out.fill_(3.0)
    with pytest.raises(kattn.KattnError) as e:
        kattn.kattn_decode_noalloc(out, q, kn, vn, kc, vc, cap, used, 1, B, H, G)
    assert e.value.code == kattn.KATTN_EBOUNDS and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool(torch.all(out == 3.0))  # nothing ran
