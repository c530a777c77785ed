"""KATTN_CHECK=1: device tables validated on the host before any work is queued.

Each malformed table makes the call return KATTN_EBOUNDS, and the outputs and caches keep
their sentinel values (nothing ran).  Valid tables, including the idle decode slots and the
short cu of a fixed-shape call, pass and give the oracle's results.  Before any test runs,
the module confirms that the check is on with a decode call whose used length exceeds
max_used (a sequence the decode kernel skips in any case), so no malformed table reaches a
kernel.
"""
import dataclasses
import os

import numpy as np
import pytest
import torch

import oracle
from transformer_attention_varlen_amd import kattn, workloads as wl
from transformer_attention_varlen_amd.session import ChunkRun, DecodeRun, PrefillRun

pytestmark = pytest.mark.gpu

ATOL = 2e-5
SENTINEL = -123.0


def _decode_case(used):
    case = wl.make_decode(len(used), 9, 3, 512, 1, 512, seed=61)
    return dataclasses.replace(case, used=np.asarray(used, np.int32))


@pytest.fixture(scope="module", autouse=True)
def _checks_on():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kattn.lib()
    before = os.environ.get("KATTN_CHECK")
    os.environ["KATTN_CHECK"] = "1"
    probe = DecodeRun(_decode_case([600]))
    probe.max_used = 512
    with pytest.raises(kattn.KattnError) as e:
        probe.step()
    assert e.value.code == kattn.KATTN_EBOUNDS, "KATTN_CHECK=1 is not in effect"
    del probe
    yield
    if before is None:
        del os.environ["KATTN_CHECK"]
    else:
        os.environ["KATTN_CHECK"] = before


def _ebounds(fn):
    with pytest.raises(kattn.KattnError) as e:
        fn()
    assert e.value.code == kattn.KATTN_EBOUNDS, str(e.value)
    return str(e.value)


def test_decode_used_beyond_max_used_is_rejected_and_nothing_runs():
    run = DecodeRun(_decode_case([100, 600, 7]))
    run.max_used = 512
    run.out.fill_(SENTINEL)
    k0 = run.k_cache.clone()
    msg = _ebounds(run.step)
    assert "used[1]=600" in msg
    torch.cuda.synchronize()
    assert bool(torch.all(run.out == SENTINEL))
    assert torch.equal(run.k_cache, k0)


def test_decode_idle_slots_pass_the_check_and_are_skipped():
    case = _decode_case([100, 0, 7, 0])
    run = DecodeRun(case)
    run.out.fill_(SENTINEL)
    run.step()
    torch.cuda.synchronize()
    got = run.out.cpu().numpy()
    live = case.used > 0
    ref, _, _ = oracle.decode(case.q_new[live], case.k_new[live], case.v_new[live],
                              case.k_cache[live], case.v_cache[live], case.used[live], 9, 3,
                              tables=oracle.rope_tables(case.theta, case.cap), threads=16)
    assert float(np.max(np.abs(got[live] - ref))) <= ATOL
    assert np.all(got[~live] == SENTINEL)


@pytest.mark.parametrize("bad,what", [([0, 40, 30, 90], "cu decreases"),
                                      ([5, 40, 70, 90], "cu[0]=5"),
                                      ([0, 40, 70, 200], "cu[S]=200"),
                                      ([0, 1, 70, 90], "longer than max_seqlen")])
def test_prefill_malformed_cu_is_rejected_and_nothing_runs(bad, what):
    case = wl.make_prefill([40, 30, 20], 9, 3, packed=False, causal=True, seed=62)
    run = PrefillRun(case)
    run.out.fill_(SENTINEL)
    # "longer than max_seqlen": a 69-row sequence against the valid batch's max_seqlen of 40
    run.cu.copy_(torch.tensor(bad, dtype=torch.int32))
    for call in (run.attention, run.attention_rope):
        assert what in _ebounds(call)
    torch.cuda.synchronize()
    assert bool(torch.all(run.out == SENTINEL))


def test_prefill_short_cu_of_a_fixed_shape_call_passes():
    case = wl.make_prefill([40, 30, 20], 9, 3, packed=False, causal=True, seed=63)
    run = PrefillRun(case)
    run.out.fill_(SENTINEL)
    # the bucket holds 3 sequences and 90 rows; this call fills the first two only
    run.cu.copy_(torch.tensor([0, 40, 70, 70], dtype=torch.int32))
    run.attention_rope()
    torch.cuda.synchronize()
    part = dataclasses.replace(wl.make_prefill([40, 30], 9, 3, packed=False, causal=True),
                               q=case.q[:70], k=case.k[:70], v=case.v[:70])
    ref = oracle.varlen_attention(part.q, part.k, part.v, part.cu, 9, 3, -1, True,
                                  tables=oracle.rope_tables(part.theta, 40), threads=16)
    got = run.out.cpu().numpy()
    assert float(np.max(np.abs(got[:70] - ref))) <= ATOL
    assert np.all(got[70:] == SENTINEL)


def test_rope_position_outside_the_table_is_rejected_and_nothing_runs():
    case = wl.make_prefill([40, 30], 4, 2, packed=False, seed=64)
    run = PrefillRun(case)
    q0 = run.q.clone()
    bad = run.pos.clone()
    bad[17] = run.table_len
    run.pos.copy_(bad)
    assert f"pos[17]={run.table_len}" in _ebounds(run.rope)
    torch.cuda.synchronize()
    assert torch.equal(run.q, q0)


def test_chunked_prefill_offset_past_max_ctx_is_rejected_and_nothing_runs():
    case = wl.make_chunked([20, 10], [5, 40], 9, 3, 128, seed=65)
    run = ChunkRun(case)
    run.out.fill_(SENTINEL)
    k0 = run.k_cache.clone()
    # max_ctx as the call is sized (50) against an offset table that moved on: 45 + 10 rows
    run.offsets.copy_(torch.tensor([5, 45], dtype=torch.int32))
    assert "offset[1]=45" in _ebounds(run.step)
    torch.cuda.synchronize()
    assert bool(torch.all(run.out == SENTINEL))
    assert torch.equal(run.k_cache, k0)
