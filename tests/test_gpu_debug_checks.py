"""MLA_DEBUG_CHECKS: with it set, a decode call first runs the device-side
input check on its stream and refuses out-of-range lengths and block-table
entries, naming the first bad sequence, before any decode kernel runs.

The bad inputs here stay inside the memory the call is given a view of or
its underlying allocation (the refused page exists physically; the refused
length reaches the next table row), so nothing could read out of bounds
even if the refusal failed."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_head_amd as mla
import synth
from tests.harness import assert_close, run, to_device

pytestmark = pytest.mark.gpu


def workload(h_q):
    return synth.make_workload("dbg", batch=4, h_q=h_q, s_q=1, seqlens=[300, 64, 129, 1000], seed=71,
                               max_pages_per_seq=16)


def decode(w, p, q, kv, bt, sl):
    plan = mla.DecodePlan(p, q.device)
    out = torch.empty((w.batch, w.s_q, w.h_q, 512), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((w.batch, w.s_q, w.h_q), dtype=torch.float32, device=q.device)
    plan.metadata(sl)
    plan.decode(q, kv, bt, sl, None, out, lse)
    torch.cuda.synchronize()


@pytest.mark.parametrize("h_q", [16, 128])
def test_good_inputs_pass_and_match_the_oracle(monkeypatch, h_q):
    monkeypatch.setenv("MLA_DEBUG_CHECKS", "1")
    w = workload(h_q)
    out, lse = run(w)
    ref_out, ref_lse = oracle.mla_decode(w)
    assert_close(out, lse, ref_out, ref_lse, what=f"MLA_DEBUG_CHECKS=1, h_q {h_q}")


@pytest.mark.parametrize("h_q", [16, 128])
def test_out_of_range_page_is_refused(monkeypatch, h_q):
    monkeypatch.setenv("MLA_DEBUG_CHECKS", "1")
    w = workload(h_q)
    q, kv, bt, sl, _ = to_device(w)
    # the largest physical page any visible position reaches: a pool that
    # ends just below it makes that entry out of range for exactly the
    # sequence that holds it
    reach = [(b, int(w.block_table[b, j])) for b in range(w.batch)
             for j in range(-(-int(w.cache_seqlens[b]) // 64))]
    b_bad, v = max(reach, key=lambda t: t[1])
    p = mla.problem_for(w)
    p.num_pages = v
    print(f"h_q {h_q}: pool cut to {v} pages, sequence {b_bad} reaches page {v}", flush=True)
    with pytest.raises(ValueError, match=rf"block_table.*first: sequence {b_bad} \(MLA_DEBUG_CHECKS\)"):
        decode(w, p, q, kv[:v], bt, sl)


def test_too_long_sequence_is_refused(monkeypatch):
    monkeypatch.setenv("MLA_DEBUG_CHECKS", "1")
    w = workload(128)
    q, kv, bt, sl, _ = to_device(w)
    sl_bad = sl.clone()
    sl_bad[0] = 16 * 64 + 1  # one page past row 0 of the table: that is row 1's first entry
    p = mla.problem_for(w)
    with pytest.raises(ValueError, match=r"cache_seqlens.*first: sequence 0 \(MLA_DEBUG_CHECKS\)"):
        decode(w, p, q, kv, bt, sl_bad)
    # the same call without the variable set is not exercised: it would hand
    # the kernels a length the preconditions exclude
    monkeypatch.delenv("MLA_DEBUG_CHECKS")
    out, lse = run(w, tensors=(q, kv, bt, sl, None))
    ref_out, ref_lse = oracle.mla_decode(w)
    assert_close(out, lse, ref_out, ref_lse, what="after the refusal, variable unset")
