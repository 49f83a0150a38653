"""The allocation-free entry point mla_decode_paged_noalloc against the
workspace entry points (mla_decode_paged, then mla_decode_combine) on the same
inputs and metadata.  Both run the same kernels on the same schedule, so the
results must agree bit for bit.  The calls come in a row, each on a smaller
problem than the one before, so the static scratch still holds the previous
call's partials when the next one runs; the last call repeats the first
shape (new seed) after the smaller ones."""

import numpy as np
import pytest
import torch

import paged_kv_head_amd as mla
import synth
from tests.harness import problem, to_device

pytestmark = pytest.mark.gpu

# (name, batch, h_q, s_q, seqlens, kv_format, topk, causal, num_parts)
CALLS = [
    ("dense bf16, 72 MiB of partials", 32, 128, 2, synth.Uniform(1000, 8000), synth.KV_BF16, 0, 1, 256),
    ("dense FP8, smaller", 5, 128, 1, [0, 1, 100, 3000, 700], synth.KV_FP8_656, 0, 0, 37),
    ("sparse FP8", 3, 128, 2, [900, 2100, 400], synth.KV_FP8_656, 300, 0, 19),
    ("small heads bf16", 4, 16, 1, [5, 64, 1000, 2500], synth.KV_BF16, 0, 0, 11),
]


def run_both(w, num_parts):
    p = problem(w)
    q, kv, bt, sl, idx = to_device(w)
    plan = mla.DecodePlan(p, q.device, num_parts)
    need = mla.mla_decode_workspace_bytes(p, plan.num_parts)
    assert need <= mla.NOALLOC_SCRATCH_BYTES
    plan.metadata(sl)
    res = []
    for noalloc in (False, True):
        out = torch.full((w.batch, w.s_q, w.h_q, 512), float("nan"), dtype=torch.bfloat16, device=q.device)
        lse = torch.full((w.batch, w.s_q, w.h_q), float("nan"), dtype=torch.float32, device=q.device)
        if noalloc:
            mla.mla_decode_paged_noalloc(p, q, kv, bt, sl, idx, plan.sched, plan.num_parts,
                                         plan.num_splits, out, lse)
        else:
            plan.decode(q, kv, bt, sl, idx, out, lse)
        torch.cuda.synchronize()
        res.append((out.view(torch.int16).cpu().numpy(), lse.view(torch.int32).cpu().numpy()))
    splits = int(plan.num_splits[-1].item())
    return res, need, splits


def check_call(i, call):
    name, batch, h_q, s_q, seqlens, fmt, topk, causal, parts = call
    w = synth.make_workload(f"noalloc{i}", batch=batch, h_q=h_q, s_q=s_q, seqlens=seqlens, seed=90 + i,
                            kv_format=fmt, topk=topk, is_causal=causal)
    print(f"call {i}: {name}: batch {batch} h_q {h_q} s_q {s_q} fmt {fmt} topk {topk} parts {parts}",
          flush=True)
    ((o_ws, l_ws), (o_na, l_na)), need, splits = run_both(w, parts)
    print(f"   partials {need / 2**20:.1f} MiB, {splits} segments", flush=True)
    assert np.array_equal(o_ws, o_na), f"{name}: out differs"
    assert np.array_equal(l_ws, l_na), f"{name}: lse differs"
    return splits


def test_noalloc_equals_workspace_path_on_calls_in_a_row():
    segs = [check_call(i, c) for i, c in enumerate(CALLS)]
    assert segs[0] > 32 and segs[1] > 5  # both dense calls really split and use the scratch
    check_call(len(CALLS), CALLS[0])     # the first shape again, after the smaller ones


def test_noalloc_rejects_problems_beyond_the_scratch():
    w = synth.make_workload("noalloc_big", batch=2, h_q=128, s_q=2, seqlens=[100, 200], seed=99)
    p = problem(w)
    parts = 2048  # (2048 + 2) slots x 256 rows x 1028 B: far beyond 96 MiB
    assert mla.mla_decode_workspace_bytes(p, parts) > mla.NOALLOC_SCRATCH_BYTES
    q, kv, bt, sl, idx = to_device(w)
    plan = mla.DecodePlan(p, q.device, parts)
    plan.metadata(sl)
    out = torch.empty((2, 2, 128, 512), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((2, 2, 128), dtype=torch.float32, device=q.device)
    with pytest.raises(mla.MlaError) as e:
        mla.mla_decode_paged_noalloc(p, q, kv, bt, sl, idx, plan.sched, parts, plan.num_splits, out, lse)
    assert e.value.status == mla.MLA_ERR_WORKSPACE_TOO_SMALL
    assert "static scratch" in str(e.value)
