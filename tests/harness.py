"""Shared helpers for the GPU tests: move a synthetic workload to the device,
run the library through its C ABI, and compare with the oracle."""

from __future__ import annotations

import numpy as np
import torch

import paged_kv_head_amd as mla
import synth

# Tolerance stated for this path: bf16 outputs within 1e-2 * max|ref| + 2e-3,
# lse within 1e-3 (log2 units); -inf lse entries must match exactly.
OUT_REL = 1e-2
OUT_ABS = 2e-3
LSE_ABS = 1e-3


def to_device(w: synth.Workload, device="cuda"):
    return mla.workload_tensors(w, device)


def problem(w: synth.Workload, natural=False, softmax_scale=None) -> mla.Problem:
    return mla.problem_for(w, natural=natural, softmax_scale=softmax_scale)


def run(w: synth.Workload, *, num_parts=None, natural=False, tensors=None, softmax_scale=None,
        return_meta=False):
    """Metadata + decode + combine through the C ABI; returns numpy
    (out float32 [B, s_q, h_q, 512], lse float32 [B, s_q, h_q])."""
    p = problem(w, natural, softmax_scale)
    q, kv, bt, sl, idx = tensors if tensors is not None else to_device(w)
    plan = mla.DecodePlan(p, q.device, num_parts)
    out = torch.full((w.batch, w.s_q, w.h_q, 512), float("nan"), dtype=torch.bfloat16, device=q.device)
    lse = torch.full((w.batch, w.s_q, w.h_q), float("nan"), dtype=torch.float32, device=q.device)
    plan.metadata(sl)
    plan.decode(q, kv, bt, sl, idx, out, lse)
    torch.cuda.synchronize()
    res = (out.float().cpu().numpy(), lse.cpu().numpy())
    if return_meta:
        return res + (plan.sched.cpu().numpy(), plan.num_splits.cpu().numpy(), plan.num_parts)
    return res


def assert_close(out, lse, ref_out, ref_lse, mask=None, what=""):
    """Element-wise comparison at the stated tolerance (optionally on a
    subset of (b, i) units given by a boolean mask [B, s_q])."""
    if mask is not None:
        out, lse, ref_out, ref_lse = out[mask], lse[mask], ref_out[mask], ref_lse[mask]
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    ninf = ref_lse == -np.inf
    assert np.array_equal(lse == -np.inf, ninf), f"{what}: -inf lse pattern differs"
    assert np.all(np.isfinite(lse[~ninf])), f"{what}: non-finite lse"
    err = np.abs(out.astype(np.float64) - ref_out).max() if out.size else 0.0
    bound = OUT_REL * (np.abs(ref_out).max() if ref_out.size else 0.0) + OUT_ABS
    assert err <= bound, f"{what}: max |out - ref| = {err:.3g} > {bound:.3g}"
    if (~ninf).any():
        lerr = np.abs(lse[~ninf].astype(np.float64) - ref_lse[~ninf]).max()
        assert lerr <= LSE_ABS, f"{what}: max |lse - ref| = {lerr:.3g} > {LSE_ABS}"
    return err, bound
