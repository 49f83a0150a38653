"""GPU parity of sparse prefill (mla_sparse_prefill) against the numpy fp64
prefill oracle, at the decode path's tolerance."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_head_amd as mla
import synth
from oracle.sparse_prefill import sparse_prefill
from tests.harness import assert_close

pytestmark = pytest.mark.gpu


def gpu_prefill(w: synth.PrefillWorkload, natural=False, num_parts=None):
    dev = torch.device("cuda")
    q = torch.from_numpy(w.q.view(np.int16)).to(dev).view(torch.bfloat16)
    kv = torch.from_numpy(w.kv).to(dev)
    if w.kv_format == 0:
        kv = kv.view(torch.bfloat16)
    idx = torch.from_numpy(w.indices).to(dev)
    out = torch.full((w.s_q, w.h_q, 512), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((w.s_q, w.h_q), float("nan"), dtype=torch.float32, device=dev)
    mla.mla_sparse_prefill(q, kv, idx, w.softmax_scale, kv_format=w.kv_format,
                           natural_base=natural, num_parts=num_parts, out=out, lse=lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("s_q, h_q, s_kv, topk, fmt, invalid", [
    (1, 128, 64, 64, 0, 0.0),       # every position of one page
    (37, 128, 1000, 256, 0, 0.05),  # ragged last page, some -1 entries
    (9, 64, 70, 70, 1, 0.0),        # FP8 rows, all positions, s_kv not a page multiple
    (20, 128, 3000, 300, 1, 0.1),   # FP8, topk not a tile multiple
    (6, 16, 200, 5, 0, 0.0),        # tiny topk: one partial tile
])
def test_prefill_matches_oracle(s_q, h_q, s_kv, topk, fmt, invalid):
    w = synth.make_sparse_prefill(f"prefill_{s_q}_{s_kv}", s_q=s_q, h_q=h_q, s_kv=s_kv, topk=topk,
                                  seed=s_q * 31 + s_kv, kv_format=fmt, invalid_frac=invalid)
    out, lse = gpu_prefill(w)
    ref_out, ref_lse = sparse_prefill(w.q, w.kv, w.indices, w.softmax_scale, fmt)
    assert_close(out, lse, ref_out, ref_lse, what=f"prefill {s_q}x{h_q} s_kv {s_kv} topk {topk}")


def test_prefill_natural_base_and_edge_rows():
    """Natural base; a query whose indices are all invalid (lse -inf, out 0);
    duplicates and out-of-range entries."""
    w = synth.make_sparse_prefill("prefill_edges", s_q=8, h_q=32, s_kv=500, topk=100, seed=4)
    w.indices[2, :] = -1
    w.indices[3, :50] = w.indices[3, 50:]
    w.indices[4, ::3] = 500 + np.arange(34, dtype=np.int32)
    for natural in (False, True):
        out, lse = gpu_prefill(w, natural=natural)
        ref_out, ref_lse = sparse_prefill(w.q, w.kv, w.indices, w.softmax_scale, 0, natural)
        assert_close(out, lse, ref_out, ref_lse, what=f"prefill edges natural={natural}")
        assert np.all(out[2] == 0) and np.isneginf(lse[2]).all()


@pytest.mark.parametrize("num_parts", [1, 7, 300])
def test_prefill_crosses_chunks_and_split_counts(num_parts):
    """More query tokens than one chunk (2048), with few and many parts."""
    w = synth.make_sparse_prefill("prefill_chunks", s_q=2100, h_q=16, s_kv=4096, topk=128, seed=12)
    out, lse = gpu_prefill(w, num_parts=num_parts)
    ref_out, ref_lse = sparse_prefill(w.q, w.kv, w.indices, w.softmax_scale, 0)
    assert_close(out, lse, ref_out, ref_lse, what=f"prefill chunks parts={num_parts}")


def test_prefill_empty_is_a_no_op():
    w = synth.make_sparse_prefill("prefill_empty", s_q=1, h_q=16, s_kv=64, topk=8, seed=1)
    dev = torch.device("cuda")
    q = torch.empty((0, 16, 576), dtype=torch.bfloat16, device=dev)
    kv = torch.from_numpy(w.kv).to(dev)
    idx = torch.empty((0, 8), dtype=torch.int32, device=dev)
    out, lse = mla.mla_sparse_prefill(q, kv, idx, 0.1, kv_format=0)
    torch.cuda.synchronize()
    assert out.shape == (0, 16, 512) and lse.shape == (0, 16)


def test_prefill_full_size_sampled():
    """The benchmark's shape (s_q 4096, h_q 128, s_kv 32768, topk 2048, bf16)
    in the benchmark's launch configuration; a seeded sample of query
    tokens is checked against the oracle."""
    w = synth.make_sparse_prefill("prefill_s4096_kv32768_topk2048", s_q=4096, h_q=128, s_kv=32768,
                                  topk=2048, seed=77)
    out, lse = gpu_prefill(w)
    pick = np.sort(np.random.default_rng(0).choice(w.s_q, size=12, replace=False))
    ref_out, ref_lse = sparse_prefill(w.q[pick], w.kv, w.indices[pick], w.softmax_scale, 0)
    assert_close(out[pick], lse[pick], ref_out, ref_lse, what="prefill full size sample")
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def prefill_case(seed: int):
    rng = np.random.default_rng(40_000 + seed)
    s_q = int(rng.integers(1, 90))
    h_q = int(rng.choice([1, 16, 33, 64, 128]))
    s_kv = int(rng.integers(1, 3000))
    topk = int(rng.integers(1, min(s_kv, 400) + 1))
    return dict(s_q=s_q, h_q=h_q, s_kv=s_kv, topk=topk, fmt=int(rng.integers(0, 2)),
                invalid=float(rng.choice([0.0, 0.0, 0.1, 0.5])), natural=bool(rng.random() < 0.3),
                parts=[None, None, 1, 5, 200][int(rng.integers(0, 5))])


@pytest.mark.parametrize("seed", range(30))
def test_prefill_random_shapes(seed):
    """Seeded random shapes: query tokens, heads, cache size, top-k, format,
    invalid entries, base and forced split counts."""
    c = prefill_case(seed)
    print(f"prefill sweep {seed}: {c}", flush=True)
    w = synth.make_sparse_prefill(f"prefill_sweep_{seed}", s_q=c["s_q"], h_q=c["h_q"], s_kv=c["s_kv"],
                                  topk=c["topk"], seed=50_000 + seed, kv_format=c["fmt"],
                                  invalid_frac=c["invalid"])
    out, lse = gpu_prefill(w, natural=c["natural"], num_parts=c["parts"])
    ref_out, ref_lse = sparse_prefill(w.q, w.kv, w.indices, w.softmax_scale, c["fmt"], c["natural"])
    assert_close(out, lse, ref_out, ref_lse, what=f"prefill sweep {seed} {c}")
