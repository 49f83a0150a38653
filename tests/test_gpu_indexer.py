"""GPU parity of the FP8 top-k indexer (mla_fp8_index_top_k) against the fp64
oracle, and the indexer -> sparse decode chain against the decode oracle.

The selected set is not unique when scores tie or nearly tie, so each token's
result is checked for validity rather than equality: indices distinct, in
ascending order and visible; as many as min(topk, visible rows), then -1
(scores -inf); every returned score within the error bound of the oracle's
value; and no unselected row whose oracle score exceeds a selected row's by
more than the two bounds together.

Error bound.  The kernels sum the heads first, Qsum[d] = sum_h qs[h][t(d)] *
e4m3(q[h][d]) (one fp32 fma per head), then per row two fp32 dot products of
16 dims per lane, the tile scales and a 16-lane sum; every e4m3 value is
exact in fp32.  Each of those at most h + 24 roundings is off by at most
2^-24 of a partial sum bounded by the same sums over absolute values, so
|S_gpu - S| <= (h + 32) * 2^-24 * A, A = oracle.indexer.abs_scores."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_head_amd as mla
import synth
from oracle import indexer as ix
from tests.harness import assert_close

pytestmark = pytest.mark.gpu

def rel_bound(h):
    return (h + 32) * 2.0 ** -24


def run_index(w, with_scores=True, tensors=None):
    p = mla.index_problem_for(w)
    qc, qs, kv, bt, sl = tensors if tensors is not None else mla.index_tensors(w)
    ws = torch.empty(mla.mla_fp8_index_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    idx = torch.full((w.batch, w.s_q, w.topk), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((w.batch, w.s_q, w.topk), float("nan"), dtype=torch.float32, device="cuda") if with_scores else None
    mla.mla_fp8_index_top_k(p, qc, qs, kv, bt, sl, ws, idx, sc)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), (sc.cpu().numpy() if with_scores else None)


def check_token(w, b, i, idx, sc, what=""):
    """Validity of one token's selection; returns (agreement with the
    oracle's own selection, max |S_gpu - S| / A)."""
    S = ix.scores(w, b, i)
    A = ix.abs_scores(w, b, i)
    n, k = S.shape[0], w.topk
    m = min(k, n)
    got = idx[b, i]
    assert np.all(got[m:] == -1), f"{what}: fill"
    assert np.all(np.isneginf(sc[b, i, m:])), f"{what}: fill scores"
    sel = got[:m]
    assert np.all((sel >= 0) & (sel < n)), f"{what}: index out of the visible range"
    assert np.all(np.diff(sel) > 0), f"{what}: not strictly ascending"
    if m == 0:
        return 1.0, 0.0
    tol = rel_bound(w.h) * A
    err = np.abs(sc[b, i, :m].astype(np.float64) - S[sel])
    assert np.all(err <= tol[sel]), f"{what}: score off by {np.max(err / tol[sel]):.3g} x the bound"
    if m < n:
        mask = np.ones(n, dtype=bool)
        mask[sel] = False
        lo = np.min(S[sel] + tol[sel])
        hi = np.max(S[mask] - tol[mask])
        assert lo >= hi, f"{what}: an unselected row outscores a selected one beyond the bound"
    ref = ix.select(S, k)
    agree = np.intersect1d(ref, sel).shape[0] / m
    return agree, float(np.max(err / np.maximum(A[sel], 1e-300)))


CASES = [
    # h, s_q, causal, kpool, seqlens, topk
    (16, 1, 0, 1, [1, 63, 64, 65, 300], 32),
    (128, 2, 0, 1, [70, 2000, 130], 64),
    (128, 2, 1, 1, [2, 129, 1000], 100),
    (64, 3, 1, 4, [5, 700, 257], 20),
    (8, 4, 0, 1, [90, 3000], 16),
    (40, 2, 0, 2, [1000, 77, 5], 50),
    (256, 2, 1, 1, [600, 64], 128),
    (1, 1, 0, 1, [500, 2], 8),
    (32, 1, 0, 1, [10, 0, 64], 16),
    (128, 1, 0, 1, [5000], 4096),
    (64, 1, 0, 1, [20000, 9000], 10000),  # k above 8192: rows stored lane by lane (also all of a shorter row set)
    (4096, 1, 0, 1, [700, 64], 100),   # the most index heads the call takes
    (1000, 2, 1, 3, [2000, 333], 77),  # many heads, not a multiple of 16
]


@pytest.mark.parametrize("h,s_q,causal,kpool,lens,topk", CASES)
def test_index_shapes(h, s_q, causal, kpool, lens, topk):
    w = synth.make_index_workload("idx", batch=len(lens), s_q=s_q, h=h, seqlens=lens, seed=200 + h + s_q,
                                  topk=topk, kpool=kpool, is_causal=causal)
    print(f"h {h} s_q {s_q} causal {causal} kpool {kpool} lens {lens} topk {topk}", flush=True)
    idx, sc = run_index(w)
    agree = []
    for b in range(w.batch):
        for i in range(s_q):
            a, _ = check_token(w, b, i, idx, sc, what=f"b={b} i={i}")
            agree.append(a)
    print(f"   agreement with the oracle's selection: min {min(agree):.4f}", flush=True)


def test_index_full_length_sample():
    """Sequences of 65536 tokens (the sparse decode benchmark's cache), topk
    2048, 128 heads, two query tokens: sampled tokens against the oracle."""
    w = synth.make_index_workload("idx_full", batch=8, s_q=2, h=128, seqlens=[65536] * 8, seed=301,
                                  topk=2048)
    idx, sc = run_index(w)
    rng = np.random.default_rng(0)
    for b, i in [(0, 0), (3, 1), (7, 0), (int(rng.integers(8)), 1)]:
        a, e = check_token(w, b, i, idx, sc, what=f"b={b} i={i}")
        print(f"token ({b}, {i}): agreement {a:.4f}, max |S_gpu - S| / A {e:.3g}", flush=True)
        assert a >= 0.99


def test_index_bit_identity_and_page_permutation():
    w = synth.make_index_workload("idx_bits", batch=3, s_q=2, h=64, seqlens=[3000, 64, 1500], seed=302,
                                  topk=200)
    i1, s1 = run_index(w)
    i2, s2 = run_index(w)
    assert np.array_equal(i1, i2) and np.array_equal(s1.view(np.int32), s2.view(np.int32))
    perm = np.random.default_rng(8).permutation(w.num_pages)
    kv2 = np.empty_like(w.kv)
    kv2[perm] = w.kv
    w.kv = kv2
    w.block_table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    i3, s3 = run_index(w)
    assert np.array_equal(i1, i3) and np.array_equal(s1.view(np.int32), s3.view(np.int32))


def test_index_without_scores_output():
    w = synth.make_index_workload("idx_ns", batch=2, s_q=1, h=32, seqlens=[700, 100], seed=303, topk=64)
    i1, _ = run_index(w)
    i2, _ = run_index(w, with_scores=False)
    assert np.array_equal(i1, i2)


@pytest.mark.parametrize("topk", [256, 2048])
def test_indexer_then_sparse_decode(topk):
    """The indexer's output drives mla_decode_sparse_fp8 directly: the decode
    over the selected rows matches the decode oracle on the same indices, and
    the selection is valid."""
    lens = [3000, 5000, 200, 64]
    w = synth.make_index_workload("idx_e2e", batch=4, s_q=2, h=128, seqlens=lens, seed=304, topk=topk)
    idx, sc = run_index(w)
    for b in range(w.batch):
        for i in range(w.s_q):
            check_token(w, b, i, idx, sc, what=f"b={b} i={i}")
    d = synth.Workload(name="e2e", batch=w.batch, s_q=w.s_q, h_q=w.h, page_size=64,
                       kv_format=synth.KV_FP8_656, topk=topk, is_causal=0,
                       softmax_scale=float(np.float32(1.0 / np.sqrt(576.0))), q=w.q_bf16, kv=w.kv,
                       block_table=w.block_table, cache_seqlens=w.cache_seqlens, indices=idx)
    p = mla.problem_for(d)
    q, kv, bt, sl, ind = mla.workload_tensors(d)
    plan = mla.DecodePlan(p, q.device)
    out = torch.empty((d.batch, d.s_q, d.h_q, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((d.batch, d.s_q, d.h_q), dtype=torch.float32, device="cuda")
    plan.metadata(sl)
    plan.decode(q, kv, bt, sl, ind, out, lse)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.mla_decode(d)
    assert_close(out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, what=f"topk={topk}")


def test_two_phases_equal_the_one_call():
    """mla_fp8_index_scores + mla_fp8_index_select give the one call's bits;
    the workspace holds every visible row's score within the bound."""
    w = synth.make_index_workload("idx_ph", batch=3, s_q=2, h=128, seqlens=[2500, 700, 64], seed=305,
                                  topk=100, is_causal=1)
    i1, s1 = run_index(w)
    p = mla.index_problem_for(w)
    qc, qs, kv, bt, sl = mla.index_tensors(w)
    ws = torch.empty(mla.mla_fp8_index_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    idx = torch.empty((w.batch, w.s_q, w.topk), dtype=torch.int32, device="cuda")
    sc = torch.empty((w.batch, w.s_q, w.topk), dtype=torch.float32, device="cuda")
    mla.mla_fp8_index_scores(p, qc, qs, kv, bt, sl, ws)
    mla.mla_fp8_index_select(p, sl, ws, idx, sc)
    torch.cuda.synchronize()
    assert np.array_equal(i1, idx.cpu().numpy())
    assert np.array_equal(s1.view(np.int32), sc.cpu().numpy().view(np.int32))
    S_all = ws[:w.batch * w.s_q * w.max_pages_per_seq * 64 * 4].view(torch.float32).cpu().numpy()
    S_all = S_all.reshape(w.batch, w.s_q, -1)
    for b in range(w.batch):
        for i in range(w.s_q):
            S, A = ix.scores(w, b, i), ix.abs_scores(w, b, i)
            n = S.shape[0]
            assert np.all(np.abs(S_all[b, i, :n] - S) <= rel_bound(w.h) * A)


@pytest.mark.parametrize("L", [5000, 20000])
def test_index_all_scores_equal(L):
    """Every row identical, so every score ties: the k smallest rows are
    selected.  5000 rows take the selection's compacted path, 20000 rows its
    fallback for a band too wide to compact."""
    w = synth.make_index_workload("idx_ties", batch=1, s_q=1, h=8, seqlens=[L], seed=306, topk=300)
    first = w.kv[w.block_table[0, 0], 0].copy()
    for j in range(L):
        w.kv[w.block_table[0, j // 64], j % 64] = first
    idx, sc = run_index(w)
    assert idx[0, 0].tolist() == list(range(300))
    assert np.all(sc[0, 0] == sc[0, 0, 0])
    check_token(w, 0, 0, idx, sc, what=f"ties L={L}")


def test_index_benchmark_workload_sampled():
    """The benchmark's workload in its launch configuration (128 sequences of
    65536 FP8 rows, two query tokens of 128 heads, topk 2048): sampled
    tokens against the oracle."""
    import bench

    c = bench.INDEX_WORKLOAD
    w = synth.make_index_workload(c["name"], batch=c["batch"], s_q=c["s_q"], h=c["h"],
                                  seqlens=[c["seqlen"]] * c["batch"], seed=c["seed"], topk=c["topk"])
    print(f"{w.name}: {w.batch} x {c['seqlen']} rows", flush=True)
    idx, sc = run_index(w)
    rng = np.random.default_rng(1)
    for u in rng.choice(w.batch * w.s_q, size=4, replace=False):
        b, i = int(u) // w.s_q, int(u) % w.s_q
        a, e = check_token(w, b, i, idx, sc, what=f"b={b} i={i}")
        print(f"token ({b}, {i}): agreement {a:.4f}, max |S_gpu - S| / A {e:.3g}", flush=True)
    # every token: a full, ascending, in-range list (no -1: 65536 rows > 2048)
    assert np.all(idx >= 0) and np.all(idx < c["seqlen"])
    assert np.all(np.diff(idx, axis=-1) > 0)


@pytest.mark.parametrize("seed", range(20))
def test_index_random_shapes(seed):
    """Seeded random shapes: heads 1-160, query tokens 1-6, lengths 0-3000
    (some 0), pooling 1-3, causal or not, topk 1-400."""
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 5))
    h = int(rng.integers(1, 161))
    s_q = int(rng.integers(1, 7))
    kpool = int(rng.integers(1, 4))
    causal = int(rng.integers(0, 2))
    lens = [int(x) if rng.random() > 0.15 else 0 for x in rng.integers(1, 3001, size=B)]
    topk = int(rng.integers(1, 401))
    print(f"seed {seed}: B {B} h {h} s_q {s_q} kpool {kpool} causal {causal} lens {lens} topk {topk}", flush=True)
    w = synth.make_index_workload("idx_rand", batch=B, s_q=s_q, h=h, seqlens=lens, seed=2000 + seed,
                                  topk=topk, kpool=kpool, is_causal=causal)
    w.topk = min(topk, 64 * w.max_pages_per_seq)  # the call's limit: rows the table can hold
    idx, sc = run_index(w)
    for b in range(B):
        for i in range(s_q):
            check_token(w, b, i, idx, sc, what=f"seed {seed} b={b} i={i}")


@pytest.mark.parametrize("k,want_nan", [(290, []), (299, [5, 17]), (300, [5, 17, 200])])
def test_index_nan_scores_rank_last(k, want_nan):
    """Rows whose tile scale is NaN score NaN and rank below every other row:
    they are selected only when k exceeds the rows with a number, the
    smallest first."""
    w = synth.make_index_workload("idx_nan", batch=1, s_q=1, h=32, seqlens=[300], seed=307, topk=k)
    for j in (5, 17, 200):
        w.kv[w.block_table[0, j // 64], j % 64, 512:516] = 0xFF  # scale of tile 0: NaN
    idx, sc = run_index(w)
    S = ix.scores(w, 0, 0)
    assert np.isnan(S[[5, 17, 200]]).all() and np.isfinite(np.delete(S, [5, 17, 200])).all()
    got = idx[0, 0]
    nan_rows = [j for j in got.tolist() if j in (5, 17, 200)]
    assert nan_rows == want_nan
    numbered = np.array([j for j in got.tolist() if j >= 0 and j not in (5, 17, 200)])
    assert len(numbered) == min(k, 297)
    if len(numbered) < 297:  # the numbered part is a valid top-k of the rows with a number
        A = ix.abs_scores(w, 0, 0)
        tol = rel_bound(w.h) * A
        rest = np.setdiff1d(np.setdiff1d(np.arange(300), numbered), [5, 17, 200])
        assert np.min(S[numbered] + tol[numbered]) >= np.max(S[rest] - tol[rest])
    assert np.isnan(sc[0, 0][np.isin(got, [5, 17, 200])]).all()
