"""Pins of the FP8 top-k indexer oracle (CPU only).

Each test fixes a value the definition determines independently of the
oracle's own code: a query with one nonzero code reads back one dequantised
cache value (decoded here by torch's float8_e4m3fn, not the oracle's codec);
two such heads add; with unit scales a score is the dot product of the
dequantised rows; hand-counted visible rows; hand-worked selections with ties,
NaN and -1 fill; invariance under page and head permutation; linearity in the
query scales."""

import numpy as np
import pytest
import torch

import synth
from oracle import indexer as ix

ONE = 0x38  # e4m3fn code of 1.0


def torch_e4m3(codes) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def row_bytes(w, b, j):
    return w.kv[w.block_table[b, j // 64], j % 64]


def row_scale(w, b, j, t):
    return float(np.frombuffer(row_bytes(w, b, j)[512 + 4 * t:516 + 4 * t].tobytes(), dtype=np.float32)[0])


def tiny(**kw):
    d = dict(batch=2, s_q=1, h=3, seqlens=[70, 5], seed=5, topk=8)
    d.update(kw)
    return synth.make_index_workload("pin", **d)


def test_one_hot_query_reads_one_dequantised_value():
    w = tiny()
    w.q_codes[:] = 0
    w.q_scales[:] = 0
    w.q_codes[:, 0, 1, 300] = ONE      # head 1, dim 300 (tile 2)
    w.q_scales[:, 0, 1, 2] = 0.5
    for b in range(2):
        S = ix.scores(w, b, 0)
        assert S.shape == (int(w.cache_seqlens[b]),)
        for j in range(S.shape[0]):
            want = 0.5 * row_scale(w, b, j, 2) * torch_e4m3([row_bytes(w, b, j)[300]])[0]
            assert S[j] == want


def test_heads_are_summed():
    w = tiny()
    w.q_codes[:] = 0
    w.q_scales[:] = 0
    w.q_codes[:, 0, 0, 5] = 0x40       # 2.0, tile 0
    w.q_scales[:, 0, 0, 0] = 3.0
    w.q_codes[:, 0, 2, 511] = 0xB8     # -1.0, tile 3
    w.q_scales[:, 0, 2, 3] = 0.25
    S = ix.scores(w, 0, 0)
    for j in range(S.shape[0]):
        r = row_bytes(w, 0, j)
        a = 3.0 * 2.0 * row_scale(w, 0, j, 0) * torch_e4m3([r[5]])[0]
        c = 0.25 * -1.0 * row_scale(w, 0, j, 3) * torch_e4m3([r[511]])[0]
        assert S[j] == pytest.approx(a + c, rel=1e-15, abs=0)


def test_unit_scales_reduce_to_a_dot_product_of_dequantised_rows():
    w = tiny(h=1, seqlens=[130, 64])
    rng = np.random.default_rng(0)
    valid = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    w.q_codes[:] = rng.choice(valid, size=w.q_codes.shape)
    w.q_scales[:] = 1.0
    ones = np.ones(4, dtype=np.float32).view(np.uint8)
    for b in range(2):
        for j in range(int(w.cache_seqlens[b])):
            r = row_bytes(w, b, j)
            r[:512] = rng.choice(valid, size=512)
            r[512:528] = ones
    for b in range(2):
        n = int(w.cache_seqlens[b])
        K = np.stack([torch_e4m3(row_bytes(w, b, j)[:512]) for j in range(n)])
        want = K @ torch_e4m3(w.q_codes[b, 0, 0])
        np.testing.assert_allclose(ix.scores(w, b, 0), want, rtol=1e-13, atol=1e-9)


def test_visible_row_counts():
    assert [ix.visible_rows(130, 3, i, 1, 1) for i in range(3)] == [128, 129, 130]
    assert [ix.visible_rows(130, 3, i, 4, 1) for i in range(3)] == [32, 33, 33]
    assert [ix.visible_rows(130, 3, i, 1, 0) for i in range(3)] == [130, 130, 130]
    assert ix.visible_rows(130, 3, 0, 4, 0) == 33
    assert ix.visible_rows(0, 1, 0, 1, 0) == 0
    assert [ix.visible_rows(1, 2, i, 1, 1) for i in range(2)] == [0, 1]
    assert ix.visible_rows(64, 1, 0, 64, 0) == 1 and ix.visible_rows(65, 1, 0, 64, 0) == 2


def selection_workload(values):
    """One sequence whose row j scores exactly values[j] (one-hot query on
    dim 0, unit scales, code of the value at dim 0 of every row)."""
    n = len(values)
    w = tiny(batch=1, h=1, seqlens=[n], topk=4)
    w.q_codes[:] = 0
    w.q_scales[:] = 0
    w.q_codes[0, 0, 0, 0] = ONE
    w.q_scales[0, 0, 0, 0] = 1.0
    codes = {1.0: 0x38, 3.0: 0x44, 2.0: 0x40, -1.0: 0xB8, 0.5: 0x30, "nan": 0x7F}
    ones = np.ones(4, dtype=np.float32).view(np.uint8)
    for j, v in enumerate(values):
        r = row_bytes(w, 0, j)
        r[0] = codes[v]
        r[512:528] = ones
    return w


def test_selection_ties_nan_and_fill():
    vals = [1.0, 3.0, 2.0, 3.0, -1.0, 0.5, 3.0, "nan", 2.0, 1.0]
    w = selection_workload(vals)
    S = ix.scores(w, 0, 0)
    assert np.isnan(S[7]) and S[1] == 3.0 and S[4] == -1.0
    for k, want in [(4, [1, 2, 3, 6]),                        # three 3.0s, then the first 2.0
                    (1, [1]),
                    (6, [0, 1, 2, 3, 6, 8]),                  # 3,3,3,2,2 then the first 1.0
                    (9, [0, 1, 2, 3, 4, 5, 6, 8, 9]),         # everything but the NaN row
                    (12, list(range(10)) + [-1, -1])]:        # fewer rows than k
        w.topk = k
        idx, sc = ix.top_k(w)
        assert idx[0, 0].tolist() == want
        got = sc[0, 0]
        assert np.all(np.isneginf(got[idx[0, 0] < 0]))


def test_masking_by_length_and_causality():
    w = tiny(batch=2, s_q=3, h=2, seqlens=[2, 100], topk=3, is_causal=1)
    idx, _ = ix.top_k(w)
    assert idx[0, 0].tolist() == [-1, -1, -1]      # t_max = -1
    assert sorted(idx[0, 1].tolist()) == [-1, -1, 0]
    assert sorted(idx[0, 2].tolist()) == [-1, 0, 1]
    assert idx[1].max() <= 99 and (idx[1] >= 0).all()
    assert idx[1, 0].max() <= 97                    # token 0 of 3 sees rows 0..97


def test_page_permutation_invariance():
    w = tiny(seqlens=[200, 130], topk=16)
    idx1, sc1 = ix.top_k(w)
    perm = np.random.default_rng(3).permutation(w.num_pages)
    kv2 = np.empty_like(w.kv)
    kv2[perm] = w.kv
    w.kv = kv2
    w.block_table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    idx2, sc2 = ix.top_k(w)
    assert np.array_equal(idx1, idx2) and np.array_equal(sc1, sc2)


def test_head_permutation_and_query_scale_linearity():
    w = tiny(h=8, seqlens=[150, 90], topk=10)
    idx1, sc1 = ix.top_k(w)
    p = np.random.default_rng(4).permutation(8)
    w.q_codes = np.ascontiguousarray(w.q_codes[:, :, p])
    w.q_scales = np.ascontiguousarray(w.q_scales[:, :, p])
    idx2, sc2 = ix.top_k(w)
    assert np.array_equal(idx1, idx2)
    np.testing.assert_allclose(sc2, sc1, rtol=1e-12)
    w.q_scales = w.q_scales * np.float32(2.0)
    idx3, sc3 = ix.top_k(w)
    assert np.array_equal(idx1, idx3)
    fin = np.isfinite(sc2)
    assert np.array_equal(sc3[fin], 2.0 * sc2[fin])


def test_absolute_sums_bound_the_scores():
    w = tiny(h=4, seqlens=[300, 64])
    for b in range(2):
        S, A = ix.scores(w, b, 0), ix.abs_scores(w, b, 0)
        assert np.all(np.abs(S) <= A * (1 + 1e-12))
        assert np.all(A > 0)
