"""Pins of the sparse prefill oracle (oracle/sparse_prefill.py) against
results fixed independently of it: the C oracle's sparse decode over an
identity block table, torch's float64 attention when every position is
listed, and closed forms."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.sparse_prefill import latent_rows, sparse_prefill


def as_decode_workload(w: synth.PrefillWorkload, pages_pad_rows=64):
    """The same problem as a batch-1 paged decode: pages of 64 consecutive
    rows of the flat cache, identity block table, cache length s_kv.
    Rows past s_kv in the last page are NaN poison."""
    pages = -(-w.s_kv // 64)
    row = w.kv.shape[1]
    pool = np.full((pages * 64, row), 0xFF, dtype=np.uint8)
    pool[:w.s_kv] = w.kv
    return synth.Workload(name=w.name, batch=1, s_q=w.s_q, h_q=w.h_q, page_size=64,
                          kv_format=w.kv_format, topk=w.topk, is_causal=0,
                          softmax_scale=w.softmax_scale, q=w.q[None],
                          kv=pool.reshape(pages, 64, row),
                          block_table=np.arange(pages, dtype=np.int32)[None],
                          cache_seqlens=np.array([w.s_kv], dtype=np.int32),
                          indices=w.indices[None])


@pytest.mark.parametrize("kv_format", [0, 1])
@pytest.mark.parametrize("natural", [False, True])
def test_prefill_matches_c_oracle_sparse_decode(kv_format, natural):
    w = synth.make_sparse_prefill("pin", s_q=6, h_q=16, s_kv=300, topk=40, seed=5,
                                  kv_format=kv_format, invalid_frac=0.1)
    w.indices[0, :5] = [299, 299, 300, 10 ** 6, -7]  # duplicate, out of range, negative
    w.indices[1, :] = -1                             # nothing visible
    out, lse = sparse_prefill(w.q, w.kv, w.indices, w.softmax_scale, kv_format, natural)
    ref_out, ref_lse = oracle.mla_decode(as_decode_workload(w), natural=natural)
    assert np.isneginf(lse[1]).all() and np.all(out[1] == 0)
    fin = np.isfinite(ref_lse[0])
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref_lse[0]))
    np.testing.assert_allclose(lse[np.isfinite(lse)], ref_lse[0][fin], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out, ref_out[0], rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("natural", [False, True])
def test_prefill_all_positions_matches_sdpa(natural):
    """Every query lists every position (in shuffled order): the result is
    ordinary attention over the whole cache; base 2 is natural attention
    with the scale times ln 2 and lse divided by ln 2."""
    w = synth.make_sparse_prefill("sdpa", s_q=4, h_q=8, s_kv=50, topk=50, seed=7)
    out, lse = sparse_prefill(w.q, w.kv, w.indices, w.softmax_scale, 0, natural)
    Q = torch.from_numpy(synth.bf16_bits_to_f32(w.q).astype(np.float64))      # [s_q, h, 576]
    K = torch.from_numpy(latent_rows(w.kv, 0))                                # [s_kv, 576]
    s = float(np.float32(w.softmax_scale)) * (1.0 if natural else math.log(2.0))
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q[:, :, None], K[None, None].expand(w.s_q, w.h_q, -1, -1),
        K[None, None, :, :512].expand(w.s_q, w.h_q, -1, -1), scale=s)[:, :, 0]
    ref_lse = torch.logsumexp((Q @ K.T) * s, dim=-1)
    if not natural:
        ref_lse = ref_lse / math.log(2.0)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=1e-12, atol=1e-12)


def test_prefill_single_index_returns_the_row():
    """topk = 1: the only weight is 2^0 = 1, so out is the gathered row's
    first 512 values exactly."""
    w = synth.make_sparse_prefill("one", s_q=5, h_q=4, s_kv=90, topk=1, seed=3)
    out, lse = sparse_prefill(w.q, w.kv, w.indices, w.softmax_scale)
    K = latent_rows(w.kv, 0)
    for i in range(w.s_q):
        assert np.array_equal(out[i], np.broadcast_to(K[w.indices[i, 0], :512], out[i].shape))
        assert np.all(np.isfinite(lse[i]))


def test_prefill_duplicate_index_adds_log2_of_two():
    """Listing every index twice doubles every weight's numerator and the
    sum: out is unchanged and lse grows by exactly log2(2) = 1."""
    w = synth.make_sparse_prefill("dup", s_q=3, h_q=4, s_kv=70, topk=20, seed=8)
    out1, lse1 = sparse_prefill(w.q, w.kv, w.indices, w.softmax_scale)
    out2, lse2 = sparse_prefill(w.q, w.kv, np.concatenate([w.indices, w.indices], axis=1),
                                w.softmax_scale)
    np.testing.assert_allclose(out2, out1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse2, lse1 + 1.0, rtol=0, atol=1e-12)
