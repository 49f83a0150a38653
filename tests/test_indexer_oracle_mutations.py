"""The indexer oracle's pins catch plausible mistakes: each case plants one
mistake in the oracle (on the CPU, by replacing one of its functions) and
checks that a pin in tests/test_indexer_oracle.py fails."""

import numpy as np
import pytest

from oracle import indexer as ix
from tests import test_indexer_oracle as pins

_scores = ix.scores
_select = ix.select
_visible = ix.visible_rows


def scores_mean_over_heads(w, b, i):
    return _scores(w, b, i) / w.h


def scores_tile_scales_reversed(w, b, i):
    n = ix.visible_rows(int(w.cache_seqlens[b]), w.s_q, i, w.kpool, w.is_causal)
    if n == 0:
        return np.zeros(0)
    E = ix.e4m3_table()
    rows = ix.gather_rows(w, b, n)
    kc = E[rows[:, :512]]
    ks = np.ascontiguousarray(rows[:, 512:528]).view(np.float32).astype(np.float64)[:, ::-1]
    qc = E[w.q_codes[b, i]]
    qs = w.q_scales[b, i].astype(np.float64)
    S = np.zeros(n)
    for t in range(4):
        cols = slice(128 * t, 128 * (t + 1))
        S += ks[:, t] * ((kc[:, cols] @ qc[:, cols].T) @ qs[:, t])
    return S


def select_ties_to_larger_rows(S, topk):
    n = S.shape[0]
    j = np.arange(n)
    nan = np.isnan(S)
    order = np.lexsort((-j, np.where(nan, 0.0, -S), nan))
    return np.sort(order[:min(topk, n)])


def visible_causal_off_by_one(L, s_q, i, kpool, is_causal):
    return _visible(L - 1 if is_causal else L, s_q, i, kpool, is_causal)


def scores_without_query_scales(w, b, i):
    saved = w.q_scales
    w.q_scales = np.ones_like(saved)
    try:
        return _scores(w, b, i)
    finally:
        w.q_scales = saved


@pytest.mark.parametrize("attr,mutant,pin", [
    ("scores", scores_mean_over_heads, pins.test_heads_are_summed),
    ("scores", scores_mean_over_heads, pins.test_one_hot_query_reads_one_dequantised_value),
    ("scores", scores_tile_scales_reversed, pins.test_one_hot_query_reads_one_dequantised_value),
    ("scores", scores_without_query_scales, pins.test_heads_are_summed),
    ("select", select_ties_to_larger_rows, pins.test_selection_ties_nan_and_fill),
    ("visible_rows", visible_causal_off_by_one, pins.test_visible_row_counts),
])
def test_planted_mistake_is_caught(monkeypatch, attr, mutant, pin):
    monkeypatch.setattr(ix, attr, mutant)
    with pytest.raises(AssertionError):
        pin()
