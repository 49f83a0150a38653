"""CPU oracle of the FP8 top-k indexer -- test infrastructure only (the
tests, the smoke check and the benchmark's CPU baseline call it; the library
never does).

It follows "max.nn.kernels 内核封装模块全解析", section 稀疏注意力（MSA）与 MLA
索引内核 (mla_fp8_index_top_k: FP8 query against the quantised K cache with
their scales, aggregated over heads, masked, top-k row indices as int32 with
-1 where no valid row is left; pooled rows with kpool > 1), with these
readings of what the passage leaves open:

  * the quantised K of a row is the FP8 part of its 656-byte cache row: 512
    e4m3fn codes and four fp32 scales, one per 128-dim tile; the bf16 RoPE
    part is not quantised and is not scored;
  * the FP8 query has per head the same tiling (512 codes, four scales);
  * the aggregation over heads is their sum;
  * visible rows of token (b, i): j < ceil((t_max + 1) / kpool), t_max =
    L_b - 1, or L_b - s_q + i when causal (none when t_max < 0);
  * selection: largest score first, equal scores toward the smaller row, NaN
    below everything; output in ascending row order, then -1.

Everything is computed in float64 from the exact values of the codes (the
oracle's own e4m3fn decoder) and the scales: no step rounds to a narrower
type, so the scores are the definition's values up to float64 rounding.
"""

from __future__ import annotations

from typing import Tuple

import numpy as np

from . import e4m3_value

D = 512
TILE = 128
ROW_BYTES = 656
_E4M3 = None


def e4m3_table() -> np.ndarray:
    """float64 value of every e4m3fn code (NaN for the two NaN codes)."""
    global _E4M3
    if _E4M3 is None:
        _E4M3 = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
    return _E4M3


def visible_rows(L: int, s_q: int, i: int, kpool: int, is_causal: int) -> int:
    """Rows of the (pooled) cache token i of a sequence of L tokens sees."""
    t_max = (L - s_q + i) if is_causal else (L - 1)
    if t_max < 0:
        return 0
    return -(-(t_max + 1) // kpool)


def gather_rows(w, b: int, n: int) -> np.ndarray:
    """Cache rows 0..n-1 of sequence b: row j is slot j % 64 of page
    block_table[b][j // 64] (uint8 [n, 656])."""
    j = np.arange(n, dtype=np.int64)
    pages = w.block_table[b, j // 64].astype(np.int64)
    return w.kv[pages, j % 64]


def scores(w, b: int, i: int) -> np.ndarray:
    """float64 score of every visible row of token (b, i):
    S_j = sum_h sum_t qs[h, t] * s_j[t] * sum_{d in tile t} q[h, d] * c_j[d]."""
    n = visible_rows(int(w.cache_seqlens[b]), w.s_q, i, w.kpool, w.is_causal)
    if n == 0:
        return np.zeros(0, dtype=np.float64)
    E = e4m3_table()
    rows = gather_rows(w, b, n)
    kc = E[rows[:, :D]]                                                    # [n, 512]
    ks = np.ascontiguousarray(rows[:, D:D + 16]).view(np.float32).astype(np.float64)  # [n, 4]
    qc = E[w.q_codes[b, i]]                                                # [h, 512]
    qs = w.q_scales[b, i].astype(np.float64)                               # [h, 4]
    S = np.zeros(n, dtype=np.float64)
    for t in range(D // TILE):
        cols = slice(TILE * t, TILE * (t + 1))
        prod = kc[:, cols] @ qc[:, cols].T          # [n, h]: code products of tile t
        S += ks[:, t] * (prod @ qs[:, t])           # scaled, summed over heads
    return S


def abs_scores(w, b: int, i: int) -> np.ndarray:
    """The same sums over absolute values: sum_h sum_t |qs| |s_j| sum_d |q| |c_j|.
    Bounds the rounding error of any evaluation of S in a narrower type."""
    n = visible_rows(int(w.cache_seqlens[b]), w.s_q, i, w.kpool, w.is_causal)
    if n == 0:
        return np.zeros(0, dtype=np.float64)
    E = np.abs(e4m3_table())
    rows = gather_rows(w, b, n)
    kc = E[rows[:, :D]]
    ks = np.abs(np.ascontiguousarray(rows[:, D:D + 16]).view(np.float32).astype(np.float64))
    qc = E[w.q_codes[b, i]]
    qs = np.abs(w.q_scales[b, i].astype(np.float64))
    A = np.zeros(n, dtype=np.float64)
    for t in range(D // TILE):
        cols = slice(TILE * t, TILE * (t + 1))
        A += ks[:, t] * ((kc[:, cols] @ qc[:, cols].T) @ qs[:, t])
    return A


def select(S: np.ndarray, topk: int) -> np.ndarray:
    """Rows of the min(topk, len(S)) largest scores (ties toward the smaller
    row, NaN lowest), in ascending row order."""
    n = S.shape[0]
    j = np.arange(n)
    nan = np.isnan(S)
    key = np.where(nan, 0.0, -S)
    order = np.lexsort((j, key, nan))   # NaN last, then descending S, then ascending j
    return np.sort(order[:min(topk, n)])


def top_k(w, tokens=None) -> Tuple[np.ndarray, np.ndarray]:
    """Indices int32 [B, s_q, topk] and their float64 scores (-inf beside -1)
    for every token, or only for the (b, i) pairs in ``tokens`` (other entries
    left at -1 / -inf)."""
    idx = np.full((w.batch, w.s_q, w.topk), -1, dtype=np.int32)
    sc = np.full((w.batch, w.s_q, w.topk), -np.inf, dtype=np.float64)
    pairs = tokens if tokens is not None else [(b, i) for b in range(w.batch) for i in range(w.s_q)]
    for b, i in pairs:
        S = scores(w, b, i)
        sel = select(S, w.topk)
        idx[b, i, :sel.shape[0]] = sel
        sc[b, i, :sel.shape[0]] = S[sel]
    return idx, sc
