"""CPU oracle for sparse MLA prefill -- test infrastructure only.

Plain numpy float64 written from the sparse-prefill semantics on the page
"为什么 FlashMLA 的解码内核能跑到 660 TFLOPS——内核里的 5 个关键设计", section
上手示例: the prefill call takes q [s_q, h_q, d_qk], a flat latent cache
kv [s_kv, 1, d_qk] (one KV head, no batch dimension, no block table) and
indices [s_q, 1, topk]; it gathers kv[indices] per query token, scores
P = (Q K^T) * sm_scale, takes lse = log2 of the sum of 2^P and returns
out = 2^(P - lse) times the gathered rows.

Readings (where the page is silent): the output keeps the first 512 latent
dims (d_v = 512, V = K[:, :512], "Modular Platform 设计文档全景导读",
section 九); indices outside [0, s_kv) (e.g. -1) are skipped, duplicates count
with multiplicity; an empty set gives lse = -inf and out = 0; the scale is
an fp32 value; with ``natural=True`` the base is e (lse in natural log).
Only the tests and the benchmark's CPU baseline use this module.
"""

from __future__ import annotations

import numpy as np

from . import decode_row

D_QK = 576
D_V = 512


def latent_rows(kv: np.ndarray, kv_format: int) -> np.ndarray:
    """Flat cache bytes [s_kv, row_bytes] -> float64 values [s_kv, 576]."""
    kv = np.ascontiguousarray(kv, dtype=np.uint8)
    if kv_format == 0:
        bits = kv.reshape(kv.shape[0], D_QK * 2).view(np.uint16)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.stack([decode_row(r, kv_format) for r in kv]).astype(np.float64)


def sparse_prefill(q_bits: np.ndarray, kv: np.ndarray, indices: np.ndarray, softmax_scale: float,
                   kv_format: int = 0, natural: bool = False):
    """q_bits uint16 bf16 [s_q, h_q, 576]; kv uint8 [s_kv, row_bytes];
    indices int32 [s_q, topk].  Returns (out float64 [s_q, h_q, 512],
    lse float64 [s_q, h_q])."""
    s_q, h_q, d = q_bits.shape
    assert d == D_QK
    K = latent_rows(kv, kv_format)
    s_kv = K.shape[0]
    Q = (np.ascontiguousarray(q_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    Q = Q.astype(np.float64)
    scale = float(np.float32(softmax_scale))
    out = np.zeros((s_q, h_q, D_V), dtype=np.float64)
    lse = np.full((s_q, h_q), -np.inf, dtype=np.float64)
    for i in range(s_q):
        idx = np.asarray(indices[i], dtype=np.int64)
        idx = idx[(idx >= 0) & (idx < s_kv)]
        if idx.size == 0:
            continue
        G = K[idx]                           # gathered rows [n, 576]
        P = (Q[i] @ G.T) * scale             # scores [h_q, n]
        if natural:
            m = P.max(axis=1, keepdims=True)
            lse_i = m[:, 0] + np.log(np.exp(P - m).sum(axis=1))
            S = np.exp(P - lse_i[:, None])
        else:
            m = P.max(axis=1, keepdims=True)
            lse_i = m[:, 0] + np.log2(np.exp2(P - m).sum(axis=1))
            S = np.exp2(P - lse_i[:, None])
        lse[i] = lse_i
        out[i] = S @ G[:, :D_V]
    return out, lse
