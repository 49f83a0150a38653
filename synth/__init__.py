"""Seeded synthetic decode workloads for paged MLA decode.

This module only draws inputs: sequence lengths, a page permutation, query and
latent-cache values, and top-k index lists.  It holds no attention arithmetic.
Both the CPU oracle and the GPU library consume exactly the arrays built here.

Recipe (all draws from ``numpy.random.Generator(PCG64(seed))``, in this order):

1. ``cache_seqlens`` (fixed list, or uniform integers in ``[lo, hi]``).
2. Page permutation: the pool holds ``ceil(1.1 * N)`` pages (``N`` = pages the
   sequences need; exactly ``N`` when ``slack`` is 0).  Sequence ``b`` gets the
   next ``ceil(L_b / page_size)`` entries of one random permutation of the pool.
   Unused block-table slots are -1.
3. Q: ``[B, s_q, h_q, 576]`` standard normal float32, rounded to bf16 (RNE).
4. Top-k indices (sparse workloads only): per (b, i), ``topk`` distinct
   positions drawn uniformly without replacement from ``[0, L_b)``.
5. KV: one standard normal float32 row of 576 values per *referenced* token,
   in ascending (b, t) order, rounded to bf16.  Rows are drawn in chunks of
   ``kv_chunk_rows`` tokens; chunk c uses its own stream
   ``PCG64(SeedSequence([seed, 1, c]))`` so chunks can be filled in parallel.  Dense workloads reference
   every ``t < L_b``; sparse workloads reference the union of their indices.
   Every other byte of the pool (page tails, slack pages, unreferenced rows)
   is 0xFF: NaN in bf16, e4m3fn and fp32, so any read of it shows up.

Latent rows in the 656-byte FP8 layout: the first 512 (NoPE) values of the
bf16 row are encoded per 1x128 tile with scale = amax / 448 (float32) and
codes = float8_e4m3fn(x / scale) (torch's cast, clamped to +-448; an all-zero
tile gets scale 0 and zero codes); bytes [512, 528) hold the four float32
scales, bytes [528, 656) the 64 RoPE values as bf16.  This is input encoding
only; decoding is done separately by each consumer.
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import List, Optional, Sequence

import numpy as np

D_QK = 576
D_V = 512
D_NOPE = 512
D_ROPE = 64
ROW_BYTES_BF16 = D_QK * 2  # 1152
ROW_BYTES_FP8 = D_NOPE + 4 * 4 + D_ROPE * 2  # 656
KV_BF16 = 0
KV_FP8_656 = 1


@dataclasses.dataclass
class Workload:
    """One decode batch: every array is host (numpy) memory."""

    name: str
    batch: int
    s_q: int
    h_q: int
    page_size: int
    kv_format: int
    topk: int
    is_causal: int
    softmax_scale: float  # float32 value
    q: np.ndarray  # uint16 [B, s_q, h_q, 576] bf16 bit patterns
    kv: np.ndarray  # uint8 [num_pages, page_size, row_bytes]
    block_table: np.ndarray  # int32 [B, max_pages_per_seq]
    cache_seqlens: np.ndarray  # int32 [B]
    indices: Optional[np.ndarray]  # int32 [B, s_q, topk] or None

    @property
    def num_pages(self) -> int:
        return int(self.kv.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def row_bytes(self) -> int:
        return int(self.kv.shape[2])

    def flops(self) -> int:
        """2*h_q*s_q*s_k*(d_qk+d_v) summed over the batch (s_k = L_b, or topk)."""
        if self.topk > 0:
            sk = self.batch * self.topk
        else:
            sk = int(self.cache_seqlens.astype(np.int64).sum())
        return 2 * self.h_q * self.s_q * sk * (D_QK + D_V)

    def algorithmic_bytes(self) -> int:
        """Bytes the method must move once: visible KV rows once per fetching
        query set, Q, out (bf16), lse (fp32), block-table and index reads."""
        L = self.cache_seqlens.astype(np.int64)
        if self.topk > 0:
            kv_rows = self.batch * self.s_q * self.topk
            table = 4 * kv_rows
            idx = 4 * kv_rows
        else:
            kv_rows = int(L.sum())
            table = 4 * int(((L + self.page_size - 1) // self.page_size).sum())
            idx = 0
        rows = self.batch * self.s_q * self.h_q
        return (kv_rows * self.row_bytes + rows * D_QK * 2 + rows * D_V * 2
                + rows * 4 + table + idx + 4 * self.batch)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns via torch's round-to-nearest-even cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def encode_fp8_rows(rows_bf16: np.ndarray) -> np.ndarray:
    """bf16 bit rows [n, 576] -> 656-byte rows [n, 656] (input encoding)."""
    import torch

    n = rows_bf16.shape[0]
    x = bf16_bits_to_f32(rows_bf16)
    nope = x[:, :D_NOPE].reshape(n, 4, 128)
    amax = np.abs(nope).max(axis=2).astype(np.float32)  # [n, 4]
    scale = (amax / np.float32(448.0)).astype(np.float32)
    safe = np.where(scale == 0, np.float32(1.0), scale)
    y = np.clip(nope / safe[:, :, None], -448.0, 448.0).astype(np.float32)
    y = np.where(scale[:, :, None] == 0, np.float32(0.0), y)
    codes = torch.from_numpy(y.reshape(n, D_NOPE)).to(torch.float8_e4m3fn)
    codes = codes.view(torch.uint8).numpy()
    out = np.empty((n, ROW_BYTES_FP8), dtype=np.uint8)
    out[:, :D_NOPE] = codes
    out[:, D_NOPE:D_NOPE + 16] = scale.view(np.uint8).reshape(n, 16)
    out[:, D_NOPE + 16:] = rows_bf16[:, D_NOPE:].copy().view(np.uint8).reshape(n, 128)
    return out


@dataclasses.dataclass(frozen=True)
class Uniform:
    """Sequence lengths drawn uniformly from the closed range [lo, hi]."""

    lo: int
    hi: int


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def make_workload(name: str, *, batch: int, h_q: int, s_q: int, seqlens,
                  seed: int, kv_format: int = KV_BF16, topk: int = 0,
                  is_causal: int = 0, page_size: int = 64, slack: float = 0.1,
                  softmax_scale: Optional[float] = None,
                  max_pages_per_seq: Optional[int] = None,
                  kv_chunk_rows: int = 1 << 15) -> Workload:
    """Build one seeded workload following the recipe in the module docstring.

    ``seqlens`` is either a sequence of ints (one per batch entry) or a
    :class:`Uniform` for uniform integers in a closed range.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if isinstance(seqlens, Uniform):
        L = rng.integers(seqlens.lo, seqlens.hi, size=batch, endpoint=True).astype(np.int32)
    else:
        L = np.asarray(list(seqlens), dtype=np.int32)
        assert L.shape == (batch,)
    n_pages = [_ceil_div(int(l), page_size) for l in L]
    need = int(sum(n_pages))
    pool = max(1, need if slack == 0 else int(math.ceil((1.0 + slack) * need)))
    perm = rng.permutation(pool).astype(np.int32)
    width = max_pages_per_seq if max_pages_per_seq is not None else max(1, max(n_pages) if n_pages else 1)
    table = np.full((batch, width), -1, dtype=np.int32)
    off = 0
    for b in range(batch):
        table[b, :n_pages[b]] = perm[off:off + n_pages[b]]
        off += n_pages[b]

    q32 = rng.standard_normal((batch, s_q, h_q, D_QK), dtype=np.float32)
    q = bf16_bits_from_f32(q32)
    del q32

    indices = None
    if topk > 0:
        indices = np.empty((batch, s_q, topk), dtype=np.int32)
        for b in range(batch):
            for i in range(s_q):
                assert topk <= L[b], "topk distinct positions need topk <= L_b"
                indices[b, i] = rng.choice(int(L[b]), size=topk, replace=False).astype(np.int32)

    row_bytes = ROW_BYTES_BF16 if kv_format == KV_BF16 else ROW_BYTES_FP8
    kv = np.full((pool, page_size, row_bytes), 0xFF, dtype=np.uint8)
    # referenced tokens in ascending (b, t) order
    refs_b: List[np.ndarray] = []
    refs_t: List[np.ndarray] = []
    for b in range(batch):
        if topk > 0:
            t = np.unique(indices[b].reshape(-1))
        else:
            t = np.arange(int(L[b]), dtype=np.int64)
        refs_b.append(np.full(t.shape, b, dtype=np.int64))
        refs_t.append(t.astype(np.int64))
    rb = np.concatenate(refs_b) if refs_b else np.zeros(0, np.int64)
    rt = np.concatenate(refs_t) if refs_t else np.zeros(0, np.int64)
    pages = table[rb, rt // page_size].astype(np.int64)
    dest = pages * page_size + rt % page_size
    flat = kv.reshape(pool * page_size, row_bytes)
    # KV rows come in fixed chunks of kv_chunk_rows referenced tokens; chunk c
    # draws from its own stream PCG64(SeedSequence([seed, 1, c])), so the
    # values do not depend on how many threads fill the chunks.
    n_chunks = -(-rb.shape[0] // kv_chunk_rows)

    def fill(c):
        s0 = c * kv_chunk_rows
        e0 = min(rb.shape[0], s0 + kv_chunk_rows)
        crng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1, c])))
        x = crng.standard_normal((e0 - s0, D_QK), dtype=np.float32)
        bits = bf16_bits_from_f32(x)
        if kv_format == KV_BF16:
            flat[dest[s0:e0]] = bits.view(np.uint8).reshape(e0 - s0, row_bytes)
        else:
            flat[dest[s0:e0]] = encode_fp8_rows(bits)

    workers = max(1, min(16, os.cpu_count() or 1))
    if n_chunks <= 1 or workers == 1:
        for c in range(n_chunks):
            fill(c)
    else:
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(n_chunks)))
    scale = np.float32(1.0 / math.sqrt(D_QK)) if softmax_scale is None else np.float32(softmax_scale)
    return Workload(name=name, batch=batch, s_q=s_q, h_q=h_q, page_size=page_size,
                    kv_format=kv_format, topk=topk, is_causal=is_causal,
                    softmax_scale=float(scale), q=q, kv=kv, block_table=table,
                    cache_seqlens=L, indices=indices)


# The five decode configurations, by number.  ``batch`` may be overridden to
# build a smaller batch of the same shape for parity runs.
BENCH_WORKLOADS = {
    1: dict(name="c1_tiny_bf16", batch=2, h_q=16, s_q=1, seqlens=[100, 257],
            kv_format=KV_BF16, slack=0.0),
    2: dict(name="c2_dense_bf16_b64_sq1", batch=64, h_q=128, s_q=1, seqlens=Uniform(1024, 8192),
            kv_format=KV_BF16, max_pages_per_seq=128),
    3: dict(name="c3_dense_bf16_b128_sq2_causal", batch=128, h_q=128, s_q=2, seqlens=4096,
            kv_format=KV_BF16, is_causal=1),
    4: dict(name="c4_dense_fp8_b128_sq2", batch=128, h_q=128, s_q=2, seqlens=Uniform(8192, 32768),
            kv_format=KV_FP8_656, max_pages_per_seq=512),
    5: dict(name="c5_sparse_fp8_b128_sq2_topk2048", batch=128, h_q=128, s_q=2, seqlens=65536,
            kv_format=KV_FP8_656, topk=2048),
}


def config_workload(n: int, batch: Optional[int] = None, seed: Optional[int] = None) -> Workload:
    """Workload of configuration ``n`` (seed 1000 + n unless given)."""
    c = dict(BENCH_WORKLOADS[n])
    b = batch if batch is not None else c["batch"]
    c["batch"] = b
    if isinstance(c["seqlens"], int):
        c["seqlens"] = [c["seqlens"]] * b
    return make_workload(seed=1000 + n if seed is None else seed, **c)


@dataclasses.dataclass
class AppendWorkload:
    """Inputs of one FP8 KV append: new latent rows, their start positions,
    a block table and the pool they are written into."""

    name: str
    kv_new: np.ndarray       # uint16 bf16 bits [B, n_new, 576]
    start_pos: np.ndarray    # int32 [B]
    block_table: np.ndarray  # int32 [B, max_pages]
    pool: np.ndarray         # uint8 [num_pages, page_size, 656], initial contents

    @property
    def tokens(self) -> int:
        return int(self.kv_new.shape[0] * self.kv_new.shape[1])


def make_append(name: str, *, batch: int, n_new: int, start_pos, seed: int,
                max_pages_per_seq: Optional[int] = None, page_size: int = 64,
                slack: float = 0.1, value_scale=None, pool_fill: Optional[int] = 0xFF
                ) -> AppendWorkload:
    """Seeded append workload.  Draw order from PCG64(seed): start positions
    (if given as a Uniform), page permutation (pool of ceil((1 + slack) * N)
    pages for the N pages the appended positions reach, assigned row-major to
    the block table, unused slots -1), then the new rows: standard normal
    float32 times ``value_scale`` (a scalar or one factor per row drawn as
    10^U[-3, 3] when ``value_scale == "mixed"``), rounded to bf16.  The
    pool starts as ``pool_fill`` bytes (0xFF = NaN everywhere) or, with
    ``pool_fill=None``, random bytes."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if isinstance(start_pos, Uniform):
        sp = rng.integers(start_pos.lo, start_pos.hi, size=batch, endpoint=True).astype(np.int32)
    else:
        sp = np.asarray(list(start_pos), dtype=np.int32)
        assert sp.shape == (batch,)
    end_pages = [_ceil_div(max(0, int(s) + n_new), page_size) for s in sp]
    width = max_pages_per_seq if max_pages_per_seq is not None else max(1, max(end_pages))
    n_pages = [min(e, width) for e in end_pages]
    need = int(sum(n_pages))
    pool_pages = max(1, int(math.ceil((1.0 + slack) * need)))
    perm = rng.permutation(pool_pages).astype(np.int32)
    table = np.full((batch, width), -1, dtype=np.int32)
    off = 0
    for b in range(batch):
        table[b, :n_pages[b]] = perm[off:off + n_pages[b]]
        off += n_pages[b]
    x = rng.standard_normal((batch, n_new, D_QK), dtype=np.float32)
    if isinstance(value_scale, str) and value_scale == "mixed":
        x *= (10.0 ** rng.uniform(-3, 3, (batch, n_new, 1))).astype(np.float32)
    elif value_scale is not None:
        x *= np.float32(value_scale)
    kv_new = bf16_bits_from_f32(x)
    if pool_fill is None:
        pool = rng.integers(0, 256, (pool_pages, page_size, ROW_BYTES_FP8), dtype=np.uint8)
    else:
        pool = np.full((pool_pages, page_size, ROW_BYTES_FP8), pool_fill, dtype=np.uint8)
    return AppendWorkload(name=name, kv_new=kv_new, start_pos=sp, block_table=table, pool=pool)


@dataclasses.dataclass
class PrefillWorkload:
    """Inputs of one sparse prefill: queries, a flat latent cache (no
    batch dimension, no block table) and per-query index lists."""

    name: str
    q: np.ndarray        # uint16 bf16 bits [s_q, h_q, 576]
    kv: np.ndarray       # uint8 [s_kv, row_bytes]
    indices: np.ndarray  # int32 [s_q, topk]
    kv_format: int
    softmax_scale: float

    @property
    def s_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def h_q(self) -> int:
        return int(self.q.shape[1])

    @property
    def s_kv(self) -> int:
        return int(self.kv.shape[0])

    @property
    def topk(self) -> int:
        return int(self.indices.shape[1])

    def flops(self) -> int:
        return 2 * self.h_q * self.s_q * self.topk * (D_QK + D_V)

    def algorithmic_bytes(self) -> int:
        """Bytes the method must move at least once: every distinct cache row
        some query lists, the index lists, Q, out and lse.  Rows listed by
        several queries are counted once (they can be served from cache)."""
        row = ROW_BYTES_BF16 if self.kv_format == KV_BF16 else ROW_BYTES_FP8
        valid = self.indices[(self.indices >= 0) & (self.indices < self.s_kv)]
        distinct = int(np.unique(valid).size)
        rows = self.s_q * self.h_q
        return (distinct * row + self.indices.size * 4 + rows * D_QK * 2 + rows * D_V * 2
                + rows * 4)


def make_sparse_prefill(name: str, *, s_q: int, h_q: int, s_kv: int, topk: int, seed: int,
                        kv_format: int = KV_BF16, invalid_frac: float = 0.0,
                        softmax_scale: Optional[float] = None) -> PrefillWorkload:
    """Seeded sparse prefill.  Draw order from PCG64(seed): Q [s_q, h_q, 576]
    standard normal rounded to bf16; KV [s_kv, 576] standard normal rounded
    to bf16 (FP8: encoded as in the decode workloads); per query token,
    ``topk`` distinct positions uniform without replacement from
    [0, s_kv); then, if ``invalid_frac`` > 0, that fraction of all entries
    (uniform positions) replaced by -1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = bf16_bits_from_f32(rng.standard_normal((s_q, h_q, D_QK), dtype=np.float32))
    kv_bits = bf16_bits_from_f32(rng.standard_normal((s_kv, D_QK), dtype=np.float32))
    kv = kv_bits.view(np.uint8).reshape(s_kv, ROW_BYTES_BF16) if kv_format == KV_BF16 \
        else encode_fp8_rows(kv_bits)
    assert topk <= s_kv
    indices = np.empty((s_q, topk), dtype=np.int32)
    for i in range(s_q):
        indices[i] = rng.choice(s_kv, size=topk, replace=False).astype(np.int32)
    if invalid_frac > 0:
        hit = rng.random((s_q, topk)) < invalid_frac
        indices[hit] = -1
    scale = np.float32(1.0 / math.sqrt(D_QK)) if softmax_scale is None else np.float32(softmax_scale)
    return PrefillWorkload(name=name, q=q, kv=np.ascontiguousarray(kv), indices=indices,
                           kv_format=kv_format, softmax_scale=float(scale))


@dataclasses.dataclass
class IndexWorkload:
    """Inputs of one FP8 top-k indexer call, plus the bf16 query the FP8
    query was encoded from (the query of the sparse decode that follows).

    Recipe: a dense FP8 decode workload (``make_workload`` with the same seed)
    over the cache's rows (``ceil(L_b / kpool)`` pooled rows per sequence), its
    bf16 query ``[B, s_q, h, 576]`` as drawn there; the FP8 query is the first
    512 values of each (b, i, h) query row encoded like a cache row (per
    1x128 tile, scale = amax / 448, e4m3fn codes).  ``cache_seqlens`` holds
    the token counts ``L_b``."""

    name: str
    batch: int
    s_q: int
    h: int
    topk: int
    kpool: int
    is_causal: int
    q_bf16: np.ndarray       # uint16 [B, s_q, h, 576]
    q_codes: np.ndarray      # uint8 [B, s_q, h, 512]
    q_scales: np.ndarray     # float32 [B, s_q, h, 4]
    kv: np.ndarray           # uint8 [num_pages, 64, 656]
    block_table: np.ndarray  # int32 [B, max_pages_per_seq]
    cache_seqlens: np.ndarray  # int32 [B], tokens

    @property
    def num_pages(self) -> int:
        return int(self.kv.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    def rows(self) -> np.ndarray:
        """Cached (pooled) rows per sequence."""
        L = self.cache_seqlens.astype(np.int64)
        return (L + self.kpool - 1) // self.kpool

    def flops(self) -> int:
        """2 * h * 512 multiply-adds per (query token, cached row) pair."""
        return 2 * self.h * D_NOPE * self.s_q * int(self.rows().sum())

    def algorithmic_bytes(self) -> int:
        """The quantised part of every cached row once (512 codes + 16 bytes
        of scales), the FP8 query with its scales, the block-table entries and
        lengths read, and the int32 indices written."""
        pages = (self.rows() + self.page_size - 1) // self.page_size
        q = self.batch * self.s_q * self.h * (D_NOPE + 16)
        return (int(self.rows().sum()) * (D_NOPE + 16) + q + 4 * int(pages.sum()) + 4 * self.batch
                + 4 * self.batch * self.s_q * self.topk)

    page_size: int = 64


def make_index_workload(name: str, *, batch: int, s_q: int, h: int, seqlens, seed: int, topk: int,
                        kpool: int = 1, is_causal: int = 0, max_pages_per_seq: Optional[int] = None,
                        slack: float = 0.1) -> IndexWorkload:
    """Seeded indexer workload (recipe in :class:`IndexWorkload`)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if isinstance(seqlens, Uniform):
        L = rng.integers(seqlens.lo, seqlens.hi, size=batch, endpoint=True).astype(np.int32)
    else:
        L = np.asarray(list(seqlens), dtype=np.int32)
        assert L.shape == (batch,)
    rows = [(-(-int(l) // kpool)) for l in L]
    w = make_workload(name, batch=batch, h_q=h, s_q=s_q, seqlens=rows, seed=seed + 1,
                      kv_format=KV_FP8_656, slack=slack, max_pages_per_seq=max_pages_per_seq)
    enc = encode_fp8_rows(w.q.reshape(-1, D_QK))
    q_codes = np.ascontiguousarray(enc[:, :D_NOPE]).reshape(batch, s_q, h, D_NOPE)
    q_scales = np.ascontiguousarray(enc[:, D_NOPE:D_NOPE + 16]).view(np.float32).reshape(batch, s_q, h, 4)
    return IndexWorkload(name=name, batch=batch, s_q=s_q, h=h, topk=topk, kpool=kpool,
                         is_causal=is_causal, q_bf16=w.q, q_codes=q_codes, q_scales=q_scales,
                         kv=w.kv, block_table=w.block_table, cache_seqlens=L)
