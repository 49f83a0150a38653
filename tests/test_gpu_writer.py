"""GPU parity of the FP8 KV writer (mla_kv_quantize_fp8) against the oracle's
quantiser and append: every byte of the pool must match (codes, scales,
RoPE, untouched rows)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_head_amd as mla
import synth

pytestmark = pytest.mark.gpu


def gpu_append(w: synth.AppendWorkload, pool=None) -> np.ndarray:
    dev = torch.device("cuda")
    kv_new = torch.from_numpy(w.kv_new.view(np.int16)).to(dev).view(torch.bfloat16)
    sp = torch.from_numpy(w.start_pos).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    pool_t = torch.from_numpy(w.pool if pool is None else pool).to(dev)
    mla.mla_kv_quantize_fp8(kv_new, sp, bt, pool_t)
    torch.cuda.synchronize()
    return pool_t.cpu().numpy()


def oracle_append(w: synth.AppendWorkload) -> np.ndarray:
    return oracle.kv_append_fp8(w.kv_new, w.start_pos, w.block_table, w.pool)


def assert_pools_equal(got, ref):
    if not np.array_equal(got, ref):
        diff = np.argwhere(got != ref)
        page, slot, byte = diff[0]
        raise AssertionError(f"{len(diff)} bytes differ; first at page {page} slot {slot} byte {byte}: "
                             f"gpu {got[page, slot, byte]:#04x} oracle {ref[page, slot, byte]:#04x}")


@pytest.mark.parametrize("seed, batch, n_new, scale", [
    (1, 1, 1, None),
    (2, 5, 37, "mixed"),
    (3, 7, 130, None),
    (4, 16, 64, "mixed"),
    (5, 3, 257, 1e-3),
])
def test_writer_matches_oracle(seed, batch, n_new, scale):
    w = synth.make_append(f"append_{seed}", batch=batch, n_new=n_new,
                          start_pos=synth.Uniform(0, 200), seed=seed, value_scale=scale,
                          pool_fill=None)
    assert_pools_equal(gpu_append(w), oracle_append(w))


def test_writer_skips_out_of_range_tokens():
    """Negative positions, -1 and too-large block-table entries and positions
    past the table's last page write nothing."""
    w = synth.make_append("append_skip", batch=4, n_new=80, start_pos=[-5, 0, 100, 190], seed=9,
                          max_pages_per_seq=4, pool_fill=None)
    num_pages = w.pool.shape[0]
    w.block_table[1, 0] = -1
    w.block_table[2, 1] = num_pages + 3
    w.block_table[2, 2] = num_pages
    ref = oracle_append(w)
    got = gpu_append(w)
    assert_pools_equal(got, ref)
    # the oracle agrees that something was skipped: fewer rows changed than tokens
    changed = np.any(ref != w.pool, axis=2).sum()
    assert 0 < changed < w.tokens


def encoder_rows(amax_bits: int, rng) -> np.ndarray:
    """Rows whose NoPE tiles each hold +-amax once (fixing the tile scale)
    and then every finite bf16 value of magnitude <= amax, in both signs."""
    amax = synth.bf16_bits_to_f32(np.array([amax_bits], dtype=np.uint16))[0]
    pos = np.arange(0, 0x7F80, dtype=np.uint16)  # all finite non-negative bf16 patterns
    pos = pos[synth.bf16_bits_to_f32(pos) <= amax]
    vals = np.concatenate([pos, pos | np.uint16(0x8000)])
    rng.shuffle(vals)
    n_tiles = -(-vals.shape[0] // 127)
    vals = np.concatenate([vals, np.zeros(n_tiles * 127 - vals.shape[0], dtype=np.uint16)])
    tiles = np.empty((n_tiles, 128), dtype=np.uint16)
    tiles[:, 0] = amax_bits | np.where(np.arange(n_tiles) % 2 == 1, 0x8000, 0).astype(np.uint16)
    tiles[:, 1:] = vals.reshape(n_tiles, 127)
    for t in tiles:
        rng.shuffle(t)
    n_rows = -(-n_tiles // 4)
    nope = np.zeros((n_rows * 4, 128), dtype=np.uint16)
    nope[:n_tiles] = tiles
    rows = np.empty((n_rows, 576), dtype=np.uint16)
    rows[:, :512] = nope.reshape(n_rows, 512)
    rows[:, 512:] = synth.bf16_bits_from_f32(rng.standard_normal((n_rows, 64)).astype(np.float32))
    return rows


@pytest.mark.parametrize("amax", [448.0, 1.0, 3.0e-5, 1.0e30, 0.7109375, 2.0 ** -120])
def test_writer_encoder_over_all_bf16_values(amax):
    """Every finite bf16 value below a tile's maximum, for maxima that make
    the scale exact (448), inexact (1, 0.71...), tiny (subnormal codes of
    tiny values, an fp32-subnormal-range scale) and huge."""
    rng = np.random.default_rng(17)
    amax_bits = int(synth.bf16_bits_from_f32(np.array([amax], dtype=np.float32))[0])
    rows = encoder_rows(amax_bits, rng)
    n = rows.shape[0]
    pages = -(-n // 64)
    w = synth.AppendWorkload(name="encoder", kv_new=rows[None], start_pos=np.zeros(1, np.int32),
                             block_table=np.arange(pages, dtype=np.int32)[None],
                             pool=np.zeros((pages, 64, 656), dtype=np.uint8))
    got = gpu_append(w).reshape(pages * 64, 656)[:n]
    ref = np.stack([oracle.quantize_row_fp8(r) for r in rows])
    assert_pools_equal(got[None], ref[None])


def test_writer_special_tiles():
    """All-zero tiles, negative zeros, a tile of one nonzero value and RoPE
    extremes."""
    rows = np.zeros((6, 576), dtype=np.uint16)
    rows[1, :128] = 0x8000                    # -0 everywhere: scale 0, codes 0x00
    rows[2, 5] = 0x3F80                       # a single 1.0
    rows[3, 128:256] = 0x0001                 # smallest bf16 subnormal
    rows[4, 256:384] = np.arange(128, dtype=np.uint16) | 0x8000  # negative subnormals
    rows[5, :512] = 0x7F7F                    # the largest finite bf16
    rows[:, 512:] = np.arange(64, dtype=np.uint16) * 0x0401
    w = synth.AppendWorkload(name="special", kv_new=rows[None], start_pos=np.array([3], np.int32),
                             block_table=np.array([[1, 0]], dtype=np.int32),
                             pool=np.full((2, 64, 656), 0xAB, dtype=np.uint8))
    assert_pools_equal(gpu_append(w), oracle_append(w))


def test_writer_full_size_fill_sampled():
    """The benchmark's fill (128 sequences x 4096 new tokens from position 0,
    permuted block table): every unwritten byte keeps its poison and a seeded
    sample of written rows matches the oracle's quantiser."""
    w = synth.make_append("fill_b128_n4096", batch=128, n_new=4096, start_pos=[0] * 128,
                          seed=2024)
    got = gpu_append(w)
    rng = np.random.default_rng(0)
    for tok in rng.choice(w.tokens, size=512, replace=False):
        b, j = divmod(int(tok), 4096)
        page, slot = w.block_table[b, j // 64], j % 64
        assert np.array_equal(got[page, slot], oracle.quantize_row_fp8(w.kv_new[b, j])), (b, j)
    used = np.zeros(w.pool.shape[0], dtype=bool)
    used[w.block_table[w.block_table >= 0]] = True
    assert np.all(got[~used] == 0xFF)
    # every written row has finite scales (no poison left in a referenced row)
    scales = got[used][:, :, 512:528].copy().view(np.float32)
    assert np.isfinite(scales).all()


def test_writer_then_fp8_decode_end_to_end():
    """Decode over a cache the GPU writer filled equals the oracle's decode
    over the cache the oracle's writer filled (the two caches are
    byte-identical, and the FP8 decode reads them the same way)."""
    import math

    from tests.harness import assert_close, run

    rng = np.random.default_rng(31)
    B, s_q, h_q = 3, 2, 128
    lens = np.array([300, 1, 777], dtype=np.int32)
    w = synth.make_workload("writer_e2e", batch=B, h_q=h_q, s_q=s_q, seqlens=lens, seed=32,
                            kv_format=synth.KV_FP8_656, is_causal=1)
    n_new = int(lens.max())
    rows = synth.bf16_bits_from_f32(rng.standard_normal((B, n_new, 576)).astype(np.float32))
    app = synth.AppendWorkload(name="e2e", kv_new=rows, start_pos=np.zeros(B, np.int32),
                               block_table=w.block_table, pool=w.kv.copy())
    # positions past a sequence's length fill its last page's tail (masked by the decode)
    # or have no page (-1 in the table): skipped
    gpu_pool = gpu_append(app)
    ref_pool = oracle_append(app)
    assert_pools_equal(gpu_pool, ref_pool)
    w.kv = gpu_pool
    out, lse = run(w)
    w.kv = ref_pool
    ref_out, ref_lse = oracle.mla_decode(w)
    assert_close(out, lse, ref_out, ref_lse, what="writer -> fp8 decode")
    assert math.isfinite(float(np.abs(out).max()))


@pytest.mark.parametrize("seed", range(20))
def test_writer_random_shapes(seed):
    """Seeded random shapes: batch, new tokens, start positions (negative
    ones included), value scales, tables narrower than the appended range
    and holes (-1) in the table; the pool must match the oracle's byte for
    byte."""
    rng = np.random.default_rng(60_000 + seed)
    batch = int(rng.integers(1, 12))
    n_new = int(rng.integers(1, 300))
    start = [int(x) for x in rng.integers(-40, 400, size=batch)]
    width = [None, 2, 5][int(rng.integers(0, 3))]
    scale = [None, "mixed", 1e-4, 30.0][int(rng.integers(0, 4))]
    print(f"writer sweep {seed}: batch {batch} n_new {n_new} width {width} scale {scale}", flush=True)
    w = synth.make_append(f"append_sweep_{seed}", batch=batch, n_new=n_new, start_pos=start,
                          seed=70_000 + seed, max_pages_per_seq=width, value_scale=scale, pool_fill=None)
    holes = rng.random(w.block_table.shape) < 0.1
    w.block_table = np.where(holes, -1, w.block_table).astype(np.int32)
    assert_pools_equal(gpu_append(w), oracle_append(w))
