"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs, at sizes the oracle finishes in seconds (several tiles,
ragged tails), plus bit-exact layout probes and invariances."""

import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_head_amd as mla
import synth
from oracle.schedule import blocks_per_unit, schedule
from tests.harness import assert_close, run, to_device

pytestmark = pytest.mark.gpu


def reduced(n, batch, seed=None):
    return synth.config_workload(n, batch=batch, seed=seed)


# ------------------------------------------------------------ configs ---

@pytest.mark.parametrize("n,batch", [(1, None), (2, 4), (3, 3), (4, 2), (5, 2)])
def test_config_parity(n, batch):
    w = synth.config_workload(n, batch=batch)
    print(f"config {n} batch {w.batch} seqlens {w.cache_seqlens.tolist()}", flush=True)
    out, lse = run(w)
    ref_out, ref_lse = oracle.mla_decode(w)
    assert_close(out, lse, ref_out, ref_lse, what=f"config {n}")


@pytest.mark.parametrize("n", [1, 3, 5])
def test_natural_base(n):
    w = synth.config_workload(n, batch=2)
    out, lse = run(w, natural=True)
    ref_out, ref_lse = oracle.mla_decode(w, natural=True)
    # lse tolerance is stated in log2 units; natural-log lse is ln2 times it
    assert_close(out, lse / math.log(2), ref_out, ref_lse / math.log(2), what="natural")


@pytest.mark.parametrize("n,scale", [(1, -1.0 / 24), (1, 0.0), (3, -0.3), (3, 0.0), (5, -1.0 / 24), (4, 0.0)])
def test_scale_sign_and_zero(n, scale):
    """Any finite softmax_scale: negative scales and zero take their own
    kernel path (a sign flip or zeroing of Q); the oracle uses the scale as
    given (zero: uniform weights, lse = log2 of the visible count)."""
    w = synth.config_workload(n, batch=2)
    out, lse = run(w, softmax_scale=scale)
    ref_out, ref_lse = oracle.mla_decode(w, softmax_scale=scale)
    assert_close(out, lse, ref_out, ref_lse, what=f"config {n} scale {scale}")


@pytest.mark.parametrize("parts", [1, 2, 3, 7, 64, 300, 1000])
def test_forced_split_counts(parts):
    w = synth.make_workload("t", batch=3, h_q=128, s_q=2, seqlens=[700, 129, 1], seed=31, is_causal=1)
    out, lse = run(w, num_parts=parts)
    ref_out, ref_lse = oracle.mla_decode(w)
    assert_close(out, lse, ref_out, ref_lse, what=f"num_parts={parts}")


@pytest.mark.parametrize("h_q,s_q,causal", [(16, 1, 0), (20, 3, 1), (64, 2, 1), (100, 1, 0),
                                            (128, 1, 0), (192, 1, 0), (256, 2, 1)])
def test_head_shapes(h_q, s_q, causal):
    w = synth.make_workload("t", batch=2, h_q=h_q, s_q=s_q, seqlens=[65, 300], seed=32, is_causal=causal)
    out, lse = run(w)
    ref_out, ref_lse = oracle.mla_decode(w)
    assert_close(out, lse, ref_out, ref_lse, what=f"h_q={h_q} s_q={s_q}")


@pytest.mark.parametrize("h_q,kv_format,L", [(128, synth.KV_BF16, 120_000), (16, synth.KV_BF16, 200_000),
                                             (64, synth.KV_FP8_656, 120_000)])
def test_long_sequence(h_q, kv_format, L):
    """One long sequence beside a short one: the scheduler cuts the long unit
    over most parts and the combine merges all of its splits."""
    w = synth.make_workload("t", batch=2, h_q=h_q, s_q=1, seqlens=[L, 77], seed=37, kv_format=kv_format)
    out, lse, _, splits, parts = run(w, return_meta=True)
    assert splits[1] - splits[0] > parts // 2  # the long unit really is split many ways
    ref_out, ref_lse = oracle.mla_decode(w)
    assert_close(out, lse, ref_out, ref_lse, what=f"long sequence h_q={h_q} fmt={kv_format}")


@pytest.mark.parametrize("kv_format", [synth.KV_BF16, synth.KV_FP8_656])
@pytest.mark.parametrize("h_q,s_q", [(128, 8), (96, 7)])
def test_many_query_tokens(h_q, s_q, kv_format):
    """Up to 1024 query rows per sequence: eight 128-row groups of one unit
    spread over the XCD mapping, causal rows of eight positions."""
    w = synth.make_workload("t", batch=3, h_q=h_q, s_q=s_q, seqlens=[5, 300, 1000], seed=36,
                            is_causal=1, kv_format=kv_format)
    out, lse = run(w)
    ref_out, ref_lse = oracle.mla_decode(w)
    assert_close(out, lse, ref_out, ref_lse, what=f"h_q={h_q} s_q={s_q} fmt={kv_format}")


@pytest.mark.parametrize("kv_format", [synth.KV_BF16, synth.KV_FP8_656])
def test_edge_lengths(kv_format):
    """Empty sequences, one token, page boundaries, causal with L < s_q."""
    w = synth.make_workload("t", batch=7, h_q=32, s_q=2, seqlens=[0, 1, 63, 64, 65, 128, 2],
                            seed=33, is_causal=1, kv_format=kv_format)
    out, lse = run(w, num_parts=5)
    ref_out, ref_lse = oracle.mla_decode(w)
    assert_close(out, lse, ref_out, ref_lse, what="edges")
    assert np.all(lse[0] == -np.inf) and np.all(out[0] == 0)
    assert np.all(lse[1, 0] == -np.inf) and np.all(out[1, 0] == 0)  # L=1, s_q=2: query 0 sees nothing


def test_empty_batch_entries_only():
    w = synth.make_workload("t", batch=3, h_q=16, s_q=1, seqlens=[0, 0, 0], seed=34)
    out, lse = run(w)
    assert np.all(lse == -np.inf) and np.all(out == 0)


@pytest.mark.parametrize("topk", [1, 63, 64, 65, 200])
def test_sparse_topk_sizes(topk):
    w = synth.make_workload("t", batch=2, h_q=128, s_q=2, seqlens=[300, 1000], seed=35,
                            kv_format=synth.KV_FP8_656, topk=topk)
    out, lse = run(w)
    ref_out, ref_lse = oracle.mla_decode(w)
    assert_close(out, lse, ref_out, ref_lse, what=f"topk={topk}")


def test_sparse_invalid_and_duplicate_indices():
    sp = synth.make_workload("t", batch=2, h_q=64, s_q=2, seqlens=[300, 90], seed=36,
                             kv_format=synth.KV_FP8_656, topk=80)
    # same shapes with every cache row filled, so edited indices reach data
    w = synth.make_workload("t", batch=2, h_q=64, s_q=2, seqlens=[300, 90], seed=36,
                            kv_format=synth.KV_FP8_656)
    w.topk = 80
    idx = sp.indices.copy()
    idx[0, 0, ::7] = -1
    idx[0, 1, 5:20] = 299          # duplicates of a valid position
    idx[1, 0, :] = -1              # nothing visible
    idx[1, 1, 3] = 90              # == L: skipped
    idx[1, 1, 4] = 2 ** 30         # far out of range: skipped
    w.indices = idx
    out, lse = run(w)
    ref_out, ref_lse = oracle.mla_decode(w)
    assert_close(out, lse, ref_out, ref_lse, what="sparse invalid/dup")
    assert np.all(lse[1, 0] == -np.inf)


def test_bf16_sparse():
    w = synth.make_workload("t", batch=2, h_q=32, s_q=1, seqlens=[500, 170], seed=37, topk=100)
    out, lse = run(w)
    ref_out, ref_lse = oracle.mla_decode(w)
    assert_close(out, lse, ref_out, ref_lse, what="bf16 sparse")


# ------------------------------------------------------ bit-exact probes ---

@pytest.mark.parametrize("kv_format", [synth.KV_BF16, synth.KV_FP8_656])
def test_single_key_returns_dequantised_row_bit_exact(kv_format):
    """topk = 1: weight is exactly 1, so out is the bf16 latent row itself."""
    L = 200
    # a dense workload references (and fills) every token; then use it sparsely
    full = synth.make_workload("t", batch=1, h_q=16, s_q=6, seqlens=[L], seed=38, kv_format=kv_format)
    full.topk = 1
    full.indices = np.array([[[0], [63], [64], [65], [127], [L - 1]]], dtype=np.int32)
    out, lse = run(full)
    for i, t in enumerate(full.indices[0, :, 0]):
        page = full.block_table[0, t // 64]
        row = oracle.decode_row(full.kv[page, t % 64], kv_format)
        assert np.array_equal(out[0, i], np.broadcast_to(row[:512], (16, 512))), f"token {t}"


def test_fp8_codes_all_values_bit_exact():
    """Every finite e4m3 code, under several scales, dequantises exactly as
    the oracle's codec does (read back through a one-key attention)."""
    w = synth.make_workload("t", batch=1, h_q=16, s_q=4, seqlens=[64], seed=39,
                            kv_format=synth.KV_FP8_656, slack=0)  # every row filled
    w.topk = 1
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    kv = w.kv.copy()
    scales = np.array([1.0, 2.0 ** -7, 3.3e-3, 0.731], dtype=np.float32)
    for slot in range(4):
        row = np.zeros(656, dtype=np.uint8)
        row[:254] = codes
        row[254:508] = codes
        row[508:512] = codes[:4]
        row[512:528] = np.roll(scales, slot).view(np.uint8)
        row[528:] = kv[0, slot, 528:]
        kv[0, slot] = row
    w.kv = kv
    w.indices = np.array([[[0], [1], [2], [3]]], dtype=np.int32)
    out, lse = run(w)
    for i in range(4):
        ref = oracle.decode_row(kv[0, i], synth.KV_FP8_656)
        assert np.array_equal(out[0, i, 0], ref[:512])


def test_lse_one_hot_probe_bit_exact():
    """q one-hot at RoPE dim h with scale 1 and one key: lse == K[512+h] exactly."""
    w = synth.make_workload("t", batch=1, h_q=64, s_q=1, seqlens=[100], seed=40)  # every row filled
    w.topk = 1
    q = np.zeros_like(w.q)
    for h in range(64):
        q[0, 0, h, 512 + h] = 0x3F80  # bf16 1.0
    w.q = q
    w.indices = np.array([[[77]]], dtype=np.int32)
    out, lse = run(w, softmax_scale=1.0)
    page = w.block_table[0, 77 // 64]
    row = oracle.decode_row(w.kv[page, 77 % 64], 0)
    assert np.array_equal(lse[0, 0], row[512:576])


# --------------------------------------------------------- invariances ---

@pytest.mark.parametrize("kv_format", [synth.KV_BF16, synth.KV_FP8_656])
def test_page_permutation_bit_identical(kv_format):
    w = synth.make_workload("t", batch=3, h_q=128, s_q=2, seqlens=[300, 64, 129], seed=41,
                            kv_format=kv_format, is_causal=1)
    out1, lse1 = run(w)
    perm = np.random.default_rng(5).permutation(w.num_pages)
    kv2 = np.empty_like(w.kv)
    kv2[perm] = w.kv
    w.block_table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    w.kv = kv2
    out2, lse2 = run(w)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


def test_repeat_runs_bit_identical():
    w = synth.config_workload(2, batch=4)
    t = to_device(w)
    a = run(w, tensors=t)
    b = run(w, tensors=t)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("n", [2, 4, 5])
def test_metadata_matches_cpu_reference(n):
    w = synth.config_workload(n, batch=16)
    out, lse, sched, splits, parts = run(w, return_meta=True)
    nb = blocks_per_unit(w.cache_seqlens, w.s_q, w.topk)
    ref_sched, ref_splits = schedule(nb, parts, int(sched[6]))
    assert np.array_equal(sched.reshape(parts, 8), np.array(ref_sched, dtype=np.int32))
    assert np.array_equal(splits, np.array(ref_splits, dtype=np.int32))


@pytest.mark.parametrize("kv_format,topk", [(synth.KV_BF16, 0), (synth.KV_FP8_656, 0),
                                            (synth.KV_BF16, 200), (synth.KV_FP8_656, 200)])
def test_restart_pass_growing_scores(kv_format, topk):
    """Scores that climb by far more than the restart margin along the
    sequence (~370 in log2 units) send the main kernel's workgroups through a
    second pass against the exact row maxima, on every instance (bf16 and FP8,
    dense and sparse); results must still match the oracle."""
    L = 640
    w = synth.make_workload("t", batch=2, h_q=128, s_q=1, seqlens=[L, 300], seed=42, slack=0,
                            kv_format=kv_format, topk=topk)
    kv = w.kv.copy()
    for b in range(2):
        for t in range(int(w.cache_seqlens[b])):
            page, slot = w.block_table[b, t // 64], t % 64
            x = np.full(576, 0.05 * t, dtype=np.float32)  # scores grow ~ linearly in t
            x[:512] += np.float32(np.sin(t))
            bits = synth.bf16_bits_from_f32(x)
            kv[page, slot] = (bits.view(np.uint8) if kv_format == synth.KV_BF16
                              else synth.encode_fp8_rows(bits[None])[0])
    w.kv = kv
    if topk:
        w.indices = np.sort(w.indices, axis=-1)  # ascending positions: the scores climb tile by tile
    q = np.full(w.q.shape, 0x3F80, dtype=np.uint16)  # all-ones queries
    w.q = q
    for parts in (None, 3):
        out, lse = run(w, num_parts=parts, softmax_scale=0.02)
        ref_out, ref_lse = oracle.mla_decode(w, softmax_scale=0.02)
        assert_close(out, lse, ref_out, ref_lse, what=f"restart fmt={kv_format} topk={topk} parts={parts}")


def test_check_inputs_finds_bad_lengths_and_pages():
    """The device-side check flags lengths outside [0, max_pages * 64] and
    reachable block-table entries outside the pool, and nothing else."""
    w = synth.make_workload("t", batch=6, h_q=16, s_q=1, seqlens=[100, 0, 64, 300, 1, 129], seed=45,
                            max_pages_per_seq=6)
    p = mla.Problem.make(batch=w.batch, s_q=1, h_q=16, num_pages=w.num_pages,
                         max_pages_per_seq=w.max_pages_per_seq, softmax_scale=w.softmax_scale)
    _, _, bt, sl, _ = to_device(w)
    assert mla.mla_decode_check_inputs(p, bt, sl) == (0, -1)
    bt_bad = w.block_table.copy()
    bt_bad[3, 4] = w.num_pages         # reachable page (L = 300 uses pages 0..4): bad
    bt_bad[0, 5] = -7                  # unreachable slot (L = 100 uses pages 0..1): ignored
    sl_bad = w.cache_seqlens.copy()
    sl_bad[5] = 6 * 64 + 1             # longer than the table row allows
    sl_bad[1] = -1
    n, first = mla.mla_decode_check_inputs(p, torch.from_numpy(bt_bad).cuda(),
                                           torch.from_numpy(sl_bad).cuda())
    assert (n, first) == (3, 1)


@pytest.mark.parametrize("seed", range(10))
def test_metadata_random_shapes(seed):
    """The scheduler alone, bit for bit against the CPU mirror, over random
    shapes: dense and sparse units, empty sequences, more parts than blocks,
    and unit counts above the 1024 threads of the metadata workgroup."""
    rng = np.random.default_rng(700 + seed)
    sparse = seed % 3 == 2
    s_q = int(rng.integers(1, 4))
    if seed < 6:
        batch, parts = int(rng.integers(1, 300)), int(rng.integers(1, 3000))
    else:
        units, parts = int(rng.integers(1025, 5000)), int(rng.integers(1, 400))
        batch = units // s_q if sparse else units
    mp = int(rng.integers(1, 40))
    topk = int(rng.integers(1, 64 * mp + 1)) if sparse else 0
    seqlens = rng.integers(0, 64 * mp + 1, size=batch).astype(np.int32)
    seqlens[rng.random(batch) < 0.2] = 0
    p = mla.Problem.make(batch=batch, s_q=s_q, h_q=64, num_pages=batch * mp, max_pages_per_seq=mp,
                         softmax_scale=0.05, topk=topk,
                         kv_format=synth.KV_FP8_656 if sparse else synth.KV_BF16)
    n_sched, n_splits = mla.mla_decode_metadata_size(p, parts)
    sched = torch.full((n_sched,), -7, dtype=torch.int32, device="cuda")
    splits = torch.full((n_splits,), -7, dtype=torch.int32, device="cuda")
    print(f"seed {seed}: units {mla.mla_decode_num_units(p)} parts {parts} topk {topk}", flush=True)
    mla.mla_decode_get_metadata(p, torch.from_numpy(seqlens).cuda(), parts, sched, splits)
    got_sched, got_splits = sched.cpu().numpy(), splits.cpu().numpy()
    nb = blocks_per_unit(seqlens, s_q, topk)
    ref_sched, ref_splits = schedule(nb, parts, int(got_sched[6]))
    assert np.array_equal(got_sched.reshape(parts, 8), np.array(ref_sched, dtype=np.int32))
    assert np.array_equal(got_splits, np.array(ref_splits, dtype=np.int32))
