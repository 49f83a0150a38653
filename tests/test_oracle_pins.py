"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test ties one part of the oracle to something other than its own code:
a library routine (torch's float8/bf16 casts, scaled_dot_product_attention in
float64), a closed form, an invariance, brute force on tiny inputs, or a
figure printed on the pages (tests/golden/page_figures.json).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


# ---------------------------------------------------------------- numerics ---

def test_e4m3_all_codes_match_torch():
    """All 256 e4m3fn codes decode as torch's float8_e4m3fn does."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert nan.sum() == 2  # 0x7F and 0xFF only: e4m3fn has no infinities
    assert np.array_equal(ref[~nan], ours[~nan])
    # fixed points of the format: max 448, smallest subnormal 2^-9, one
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x38] == 1.0


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    # force exact ties and near-ties at the bf16 boundary
    bits[:2000] = (bits[:2000] & 0xFFFF0000) | 0x8000
    bits[2000:4000] = (bits[2000:4000] & 0xFFFF0000) | 0x7FFF
    x = bits.view(np.float32)
    finite = np.isfinite(x)
    x = x[finite]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = np.array([oracle.bf16_round(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(ref, ours)


def test_fp8_row_decode_matches_library_dequant():
    """656-byte row: codes times the tile's fp32 scale, rounded once to bf16
    (torch's float8 and bf16 casts); RoPE bf16 passes through."""
    w = synth.make_workload("t", batch=1, h_q=1, s_q=1, seqlens=[64], seed=3,
                            kv_format=synth.KV_FP8_656, slack=0)
    for slot in (0, 17, 63):
        row = w.kv[w.block_table[0, 0], slot]
        codes = torch.from_numpy(row[:512].copy()).view(torch.float8_e4m3fn).float()
        scales = torch.from_numpy(row[512:528].copy().view(np.float32))
        ref = (codes.view(4, 128) * scales[:, None]).reshape(512).to(torch.bfloat16).float().numpy()
        rope = (row[528:656].copy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
        got = oracle.decode_row(row, synth.KV_FP8_656)
        assert np.array_equal(got[:512], ref)
        assert np.array_equal(got[512:], rope)


def test_fp8_row_zero_tile():
    row = np.zeros(656, dtype=np.uint8)
    rope_bits = (np.full(64, 1.5, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    row[528:] = rope_bits.view(np.uint8)
    got = oracle.decode_row(row, synth.KV_FP8_656)
    assert np.all(got[:512] == 0) and np.all(got[512:] == 1.5)


# -------------------------------------------------- attention: brute force ---

def _logical_rows(w, b):
    """Dequantised logical rows 0..L_b-1 of sequence b, gathered by the test
    itself with numpy fancy indexing (t // ps, t % ps)."""
    L = int(w.cache_seqlens[b])
    t = np.arange(L)
    rows = w.kv[w.block_table[b, t // w.page_size], t % w.page_size]
    return np.stack([oracle.decode_row(r, w.kv_format) for r in rows]) if L else np.zeros((0, 576), np.float32)


def _sdpa(q, K, scale, natural, mask=None):
    """torch SDPA in float64 with V = K[:, :512]; base 2 = natural with scale*ln2."""
    qt = torch.from_numpy(q.astype(np.float64))[None]  # [1, H, 576]
    Kt = torch.from_numpy(K.astype(np.float64))[None]
    Vt = Kt[..., :512].contiguous()
    s = float(scale) if natural else float(scale) * math.log(2.0)
    am = None if mask is None else torch.from_numpy(mask)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=am, scale=s)
    logits = (qt @ Kt.transpose(-1, -2)) * s
    if am is not None:
        logits = logits.masked_fill(~am, float("-inf"))
    lse = torch.logsumexp(logits, dim=-1)
    if not natural:
        lse = lse / math.log(2.0)
    return o[0].numpy(), lse[0].numpy()


def _q64(w):
    return (w.q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("kv_format", [synth.KV_BF16, synth.KV_FP8_656])
@pytest.mark.parametrize("natural", [False, True])
@pytest.mark.parametrize("page_size", [16, 64])
def test_dense_matches_sdpa(kv_format, natural, page_size):
    w = synth.make_workload("t", batch=3, h_q=4, s_q=1, seqlens=[1, 63, 130], seed=11,
                            kv_format=kv_format, page_size=page_size)
    out, lse = oracle.mla_decode(w, natural=natural)
    q = _q64(w)
    for b in range(w.batch):
        K = _logical_rows(w, b)
        o_ref, l_ref = _sdpa(q[b, 0], K, np.float32(w.softmax_scale), natural)
        np.testing.assert_allclose(out[b, 0], o_ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[b, 0], l_ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("s_q", [2, 3])
def test_causal_matches_masked_sdpa(s_q):
    w = synth.make_workload("t", batch=2, h_q=3, s_q=s_q, seqlens=[5, 70], seed=12, is_causal=1)
    out, lse = oracle.mla_decode(w)
    q = _q64(w)
    for b in range(w.batch):
        K = _logical_rows(w, b)
        L = K.shape[0]
        for i in range(s_q):
            mask = np.broadcast_to(np.arange(L)[None, :] <= L - s_q + i, (3, L)).copy()
            o_ref, l_ref = _sdpa(q[b, i], K, np.float32(w.softmax_scale), False, mask=mask)
            np.testing.assert_allclose(out[b, i], o_ref, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse[b, i], l_ref, rtol=1e-12, atol=1e-12)


def test_brute_force_numpy_tiny():
    """Materialise every score and weight in numpy fp64 (tiny sizes)."""
    w = synth.make_workload("t", batch=2, h_q=2, s_q=2, seqlens=[3, 9], seed=13, page_size=4,
                            is_causal=1)
    out, lse = oracle.mla_decode(w)
    q = _q64(w)
    for b in range(2):
        K = _logical_rows(w, b).astype(np.float64)
        L = K.shape[0]
        for i in range(2):
            for h in range(2):
                vis = [t for t in range(L) if t <= L - 2 + i]
                P = np.array([np.float64(np.float32(w.softmax_scale)) * sum(q[b, i, h, d] * K[t, d] for d in range(576)) for t in vis])
                l2 = np.log2(np.sum(2.0 ** P))
                o = sum((2.0 ** (P[k] - l2)) * K[t, :512] for k, t in enumerate(vis))
                assert abs(lse[b, i, h] - l2) < 1e-12
                np.testing.assert_allclose(out[b, i, h], o, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------- closed forms ---

def test_single_key_closed_form():
    w = synth.make_workload("t", batch=1, h_q=4, s_q=1, seqlens=[1], seed=14)
    out, lse = oracle.mla_decode(w)
    K = _logical_rows(w, 0)
    q = _q64(w)[0, 0]
    assert np.array_equal(out[0, 0], np.broadcast_to(K[0, :512].astype(np.float64), (4, 512)))
    P = (q @ K[0].astype(np.float64)) * np.float64(np.float32(w.softmax_scale))
    np.testing.assert_allclose(lse[0, 0], P, rtol=1e-13)


def test_zero_scale_is_mean_and_log2_length():
    w = synth.make_workload("t", batch=1, h_q=2, s_q=1, seqlens=[37], seed=15)
    out, lse = oracle.mla_decode(w, softmax_scale=0.0)
    K = _logical_rows(w, 0).astype(np.float64)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(K[:, :512].mean(0), (2, 512)), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], math.log2(37), rtol=1e-14)


def test_identical_rows_closed_form():
    w = synth.make_workload("t", batch=1, h_q=2, s_q=1, seqlens=[50], seed=16, slack=0)
    kv = w.kv.copy()
    first = kv[w.block_table[0, 0], 0].copy()
    kv[:, :, :] = first  # every row (all pages, all slots) identical
    out, lse = oracle.mla_decode(w, kv=kv)
    K0 = oracle.decode_row(first, 0).astype(np.float64)
    P = (_q64(w)[0, 0] @ K0) * np.float64(np.float32(w.softmax_scale))
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(K0[:512], (2, 512)), rtol=1e-13)
    np.testing.assert_allclose(lse[0, 0], P + math.log2(50), rtol=1e-13)


def test_two_keys_weight():
    w = synth.make_workload("t", batch=1, h_q=1, s_q=1, seqlens=[2], seed=17)
    out, lse = oracle.mla_decode(w)
    K = _logical_rows(w, 0).astype(np.float64)
    s = np.float64(np.float32(w.softmax_scale))
    P0, P1 = (_q64(w)[0, 0, 0] @ K.T) * s
    w0 = 1.0 / (1.0 + 2.0 ** (P1 - P0))
    np.testing.assert_allclose(out[0, 0, 0], w0 * K[0, :512] + (1 - w0) * K[1, :512], rtol=1e-12, atol=1e-14)


def test_empty_sequence():
    w = synth.make_workload("t", batch=2, h_q=2, s_q=2, seqlens=[0, 3], seed=18, is_causal=1)
    out, lse = oracle.mla_decode(w)
    assert np.all(lse[0] == -np.inf) and np.all(out[0] == 0)
    # causal with L=3, s_q=2: query 0 sees 2 keys, query 1 sees 3
    assert np.all(np.isfinite(lse[1]))


def test_causal_shorter_query_sees_fewer_keys():
    """Causal s_q=2 equals two non-causal calls with L-1 and L keys."""
    w = synth.make_workload("t", batch=2, h_q=3, s_q=2, seqlens=[65, 128], seed=19, is_causal=1)
    out, lse = oracle.mla_decode(w)
    for i, shift in ((0, 1), (1, 0)):
        qi = np.ascontiguousarray(w.q[:, i:i + 1])
        o1, l1 = oracle.mla_decode(w, q=qi, is_causal=0, cache_seqlens=w.cache_seqlens - shift)
        assert np.array_equal(out[:, i], o1[:, 0]) and np.array_equal(lse[:, i], l1[:, 0])


# ----------------------------------------------------------- invariances ---

@pytest.mark.parametrize("kv_format", [synth.KV_BF16, synth.KV_FP8_656])
def test_page_permutation_bit_identical_and_poison_unread(kv_format):
    w = synth.make_workload("t", batch=3, h_q=4, s_q=2, seqlens=[64, 100, 200], seed=20,
                            kv_format=kv_format)
    out, lse = oracle.mla_decode(w)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))  # poisoned tails never read
    rng = np.random.default_rng(0)
    perm = rng.permutation(w.num_pages)  # new physical position of each page
    kv2 = np.empty_like(w.kv)
    kv2[perm] = w.kv
    bt2 = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    out2, lse2 = oracle.mla_decode(w, kv=kv2, block_table=bt2)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("n", [2, 3, 7, 100])
def test_split_merge_invariance(n):
    w = synth.make_workload("t", batch=2, h_q=4, s_q=2, seqlens=[100, 33], seed=21, is_causal=1)
    out, lse = oracle.mla_decode(w)
    out2, lse2 = oracle.mla_decode(w, n_splits=n)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-12, atol=1e-12)


def test_sparse_arange_equals_dense():
    w = synth.make_workload("t", batch=2, h_q=4, s_q=2, seqlens=[70, 129], seed=22)
    dense, dl = oracle.mla_decode(w)
    L = int(w.cache_seqlens.max())
    idx = np.full((2, 2, L), -1, dtype=np.int32)
    for b in range(2):
        idx[b, :, :w.cache_seqlens[b]] = np.arange(w.cache_seqlens[b])
    sp, sl = oracle.mla_decode(w, indices=idx, topk=L)
    assert np.array_equal(sp, dense) and np.array_equal(sl, dl)


def test_sparse_invalid_entries_are_skipped_and_order_free():
    w = synth.make_workload("t", batch=1, h_q=4, s_q=2, seqlens=[300], seed=23,
                            kv_format=synth.KV_FP8_656, topk=40)
    base, bl = oracle.mla_decode(w)
    idx = w.indices
    noisy = np.concatenate([idx, np.full((1, 2, 5), -1, np.int32),
                            np.full((1, 2, 3), 300, np.int32), np.full((1, 2, 2), 10 ** 6, np.int32)], axis=2)
    rng = np.random.default_rng(1)
    noisy = np.ascontiguousarray(noisy[:, :, rng.permutation(noisy.shape[2])])
    o2, l2 = oracle.mla_decode(w, indices=noisy, topk=noisy.shape[2])
    np.testing.assert_allclose(o2, base, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l2, bl, rtol=1e-12, atol=1e-12)
    allbad = np.full((1, 2, 4), -1, np.int32)
    o3, l3 = oracle.mla_decode(w, indices=allbad, topk=4)
    assert np.all(l3 == -np.inf) and np.all(o3 == 0)


def test_sparse_duplicate_doubles_weight():
    """Keys {a, a, b}: weight of a is 2*2^Pa / (2*2^Pa + 2^Pb)."""
    w = synth.make_workload("t", batch=1, h_q=1, s_q=1, seqlens=[10], seed=24)
    idx = np.array([[[3, 3, 7]]], dtype=np.int32)
    out, lse = oracle.mla_decode(w, indices=idx, topk=3)
    K = _logical_rows(w, 0).astype(np.float64)
    s = np.float64(np.float32(w.softmax_scale))
    Pa, Pb = (_q64(w)[0, 0, 0] @ K[[3, 7]].T) * s
    wa = 2 * 2.0 ** Pa / (2 * 2.0 ** Pa + 2.0 ** Pb)
    np.testing.assert_allclose(out[0, 0, 0], wa * K[3, :512] + (1 - wa) * K[7, :512], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0, 0], math.log2(2 * 2.0 ** Pa + 2.0 ** Pb), rtol=1e-13)


def test_unit_mask_computes_subset_only():
    w = synth.make_workload("t", batch=3, h_q=2, s_q=2, seqlens=[10, 20, 30], seed=25)
    full, fl = oracle.mla_decode(w)
    m = np.array([0, 1, 0, 0, 1, 1], dtype=np.uint8)
    part, pl = oracle.mla_decode(w, unit_mask=m)
    mm = m.reshape(3, 2).astype(bool)
    assert np.array_equal(part[mm], full[mm]) and np.all(np.isnan(part[~mm]))


# ------------------------------------------------ figures on the pages ---

def test_page_figures_pin_layout_and_flop_model():
    g = json.load(open(GOLDEN))
    f8 = g["fp8_token_bytes"]
    assert synth.ROW_BYTES_FP8 == f8["value"] == sum(f8["parts"].values())
    assert synth.ROW_BYTES_BF16 == g["bf16_token_bytes"]["value"]
    assert round(100 * (1 - synth.ROW_BYTES_FP8 / synth.ROW_BYTES_BF16)) == g["fp8_saving_percent"]["value"]
    fac = g["kv_bytes_per_128k_request_bf16"]
    assert fac["factors"][0] == synth.D_QK
    assert round(np.prod(fac["factors"], dtype=np.float64) / 2 ** 30, 2) == fac["gib"]
    shape = g["mla_shape"]
    assert (synth.D_QK, synth.D_V, synth.D_ROPE) == (shape["d_qk"], shape["d_v"], shape["rope_dims"])
    # FLOP model: flops / bytes ~ 2*h_q*s_q when d_v ~ d_k (only KV bytes counted)
    w = synth.make_workload("t", batch=1, h_q=128, s_q=1, seqlens=[4096], seed=1)
    kv_bytes = 4096 * synth.ROW_BYTES_BF16
    ratio = w.flops() / kv_bytes
    assert abs(ratio - 128 * (576 + 512) / 576) < 1e-9
    im = g["intensity_model"]
    assert im["h800_ridge_flop_per_byte"] // 2 == im["compute_bound_threshold_hq_sq"] + 1
    assert g["e4m3_format"]["exponent_bits"] == 4 and g["e4m3_format"]["mantissa_bits"] == 3
    # natural exp overflow point quoted for float32
    x = g["fp32_exp_overflow"]["value"]
    with np.errstate(over="ignore"):
        assert np.isfinite(np.exp(np.float32(x - 1e-5), dtype=np.float32))
        assert np.isinf(np.exp(np.float32(x + 1e-4), dtype=np.float32))


# ------------------------------------------------ FP8 writer (quantiser) ---

def test_e4m3_encode_exact_codes_round_trip():
    """Every finite code's value encodes back to that code (both signs)."""
    for c in range(0x7F):
        v = oracle.e4m3_value(c)
        assert oracle.e4m3_encode(v) == c, hex(c)
        assert oracle.e4m3_encode(-v) == (c | 0x80), hex(c)


def test_e4m3_encode_midpoints_go_to_even_and_saturate():
    """Halfway between neighbouring codes the even code wins; beyond 448 the
    code saturates (e4m3fn has no infinity and 0x7F is NaN)."""
    for c in range(0x7E):
        lo, hi = oracle.e4m3_value(c), oracle.e4m3_value(c + 1)
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2  # the midpoint is exact in float
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(float(mid)) == want, hex(c)
        # just off the midpoint rounds to the nearer code
        assert oracle.e4m3_encode(float(np.nextafter(mid, np.float32(0)))) == c
        assert oracle.e4m3_encode(float(np.nextafter(mid, np.float32(1e9)))) == c + 1
    for v in (448.0, 449.0, 464.0, 500.0, 1e30):
        assert oracle.e4m3_encode(v) == 0x7E and oracle.e4m3_encode(-v) == 0xFE


def test_e4m3_encode_matches_torch_cast():
    """Library pin: torch's float8_e4m3fn cast (round to nearest even) agrees
    on random values across the whole range, subnormals included."""
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-0.02, 0.02, 20000),
                        np.ldexp(rng.uniform(-1, 1, 5000), rng.integers(-12, 9, 5000))]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v)) for v in x], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_quantize_row_closed_form():
    """Tile maxima 3.5, 0, 448 and 1e-3: scale = amax / 448; with amax = 3.5
    the scale is exactly 2^-7, so a value x encodes as x * 128."""
    row = np.zeros(576, dtype=np.float32)
    row[0:128] = np.linspace(-3.5, 3.5, 128)
    row[5] = 1.0
    row[256:384] = np.linspace(-448, 448, 128)
    row[384:512] = 1e-3
    row[512:] = np.arange(64) - 32
    bits = synth.bf16_bits_from_f32(row)
    out = oracle.quantize_row_fp8(bits)
    scales = out[512:528].view(np.float32)
    x = synth.bf16_bits_to_f32(bits)
    assert scales[0] == np.float32(np.abs(x[0:128]).max()) / np.float32(448.0) == np.float32(2.0 ** -7)
    assert scales[1] == 0.0 and np.all(out[128:256] == 0)
    assert scales[2] == np.float32(1.0)
    assert out[5] == 0x70  # 1.0 * 128 = 2^7: exponent field 14, mantissa 0
    assert out[256] == 0xFE and out[383] == 0x7E  # -448 and 448
    assert np.array_equal(out[528:].view(np.uint16), bits[512:])  # RoPE copied


def test_quantize_row_matches_input_generator():
    """The input generator's encoding (numpy float32 divisions + torch's
    cast) and the oracle's quantiser agree byte for byte."""
    rng = np.random.default_rng(11)
    rows = synth.bf16_bits_from_f32((rng.standard_normal((64, 576)) * rng.uniform(0.01, 100, (64, 1))).astype(np.float32))
    rows[3, 0:128] = 0  # an all-zero tile
    rows[4, 128:256] = 0x8000  # negative zeros
    ref = synth.encode_fp8_rows(rows)
    got = np.stack([oracle.quantize_row_fp8(r) for r in rows])
    assert np.array_equal(got, ref)


def test_kv_append_places_rows_through_block_table():
    """Appended tokens land at slot t mod 64 of page block_table[b][t div 64];
    decoding them through the block table gives the dequantised rows; every
    other byte of the pool is untouched; out-of-range positions are skipped."""
    rng = np.random.default_rng(3)
    B, n_new, pages_per_seq = 3, 70, 4
    num_pages = B * pages_per_seq + 2
    perm = rng.permutation(num_pages)[:B * pages_per_seq].reshape(B, pages_per_seq).astype(np.int32)
    start = np.array([0, 60, 250], dtype=np.int32)  # the last sequence runs past its 4 pages
    new = synth.bf16_bits_from_f32(rng.standard_normal((B, n_new, 576)).astype(np.float32))
    pool0 = rng.integers(0, 256, (num_pages, 64, 656), dtype=np.uint8)
    pool = oracle.kv_append_fp8(new, start, perm, pool0)
    written = np.zeros(pool.shape[:2], dtype=bool)
    for b in range(B):
        for j in range(n_new):
            t = start[b] + j
            if t // 64 >= pages_per_seq:
                continue
            page, slot = perm[b, t // 64], t % 64
            written[page, slot] = True
            assert np.array_equal(pool[page, slot], oracle.quantize_row_fp8(new[b, j]))
    assert np.array_equal(pool[~written], pool0[~written])
    assert written.sum() == 70 + 70 + (256 - 250)
