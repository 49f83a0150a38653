"""GPU parity of decode at small head counts (h_q * s_q <= 64, dense, bf16
and FP8 caches): units of at most 32 rows (either format) run on
their own kernel, larger ones on the main kernel; row counts below and between 16-row blocks, causal rows, the restart pass, forced split counts, bit identity under page
permutation and across runs, and a seeded sample at the benchmark's size."""

import numpy as np
import pytest

import oracle
import synth
from tests.harness import assert_close, run, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("h_q,s_q,causal", [(1, 1, 0), (3, 1, 0), (4, 3, 1), (8, 2, 1), (16, 1, 0),
                                            (5, 3, 1), (16, 1, 1), (17, 1, 0), (16, 2, 1), (32, 1, 0),
                                            (11, 3, 1), (48, 1, 0), (16, 4, 1), (64, 1, 0), (21, 3, 1)])
@pytest.mark.parametrize("kv_format", [synth.KV_BF16, synth.KV_FP8_656])
def test_small_head_shapes(h_q, s_q, causal, kv_format):
    w = synth.make_workload("small", batch=5, h_q=h_q, s_q=s_q, seqlens=[1, 2, 64, 300, 1000],
                            seed=60 + h_q * 4 + s_q, is_causal=causal, kv_format=kv_format)
    print(f"h_q {h_q} s_q {s_q} causal {causal} kv_format {kv_format}", flush=True)
    out, lse = run(w)
    ref_out, ref_lse = oracle.mla_decode(w)
    assert_close(out, lse, ref_out, ref_lse, what=f"h_q={h_q} s_q={s_q} causal={causal} fmt={kv_format}")


@pytest.mark.parametrize("h_q,s_q,kv_format", [(16, 1, synth.KV_BF16), (40, 1, synth.KV_BF16),
                                              (16, 1, synth.KV_FP8_656), (8, 1, synth.KV_FP8_656),
                                              (32, 1, synth.KV_FP8_656), (16, 2, synth.KV_FP8_656)])
@pytest.mark.parametrize("parts", [1, 2, 5, 64, 700])
def test_small_heads_forced_splits(parts, h_q, s_q, kv_format):
    """Forced split counts on every small-head variant, including the FP8
    two-row-block one (17-32 rows)."""
    w = synth.make_workload("small_split", batch=6, h_q=h_q, s_q=s_q, seqlens=synth.Uniform(1, 3000),
                            seed=71, kv_format=kv_format, is_causal=int(s_q > 1))
    out, lse = run(w, num_parts=parts)
    ref_out, ref_lse = oracle.mla_decode(w)
    assert_close(out, lse, ref_out, ref_lse, what=f"parts={parts}")


@pytest.mark.parametrize("kv_format", [synth.KV_BF16, synth.KV_FP8_656])
@pytest.mark.parametrize("natural, scale", [(True, None), (False, -0.05), (False, 0.0)])
def test_small_heads_base_and_scale(natural, scale, kv_format):
    w = synth.make_workload("small_scale", batch=3, h_q=16, s_q=1, seqlens=[100, 700, 65], seed=72,
                            kv_format=kv_format)
    out, lse = run(w, natural=natural, softmax_scale=scale)
    ref_out, ref_lse = oracle.mla_decode(w, natural=natural, softmax_scale=scale)
    assert_close(out, lse, ref_out, ref_lse, what=f"natural={natural} scale={scale}")


@pytest.mark.parametrize("h_q,kv_format", [(16, synth.KV_BF16), (32, synth.KV_BF16),
                                          (128, synth.KV_BF16), (16, synth.KV_FP8_656),
                                          (32, synth.KV_FP8_656)])
def test_small_heads_growing_scores_rescale(h_q, kv_format):
    """Scores that climb by far more than any lag the running max may have
    (here by ~500 in log2 units over the sequence) force the recovery path:
    a second pass of the segment on the small-head kernel (h_q 16, 32) and
    on the main kernel (h_q 128)."""
    w = synth.make_workload("small_grow", batch=2, h_q=h_q, s_q=1, seqlens=[900, 300], seed=73,
                            slack=0, kv_format=kv_format)
    kv = w.kv.copy()
    for b in range(2):
        for t in range(int(w.cache_seqlens[b])):
            page, slot = w.block_table[b, t // 64], t % 64
            x = np.full(576, 0.05 * t, dtype=np.float32)
            x[:512] += np.float32(np.sin(t))
            bits = synth.bf16_bits_from_f32(x)
            kv[page, slot] = (bits.view(np.uint8) if kv_format == synth.KV_BF16
                              else synth.encode_fp8_rows(bits[None])[0])
    w.kv = kv
    w.q = np.full(w.q.shape, 0x3F80, dtype=np.uint16)
    for parts in (None, 3):
        out, lse = run(w, num_parts=parts, softmax_scale=0.02)
        ref_out, ref_lse = oracle.mla_decode(w, softmax_scale=0.02)
        assert_close(out, lse, ref_out, ref_lse, what=f"growing parts={parts}")


@pytest.mark.parametrize("h_q,s_q,kv_format", [(24, 2, synth.KV_BF16), (8, 2, synth.KV_FP8_656),
                                                (12, 2, synth.KV_FP8_656)])
def test_small_heads_bit_identity(h_q, s_q, kv_format):
    """Same results bit for bit across runs and after permuting the physical
    pages (the block table rewritten to match)."""
    w = synth.make_workload("small_bits", batch=4, h_q=h_q, s_q=s_q, seqlens=[700, 64, 129, 2000],
                            seed=74, is_causal=1, kv_format=kv_format)
    t = to_device(w)
    out1, lse1 = run(w, tensors=t)
    out2, lse2 = run(w, tensors=t)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)
    perm = np.random.default_rng(6).permutation(w.num_pages)
    kv2 = np.empty_like(w.kv)
    kv2[perm] = w.kv
    w.block_table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    w.kv = kv2
    out3, lse3 = run(w)
    assert np.array_equal(out1, out3) and np.array_equal(lse1, lse3)


@pytest.mark.parametrize("name,h_q,s_q,lo,hi,kv_format,seed,max_pages", [
    ("b128_h16_sq1", 16, 1, 1024, 8192, synth.KV_BF16, 1006, 128),
    ("b128_h16_sq1_fp8", 16, 1, 1024, 8192, synth.KV_FP8_656, 1007, 128),
    ("b128_h16_sq1_fp8_l8k_32k", 16, 1, 8192, 32768, synth.KV_FP8_656, 1008, 512),
    ("b128_h16_sq2_fp8_l8k_32k", 16, 2, 8192, 32768, synth.KV_FP8_656, 1009, 512),
])
def test_small_heads_full_size(name, h_q, s_q, lo, hi, kv_format, seed, max_pages):
    """The small-head benchmark shapes at batch 128 in the default launch
    configuration, every query row against the oracle: 16 heads over the bf16
    and FP8 caches (the FP8 one also at the benchmark's lengths U[8192,
    32768], same seed), and 16 heads x 2 causal query tokens over the FP8
    cache at lengths U[8192, 32768] (the two-row-block variant)."""
    w = synth.make_workload(name, batch=128, h_q=h_q, s_q=s_q, seqlens=synth.Uniform(lo, hi),
                            seed=seed, max_pages_per_seq=max_pages, kv_format=kv_format,
                            is_causal=int(s_q > 1))
    out, lse = run(w)
    ref_out, ref_lse = oracle.mla_decode(w)
    err, bound = assert_close(out, lse, ref_out, ref_lse, what=name)
    print(f"{name}: max |out - ref| {err:.3g} (bound {bound:.3g})", flush=True)
    assert np.isfinite(out).all() and np.isfinite(lse).all()


@pytest.mark.parametrize("kv_format", [synth.KV_BF16, synth.KV_FP8_656])
def test_small_heads_single_key_bit_exact(kv_format):
    """A one-token sequence: the weight is exactly 1, so every head's output
    is the dequantised latent row bit for bit (the FP8 dequantisation of the
    small-head kernel matches the oracle's codec)."""
    w = synth.make_workload("small_one", batch=3, h_q=16, s_q=1, seqlens=[1, 1, 1], seed=75,
                            kv_format=kv_format)
    out, lse = run(w)
    for b in range(3):
        row = oracle.decode_row(w.kv[w.block_table[b, 0], 0], kv_format)
        assert np.array_equal(out[b, 0], np.broadcast_to(row[:512], (16, 512))), b

