"""Bit-exact pins of the FP8 K dequantisation on the GPU, one per kernel that
dequantises K: the small-head kernel (in registers), the main kernel
(dense and sparse, into the bf16 tile).

One key per sequence and one-hot queries make each head's score a single
dequantised K element, and its base-2 LSE (softmax scale 1) that element
itself: every head's LSE must equal the oracle's bf16(float(code) * tile
scale), the 656-byte row's rule ("为什么 FlashMLA 的解码内核能跑到 660
TFLOPS", section 设计 2), bit for bit, for every finite e4m3 code
(subnormals and negative zero included) in every 128-dim tile.  The output
of a one-key sequence must be the dequantised V row."""

import numpy as np
import pytest

import oracle
import synth
from tests.harness import run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("h_q,topk", [(16, 0), (128, 0), (128, 1)],
                         ids=["small-head", "main-dense", "main-sparse"])
def test_fp8_scores_dequantise_exactly(h_q, topk):
    rng = np.random.default_rng(76 + h_q + topk)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    combos = [(int(c), t) for c in codes for t in range(4)]
    rng.shuffle(combos)
    H = h_q
    B = -(-len(combos) // H)
    w = synth.make_workload(f"fp8_exact_scores_h{h_q}_k{topk}", batch=B, h_q=H, s_q=1, seqlens=[1] * B,
                            seed=77, kv_format=synth.KV_FP8_656, softmax_scale=1.0, topk=topk)
    q = np.zeros(w.q.shape, dtype=np.uint16)
    pos = np.zeros((B, H), dtype=np.int64)
    for b in range(B):
        row = np.empty(656, dtype=np.uint8)
        row[:512] = rng.choice(codes, size=512)
        scales = (np.exp2(rng.integers(-60, 61, size=4)) * rng.uniform(1, 2, size=4)).astype(np.float32)
        row[512:528] = scales.view(np.uint8)
        row[528:] = synth.bf16_bits_from_f32(rng.standard_normal(64).astype(np.float32)).view(np.uint8)
        cols = rng.permutation(128)  # distinct columns, so distinct positions
        for h in range(H):
            c, t = combos[(b * H + h) % len(combos)]
            pos[b, h] = 128 * t + int(cols[h])
            row[pos[b, h]] = c
            q[b, 0, h, pos[b, h]] = 0x3F80  # 1.0
        w.kv[w.block_table[b, 0], 0] = row
    w.q = q
    print(f"h_q {h_q} topk {topk}: {B} one-key sequences", flush=True)
    out, lse = run(w)
    expect = np.zeros((B, 1, H), dtype=np.float32)
    for b in range(B):
        row = oracle.decode_row(w.kv[w.block_table[b, 0], 0], synth.KV_FP8_656)
        # + 0: a zero element gives +0 in the fp32 accumulator
        expect[b, 0] = row[pos[b]].astype(np.float32) + np.float32(0.0)
        assert np.array_equal(out[b, 0], np.broadcast_to(row[:512], (H, 512))), b
    bad = np.argwhere(lse.view(np.uint32) != expect.view(np.uint32))
    if len(bad):
        b, _, h = bad[0]
        raise AssertionError(f"{len(bad)} heads differ; first b={b} h={h} pos={pos[b, h]}: "
                             f"gpu {lse[b, 0, h]!r} expected {expect[b, 0, h]!r}")
