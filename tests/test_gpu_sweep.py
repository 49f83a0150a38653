"""GPU parity over a seeded random sweep of shapes: batch, heads, query
tokens, lengths (zero, ragged, past a page), cache format, causal or sparse
(top-k, with invalid entries) and forced split counts, each case against the
oracle at the stated tolerance.  The cases cross every dispatch boundary of
the decode entry point: the small-head kernel (up to 32 rows
per unit), the main kernel with one or several 128-row groups, dense and
sparse."""

import numpy as np
import pytest

import oracle
import synth
from tests.harness import assert_close, run

pytestmark = pytest.mark.gpu

N_CASES = 80


def sweep_case(seed: int):
    rng = np.random.default_rng(10_000 + seed)
    batch = int(rng.integers(1, 7))
    h_q = int(rng.choice([1, 2, 5, 8, 16, 20, 32, 48, 64, 100, 128]))
    s_q = int(rng.choice([1, 1, 2, 3, 4]))
    kv_format = int(rng.choice([synth.KV_BF16, synth.KV_FP8_656]))
    sparse = rng.random() < 0.3
    if sparse:
        topk = int(rng.choice([1, 7, 64, 65, 130]))
        lens = rng.integers(topk, topk + 700, size=batch)
        causal = 0
    else:
        topk = 0
        lens = rng.integers(0, 1500, size=batch)
        lens[rng.random(batch) < 0.15] = 0
        causal = int(rng.random() < 0.5)
    parts = [None, None, 1, 3, 17, 300][int(rng.integers(0, 6))]
    return dict(batch=batch, h_q=h_q, s_q=s_q, kv_format=kv_format, topk=topk, causal=causal,
                seqlens=[int(x) for x in lens], parts=parts, invalid=sparse and rng.random() < 0.5)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape_parity(seed):
    c = sweep_case(seed)
    print(f"sweep {seed}: {c}", flush=True)
    w = synth.make_workload(f"sweep_{seed}", batch=c["batch"], h_q=c["h_q"], s_q=c["s_q"],
                            seqlens=c["seqlens"], seed=20_000 + seed, kv_format=c["kv_format"],
                            topk=c["topk"], is_causal=c["causal"])
    if c["invalid"]:
        # some entries -1 or past the sequence end: skipped by both sides
        rng = np.random.default_rng(30_000 + seed)
        idx = w.indices
        hit = rng.random(idx.shape) < 0.2
        bad = np.where(rng.random(idx.shape) < 0.5, -1, w.cache_seqlens[:, None, None] + 3)
        w.indices = np.where(hit, bad, idx).astype(np.int32)
    out, lse = run(w, num_parts=c["parts"])
    ref_out, ref_lse = oracle.mla_decode(w)
    assert_close(out, lse, ref_out, ref_lse, what=f"sweep {seed} {c}")
