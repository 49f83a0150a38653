"""Many work units: the scheduler at and near its unit limit (16384 units,
more units than parts, several segments per part, per-thread scan chunks
of more than one unit) on both decode kernels, against the oracle."""

import numpy as np
import pytest

import oracle
import synth
from tests.harness import assert_close, run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,batch,h_q,lo,hi,seed", [
    ("max_units_small_heads", 16384, 16, 0, 40, 301),   # the unit limit, short ragged rows
    ("many_units_main_kernel", 2000, 128, 0, 300, 302),  # 2000 units over 256 parts
])
def test_many_units(name, batch, h_q, lo, hi, seed):
    w = synth.make_workload(name, batch=batch, h_q=h_q, s_q=1, seqlens=synth.Uniform(lo, hi), seed=seed)
    print(f"{name}: batch {batch}, h_q {h_q}, {int(w.cache_seqlens.sum())} tokens, "
          f"{int((w.cache_seqlens == 0).sum())} empty", flush=True)
    out, lse, sched, splits, parts = run(w, return_meta=True)
    assert splits[-1] >= np.count_nonzero(w.cache_seqlens)  # every non-empty unit has a segment
    ref_out, ref_lse = oracle.mla_decode(w)
    assert_close(out, lse, ref_out, ref_lse, what=name)
