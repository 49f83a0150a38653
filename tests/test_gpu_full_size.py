"""GPU parity at the full benchmark workloads, in the launch configuration
the benchmark times (default plan: one workgroup per CU), checked on a
seeded sample of query tokens that the oracle computes one by one.  The
last query token of the batch is always in the sample: its unit closes the
schedule's last part."""

import numpy as np
import pytest

import oracle
import synth
from tests.harness import assert_close, run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,sample", [(2, 8), (3, 6), (4, 3), (5, 8)])
def test_full_size_sampled(n, sample):
    w = synth.config_workload(n)
    tokens = w.batch * w.s_q
    rng = np.random.default_rng(4242 + n)
    pick = np.union1d(rng.choice(tokens, size=sample, replace=False), [tokens - 1])
    mask = np.zeros(tokens, dtype=np.uint8)
    mask[pick] = 1
    print(f"config {n} ({w.name}): query tokens {pick.tolist()} of {tokens}", flush=True)
    out, lse = run(w)
    ref_out, ref_lse = oracle.mla_decode(w, unit_mask=mask)
    sel = mask.reshape(w.batch, w.s_q).astype(bool)
    err, bound = assert_close(out, lse, ref_out, ref_lse, mask=sel, what=f"config {n} full size")
    print(f"config {n}: max |out - ref| {err:.3g} (bound {bound:.3g})", flush=True)
    # every output row of the workload is finite, sampled or not
    assert np.all(np.isfinite(out)), f"config {n}: non-finite output outside the sample"
