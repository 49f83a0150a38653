"""GPU parity at the full benchmark workloads, in the launch configuration
the benchmark times (default plan: one workgroup per CU).  Every query token
of every configuration is compared element by element with the oracle at the
stated tolerance (bf16 out within 1e-2 * max|ref| + 2e-3, lse within 1e-3)."""

import time

import numpy as np
import pytest

import oracle
import synth
from tests.harness import assert_close, run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_full_size_all_tokens(n):
    w = synth.config_workload(n)
    tokens = w.batch * w.s_q
    print(f"config {n} ({w.name}): {tokens} query tokens x {w.h_q} heads", flush=True)
    out, lse = run(w)
    t0 = time.perf_counter()
    ref_out, ref_lse = oracle.mla_decode(w)
    t_oracle = time.perf_counter() - t0
    err, bound = assert_close(out, lse, ref_out, ref_lse, what=f"config {n} full size")
    ninf = np.isneginf(ref_lse)
    lerr = float(np.abs(lse[~ninf] - ref_lse[~ninf]).max()) if (~ninf).any() else 0.0
    print(f"config {n}: all {tokens} query tokens: max |out - ref| {err:.3g} (bound {bound:.3g}), "
          f"max |lse - ref| {lerr:.3g}; oracle {t_oracle:.1f} s on {oracle.num_threads()} threads",
          flush=True)
    assert np.all(np.isfinite(out))
