"""The sparse prefill oracle's pins catch plausible mistakes: each case
builds a copy of oracle/sparse_prefill.py with one planted mistake (a text
substitution, loaded as a separate module on the CPU), hands its
sparse_prefill to the pins of tests/test_prefill_oracle.py, and checks that
one of them fails."""

import os
import types

import pytest

import oracle
from tests import test_prefill_oracle as pins

SRC = os.path.join(os.path.dirname(os.path.abspath(oracle.__file__)), "sparse_prefill.py")

# name: (original text, planted mistake, the pin that must fail)
MUTANTS = {
    "negative indices not skipped": (
        "idx = idx[(idx >= 0) & (idx < s_kv)]", "idx = idx[idx < s_kv]",
        lambda: pins.test_prefill_matches_c_oracle_sparse_decode(0, False)),
    "duplicates counted once": (
        "idx = idx[(idx >= 0) & (idx < s_kv)]", "idx = np.unique(idx[(idx >= 0) & (idx < s_kv)])",
        lambda: pins.test_prefill_duplicate_index_adds_log2_of_two()),
    "natural log of a base-2 sum": (
        "lse_i = m[:, 0] + np.log2(np.exp2(P - m).sum(axis=1))",
        "lse_i = m[:, 0] + np.log(np.exp2(P - m).sum(axis=1))",
        lambda: pins.test_prefill_all_positions_matches_sdpa(False)),
    "softmax scale dropped": (
        "P = (Q[i] @ G.T) * scale", "P = (Q[i] @ G.T)",
        lambda: pins.test_prefill_all_positions_matches_sdpa(True)),
    "values from the last 512 dims": (
        "out[i] = S @ G[:, :D_V]", "out[i] = S @ G[:, 64:]",
        lambda: pins.test_prefill_single_index_returns_the_row()),
}


def module_copy(name, original=None, mistake=None):
    src = open(SRC).read()
    if original is not None:
        assert src.count(original) == 1, f"{name}: the text to change is not unique in the oracle"
        src = src.replace(original, mistake)
    mod = types.ModuleType("oracle._prefill_copy")
    mod.__package__ = "oracle"
    exec(compile(src, SRC, "exec"), mod.__dict__)
    return mod


def test_unmodified_copy_passes_every_pin_used(monkeypatch):
    monkeypatch.setattr(pins, "sparse_prefill", module_copy("unmodified").sparse_prefill)
    for _, _, pin in MUTANTS.values():
        pin()


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_is_caught(monkeypatch, name):
    original, mistake, pin = MUTANTS[name]
    monkeypatch.setattr(pins, "sparse_prefill", module_copy(name, original, mistake).sparse_prefill)
    with pytest.raises(AssertionError):
        pin()
