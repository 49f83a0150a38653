"""The decode oracle's pins catch plausible mistakes.  Each case compiles a
temporary copy of the C oracle with one planted mistake (a text substitution,
on the CPU), points the oracle module at that copy, and checks that a pin in
tests/test_oracle_pins.py fails.  The unmodified copy passes the same pins,
so a failure is the mistake's doing."""

import ctypes
import os
import subprocess

import pytest

import oracle
import synth
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.abspath(oracle.__file__)), "mla_oracle.c")

# name: (original text, planted mistake, the pin that must fail)
MUTANTS = {
    "scores without the RoPE dims": (
        "for (int d = 0; d < ORACLE_D_QK; ++d) acc += q[d] * (double)k[d];",
        "for (int d = 0; d < ORACLE_D_NOPE; ++d) acc += q[d] * (double)k[d];",
        lambda: pins.test_dense_matches_sdpa(synth.KV_BF16, False, 64)),
    "softmax scale dropped": (
        "p[t] = acc * scale;", "p[t] = acc;",
        lambda: pins.test_brute_force_numpy_tiny()),
    "natural exponent in the base-2 sum": (
        "sum += natural ? exp(p[t] - m) : exp2(p[t] - m);", "sum += exp(p[t] - m);",
        lambda: pins.test_two_keys_weight()),
    "values from the last 512 dims": (
        "out512[j] += w[t] * (double)k[j];", "out512[j] += w[t] * (double)k[j + 64];",
        lambda: pins.test_brute_force_numpy_tiny()),
    "causal window one key short": (
        "int last = is_causal ? L - s_q + i : L - 1;", "int last = is_causal ? L - s_q + i - 1 : L - 1;",
        lambda: pins.test_causal_matches_masked_sdpa(2)),
    "page and slot swapped": (
        "int lp = t / page_size, slot = t % page_size;", "int lp = t % page_size, slot = t / page_size;",
        lambda: pins.test_page_permutation_bit_identical_and_poison_unread(synth.KV_BF16)),
    "FP8 tile scale by the wrong index": (
        "float prod = v * scale[d / 128];", "float prod = v * scale[d % 4];",
        lambda: pins.test_fp8_row_decode_matches_library_dequant()),
    "e4m3 exponent bias 8": (
        "v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 8.0, e - 8);",
        lambda: pins.test_e4m3_all_codes_match_torch()),
    "bf16 by truncation": (
        "u += 0x7fffu + keep_lsb;", "u += 0u * keep_lsb;",
        lambda: pins.test_bf16_round_matches_torch()),
    "split results merged without renormalising": (
        "double wc = natural ? exp(part_l[c] - L2) : exp2(part_l[c] - L2);",
        "double wc = natural ? exp(part_l[c] - M) : exp2(part_l[c] - M);",
        lambda: pins.test_split_merge_invariance(3)),
    "sparse indices past the end kept": (
        "if (t >= 0 && t < L) vis[n++] = t;", "if (t >= 0) vis[n++] = t;",
        lambda: pins.test_sparse_invalid_entries_are_skipped_and_order_free()),
    "quantiser scale from 240": (
        "const float scale = amax / 448.0f;", "const float scale = amax / 240.0f;",
        lambda: pins.test_quantize_row_closed_form()),
    "append one slot late": (
        "uint8_t* row = kv_pool + ((long)page * page_size + t % page_size) * ORACLE_ROW_FP8;",
        "uint8_t* row = kv_pool + ((long)page * page_size + (t + 1) % page_size) * ORACLE_ROW_FP8;",
        lambda: pins.test_kv_append_places_rows_through_block_table()),
}


def compiled_copy(tmp_path, name, original=None, mistake=None):
    src = open(SRC).read()
    if original is not None:
        assert src.count(original) == 1, f"{name}: the text to change is not unique in the oracle"
        src = src.replace(original, mistake)
    c = tmp_path / "oracle_copy.c"
    so = tmp_path / "liboracle_copy.so"
    c.write_text(src)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(c), "-lm"])
    return oracle._declare(ctypes.CDLL(str(so)))


def test_unmodified_copy_passes_every_pin_used(tmp_path, monkeypatch):
    monkeypatch.setattr(oracle, "_lib", compiled_copy(tmp_path, "unmodified"))
    for _, _, pin in MUTANTS.values():
        pin()


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, monkeypatch, name):
    original, mistake, pin = MUTANTS[name]
    monkeypatch.setattr(oracle, "_lib", compiled_copy(tmp_path, name, original, mistake))
    with pytest.raises((AssertionError, ValueError)):
        pin()
