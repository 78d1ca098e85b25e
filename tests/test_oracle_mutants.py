"""Planted mistakes in the oracle must each be rejected by some pin (CPU only).

Each mutant is the oracle's C source with one plausible mistake substituted
(a dropped term, a wrong index, a transposed operand, a swapped operand, a
wrong sign, a missing rounding, a wrong tie rule), compiled into a temporary
library.  All pins run against it, cheapest first, until one fails.  A
mutant that passes every pin means the pins leave that part of the oracle
unchecked.
"""
import os
import subprocess

import pytest

import oracle
import oracle_pins
from oracle import build as oracle_build

SOURCE = open(oracle_build.SOURCE).read()

# (name, text to find, replacement, occurrences to replace: 0 = all)
MUTANTS = [
    ("up_reads_gate_weights", "const uint16_t* urow = up_w + j * K;",
     "const uint16_t* urow = gate_w + j * K;", 0),
    ("gate_weight_transposed", "const double pg = hk * bf16_bits_to_double(grow[k]);",
     "const double pg = hk * bf16_bits_to_double(gate_w[k * N + j]);", 1),
    ("hidden_row_ignored", "const uint16_t* hrow = hidden + m * K;",
     "const uint16_t* hrow = hidden + 0 * K;", 0),
    ("first_term_dropped", "for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 1; k < K; ++k)", 0),
    ("exp_sign_flipped", "exp(-(double)g)", "exp((double)g)", 0),
    ("denominator_minus", "1.0f + e;", "1.0f - e;", 0),
    ("act_not_rounded",
     "uint16_t s_bits = rne_bf16_from_double((double)silu_f32(g));\n    float s = (float)bf16_bits_to_double(s_bits);",
     "float s = silu_f32(g);", 0),
    ("up_factor_missing", "volatile float p = s * u;", "volatile float p = s;", 0),
    ("gate_up_swapped", "out[idx] = glu_epilogue_one(g, u);", "out[idx] = glu_epilogue_one(u, g);", 0),
    ("ties_away_from_zero", "nearbyint(", "round(", 0),
    ("truncating_round", "nearbyint(", "trunc(", 0),
    ("subnormals_flushed", "(e < -126) ? -133 : e - 7", "(e < -126) ? -126 : e - 7", 0),
    ("overflow_threshold_off_by_one", "ldexp(1.0 - ldexp(1.0, -9), 128)", "ldexp(1.0 - ldexp(1.0, -9), 127)", 0),
    ("gate_not_rounded", "const uint16_t g = rne_bf16_from_double(G);",
     "const uint16_t g = float_bits_hi((float)G);", 0),
    ("linear_last_term_dropped", "for (int64_t kk = 0; kk < K; ++kk)", "for (int64_t kk = 0; kk + 1 < K; ++kk)", 0),
    ("linear_weight_row_shifted", "const uint16_t* wrow = w + (pos % N) * K;",
     "const uint16_t* wrow = w + ((pos + 1) % N) * K;", 0),
    ("linear_truncated", "out[pos] = rne_bf16_from_double(acc);", "out[pos] = float_bits_hi((float)acc);", 0),
    ("linear_hidden_row_ignored", "const uint16_t* hvec = hidden + (pos / N) * K;", "const uint16_t* hvec = hidden;", 0),
]

# cheap pins first; the exhaustive sweeps only run if nothing cheaper caught the mutant
COST_ORDER = sorted(oracle_pins.ALL_PINS,
                    key=lambda f: 1 if "exhaustive" in f.__name__ else 0)


def _build_mutant(tmp_path, name, find, repl, count):
    assert find in SOURCE, f"mutation anchor for {name} not found in the oracle source"
    src = SOURCE.replace(find, repl) if count == 0 else SOURCE.replace(find, repl, count)
    c_path = tmp_path / f"{name}.c"
    so_path = tmp_path / f"lib{name}.so"
    c_path.write_text(src)
    flags = [f for f in oracle_build.CFLAGS if f not in ("-Werror", "-Wall", "-Wextra")]
    subprocess.run(["gcc", *flags, "-w", "-o", str(so_path), str(c_path), "-lm"], check=True)
    return str(so_path)


@pytest.mark.parametrize("name,find,repl,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_rejected(tmp_path, name, find, repl, count):
    path = _build_mutant(tmp_path, name, find, repl, count)
    caught_by = None
    with oracle.using_library(path):
        for pin in COST_ORDER:
            try:
                pin()
            except AssertionError:
                caught_by = pin.__name__
                break
    assert caught_by is not None, f"no pin rejects the mutant {name}"
    print(f"{name}: rejected by {caught_by}")


def test_unmutated_source_passes_cheap_pins():
    """Control: the real oracle passes the same cheap pins the mutants are run through."""
    for pin in COST_ORDER:
        if "exhaustive" not in pin.__name__:
            pin()
