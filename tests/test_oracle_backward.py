"""The backward oracle against its pins, and planted mistakes against the pins (CPU only).

Pins: tests/oracle_pins_backward.py.  Each mutant is oracle/backward.py with one
plausible mistake substituted (a wrong operand, a dropped factor, a missing
rounding, a flipped sign), loaded as a module of its own; some pin must reject
it.
"""
import importlib.util
import os
import sys

import pytest

import oracle
import oracle_pins_backward as pins

SOURCE_PATH = os.path.join(os.path.dirname(oracle.__file__), "backward.py")
SOURCE = open(SOURCE_PATH).read()

MUTANTS = [
    ("silu_grad_factor_missing", "return (ds * sig) * (one + g * (one - sig))", "return ds * sig"),
    ("silu_grad_sign_of_exp", "e = np.exp(-g.astype(np.float64)).astype(np.float32)\n    sig",
     "e = np.exp(g.astype(np.float64)).astype(np.float32)\n    sig"),
    ("ds_times_s", "ds_bits = _rne(go32 * u)", "ds_bits = _rne(go32 * s)"),
    ("du_times_u", "du_bits = _rne(go32 * s)", "du_bits = _rne(go32 * u)"),
    ("dh_up_branch_dropped", "dh_bits = _rne(dh_g + dh_u)", "dh_bits = _rne(dh_g)"),
    ("contract_swaps_gradients", "c = contract(h, wg, wu, dg_bits, du_bits)", "c = contract(h, wg, wu, du_bits, dg_bits)"),
    ("dh_up_uses_gate_weights", "dhu_pre = du64 @ wu64", "dhu_pre = du64 @ wg64"),
    ("dwg_uses_du", "dwg_pre = dg64.T @ h64", "dwg_pre = du64.T @ h64"),
    ("dh_contributions_not_rounded", "dh_g = bits_to_f32(_rne(dhg_pre))", "dh_g = dhg_pre.astype(np.float32)"),
    ("dg_truncated", "dg_bits = _rne(silu_grad32(bits_to_f32(ds_bits), g))",
     "dg_bits = (silu_grad32(bits_to_f32(ds_bits), g).view(np.uint32) >> 16).astype(np.uint16)"),
    ("silu_unrounded_in_du", "s = bits_to_f32(_rne(_silu32(g)))", "s = _silu32(g)"),
]


def _mutant_module(name, find, repl):
    assert find in SOURCE, f"mutation anchor for {name} not found"
    src = SOURCE.replace(find, repl)
    spec = importlib.util.spec_from_loader(f"oracle._mutant_{name}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    sys.modules[spec.name] = mod
    try:
        exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    finally:
        del sys.modules[spec.name]
    return mod


@pytest.mark.parametrize("pin", pins.BACKWARD_PINS, ids=lambda f: f.__name__)
def test_backward_pin(pin):
    pin()


@pytest.mark.parametrize("name,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_backward_mutant_is_rejected(name, find, repl):
    mod = _mutant_module(name, find, repl)
    caught_by = None
    for pin in pins.BACKWARD_PINS:
        try:
            pin(mod.dual_gemv_backward)
        except AssertionError:
            caught_by = pin.__name__
            break
    assert caught_by is not None, f"no pin rejects the mutant {name}"
    print(f"{name}: rejected by {caught_by}")
