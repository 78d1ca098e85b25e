"""Pins of the oracle against facts it does not compute itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
what the pages and the mathematics fix.  test_oracle_pins.py runs them on the
oracle; test_oracle_mutants.py runs them on copies of the oracle with one
planted mistake each and requires that some pin rejects every copy.

Independent references used here:
* tests/exact.py -- exact rational arithmetic, 60-digit decimal exp;
* torch CPU ops -- fp32->bf16 casts, fp64 matmul, the bf16 composite
  silu(h @ Wg^T) * (h @ Wu^T) that a Hugging Face MLP evaluates on the CPU;
* closed forms of silu and of scaling by powers of two.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import torch

import exact
import oracle
from oracle import check
from glu_mlp_gemv_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def bits_of(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def tensor_of(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def all_bf16() -> np.ndarray:
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


# ---- rounding -------------------------------------------------------------

def pin_round_matches_torch_cast():
    """fp64 holding fp32 values: direct rounding equals torch's fp32->bf16 cast (RNE)."""
    rng = np.random.default_rng(11)
    raw = rng.integers(0, 1 << 32, 200_000, dtype=np.uint64).astype(np.uint32)
    f32 = raw.view(np.float32)
    f32 = f32[np.isfinite(f32)]
    got = oracle.round_bf16(f32.astype(np.float64))
    want = bits_of(torch.from_numpy(f32.copy()).to(torch.bfloat16))
    bad = check.compare_strict_bits(got, want)
    assert bad is None, f"{bad.size} mismatches, first input {f32[bad[0]]!r}"


def pin_round_matches_exact_for_fp64():
    """fp64 values off the fp32 grid: rounding equals the exact rational rule."""
    rng = np.random.default_rng(12)
    mant = rng.random(3000) + 1.0
    expo = rng.integers(-140, 130, 3000)
    sign = np.where(rng.random(3000) < 0.5, -1.0, 1.0)
    x = sign * np.ldexp(mant, expo)
    got = oracle.round_bf16(x)
    for xi, gi in zip(x, got):
        r = exact.round_to_format(Fraction(float(xi)), exact.BF16)
        want = exact.value_to_bf16_bits(r, negative_zero=(xi < 0))
        assert exact.bits_equal(int(gi), want), f"round({xi!r}) -> {gi:#06x}, exact {want:#06x}"


def pin_round_edges():
    """Ties to even, subnormals, overflow threshold, zeros, NaN."""
    fixture = json.load(open(os.path.join(GOLDEN, "bf16_rounding_edges.json")))
    xs = np.array([float.fromhex(c["x"]) for c in fixture["cases"]], dtype=np.float64)
    got = oracle.round_bf16(xs)
    for c, gi in zip(fixture["cases"], got):
        want = int(c["bf16"], 16)
        assert exact.bits_equal(int(gi), want), f"{c['x']}: got {gi:#06x}, want {want:#06x} ({c['why']})"


# ---- epilogue -------------------------------------------------------------

def pin_epilogue_exhaustive_unit_up():
    """Every bf16 gate value with u = 1: act and out equal the exact evaluation."""
    g = all_bf16()
    u = np.full(g.size, 0x3F80, dtype=np.uint16)
    out = oracle.epilogue(g, u)
    s = oracle.silu_bf16(g)
    for i in range(g.size):
        r = exact.epilogue_bits(int(g[i]), 0x3F80)
        assert exact.bits_equal(r["s_bits"], int(s[i])), f"act(g={g[i]:#06x}) {s[i]:#06x} != {r['s_bits']:#06x}"
        assert exact.bits_equal(r["out_bits"], int(out[i])), f"out(g={g[i]:#06x}) {out[i]:#06x} != {r['out_bits']:#06x}"


def pin_epilogue_exhaustive_random_up():
    """Every bf16 gate value with a random bf16 up value (product rounding, underflow, inf)."""
    g = all_bf16()
    rng = np.random.default_rng(13)
    u = rng.integers(0, 1 << 16, g.size).astype(np.uint16)
    out = oracle.epilogue(g, u)
    for i in range(g.size):
        r = exact.epilogue_bits(int(g[i]), int(u[i]))
        assert exact.bits_equal(r["out_bits"], int(out[i])), \
            f"out(g={g[i]:#06x}, u={u[i]:#06x}) {out[i]:#06x} != {r['out_bits']:#06x}"


def pin_silu_vs_torch_cpu(max_mismatch: int = 64):
    """torch's own bf16 silu (fp32 inside, HF's act_fn) agrees except a few 1-ULP exp cases."""
    g = all_bf16()
    finite = ~check.is_nan_bits(g) & ((g & 0x7F80) != 0x7F80)
    ours = oracle.silu_bf16(g)[finite]
    theirs = bits_of(torch.nn.functional.silu(tensor_of(g)))[finite]
    d = check.ulp_distance(ours, theirs)
    assert d.max() <= 1, f"max ULP {d.max()}"
    assert int((d > 0).sum()) <= max_mismatch, f"{int((d > 0).sum())} 1-ULP differences"


def pin_silu_closed_forms():
    """silu(+-0) = +-0; g >= 17 gives act = g; g <= -89 gives -0; |g| < 2^-25 gives g/2."""
    g = all_bf16()
    gv = check.bf16_to_f64(g)
    s = oracle.silu_bf16(g)
    assert s[0x0000] == 0x0000 and s[0x8000] == 0x8000
    big = np.isfinite(gv) & (gv >= 17.0)
    assert np.array_equal(s[big], g[big]), "1 + exp(-g) must round to 1 for g >= 17"
    neg = np.isfinite(gv) & (gv <= -89.0)
    assert np.all(s[neg] == 0x8000), "exp(-g) overflows fp32 for g <= -89: act is -0"
    tiny = (np.abs(gv) < 2.0 ** -25) & (gv != 0)
    half = bits_of(torch.from_numpy((gv[tiny] / 2).astype(np.float32)).to(torch.bfloat16))
    assert np.array_equal(s[tiny], half), "exp(-g) rounds to 1 for |g| < 2^-25: act = g/2"
    assert check.is_nan_bits(s[0x7FC0:0x7FC1]).all()
    assert s[0x7F80] == 0x7F80 and check.is_nan_bits(s[0xFF80:0xFF81]).all()


def pin_hand_worked():
    """Small cases worked by hand (derivations in tests/golden/hand_worked.json)."""
    fixture = json.load(open(os.path.join(GOLDEN, "hand_worked.json")))
    for c in fixture["cases"]:
        h = np.array([[float(v) for v in row] for row in c["hidden"]], dtype=np.float32)
        wg = np.array([[float(v) for v in row] for row in c["gate_w"]], dtype=np.float32)
        wu = np.array([[float(v) for v in row] for row in c["up_w"]], dtype=np.float32)
        to_bits = lambda a: bits_of(torch.from_numpy(a).to(torch.bfloat16))
        out = oracle.dual_gemv(to_bits(h), to_bits(wg), to_bits(wu))
        want = np.array([[int(v, 16) for v in row] for row in c["out_bf16"]], dtype=np.uint16)
        assert np.array_equal(out, want), f"{c['name']}: {out} != {want}"


# ---- dots and indexing ----------------------------------------------------

def _random_bf16(rng, shape, scale_exp=(-6, 3)):
    """Random bf16 bit patterns with varied exponents (finite, non-NaN)."""
    mant = rng.integers(0, 128, shape)
    expo = rng.integers(127 + scale_exp[0], 127 + scale_exp[1], shape)
    sign = rng.integers(0, 2, shape)
    return ((sign << 15) | (expo << 7) | mant).astype(np.uint16)


def pin_brute_force_tiny():
    """Tiny shapes: every output, g and u equal the exact rational evaluation."""
    rng = np.random.default_rng(14)
    for M, K, N in [(1, 1, 3), (1, 4, 3), (2, 8, 5), (2, 13, 4), (3, 31, 2), (1, 64, 3)]:
        h = _random_bf16(rng, (M, K))
        wg = _random_bf16(rng, (N, K))
        wu = _random_bf16(rng, (N, K))
        res = oracle.dual_gemv(h, wg, wu, with_pre=True)
        g_bits = oracle.round_bf16(res.gate_pre)
        u_bits = oracle.round_bf16(res.up_pre)
        for m in range(M):
            for j in range(N):
                r = exact.glu_out_bits(h[m].tolist(), wg[j].tolist(), wu[j].tolist())
                bound = K * 2.0 ** -53 * float(res.gate_abs[m, j]) * 1.01
                assert abs(float(r["G"]) - res.gate_pre[m, j]) <= bound, (M, K, N, m, j, "G")
                bound = K * 2.0 ** -53 * float(res.up_abs[m, j]) * 1.01
                assert abs(float(r["U"]) - res.up_pre[m, j]) <= bound, (M, K, N, m, j, "U")
                assert exact.bits_equal(r["g_bits"], int(g_bits[m, j])), (M, K, N, m, j, "g")
                assert exact.bits_equal(r["u_bits"], int(u_bits[m, j])), (M, K, N, m, j, "u")
                assert exact.bits_equal(r["out_bits"], int(res.out[m, j])), \
                    (M, K, N, m, j, hex(r["out_bits"]), hex(int(res.out[m, j])))


def pin_abs_sums():
    """The absolute sums are sum |h*w| (checked against a torch fp64 evaluation)."""
    rng = np.random.default_rng(15)
    h = _random_bf16(rng, (2, 40))
    wg = _random_bf16(rng, (6, 40))
    wu = _random_bf16(rng, (6, 40))
    res = oracle.dual_gemv(h, wg, wu, with_pre=True)
    ht = tensor_of(h).double().abs()
    np.testing.assert_allclose(res.gate_abs, (ht @ tensor_of(wg).double().abs().T).numpy(), rtol=1e-14)
    np.testing.assert_allclose(res.up_abs, (ht @ tensor_of(wu).double().abs().T).numpy(), rtol=1e-14)


def pin_torch_fp64_matmul():
    """G and U equal torch's fp64 matmul of the upcast operands (rows of Wg, Wu; h @ W^T)."""
    h, wg, wu = inputs.case("tail_k1024_n3000", M=3, seed=5)
    res = oracle.dual_gemv(bits_of(h), bits_of(wg), bits_of(wu), with_pre=True)
    G = (h.double() @ wg.double().T).numpy()
    U = (h.double() @ wu.double().T).numpy()
    tol = 1024 * 2.0 ** -52 * res.gate_abs
    assert np.all(np.abs(G - res.gate_pre) <= tol), "gate pre-activation differs from h @ Wg^T"
    tol = 1024 * 2.0 ** -52 * res.up_abs
    assert np.all(np.abs(U - res.up_pre) <= tol), "up pre-activation differs from h @ Wu^T"


def pin_torch_bf16_composite():
    """The HF composite on the CPU in bf16 lands within the parity tolerance of the oracle."""
    h, wg, wu = inputs.case("tail_k1024_n3000", M=2, seed=6)
    composite = torch.nn.functional.silu(h @ wg.T) * (h @ wu.T)
    res = oracle.dual_gemv(bits_of(h), bits_of(wg), bits_of(wu), with_pre=True)
    rep = check.compare(bits_of(composite), res, depth=1024, k_len=1024)
    assert rep.failures == 0, rep.summary()
    assert rep.bit_exact_frac >= 0.999, rep.summary()
    assert rep.mean_rel <= 3e-3, rep.summary()


def pin_linearity():
    """Before the nonlinearity the dots are linear in h: exact power-of-two scaling, additivity."""
    h, wg, wu = inputs.case("tail_k1024_n3000", M=1, seed=7)
    hb, wgb, wub = bits_of(h), bits_of(wg), bits_of(wu)
    base = oracle.dual_gemv(hb, wgb, wub, with_pre=True)
    for a in (-3, 1, 4):
        hs = bits_of((h.float() * 2.0 ** a).to(torch.bfloat16))  # exact in bf16
        sc = oracle.dual_gemv(hs, wgb, wub, with_pre=True)
        assert np.array_equal(sc.gate_pre, base.gate_pre * 2.0 ** a), f"G(2^{a} h) != 2^{a} G(h)"
        assert np.array_equal(sc.up_pre, base.up_pre * 2.0 ** a), f"U(2^{a} h) != 2^{a} U(h)"
    # h = h1 + h2 with disjoint supports (so the sum is exact in bf16)
    mask = (np.arange(h.shape[1]) % 3 == 0)
    h1 = h.clone(); h1[:, ~torch.from_numpy(mask)] = 0
    h2 = h.clone(); h2[:, torch.from_numpy(mask)] = 0
    r1 = oracle.dual_gemv(bits_of(h1), wgb, wub, with_pre=True)
    r2 = oracle.dual_gemv(bits_of(h2), wgb, wub, with_pre=True)
    tol = 3 * 1024 * 2.0 ** -53 * base.gate_abs
    assert np.all(np.abs(r1.gate_pre + r2.gate_pre - base.gate_pre) <= tol)
    tol = 3 * 1024 * 2.0 ** -53 * base.up_abs
    assert np.all(np.abs(r1.up_pre + r2.up_pre - base.up_pre) <= tol)
    # the nonlinearity sits on the gate only: zero gate weights give +-0 everywhere
    zero = np.zeros_like(wgb)
    z = oracle.dual_gemv(hb, zero, wub)
    assert np.all((z & 0x7FFF) == 0), "silu(0) * u must be a zero"


def pin_row_independence():
    """Batched row m equals the M=1 evaluation of h[m] bitwise (M=1 vs batched)."""
    h, wg, wu = inputs.case("batch_k4096_n12288", M=4, seed=0)
    n = 700  # a slice of the output rows keeps the pin quick
    wgb, wub = bits_of(wg[:n]), bits_of(wu[:n])
    batched = oracle.dual_gemv(bits_of(h), wgb, wub, with_pre=True)
    for m in range(h.shape[0]):
        single = oracle.dual_gemv(bits_of(h[m:m + 1]), wgb, wub, with_pre=True)
        assert np.array_equal(single.out[0], batched.out[m]), f"row {m}"
        assert np.array_equal(single.gate_pre[0], batched.gate_pre[m]), f"row {m} G"
        assert np.array_equal(single.up_pre[0], batched.up_pre[m]), f"row {m} U"


def pin_sampled_matches_full():
    h, wg, wu = inputs.case("tail_k1024_n3000", M=2, seed=8)
    hb, wgb, wub = bits_of(h), bits_of(wg), bits_of(wu)
    full = oracle.dual_gemv(hb, wgb, wub, with_pre=True)
    rng = np.random.default_rng(16)
    rows = rng.integers(0, 2, 300)
    cols = rng.integers(0, 3000, 300)
    smp = oracle.dual_gemv_sampled(hb, wgb, wub, rows, cols)
    assert np.array_equal(smp.out, full.out[rows, cols])
    assert np.array_equal(smp.gate_pre, full.gate_pre[rows, cols])
    assert np.array_equal(smp.up_abs, full.up_abs[rows, cols])


# ---- one projection of the grouped GEMV ------------------------------------

def pin_linear_brute_force_tiny():
    """Tiny shapes: every projection output equals the exact rational dot rounded to bf16."""
    rng = np.random.default_rng(31)
    for M, K, N in [(1, 1, 3), (1, 5, 4), (2, 8, 5), (3, 17, 3), (1, 64, 2)]:
        h = _random_bf16(rng, (M, K))
        w = _random_bf16(rng, (N, K))
        res = oracle.linear(h, w, with_pre=True)
        for m in range(M):
            for j in range(N):
                hv = [exact.bf16_bits_to_value(b) for b in h[m].tolist()]
                dot = sum((a * exact.bf16_bits_to_value(b) for a, b in zip(hv, w[j].tolist())), Fraction(0))
                r = exact.round_to_format(dot, exact.BF16)
                want = exact.value_to_bf16_bits(r, negative_zero=(r == 0 and dot < 0))
                assert exact.bits_equal(want, int(res.out[m, j])), (M, K, N, m, j, hex(want), hex(int(res.out[m, j])))
                bound = K * 2.0 ** -53 * float(res.abs[m, j]) * 1.01
                assert abs(float(dot) - res.pre[m, j]) <= bound, (M, K, N, m, j)


def pin_linear_torch():
    """The projection's dots equal torch's fp64 matmul, and torch's own bf16 linear on the CPU
    (fp32 accumulation, one rounding) lands within the parity bar of the oracle."""
    h, wg, _ = inputs.case("tail_k1024_n3000", M=3, seed=8)
    res = oracle.linear(bits_of(h), bits_of(wg), with_pre=True)
    P = (h.double() @ wg.double().T).numpy()
    assert np.all(np.abs(P - res.pre) <= 1024 * 2.0 ** -52 * res.abs), "projection differs from h @ W^T"
    A = (h.double().abs() @ wg.double().abs().T).numpy()
    np.testing.assert_allclose(res.abs, A, rtol=1e-14)
    lin = torch.nn.functional.linear(h, wg)
    rep = check.compare_linear(bits_of(lin), res, depth=1024, k_len=1024)
    assert rep.failures == 0 and rep.bit_exact_frac >= 0.999 and rep.mean_rel <= 3e-3, rep.summary()


def pin_linear_scaling():
    """Scaling h by a power of two scales every dot exactly and the rounded output by the same power."""
    h, wg, _ = inputs.case("tail_k1024_n3000", M=1, seed=9)
    base = oracle.linear(bits_of(h), bits_of(wg), with_pre=True)
    for a in (-2, 3):
        hs = (h.float() * 2.0 ** a).to(torch.bfloat16)
        sc = oracle.linear(bits_of(hs), bits_of(wg), with_pre=True)
        assert np.array_equal(sc.pre, base.pre * 2.0 ** a)
        want = bits_of((tensor_of(base.out).float() * 2.0 ** a).to(torch.bfloat16))
        assert check.compare_strict_bits(sc.out, want) is None


ALL_PINS = [
    pin_round_matches_torch_cast,
    pin_round_matches_exact_for_fp64,
    pin_round_edges,
    pin_epilogue_exhaustive_unit_up,
    pin_epilogue_exhaustive_random_up,
    pin_silu_vs_torch_cpu,
    pin_silu_closed_forms,
    pin_hand_worked,
    pin_brute_force_tiny,
    pin_abs_sums,
    pin_torch_fp64_matmul,
    pin_torch_bf16_composite,
    pin_linearity,
    pin_row_independence,
    pin_sampled_matches_full,
    pin_linear_brute_force_tiny,
    pin_linear_torch,
    pin_linear_scaling,
]
