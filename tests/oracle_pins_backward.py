"""Pins of the backward oracle (oracle/backward.py) -- CPU only.

Each pin takes the backward function to check (default: the oracle's), so the
mutant tests can run the same pins against a copy of the oracle with one
planted mistake.  What pins what:

* pin_bwd_brute_force_tiny -- every step, bitwise: an exact-rational
  evaluation of the same reading (tests/exact.py: Fractions, rounding from the
  definition of the formats, exp at 60 digits);
* pin_bwd_silu_derivative -- the silu derivative itself against a 60-digit
  central difference of silu (a closed form nowhere retyped), all finite bf16 g
  with |g| <= 80;
* pin_bwd_special_cases -- g = 0 (sigma = 1/2: dg = ds/2, silu = 0: du = 0)
  and a saturated gate (sigma = 1: dg = ds, s = g);
* pin_bwd_identities -- sum_k dh_g[m,k] h[m,k] = sum_j dg[m,j] G[m,j] and
  sum_k dWg[j,k] Wg[j,k] = sum_m dg[m,j] G[m,j] (likewise for up), which hold
  for the exact contractions whatever the values: a transposed or swapped
  operand breaks them;
* pin_bwd_torch_bf16_autograd -- torch's own CPU autograd of the composite
  silu(h @ Wg^T) * (h @ Wu^T) over bf16 tensors lands on the oracle's
  gradients up to fp32 summation order (it also fixes the fp32 operation
  order of the silu derivative that the pages leave open).
"""
from __future__ import annotations

import decimal
import math
from fractions import Fraction

import numpy as np
import torch

import exact
from oracle import LinearResult
from oracle import backward as bwd_mod
from oracle import check

_DEC = decimal.Context(prec=60, rounding=decimal.ROUND_HALF_EVEN, Emin=-999999, Emax=999999, traps=[])


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).numpy().view(np.uint16)


def tensor_of(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def _random_bf16(rng, shape, scale_exp=(-4, 2)):
    mant = rng.integers(0, 128, shape)
    expo = rng.integers(127 + scale_exp[0], 127 + scale_exp[1], shape)
    sign = rng.integers(0, 2, shape)
    return ((sign << 15) | (expo << 7) | mant).astype(np.uint16)


def _val(bits) -> float:
    v = exact.bf16_bits_to_value(int(bits))
    return float(v)


def _same_value(a_bits, b_val) -> bool:
    """bf16 bits equal an exact value (+0 and -0 alike)."""
    a = exact.bf16_bits_to_value(int(a_bits))
    return a == b_val


def _r32(q):
    return exact.round_to_format(q, exact.FP32)


def _r16(q):
    return exact.round_to_format(q, exact.BF16)


def _exact_backward(h, wg, wu, dout):
    """Exact-rational evaluation of the four steps for finite tiny inputs (values, signs of zero dropped)."""
    M, K = h.shape
    N = wg.shape[0]
    hv = [[exact.bf16_bits_to_value(int(b)) for b in row] for row in h]
    gv = [[exact.bf16_bits_to_value(int(b)) for b in row] for row in wg]
    uv = [[exact.bf16_bits_to_value(int(b)) for b in row] for row in wu]
    dg = [[None] * N for _ in range(M)]
    du = [[None] * N for _ in range(M)]
    for m in range(M):
        for j in range(N):
            r = exact.glu_out_bits(h[m].tolist(), wg[j].tolist(), wu[j].tolist())
            g = exact.bf16_bits_to_value(r["g_bits"])
            u = exact.bf16_bits_to_value(r["u_bits"])
            s = exact.bf16_bits_to_value(r["s_bits"])
            go = exact.bf16_bits_to_value(int(dout[m, j]))
            ds = _r16(go * u)
            du[m][j] = _r16(go * s)
            e = exact.exp_fp32(-g)
            sig = _r32(1 / _r32(1 + e))
            t = _r32(1 + _r32(g * _r32(1 - sig)))
            dg[m][j] = _r16(_r32(_r32(ds * sig) * t))
    dh = [[None] * K for _ in range(M)]
    for m in range(M):
        for k in range(K):
            a = _r16(sum((dg[m][j] * gv[j][k] for j in range(N)), Fraction(0)))
            b = _r16(sum((du[m][j] * uv[j][k] for j in range(N)), Fraction(0)))
            dh[m][k] = _r16(_r32(a + b))
    dwg = [[_r16(sum((dg[m][j] * hv[m][k] for m in range(M)), Fraction(0))) for k in range(K)] for j in range(N)]
    dwu = [[_r16(sum((du[m][j] * hv[m][k] for m in range(M)), Fraction(0))) for k in range(K)] for j in range(N)]
    return dg, du, dh, dwg, dwu


def pin_bwd_brute_force_tiny(backward=None):
    """Every gradient of tiny cases equals its exact-rational evaluation."""
    backward = backward or bwd_mod.dual_gemv_backward
    rng = np.random.default_rng(61)
    for M, N, K in [(1, 3, 1), (1, 3, 4), (2, 3, 8), (2, 5, 3), (3, 2, 6)]:
        h = _random_bf16(rng, (M, K))
        wg = _random_bf16(rng, (N, K))
        wu = _random_bf16(rng, (N, K))
        dout = _random_bf16(rng, (M, N))
        res = backward(h, wg, wu, dout)
        dg, du, dh, dwg, dwu = _exact_backward(h, wg, wu, dout)
        for m in range(M):
            for j in range(N):
                assert _same_value(res.dg[m, j], dg[m][j]), (M, N, K, m, j, "dg")
                assert _same_value(res.du[m, j], du[m][j]), (M, N, K, m, j, "du")
            for k in range(K):
                assert _same_value(res.dh[m, k], dh[m][k]), (M, N, K, m, k, "dh")
        for j in range(N):
            for k in range(K):
                assert _same_value(res.dwg[j, k], dwg[j][k]), (M, N, K, j, k, "dwg")
                assert _same_value(res.dwu[j, k], dwu[j][k]), (M, N, K, j, k, "dwu")


def _silu_dec(x: decimal.Decimal) -> decimal.Decimal:
    return _DEC.divide(x, _DEC.add(1, _DEC.exp(-x)))


def pin_bwd_silu_derivative(backward=None):
    """dg for ds = 1 against the derivative of silu by a 60-digit central difference.

    h = 1 at k = 0, Wg[j,0] = g_j, Wu[j,0] = 1, dout = 1 make G = g_j, u = 1 and
    ds = 1, so dg_j is the bf16 rounding of the fp32-evaluated derivative.  Any
    difference from the correctly rounded derivative must be one bf16 unit and
    sit where the derivative lies within 2^-12 (relative) of a bf16 rounding
    boundary, i.e. where a few fp32 rounding errors can move the rounding.
    """
    backward = backward or bwd_mod.dual_gemv_backward
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bwd_mod.bits_to_f32(pats)
    keep = np.isfinite(vals) & (np.abs(vals) <= 80)
    g = pats[keep]
    N = g.size
    K = 8
    h = np.zeros((1, K), dtype=np.uint16)
    h[0, 0] = 0x3F80
    wg = np.zeros((N, K), dtype=np.uint16)
    wg[:, 0] = g
    wu = np.zeros((N, K), dtype=np.uint16)
    wu[:, 0] = 0x3F80
    dout = np.full((1, N), 0x3F80, dtype=np.uint16)
    res = backward(h, wg, wu, dout)
    got = res.dg[0]
    eps = decimal.Decimal("1e-25")
    gv = vals[keep]
    mismatches = 0
    for i in range(N):
        x = decimal.Decimal(float(gv[i]))
        d = _DEC.divide(_DEC.subtract(_silu_dec(_DEC.add(x, eps)), _silu_dec(_DEC.subtract(x, eps))),
                        _DEC.multiply(2, eps))
        q = Fraction(d)
        want = _r16(q)
        have = exact.bf16_bits_to_value(int(got[i]))
        if have == want:
            continue
        mismatches += 1
        # one bf16 unit apart, with the exact derivative next to the midpoint between them
        assert not isinstance(have, float) and not isinstance(want, float), (hex(int(g[i])), have, want)
        mid = (have + want) / 2
        assert abs(have - want) <= abs(want) * Fraction(1, 64) + Fraction(1, 2 ** 133), (hex(int(g[i])), have, want)
        assert abs(q - mid) <= abs(q) * Fraction(1, 2 ** 12), (hex(int(g[i])), float(q), float(mid))
    assert mismatches <= N // 200, f"{mismatches} of {N} derivative values differ"


def pin_bwd_special_cases(backward=None):
    """g = 0: dg = ds / 2 exactly, du = 0; a saturated gate (G = 32): dg = ds, du = dout * 32."""
    backward = backward or bwd_mod.dual_gemv_backward
    rng = np.random.default_rng(62)
    M, N, K = 2, 6, 16
    h = _random_bf16(rng, (M, K))
    wu = _random_bf16(rng, (N, K))
    dout = _random_bf16(rng, (M, N))
    res = backward(h, np.zeros((N, K), dtype=np.uint16), wu, dout)
    ds = bwd_mod.bits_to_f32(res.ds).astype(np.float64)
    assert np.array_equal(bwd_mod.bits_to_f32(res.dg).astype(np.float64), ds / 2)
    assert np.all(bwd_mod.bits_to_f32(res.du) == 0)
    assert np.all(bwd_mod.bits_to_f32(res.dwu) == 0)
    assert np.all(bwd_mod.bits_to_f32(res.dh) == 0)
    # ds = bf16(dout * u) with u the rounded up projection
    u = bwd_mod.bits_to_f32(bwd_mod._rne(res.up_pre)).astype(np.float64)
    want = np.array([[_r16(Fraction(float(bwd_mod.bits_to_f32(dout)[m, j])) * Fraction(u[m, j]))
                      for j in range(N)] for m in range(M)], dtype=object)
    assert all(_same_value(res.ds[m, j], want[m, j]) for m in range(M) for j in range(N))
    # saturated: h = 2 at k = 0 only, Wg[:,0] = 16, so G = 32 and sigma rounds to 1
    h2 = np.zeros((M, K), dtype=np.uint16)
    h2[:, 0] = 0x4000
    wg2 = np.zeros((N, K), dtype=np.uint16)
    wg2[:, 0] = 0x4180
    res = backward(h2, wg2, wu, dout)
    assert np.array_equal(res.dg, res.ds)
    go = bwd_mod.bits_to_f32(dout).astype(np.float64)
    assert np.array_equal(bwd_mod.bits_to_f32(res.du).astype(np.float64), go * 32)


def pin_bwd_identities(backward=None):
    """Contractions against identities of the exact products (fp64, relative 1e-9)."""
    backward = backward or bwd_mod.dual_gemv_backward
    rng = np.random.default_rng(63)
    M, N, K = 3, 40, 24
    h = _random_bf16(rng, (M, K))
    wg = _random_bf16(rng, (N, K))
    wu = _random_bf16(rng, (N, K))
    dout = _random_bf16(rng, (M, N))
    r = backward(h, wg, wu, dout)
    f = lambda b: bwd_mod.bits_to_f32(b).astype(np.float64)  # noqa: E731
    h64, wg64, wu64, dg, du = f(h), f(wg), f(wu), f(r.dg), f(r.du)
    G, U = r.gate_pre, r.up_pre
    for pre, w, d, P in ((r.dhg_pre, wg64, dg, G), (r.dhu_pre, wu64, du, U)):
        lhs = np.sum(pre * h64, axis=1)
        rhs = np.sum(d * P, axis=1)
        scale = np.abs(d) @ (np.abs(h64) @ np.abs(w).T).T
        assert np.all(np.abs(lhs - rhs) <= 1e-9 * np.diag(scale) + 1e-300), "dh identity"
    for pre, w, d, P in ((r.dwg_pre, wg64, dg, G), (r.dwu_pre, wu64, du, U)):
        lhs = np.sum(pre * w, axis=1)
        rhs = np.sum(d * P, axis=0)
        scale = np.sum(np.abs(d) * (np.abs(h64) @ np.abs(w).T), axis=0)
        assert np.all(np.abs(lhs - rhs) <= 1e-9 * scale + 1e-300), "dW identity"
    # absolute sums are the sums of magnitudes
    np.testing.assert_allclose(r.dhg_abs, np.abs(dg) @ np.abs(wg64), rtol=1e-13)
    np.testing.assert_allclose(r.dwu_abs, np.abs(du).T @ np.abs(h64), rtol=1e-13)


def pin_bwd_torch_bf16_autograd(backward=None):
    """torch's CPU autograd of the bf16 composite against the oracle: each gradient within 2 ULP
    or its admissible interval, >= 99.9 % bit-exact (torch's fp32 summation order is its own; its
    silu backward evaluates the derivative in fp32 as the oracle reads it)."""
    backward = backward or bwd_mod.dual_gemv_backward
    g = torch.Generator().manual_seed(64)
    M, N, K = 4, 256, 192
    h = (torch.randn(M, K, generator=g)).bfloat16().requires_grad_()
    wg = (torch.randn(N, K, generator=g) * 0.1).bfloat16().requires_grad_()
    wu = (torch.randn(N, K, generator=g) * 0.1).bfloat16().requires_grad_()
    dout = torch.randn(M, N, generator=g).bfloat16()
    out = torch.nn.functional.silu(h @ wg.T) * (h @ wu.T)
    out.backward(dout)
    r = backward(bits_of(h), bits_of(wg), bits_of(wu), bits_of(dout))
    for name, t, want, pre, ab, depth, klen in (
            ("dWg", wg.grad, r.dwg, r.dwg_pre, r.dwg_abs, M, M),
            ("dWu", wu.grad, r.dwu, r.dwu_pre, r.dwu_abs, M, M)):
        rep = check.compare_linear(bits_of(t), LinearResult(want, pre, ab), depth=depth, k_len=klen)
        assert rep.failures == 0 and rep.bit_exact_frac >= 0.999, (name, rep.summary())
    rep = check.compare_grad_sum(bits_of(h.grad), r.dh, r.dhg_pre, r.dhg_abs, r.dhu_pre, r.dhu_abs,
                                 depth=N, k_len=N)
    assert rep.failures == 0 and rep.bit_exact_frac >= 0.999, ("dh", rep.summary())


BACKWARD_PINS = [pin_bwd_special_cases, pin_bwd_identities, pin_bwd_brute_force_tiny, pin_bwd_torch_bf16_autograd,
                 pin_bwd_silu_derivative]
