"""Backward of the dual-weight GLU projection -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module; it shares no code with the HIP library.

What it computes.  The dual-weight GLU (DeepSpeed PR #8602, comment "Plan B:
Dual-Weight GEMV", section "Plan B Design") is an autograd Function that keeps
hidden, gate_w and up_w for the backward, and the same comment checks that its
gradients for all three equal those of the composite silu(h @ Wg^T) *
(h @ Wu^T) (section "Verification Results", "Gradient exactness").  Read together with the forward's bf16 tensor
boundaries (PR #9057, "Changes"), the backward is autograd of that composite
over bf16 tensors: each gradient tensor is computed in fp32 (or exactly) and
rounded once to bf16, round to nearest even.  For every m < M, j < N, k < K,
given the upstream gradient dout [M,N]:

1. the forward's values: G = h[m] . Wg[j], U = h[m] . Wu[j] (fp64, exact
   products), g = RNE(G), u = RNE(U), s = RNE(silu32(g)) exactly as the
   forward oracle rounds them;
2. backward of out = s * u:  ds = RNE(dout * u),  du = RNE(dout * s)  (a
   product of two bf16 values is exact, so one rounding);
3. backward of s = silu(g), evaluated in fp32 with sigma the logistic
   function:  sig = fl32(1 / fl32(1 + fl32(exp(-g)))),
   dg = RNE(fl32(fl32(ds * sig) * fl32(1 + fl32(g * fl32(1 - sig)))));
4. backward of the two products with hidden:  dh_g = RNE(sum_j dg * Wg[j,k]),
   dh_u = RNE(sum_j du * Wu[j,k]), and hidden's gradient is the bf16 sum of
   the two contributions, dh = RNE(fl32(dh_g + dh_u));  the weights'
   gradients are dWg[j,k] = RNE(sum_m dg[m,j] * h[m,k]) and
   dWu[j,k] = RNE(sum_m du[m,j] * h[m,k]).

The sums of step 4 are fp64 matrix products of exact fp64 products (a library
routine as one step; its rounding error, at most about n * 2^-53 relative to
the sum of magnitudes, decides a bf16 rounding only for sums that nearly
cancel).  exp is the fp64 exponential rounded to fp32, as in the forward.

Reading where the pages are silent: the fp32 operation order inside step 3
(the silu derivative sig * (1 + g * (1 - sig)) applied as (ds * sig) * (...)).
Another order can move a bf16 result by one unit where the fp32 value lies
within a few fp32 units of a bf16 rounding boundary.  The formula is pinned
against a high-precision numerical derivative of silu, and the order against
torch's CPU autograd of the bf16 composite (the Hugging Face training path),
which gives these gradients bit for bit.
"""
from __future__ import annotations

from typing import NamedTuple

import numpy as np

from . import _u16, dual_gemv, round_bf16


class BackwardResult(NamedTuple):
    dh: np.ndarray        # uint16 [M,K] bf16 bits
    dwg: np.ndarray       # uint16 [N,K]
    dwu: np.ndarray       # uint16 [N,K]
    dg: np.ndarray        # uint16 [M,N]  gradient of the gate pre-activation
    du: np.ndarray        # uint16 [M,N]  gradient of the up pre-activation
    ds: np.ndarray        # uint16 [M,N]  gradient of silu(g)
    dhg_pre: np.ndarray   # fp64 [M,K]  sum_j dg * Wg[j,k]
    dhu_pre: np.ndarray   # fp64 [M,K]  sum_j du * Wu[j,k]
    dhg_abs: np.ndarray   # fp64 [M,K]  sum_j |dg * Wg[j,k]|
    dhu_abs: np.ndarray   # fp64 [M,K]
    dwg_pre: np.ndarray   # fp64 [N,K]  sum_m dg * h[m,k]
    dwu_pre: np.ndarray   # fp64 [N,K]
    dwg_abs: np.ndarray   # fp64 [N,K]  sum_m |dg * h[m,k]|
    dwu_abs: np.ndarray   # fp64 [N,K]
    gate_pre: np.ndarray  # fp64 [M,N]  G
    up_pre: np.ndarray    # fp64 [M,N]  U


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact fp32 values of bf16 bit patterns."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rne(x: np.ndarray) -> np.ndarray:
    """bf16 bits of fp32 or fp64 values, one rounding to nearest even."""
    return round_bf16(np.asarray(x, dtype=np.float64))


def _silu32(g: np.ndarray) -> np.ndarray:
    """fp32 silu of fp32 values g: g / (1 + exp(-g)), each step in fp32."""
    e = np.exp(-g.astype(np.float64)).astype(np.float32)
    d = np.float32(1) + e
    return g / d


def silu_grad32(ds: np.ndarray, g: np.ndarray) -> np.ndarray:
    """Step 3 in fp32: (ds * sig) * (1 + g * (1 - sig)), sig = 1 / (1 + exp(-g))."""
    one = np.float32(1)
    e = np.exp(-g.astype(np.float64)).astype(np.float32)
    sig = one / (one + e)
    return (ds * sig) * (one + g * (one - sig))


class ContractResult(NamedTuple):
    dh: np.ndarray        # uint16 [M,K]
    dwg: np.ndarray       # uint16 [N,K]
    dwu: np.ndarray       # uint16 [N,K]
    dhg_pre: np.ndarray
    dhu_pre: np.ndarray
    dhg_abs: np.ndarray
    dhu_abs: np.ndarray
    dwg_pre: np.ndarray
    dwu_pre: np.ndarray
    dwg_abs: np.ndarray
    dwu_abs: np.ndarray


def act_grads(g_bits: np.ndarray, u_bits: np.ndarray, dout: np.ndarray):
    """Steps 2 and 3, elementwise: (ds, du, dg) bf16 bits from the forward's bf16 g and u and dout."""
    with np.errstate(all="ignore"):
        g = bits_to_f32(_u16(g_bits))
        u = bits_to_f32(_u16(u_bits))
        s = bits_to_f32(_rne(_silu32(g)))
        go32 = bits_to_f32(_u16(dout))
        ds_bits = _rne(go32 * u)
        du_bits = _rne(go32 * s)
        dg_bits = _rne(silu_grad32(bits_to_f32(ds_bits), g))
    return ds_bits, du_bits, dg_bits


def contract(hidden: np.ndarray, gate_w: np.ndarray, up_w: np.ndarray, dg_bits: np.ndarray,
             du_bits: np.ndarray) -> ContractResult:
    """Step 4: the three gradients from the bf16 gradients dg, du [M,N] of the pre-activations."""
    with np.errstate(all="ignore"):
        dg64 = bits_to_f32(dg_bits).astype(np.float64)
        du64 = bits_to_f32(du_bits).astype(np.float64)
        h64 = bits_to_f32(_u16(hidden)).astype(np.float64)
        wg64 = bits_to_f32(_u16(gate_w)).astype(np.float64)
        wu64 = bits_to_f32(_u16(up_w)).astype(np.float64)
        dhg_pre = dg64 @ wg64
        dhu_pre = du64 @ wu64
        dhg_abs = np.abs(dg64) @ np.abs(wg64)
        dhu_abs = np.abs(du64) @ np.abs(wu64)
        dwg_pre = dg64.T @ h64
        dwu_pre = du64.T @ h64
        dwg_abs = np.abs(dg64).T @ np.abs(h64)
        dwu_abs = np.abs(du64).T @ np.abs(h64)
        dh_g = bits_to_f32(_rne(dhg_pre))
        dh_u = bits_to_f32(_rne(dhu_pre))
        dh_bits = _rne(dh_g + dh_u)
    return ContractResult(dh_bits, _rne(dwg_pre), _rne(dwu_pre), dhg_pre, dhu_pre, dhg_abs, dhu_abs,
                          dwg_pre, dwu_pre, dwg_abs, dwu_abs)


def dual_gemv_backward(hidden: np.ndarray, gate_w: np.ndarray, up_w: np.ndarray, dout: np.ndarray,
                       threads: int = 0) -> BackwardResult:
    """Gradients of the GLU projection for bf16 bit arrays hidden [M,K], gate_w/up_w [N,K], dout [M,N]."""
    h = _u16(hidden)
    wg = _u16(gate_w)
    wu = _u16(up_w)
    go = _u16(dout)
    M, K = h.shape
    N = wg.shape[0]
    if wg.shape != (N, K) or wu.shape != (N, K) or go.shape != (M, N):
        raise ValueError(f"shape mismatch: hidden {h.shape}, gate_w {wg.shape}, up_w {wu.shape}, dout {go.shape}")
    # 1. the forward's bf16 values
    fwd = dual_gemv(h, wg, wu, threads=threads, with_pre=True)
    g_bits = _rne(fwd.gate_pre)
    u_bits = _rne(fwd.up_pre)
    # 2.-3. backward of s * u and of silu
    ds_bits, du_bits, dg_bits = act_grads(g_bits, u_bits, go)
    # 4. backward of the products with hidden
    c = contract(h, wg, wu, dg_bits, du_bits)
    return BackwardResult(c.dh, c.dwg, c.dwu, dg_bits, du_bits, ds_bits, c.dhg_pre, c.dhu_pre, c.dhg_abs,
                          c.dhu_abs, c.dwg_pre, c.dwu_pre, c.dwg_abs, c.dwu_abs, fwd.gate_pre, fwd.up_pre)
