"""Comparison of a bf16 result against the oracle -- TEST INFRASTRUCTURE ONLY.

Tolerance (the parity bar for floating point):

* strict: every output within 2 bf16 ULP of the oracle's output, where the ULP
  distance of two bf16 values is the difference of their sign-magnitude
  ordered 16-bit codes (+0 and -0 are the same point; NaN matches only NaN);
* mean relative error <= 0.3% over outputs whose oracle value is non-zero;
* bit-exact fraction >= 99.9% (a single-rounding kernel also meets the first
  two bars, so this one is what pins the four bf16 roundings in the device
  path); on small outputs, where one near-tie already moves the fraction by
  more than 0.1%, up to SMALL_SAMPLE_SLACK non-exact outputs also pass.

No fp32 accumulation can hold 2 ULP on every output.  Where a dot product
nearly cancels, its relative error is unbounded; and where G lies within the
fp32 error of a bf16 rounding boundary, any summation order may round g (or u)
to either neighbour, and silu(g)*u turns that one-ULP step into up to ~3 ULP
of the output.  Both are outputs with several correct results.  An output
that fails the strict check therefore passes only if it lies in its
*admissible interval*: the oracle's epilogue applied over every gate and up
pre-activation that an fp32 sum of depth ``d`` can reach,
``G +- gamma_d * sum|h*w|`` with ``gamma_d = d*2^-24 / (1 - d*2^-24)`` (the
order-independent error bound of a floating-point inner product), widened by
2 ULP.  ``d`` counts rounding steps in units of 2^-24; a kernel whose adder
may truncate states twice its chain length.  Such outputs are counted and
reported with their condition number ``kappa = sum|h*w| / |sum h*w|``.

``compare_linear`` applies the same bars to a plain projection (one bf16
rounding of the dot, no epilogue): there the admissible interval is the
rounding of every reachable sum, ``[RNE(G - tau), RNE(G + tau)]``, exactly
(rounding is monotone), with no widening.  Where one call writes several
projections, the bit-exact fraction is a rate over all outputs of the call
(``pooled_bit_exact_ok``), as it is over all M x N outputs of one dual call;
the per-output and mean bars still hold for each projection.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from . import DualGemvResult, LinearResult, round_bf16, silu_bf16

U32 = 2.0 ** -24  # unit roundoff of fp32
SMALL_SAMPLE_SLACK = 3  # non-bit-exact outputs always allowed (each still within the ULP bar)

# Every report made in this process, so that a test session can state how much of the bar's
# slack was used: outputs admitted by the interval, of those the ones inside only its +-2 ULP
# widening, reports that met the bit-exact bar only through SMALL_SAMPLE_SLACK, and grouped
# calls that met it only as a pooled rate.
LEDGER: list = []
POOLED_ONLY: list = []


def slack_summary() -> dict:
    reps = [r for r in LEDGER]
    return {"reports": len(reps), "outputs": sum(r.n for r in reps),
            "over_2ulp": sum(r.over_2ulp for r in reps),
            "interval_pass": sum(r.interval_pass for r in reps),
            "widened_pass": sum(r.widened_pass for r in reps),
            "small_sample_slack_reports": sum(1 for r in reps if r.slack_used),
            "pooled_only_calls": len(POOLED_ONLY),
            "failures": sum(r.failures for r in reps)}


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):  # signalling NaN patterns widen quietly
        return b.view(np.float32).astype(np.float64)


def is_nan_bits(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


def ordered(bits: np.ndarray) -> np.ndarray:
    """Sign-magnitude bf16 codes mapped to integers that count ULPs (+0 == -0)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def from_ordered(o: np.ndarray) -> np.ndarray:
    o = np.asarray(o, dtype=np.int64)
    return np.where(o < 0, 0x8000 | (-o), o).astype(np.uint16)


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """ULP distance between bf16 bit arrays; NaN vs NaN is 0, NaN vs number is 2^16."""
    na, nb = is_nan_bits(a), is_nan_bits(b)
    d = np.abs(ordered(a) - ordered(b))
    d = np.where(na & nb, 0, d)
    return np.where(na ^ nb, 1 << 16, d)


def gamma(depth: int) -> float:
    du = depth * U32
    return du / (1.0 - du)


def _admissible_range(pre: float, abs_sum: float, depth: int, k_len: int):
    """Smallest and largest bf16 (ordered codes) that rounding any reachable sum can give."""
    tau = gamma(depth) * abs_sum + k_len * 2.0 ** -53 * abs_sum  # device bound + oracle's own fp64 error
    lo, hi = round_bf16(np.array([pre - tau, pre + tau]))
    return int(ordered(lo)), int(ordered(hi))


def admissible_bf16_set(pre: float, abs_sum: float, depth: int, k_len: int) -> np.ndarray:
    """Every bf16 (bits) that rounding a reachable fp32 sum of depth ``depth`` can give."""
    lo, hi = _admissible_range(pre, abs_sum, depth, k_len)
    return from_ordered(np.arange(lo, hi + 1))


def admissible_out_range(G: float, U: float, Ga: float, Ua: float, depth: int, k_len: int):
    """Ordered-code interval of outputs reachable from any admissible (g, u)."""
    g_lo, g_hi = _admissible_range(G, Ga, depth, k_len)
    u_lo, u_hi = _admissible_range(U, Ua, depth, k_len)
    g_set = from_ordered(np.arange(g_lo, g_hi + 1))
    s = bf16_to_f64(silu_bf16(g_set))
    s_min, s_max = float(np.min(s)), float(np.max(s))
    u_min, u_max = float(bf16_to_f64(from_ordered(np.array([u_lo])))[0]), \
        float(bf16_to_f64(from_ordered(np.array([u_hi])))[0])
    corners = np.array([s_min * u_min, s_min * u_max, s_max * u_min, s_max * u_max])
    # fp32 product then bf16 rounding, both monotone: the corner extremes bound the set
    p32 = corners.astype(np.float32).astype(np.float64)
    codes = ordered(round_bf16(p32))
    return int(codes.min()), int(codes.max())


@dataclass
class Report:
    n: int = 0
    max_ulp: int = 0
    over_2ulp: int = 0
    interval_pass: int = 0
    interval_max_kappa: float = 0.0
    interval_min_kappa: float = float("inf")
    widened_pass: int = 0  # interval passes inside the +-2 ULP widening only (compare)
    failures: int = 0
    bit_exact_frac: float = 1.0
    mean_rel: float = 0.0
    failure_idx: List[int] = field(default_factory=list)
    failure_info: List[dict] = field(default_factory=list)

    @property
    def bit_exact_ok(self) -> bool:
        inexact = round((1.0 - self.bit_exact_frac) * self.n)
        return self.bit_exact_frac >= 0.999 or inexact <= SMALL_SAMPLE_SLACK

    @property
    def slack_used(self) -> bool:
        """The bit-exact bar was met only through SMALL_SAMPLE_SLACK."""
        return self.bit_exact_frac < 0.999 and self.bit_exact_ok

    @property
    def ok(self) -> bool:
        return self.failures == 0 and self.bit_exact_ok and self.mean_rel <= 3e-3

    @property
    def inexact(self) -> int:
        return int(round((1.0 - self.bit_exact_frac) * self.n))

    def summary(self) -> str:
        s = (f"n={self.n} max_ulp={self.max_ulp} over2={self.over_2ulp} "
             f"interval_pass={self.interval_pass} (kappa {self.interval_min_kappa:.3g}..{self.interval_max_kappa:.3g}; "
             f"{self.widened_pass} only in the widening) "
             f"failures={self.failures} bit_exact={self.bit_exact_frac:.6f}{' (slack)' if self.slack_used else ''} "
             f"mean_rel={self.mean_rel:.3e}")
        if self.failure_info:
            s += f" first failures: {self.failure_info[:3]}"
        return s


def compare(got: np.ndarray, ref: DualGemvResult, depth: int, k_len: int,
            max_listed: int = 20) -> Report:
    """Check device output bits ``got`` against the oracle's result ``ref``.

    ``depth`` is the longest chain of fp32 additions the device sum can take for
    one output (per-lane terms plus reduction levels); ``k_len`` is K.
    """
    got = np.asarray(got, dtype=np.uint16).ravel()
    want = np.asarray(ref.out, dtype=np.uint16).ravel()
    if got.shape != want.shape:
        raise ValueError(f"size mismatch {got.shape} vs {want.shape}")
    rep = Report(n=int(got.size))
    if got.size == 0:
        return rep
    d = ulp_distance(got, want)
    rep.max_ulp = int(d.max())
    rep.bit_exact_frac = float(np.mean((got == want) | (is_nan_bits(got) & is_nan_bits(want))))
    w = bf16_to_f64(want)
    g = bf16_to_f64(got)
    nz = (w != 0) & np.isfinite(w) & np.isfinite(g)
    rep.mean_rel = float(np.mean(np.abs(g[nz] - w[nz]) / np.abs(w[nz]))) if nz.any() else 0.0
    bad = np.nonzero(d > 2)[0]
    rep.over_2ulp = int(bad.size)
    G, U = np.asarray(ref.gate_pre).ravel(), np.asarray(ref.up_pre).ravel()
    Ga, Ua = np.asarray(ref.gate_abs).ravel(), np.asarray(ref.up_abs).ravel()
    for i in bad:
        kappa = max(Ga[i] / abs(G[i]) if G[i] != 0 else np.inf,
                    Ua[i] / abs(U[i]) if U[i] != 0 else np.inf)
        o = int(ordered(got[i:i + 1])[0])
        ok = False
        lo = hi = None
        if not is_nan_bits(got[i:i + 1])[0]:
            lo, hi = admissible_out_range(float(G[i]), float(U[i]), float(Ga[i]), float(Ua[i]),
                                          depth, k_len)
            ok = lo - 2 <= o <= hi + 2
        if ok:
            rep.interval_pass += 1
            rep.widened_pass += int(not (lo <= o <= hi))
            rep.interval_max_kappa = max(rep.interval_max_kappa, float(kappa))
            rep.interval_min_kappa = min(rep.interval_min_kappa, float(kappa))
        else:
            rep.failures += 1
            if len(rep.failure_idx) < max_listed:
                rep.failure_idx.append(int(i))
                info = {"index": int(i), "got": f"{int(got[i]):#06x}", "want": f"{int(want[i]):#06x}",
                        "ulp": int(d[i]), "kappa": float(kappa), "G": float(G[i]), "U": float(U[i]),
                        "sum_abs_g": float(Ga[i]), "sum_abs_u": float(Ua[i])}
                if lo is not None:
                    info["interval"] = [lo, hi, o]
                rep.failure_info.append(info)
    LEDGER.append(rep)
    return rep


def compare_linear(got: np.ndarray, ref: LinearResult, depth: int, k_len: int, max_listed: int = 20) -> Report:
    """Check device output bits of one plain projection against the oracle's ``linear`` result."""
    got = np.asarray(got, dtype=np.uint16).ravel()
    want = np.asarray(ref.out, dtype=np.uint16).ravel()
    if got.shape != want.shape:
        raise ValueError(f"size mismatch {got.shape} vs {want.shape}")
    rep = Report(n=int(got.size))
    if got.size == 0:
        return rep
    d = ulp_distance(got, want)
    rep.max_ulp = int(d.max())
    rep.bit_exact_frac = float(np.mean((got == want) | (is_nan_bits(got) & is_nan_bits(want))))
    w = bf16_to_f64(want)
    g = bf16_to_f64(got)
    nz = (w != 0) & np.isfinite(w) & np.isfinite(g)
    rep.mean_rel = float(np.mean(np.abs(g[nz] - w[nz]) / np.abs(w[nz]))) if nz.any() else 0.0
    bad = np.nonzero(d > 2)[0]
    rep.over_2ulp = int(bad.size)
    P, A = np.asarray(ref.pre).ravel(), np.asarray(ref.abs).ravel()
    for i in bad:
        kappa = A[i] / abs(P[i]) if P[i] != 0 else np.inf
        o = int(ordered(got[i:i + 1])[0])
        ok = False
        lo = hi = None
        if not is_nan_bits(got[i:i + 1])[0]:
            lo, hi = _admissible_range(float(P[i]), float(A[i]), depth, k_len)
            ok = lo <= o <= hi
        if ok:
            rep.interval_pass += 1
            rep.interval_max_kappa = max(rep.interval_max_kappa, float(kappa))
            rep.interval_min_kappa = min(rep.interval_min_kappa, float(kappa))
        else:
            rep.failures += 1
            if len(rep.failure_idx) < max_listed:
                rep.failure_idx.append(int(i))
                info = {"index": int(i), "got": f"{int(got[i]):#06x}", "want": f"{int(want[i]):#06x}",
                        "ulp": int(d[i]), "kappa": float(kappa), "pre": float(P[i]), "sum_abs": float(A[i])}
                if lo is not None:
                    info["interval"] = [lo, hi, o]
                rep.failure_info.append(info)
    LEDGER.append(rep)
    return rep


def compare_grad_sum(got: np.ndarray, want: np.ndarray, A: np.ndarray, Aabs: np.ndarray, B: np.ndarray,
                     Babs: np.ndarray, depth: int, k_len: int, max_listed: int = 20) -> Report:
    """Check the bf16 sum of two single-rounded contractions, RNE(fl32(RNE(A) + RNE(B))) (the
    gradient of hidden in the backward), against the oracle's bits ``want``.  The same bars as
    ``compare``; an output over 2 ULP passes only inside the sum of the two admissible intervals
    (rounding and fp32 addition are monotone, so the interval's ends bound every reachable value)."""
    got = np.asarray(got, dtype=np.uint16).ravel()
    want = np.asarray(want, dtype=np.uint16).ravel()
    if got.shape != want.shape:
        raise ValueError(f"size mismatch {got.shape} vs {want.shape}")
    rep = Report(n=int(got.size))
    if got.size == 0:
        return rep
    d = ulp_distance(got, want)
    rep.max_ulp = int(d.max())
    rep.bit_exact_frac = float(np.mean((got == want) | (is_nan_bits(got) & is_nan_bits(want))))
    w = bf16_to_f64(want)
    g = bf16_to_f64(got)
    nz = (w != 0) & np.isfinite(w) & np.isfinite(g)
    rep.mean_rel = float(np.mean(np.abs(g[nz] - w[nz]) / np.abs(w[nz]))) if nz.any() else 0.0
    bad = np.nonzero(d > 2)[0]
    rep.over_2ulp = int(bad.size)
    A, Aa, B, Ba = (np.asarray(x, dtype=np.float64).ravel() for x in (A, Aabs, B, Babs))
    for i in bad:
        ok = False
        if not is_nan_bits(got[i:i + 1])[0]:
            a_lo, a_hi = _admissible_range(float(A[i]), float(Aa[i]), depth, k_len)
            b_lo, b_hi = _admissible_range(float(B[i]), float(Ba[i]), depth, k_len)
            ends = bf16_to_f64(from_ordered(np.array([a_lo, a_hi, b_lo, b_hi])))
            sums = np.array([ends[0] + ends[2], ends[1] + ends[3]]).astype(np.float32).astype(np.float64)
            lo, hi = (int(x) for x in ordered(round_bf16(sums)))
            o = int(ordered(got[i:i + 1])[0])
            ok = lo <= o <= hi
        if ok:
            rep.interval_pass += 1
        else:
            rep.failures += 1
            if len(rep.failure_idx) < max_listed:
                rep.failure_idx.append(int(i))
                rep.failure_info.append({"index": int(i), "got": f"{int(got[i]):#06x}",
                                         "want": f"{int(want[i]):#06x}", "ulp": int(d[i])})
    LEDGER.append(rep)
    return rep


def compare_strict_bits(got: np.ndarray, want: np.ndarray) -> Optional[np.ndarray]:
    """Indices where two bf16 bit arrays differ (NaN matches NaN); None when identical."""
    got = np.asarray(got, dtype=np.uint16).ravel()
    want = np.asarray(want, dtype=np.uint16).ravel()
    diff = (got != want) & ~(is_nan_bits(got) & is_nan_bits(want))
    idx = np.nonzero(diff)[0]
    return idx if idx.size else None


def pooled_bit_exact_ok(reports: List[Report]) -> bool:
    """The bit-exact bar over every output of one call that writes several projections."""
    n = sum(r.n for r in reports)
    inexact = sum(r.inexact for r in reports)
    ok = n == 0 or inexact <= 1e-3 * n or inexact <= SMALL_SAMPLE_SLACK
    if ok and not all(r.bit_exact_ok for r in reports):
        POOLED_ONLY.append((n, inexact))
    return ok
