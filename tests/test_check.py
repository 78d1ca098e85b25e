"""The parity checker (oracle/check.py) against simulated fp32 kernels (CPU only).

A kernel that sums in fp32 (any order) and then applies the exact epilogue
must pass; the same output with a planted error on a well-conditioned output
must fail; an output whose gate sits on a bf16 rounding boundary must be
admitted with either neighbour.
"""
import numpy as np
import torch

import oracle
from oracle import check
from glu_mlp_gemv_amd import inputs


def bits_of(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def fp32_kernel(h, wg, wu, order):
    """bf16 output of an fp32 accumulation in a given summation order, exact epilogue."""
    hf = h.float().numpy()
    res = []
    for w in (wg, wu):
        wf = w.float().numpy()
        prods = (hf[:, None, :] * wf[None, :, :]).astype(np.float32)  # exact bf16 products
        if order == "sequential":
            acc = np.zeros(prods.shape[:2], np.float32)
            for k in range(prods.shape[2]):
                acc = (acc + prods[:, :, k]).astype(np.float32)
        else:  # 64 strided lanes, then a pairwise tree over the lanes
            K = prods.shape[2]
            lanes = np.zeros(prods.shape[:2] + (64,), np.float32)
            for k in range(K):
                lanes[:, :, k % 64] = (lanes[:, :, k % 64] + prods[:, :, k]).astype(np.float32)
            while lanes.shape[2] > 1:
                lanes = (lanes[:, :, ::2] + lanes[:, :, 1::2]).astype(np.float32)
            acc = lanes[:, :, 0]
        res.append(acc)
    g = oracle.round_bf16(res[0].astype(np.float64))
    u = oracle.round_bf16(res[1].astype(np.float64))
    return oracle.epilogue(g, u)


def test_fp32_kernels_pass_and_planted_errors_fail():
    h, wg, wu = inputs.case("tail_k1024_n3000", M=2, seed=11)
    ref = oracle.dual_gemv(bits_of(h), bits_of(wg), bits_of(wu), with_pre=True)
    for order, depth in (("sequential", 1024), ("lanes", 1024 // 64 + 6)):
        got = fp32_kernel(h, wg, wu, order)
        rep = check.compare(got, ref, depth=depth, k_len=1024)
        assert rep.ok, (order, rep.summary())
        assert rep.bit_exact_frac > 0.999
    # plant a 4-ULP error on the best-conditioned output: must be rejected
    kappa = np.maximum(ref.gate_abs / np.abs(ref.gate_pre), ref.up_abs / np.abs(ref.up_pre)).ravel()
    i = int(np.argmin(kappa))
    bad = got.ravel().copy()
    o = check.ordered(bad[i:i + 1])[0]
    bad[i] = check.from_ordered(np.array([o + 4]))[0]
    rep = check.compare(bad, ref, depth=depth, k_len=1024)
    assert rep.failures == 1 and not rep.ok
    # a systematic 1-ULP bias on every output fails the bit-exact bar
    biased = check.from_ordered(check.ordered(got.ravel()) + 1)
    rep2 = check.compare(biased, ref, depth=depth, k_len=1024)
    assert not rep2.ok
    # the planted errors are not results of the device path: keep them out of the session's slack report
    check.LEDGER.remove(rep)
    check.LEDGER.remove(rep2)


def test_gate_on_a_rounding_boundary_admits_both_neighbours():
    # G = 2.7578125 - 3.8e-7 (just below the midpoint of bf16 2.75 and 2.765625), U = 0.584
    G = 2.7578125 - 3.8e-7
    U = 0.5840484601212665
    sums = 70.0  # sum |h*w| of a K=5120 row: kappa ~ 25
    lo, hi = check.admissible_out_range(G, U, sums, sums, depth=2 * (40 + 7), k_len=5120)
    outs = oracle.epilogue(oracle.round_bf16(np.array([2.75, 2.765625])), oracle.round_bf16(np.array([U, U])))
    codes = check.ordered(outs)
    assert lo <= codes.min() and codes.max() <= hi
    # and a gate far from any boundary with a tight depth admits a narrow range only
    lo2, hi2 = check.admissible_out_range(1.2, 0.5, 1.3, 0.6, depth=46, k_len=2560)
    assert hi2 - lo2 <= 2


def test_nan_matches_only_nan():
    a = np.array([0x7FC0, 0x7FC1, 0x3F80], np.uint16)
    b = np.array([0xFFC0, 0x3F80, 0x7FC0], np.uint16)
    d = check.ulp_distance(a, b)
    assert d[0] == 0 and d[1] == 1 << 16 and d[2] == 1 << 16
    assert check.ulp_distance(np.array([0x0000], np.uint16), np.array([0x8000], np.uint16))[0] == 0
