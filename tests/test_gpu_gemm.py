"""GPU parity of the tiled dual GEMM (M > 64) against the oracle, through the C ABI
(needs an MI355X).

The bar is the one of oracle/check.py.  Shapes cover ragged M, N and K tails
and every tile shape; the prefill-like full size (K=5120, N=17408, M=256) is
checked on sampled rows of hidden that the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import check
from glu_mlp_gemv_amd import api, inputs
from cases import GEMM_SHAPES, GEMM_TILES

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NAN = 0x7FC0
CANARY = 0x1234


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("tile", range(len(GEMM_TILES)))
@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_parity(M, N, K, tile):
    kw = dict(kernel=api.KERNEL_GEMM, **GEMM_TILES[tile])
    t = api.make_tuning(**kw)
    h, wg, wu = inputs.hidden(M, K, 41), *inputs.weights(N, K, 41)
    plan = api.plan(M, N, K, True, t)
    say(f"[gemm] M={M} N={N} K={K} {kw} plan={plan}")
    got = bits(api.dual_gemv(h.to(DEV), wg.to(DEV), wu.to(DEV), tuning=t))
    torch.cuda.synchronize()
    ref = oracle.dual_gemv(bits(h), bits(wg), bits(wu), with_pre=True)
    rep = check.compare(got, ref, depth=plan["accum_depth"], k_len=K)
    say(f"[gemm] {rep.summary()}")
    assert rep.ok, rep.summary()


def test_gemm_default_for_large_m():
    assert api.plan(65, 1000, 1024)["kernel"] == api.KERNEL_GEMM
    assert api.plan(64, 1000, 1024)["kernel"] == api.KERNEL_MFMA
    assert api.plan(33, 1000, 1024)["kernel"] == api.KERNEL_MFMA


@pytest.mark.parametrize("M,seed", [(256, 0), (96, 1)])
def test_gemm_prefill_full_size_sampled(M, seed):
    """K=5120, N=17408 with 1 % outliers (the batched workload's weights): the whole output
    from the GPU, the oracle on a sample of rows of hidden (first, last, and random)."""
    h, wg, wu = inputs.case("mfma_k5120_n17408", M=32, seed=seed)
    K = h.shape[1]
    hh = inputs.hidden(M, K, 50 + seed)
    hh[:32] = h
    plan = api.plan(M, wg.shape[0], K)
    say(f"[gemm] full size M={M} plan={plan}")
    got = bits(api.dual_gemv(hh.to(DEV), wg.to(DEV), wu.to(DEV)))
    torch.cuda.synchronize()
    rows = sorted({0, 31, M - 1, *np.random.default_rng(seed).integers(0, M, 3).tolist()})
    ref = oracle.dual_gemv(bits(hh[rows]), bits(wg), bits(wu), with_pre=True)
    rep = check.compare(got[rows], ref, depth=plan["accum_depth"], k_len=K)
    say(f"[gemm] rows {rows}: {rep.summary()}")
    assert rep.ok, rep.summary()


def test_gemm_rows_permute_bitwise():
    """Every output position is summed in the same order, so permuting the rows of hidden
    permutes the output rows bitwise (rows land in other tiles and other waves)."""
    M, N, K = 150, 700, 1024
    h, wg, wu = inputs.hidden(M, K, 42), *inputs.weights(N, K, 42)
    perm = np.random.default_rng(42).permutation(M)
    a = bits(api.dual_gemv(h.to(DEV), wg.to(DEV), wu.to(DEV)))
    b = bits(api.dual_gemv(h[perm].to(DEV), wg.to(DEV), wu.to(DEV)))
    torch.cuda.synchronize()
    assert np.array_equal(a[perm], b)
    c = bits(api.dual_gemv(h.to(DEV), wg.to(DEV), wu.to(DEV)))
    torch.cuda.synchronize()
    assert np.array_equal(a, c), "repeated calls must be bitwise equal"


@pytest.mark.parametrize("tile", [dict(), dict(gemm_tile_n=128, gemm_tile_m=128)])
def test_gemm_strided_operands_and_canaries(tile):
    """Operands inside wider buffers whose gaps hold NaN, output rows inside wider rows holding a
    canary: a read past K or a write past N shows."""
    M, N, K = 100, 300, 1032
    pads = (8, 16, 24, 5)
    h, wg, wu = inputs.hidden(M, K, 43), *inputs.weights(N, K, 43)

    def widened(x, pad):
        R, C = x.shape
        buf = torch.full((R, C + pad), NAN, dtype=torch.int16).view(torch.bfloat16)
        buf[:, :C] = x
        return buf.to(DEV)[:, :C]
    hs, gs, us = widened(h, pads[0]), widened(wg, pads[1]), widened(wu, pads[2])
    ob = torch.full((M, N + pads[3]), CANARY, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    t = api.make_tuning(kernel=api.KERNEL_GEMM, **tile)
    api.dual_gemv(hs, gs, us, out=ob[:, :N], tuning=t)
    torch.cuda.synchronize()
    got = bits(ob)
    assert (got[:, N:] == CANARY).all(), "a write landed between output rows"
    ref = oracle.dual_gemv(bits(h), bits(wg), bits(wu), with_pre=True)
    rep = check.compare(got[:, :N], ref, depth=api.plan(M, N, K, True, t)["accum_depth"], k_len=K)
    say(f"[gemm] strided {tile}: {rep.summary()}")
    assert rep.ok, rep.summary()


def test_gemm_nan_rows_stay_in_their_rows():
    """A NaN in one row of hidden and one weight row poisons exactly that output row and column."""
    M, N, K = 80, 200, 512
    h, wg, wu = inputs.hidden(M, K, 44), *inputs.weights(N, K, 44)
    hb, gb = bits(h).copy(), bits(wg).copy()
    hb[37, 100] = NAN
    gb[150, 7] = NAN
    h2 = torch.from_numpy(hb.view(np.int16)).view(torch.bfloat16)
    g2 = torch.from_numpy(gb.view(np.int16)).view(torch.bfloat16)
    got = bits(api.dual_gemv(h2.to(DEV), g2.to(DEV), wu.to(DEV)))
    torch.cuda.synchronize()
    nan = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
    want = np.zeros_like(nan)
    want[37, :] = True
    want[:, 150] = True
    assert np.array_equal(nan, want)
