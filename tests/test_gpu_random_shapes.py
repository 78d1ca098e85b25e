"""GPU parity on seeded random shapes through the default planners (needs an MI355X).

The other GPU tests pin each kernel family on chosen shapes; these draw shapes from a seeded
generator instead, so that the planner's routing (VALU, 4-row and 8-row MFMA, one launch of up to
64 rows, the tiled GEMM, the grouped GEMV's kernels, the backward's paths) is crossed with ragged
M, N and K the tables do not list.  Each case prints its shape before it runs; the bar is that of
oracle/check.py, as everywhere.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import check
from glu_mlp_gemv_amd import api, inputs

from test_gpu_backward import check_backward, run_backward
from test_gpu_grouped import check_all, weight_set

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def draw_m(rng, hi):
    # every routing band about equally often: 1, 2-8, 9-32, 33-64, above 64
    band = int(rng.integers(0, 5))
    lo_hi = ((1, 1), (2, 8), (9, 32), (33, 64), (65, hi))[band]
    return int(rng.integers(lo_hi[0], lo_hi[1] + 1))


def draw_nk(rng, M, n_hi, k_hi, budget):
    # N first, then K (a multiple of 8: the fast layout) within the oracle's budget of M*N*K
    N = int(rng.integers(1, min(n_hi, max(1, budget // (M * 64))) + 1))
    kmax = min(k_hi, budget // (M * N)) // 8
    return N, 8 * int(rng.integers(1, max(1, kmax) + 1))


def forward_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = draw_m(rng, 160)
        N, K = draw_nk(rng, M, 3000, 6400, 60_000_000)
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", forward_shapes(24, 2026))
def test_random_forward_default_plan(M, N, K):
    h, wg, wu = inputs.hidden(M, K, 91), *inputs.weights(N, K, 91)
    plan = api.plan(M, N, K)
    print(f"[random] forward M={M} N={N} K={K} plan={plan['kernel_symbol']}", flush=True)
    got = bits(api.dual_gemv(h.to(DEV), wg.to(DEV), wu.to(DEV)))
    torch.cuda.synchronize()
    ref = oracle.dual_gemv(bits(h), bits(wg), bits(wu), with_pre=True)
    rep = check.compare(got, ref, depth=plan["accum_depth"], k_len=K)
    print(f"[random] {rep.summary()}", flush=True)
    assert rep.ok, rep.summary()


def grouped_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = draw_m(rng, 100)
        step = (1, 4, 8)[int(rng.integers(0, 3))]  # projections' rows: any, multiples of 4 or of 8
        Ns = tuple(step * int(rng.integers(1, 1 + 1200 // step)) for _ in range(int(rng.integers(1, 5))))
        kmax = min(4096, 40_000_000 // (M * sum(Ns))) // 8
        out.append((Ns, 8 * int(rng.integers(1, max(1, kmax) + 1)), M))
    return out


@pytest.mark.parametrize("Ns,K,M", grouped_shapes(16, 2027))
def test_random_grouped_default_plan(Ns, K, M):
    h = inputs.hidden(M, K, 92)
    ws = weight_set(Ns, K, 92)
    outs = api.grouped_gemv(h.to(DEV), [w.to(DEV) for w in ws])
    torch.cuda.synchronize()
    check_all(h, ws, [o.cpu() for o in outs], label="random")


def backward_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = draw_m(rng, 200)
        N, K = draw_nk(rng, M, 2048, 4096, 30_000_000)
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", backward_shapes(16, 2028))
def test_random_backward_default_plan(M, N, K):
    print(f"[random] backward M={M} N={N} K={K} plan={api.backward_plan(M, N, K)}", flush=True)
    h, (wg, wu), go = inputs.hidden(M, K, 93), inputs.weights(N, K, 93), inputs.grad_out(M, N, 93)
    got, dg, du = run_backward(h, wg, wu, go)
    check_backward(h, wg, wu, go, got, dg, du, label="random")
