"""glu_dual_gemv_backward_noalloc, the backward for callers that cannot allocate: through the C ABI,
bitwise against glu_dual_gemv_backward with a workspace on the same inputs, on two calls in a
row on one GPU (the second smaller, so it runs on what the first left in the library's array).

The two entry points run the same kernels in the same order and every kernel's summation order
is fixed, so their outputs are equal bit for bit (the bar for results that are deterministic);
the workspace variant itself is held to the oracle by tests/test_gpu_backward.py.
"""
import numpy as np
import pytest
import torch

from glu_mlp_gemv_amd import api, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def one(M, N, K, seed):
    h, (wg, wu), go = inputs.hidden(M, K, seed), inputs.weights(N, K, seed), inputs.grad_out(M, N, seed)
    h, wg, wu, go = (t.to(DEV) for t in (h, wg, wu, go))
    print(f"[noalloc] M={M} N={N} K={K} plan={api.backward_plan(M, N, K)}", flush=True)
    ref = api.dual_gemv_backward(h, wg, wu, go)
    outs = tuple(torch.full(t.shape, 3.0, dtype=torch.bfloat16, device=DEV) for t in ref)
    got = api.dual_gemv_backward_noalloc(h, wg, wu, go, *outs)
    torch.cuda.synchronize()
    assert all(g is o for g, o in zip(got, outs)), "the given outputs are written in place"
    for name, a, b in zip(("dhidden", "dgate_w", "dup_w"), got, ref):
        assert np.array_equal(bits(a), bits(b)), f"{name} differs from the workspace entry point"


@pytest.mark.parametrize("first,second", [
    ((64, 9216, 2560), (16, 4096, 2560)),    # matrix-core contractions, then a smaller one
    ((128, 9216, 2560), (2, 1000, 512)),     # above 64 rows (GEMM regime), then one pass
    ((1, 9216, 2560), (5, 3000, 1024)),      # one pass, then grouped GEMV + contraction
    ((4, 12288, 4096), (1, 700, 4104)),      # K split over a workgroup, twice
])
def test_noalloc_backward_equals_workspace_entry(first, second):
    one(*first, seed=81)
    one(*second, seed=82)


def test_noalloc_empty_sums_and_limit():
    """M == 0 zero-fills both weight gradients without touching the array; a shape past the
    array's size is refused before any launch."""
    K, N = 64, 5
    dwg = torch.full((N, K), 5.0, dtype=torch.bfloat16, device=DEV)
    dwu = torch.full((N, K), 5.0, dtype=torch.bfloat16, device=DEV)
    api.dual_gemv_backward_noalloc(torch.zeros(0, K, dtype=torch.bfloat16, device=DEV),
                                   torch.ones(N, K, dtype=torch.bfloat16, device=DEV),
                                   torch.ones(N, K, dtype=torch.bfloat16, device=DEV),
                                   torch.zeros(0, N, dtype=torch.bfloat16, device=DEV),
                                   dhidden=torch.zeros(0, K, dtype=torch.bfloat16, device=DEV), dgate_w=dwg,
                                   dup_w=dwu)
    torch.cuda.synchronize()
    assert (bits(dwg) == 0).all() and (bits(dwu) == 0).all()
    M, N, K = 512, 9216, 2560
    assert api.backward_workspace_bytes(M, N, K) > api.NOALLOC_SCRATCH_BYTES
    h = torch.zeros(M, K, dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(N, K, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(api.GluError) as e:
        api.dual_gemv_backward_noalloc(h, w, w.clone(), torch.zeros(M, N, dtype=torch.bfloat16, device=DEV))
    assert e.value.status == api.GLU_ERR_SCRATCH_LIMIT
