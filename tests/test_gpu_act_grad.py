"""The backward's elementwise step on every bf16 gate value, bitwise, on each kernel that forms it
(needs an MI355X).

dg and du (the workspace head after glu_dual_gemv_backward) follow from the forward's bf16 g and u
and the upstream gradient alone.  With every row of hidden equal to e_0 (1 at column 0, zeros
elsewhere), G[m][j] = gate_w[j][0] and U[m][j] = up_w[j][0] exactly: every other product is +0,
so only -0 becomes +0 (a sum that adds +0 to -0).  gate_w[:, 0] then runs over all 65536 bf16 bit
patterns (NaN, infinities, subnormals included, spread over calls of 16384 rows), up_w[:, 0] and
dout over seeded permutations of all patterns, and dg, du must equal the oracle's elementwise
step bit for bit (a NaN only as a NaN).  The shapes pick the kernel that forms the step: the
one-pass kernel (M = 1), the 4-row MFMA kernel's epilogue (M = 4, 8 and 16 at K = 8), the separate
elementwise kernel after the grouped GEMV (M = 8 at K = 4104, M = 24 at K = 8), the slice-major
8-row kernel's epilogue (M = 16, 40, 64 at K = 2560) and the tiled GEMM's epilogue (M = 100).
"""
import numpy as np
import pytest
import torch

from oracle.backward import act_grads
from glu_mlp_gemv_amd import api

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ROWS = 16384  # weight rows per call: the slice-major kernel covers them in one launch


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def as_bf16(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(b.astype(np.uint16).view(np.int16)).view(torch.bfloat16)


def same_bits(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    nan_g = (got & 0x7FFF) > 0x7F80
    nan_r = (ref & 0x7FFF) > 0x7F80
    return np.where(nan_r, nan_g, (got == ref) & ~nan_g)


@pytest.mark.parametrize("M,K", [(1, 8), (4, 8), (8, 8), (8, 4104), (16, 8), (24, 8), (16, 2560), (40, 2560),
                                 (64, 2560), (100, 64)])
@pytest.mark.parametrize("part", range(65536 // ROWS))
def test_act_grad_every_gate_value(M, K, part):
    N = ROWS
    rng = np.random.default_rng(1000 + part)
    g_bits = np.arange(part * N, (part + 1) * N, dtype=np.uint32).astype(np.uint16)
    u_bits = rng.permutation(65536)[:N].astype(np.uint16)
    go_bits = np.stack([rng.permutation(65536)[:N] for _ in range(M)]).astype(np.uint16)
    p = api.backward_plan(M, N, K)
    fwd = api.plan(M, N, K)["kernel_symbol"]
    print(f"[act_grad] M={M} N={N} K={K} part={part} launches={p['launches']} forward={fwd}", flush=True)
    if (M, K) in ((16, 2560), (40, 2560), (64, 2560)):
        assert fwd.startswith("glu::mfma8_pass_kernel") and p["launches"] == 5  # the epilogue form
    if (M, K) in ((4, 8), (8, 8), (16, 8)):
        assert fwd.startswith("glu::mfma_kernel<") and p["launches"] in (3, 5)  # the 4-row kernel's epilogue
    if (M, K) in ((8, 4104), (24, 8)):
        assert p["launches"] in (4, 6)  # the separate elementwise kernel
    if M == 100:
        assert p["launches"] == 5

    h = torch.zeros(M, K, dtype=torch.bfloat16, device=DEV)
    h[:, 0] = 1.0
    wg = torch.zeros(N, K, dtype=torch.bfloat16, device=DEV)
    wu = torch.zeros(N, K, dtype=torch.bfloat16, device=DEV)
    wg[:, 0] = as_bf16(g_bits).to(DEV)
    wu[:, 0] = as_bf16(u_bits).to(DEV)
    go = as_bf16(go_bits).to(DEV)
    ws = torch.empty(max(api.backward_workspace_bytes(M, N, K), 1), dtype=torch.uint8, device=DEV)
    api.dual_gemv_backward(h, wg, wu, go, workspace=ws)
    torch.cuda.synchronize()
    head = bits(ws[:4 * M * N].view(torch.bfloat16)).reshape(2, M, N)

    def forward_value(b):  # the forward's bf16 value: -0 comes out as +0
        return np.where(b == 0x8000, 0, b).astype(np.uint16)

    g_eff = np.broadcast_to(forward_value(g_bits), (M, N))
    u_eff = np.broadcast_to(forward_value(u_bits), (M, N))
    _, du_ref, dg_ref = act_grads(np.ascontiguousarray(g_eff), np.ascontiguousarray(u_eff), go_bits)
    ok_g = same_bits(head[0], dg_ref)
    ok_u = same_bits(head[1], du_ref)
    bad = np.argwhere(~(ok_g & ok_u))
    if bad.size:
        m, j = bad[0]
        print(f"[act_grad] first mismatch m={m} j={j}: g={g_eff[m, j]:#06x} u={u_eff[m, j]:#06x} "
              f"go={go_bits[m, j]:#06x} dg {head[0][m, j]:#06x} vs {dg_ref[m, j]:#06x}, "
              f"du {head[1][m, j]:#06x} vs {du_ref[m, j]:#06x}", flush=True)
    assert bad.size == 0, f"{len(bad)} of {M * N} outputs differ"
