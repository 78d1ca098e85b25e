"""GPU parity of the backward (glu_dual_gemv_backward) against the oracle's backward, through
the C ABI (needs an MI355X).

Bars (oracle/check.py): dgate_w and dup_w are single roundings of sums over
the M rows of hidden (compare_linear, depth M); dhidden is the bf16 sum of two
single-rounded contractions over the N weight rows (compare_grad_sum, depth
from the backward's plan).  Every output within 2 ULP or its admissible
interval, mean relative error <= 0.3 %, >= 99.9 % bit-exact over the call.
Inputs: hidden N(0,1), weights N(0, 0.02^2), upstream gradient N(0,1).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import LinearResult, check
from oracle.backward import act_grads, contract
from oracle.backward import dual_gemv_backward as oracle_backward
from glu_mlp_gemv_amd import api, autograd, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CANARY = 0x1234


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def say(*a):
    print(*a, flush=True)


def run_backward(h, wg, wu, go, outs=()):
    """The GPU backward on host tensors; returns (dh, dwg, dwu) and the workspace's (dg, du) as bits."""
    M, K = h.shape
    N = wg.shape[0]
    ws = torch.empty(max(api.backward_workspace_bytes(M, N, K), 1), dtype=torch.uint8, device=DEV)
    got = api.dual_gemv_backward(h.to(DEV), wg.to(DEV), wu.to(DEV), go.to(DEV), *outs, workspace=ws)
    torch.cuda.synchronize()
    head = bits(ws[:4 * M * N].view(torch.bfloat16)).reshape(2, M, N)
    return got, head[0], head[1]


def check_backward(h, wg, wu, go, got, dg_gpu, du_gpu, label=""):
    """dg, du: equal to the oracle's, or to what the oracle's elementwise step gives from another
    admissible (g, u) (an fp32 forward sum next to a bf16 rounding boundary may round either way).
    The contractions: against the oracle's contraction of the device's own dg and du."""
    M, K = h.shape
    N = wg.shape[0]
    hb, gb, ub, ob = bits(h), bits(wg), bits(wu), bits(go)
    ref = oracle_backward(hb, gb, ub, ob)
    diff = np.argwhere((dg_gpu != ref.dg) | (du_gpu != ref.du))
    if diff.size:
        fwd = oracle.dual_gemv(hb, gb, ub, with_pre=True)
        # G and U come from the grouped GEMV, from the forward's kernel for the shape (whose depth the
        # backward's plan includes) or from the backward's one-pass kernel
        depth = max(api.grouped_plan(M, K, 2 * N, True, None, N % 4 == 0, N % 8 == 0)["accum_depth"],
                    api.backward_plan(M, N, K)["accum_depth"])
        for m, j in diff:
            g_set = check.admissible_bf16_set(fwd.gate_pre[m, j], fwd.gate_abs[m, j], depth, K)
            u_set = check.admissible_bf16_set(fwd.up_pre[m, j], fwd.up_abs[m, j], depth, K)
            gg, uu = np.meshgrid(g_set, u_set)
            _, du_c, dg_c = act_grads(gg.ravel(), uu.ravel(), np.full(gg.size, ob[m, j], dtype=np.uint16))
            ok = np.any((dg_c == dg_gpu[m, j]) & (du_c == du_gpu[m, j]))
            assert ok, (label, "dg/du from no admissible (g, u)", int(m), int(j), hex(int(dg_gpu[m, j])),
                        hex(int(ref.dg[m, j])), hex(int(du_gpu[m, j])), hex(int(ref.du[m, j])))
    say(f"[backward] {label} M={M} N={N} K={K}: {len(diff)} of {M * N} (dg, du) pairs from a neighbouring "
        f"admissible (g, u)")
    c = contract(hb, gb, ub, dg_gpu, du_gpu)
    dh, dwg, dwu = (bits(t) for t in got)
    plan = api.backward_plan(M, N, K)
    # the weight gradients add the M rows in order (depth M), or on the matrix cores above 8 rows,
    # whose depth the plan's accum_depth covers
    dw_depth = max(M, plan["accum_depth"]) if M > 8 else M
    reps = {
        "dwg": check.compare_linear(dwg, LinearResult(c.dwg, c.dwg_pre, c.dwg_abs), depth=dw_depth, k_len=M),
        "dwu": check.compare_linear(dwu, LinearResult(c.dwu, c.dwu_pre, c.dwu_abs), depth=dw_depth, k_len=M),
        "dh": check.compare_grad_sum(dh, c.dh, c.dhg_pre, c.dhg_abs, c.dhu_pre, c.dhu_abs,
                                     depth=plan["accum_depth"], k_len=N),
    }
    for name, rep in reps.items():
        say(f"[backward] {label} M={M} N={N} K={K} {name}: {rep.summary()}")
        assert rep.failures == 0 and rep.mean_rel <= 3e-3, (name, rep.summary())
    assert check.pooled_bit_exact_ok(list(reps.values())), {k: r.summary() for k, r in reps.items()}
    return reps


CASES = [(1, 9216, 2560), (1, 300, 1032), (2, 1000, 512), (3, 257, 8), (4, 65, 2048), (5, 1, 520),
         (8, 513, 4096), (8, 12288, 4096), (6, 3000, 1024), (7, 64, 40000),
         # one pass with K split over a workgroup: ragged last wave, two chunks a lane, hidden in LDS
         (4, 9216, 3072), (1, 12288, 4096), (2, 700, 2568), (3, 300, 8192), (2, 99, 6152), (3, 255, 4096),
         (2, 257, 2600), (1, 3, 4104), (4, 1, 2576), (4, 4104, 4096), (1, 513, 8192),
         # one pass with a wave per weight row for two rows of hidden (three: the four launches)
         (2, 9216, 2560), (3, 3000, 2048), (2, 1, 520), (3, 65, 1032), (2, 300, 2552),
         # more than 8 rows of hidden: the contractions on the matrix cores (zero-padded operands,
         # ragged row ranges and column tiles, partial 16-row tiles of hidden)
         (9, 700, 1032), (16, 2048, 2560), (33, 300, 520), (64, 1000, 1024), (64, 5, 8), (17, 1000, 2568),
         (40, 333, 520), (48, 4097, 72), (12, 31, 4096), (64, 9216, 2560),
         # 33..64 rows: g and u from one launch of the grouped GEMV's K-slice kernel (N % 8 == 0), ragged
         # stages; with only N % 4 == 0 from the tiled GEMM
         (56, 1024, 2176), (33, 2048, 2560), (36, 1004, 1032),
         # more than 64 rows: g and u from the tiled GEMM (N % 4 == 0; else the grouped GEMV in slices),
         # dh over slices of 64 rows of hidden, the weight gradients as one transposed GEMM (a ragged
         # last 32-row block of the contraction, transposes over several 64-row tiles)
         (65, 700, 1032), (100, 333, 520), (128, 1000, 1024), (96, 4097, 72), (200, 64, 2048),
         (130, 12, 8), (512, 9216, 2560)]


@pytest.mark.parametrize("M,N,K", CASES)
def test_backward_parity(M, N, K):
    h, (wg, wu), go = inputs.hidden(M, K, 71), inputs.weights(N, K, 71), inputs.grad_out(M, N, 71)
    got, dg, du = run_backward(h, wg, wu, go)
    check_backward(h, wg, wu, go, got, dg, du, label="packed")


def test_backward_outliers_and_scaled_row():
    """The batched workload's weights (1 % outliers) and a row of hidden scaled by 8."""
    h, wg, wu = inputs.case("mfma_k5120_n17408", M=16, seed=1)
    h, wg, wu = h[:8].clone(), wg[:4096].clone(), wu[:4096].clone()
    h[0] = (h[0].float() * 8).bfloat16()
    go = inputs.grad_out(8, wg.shape[0], 72)
    got, dg, du = run_backward(h, wg, wu, go)
    check_backward(h, wg, wu, go, got, dg, du, label="outliers")


def test_backward_determinism_and_given_outputs():
    M, N, K = 4, 2000, 1024
    h, (wg, wu), go = inputs.hidden(M, K, 73), inputs.weights(N, K, 73), inputs.grad_out(M, N, 73)
    hd, gd, ud, od = h.to(DEV), wg.to(DEV), wu.to(DEV), go.to(DEV)
    a = [bits(t) for t in api.dual_gemv_backward(hd, gd, ud, od)]
    ws = torch.empty(api.backward_workspace_bytes(M, N, K), dtype=torch.uint8, device=DEV)
    outs = (torch.full((M, K), 7.0, dtype=torch.bfloat16, device=DEV),
            torch.full((N, K), 7.0, dtype=torch.bfloat16, device=DEV),
            torch.full((N, K), 7.0, dtype=torch.bfloat16, device=DEV))
    for _ in range(3):
        api.dual_gemv_backward(hd, gd, ud, od, *outs, workspace=ws)
        torch.cuda.synchronize()
        assert all(np.array_equal(x, bits(y)) for x, y in zip(a, outs)), "repeated calls must be bitwise equal"


def test_backward_canaries_around_outputs():
    """Outputs as views into larger buffers holding a canary before and after: nothing outside is written."""
    M, N, K = 3, 333, 1032
    h, (wg, wu), go = inputs.hidden(M, K, 74), inputs.weights(N, K, 74), inputs.grad_out(M, N, 74)
    pad = 64  # elements; keeps 16-byte alignment of the views
    bufs = [torch.full((n + 2 * pad,), CANARY, dtype=torch.int16, device=DEV).view(torch.bfloat16)
            for n in (M * K, N * K, N * K)]
    views = [b[pad:pad + n].view(shape) for b, n, shape in zip(bufs, (M * K, N * K, N * K), ((M, K), (N, K), (N, K)))]
    _, dg, du = run_backward(h, wg, wu, go, outs=views)
    for b in bufs:
        bb = bits(b)
        assert (bb[:pad] == CANARY).all() and (bb[-pad:] == CANARY).all(), "a write landed outside an output"
    check_backward(h, wg, wu, go, views, dg, du, label="canaries")


def test_backward_empty_sums_are_zero():
    K = 64
    # N == 0: hidden's gradient is an empty sum
    dh = torch.full((2, K), 5.0, dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(0, K, dtype=torch.bfloat16, device=DEV)
    api.dual_gemv_backward(torch.ones(2, K, dtype=torch.bfloat16, device=DEV), w, w,
                           torch.zeros(2, 0, dtype=torch.bfloat16, device=DEV), dhidden=dh,
                           dgate_w=torch.zeros(0, K, dtype=torch.bfloat16, device=DEV),
                           dup_w=torch.zeros(0, K, dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert (bits(dh) == 0).all()
    # M == 0: the weights' gradients are empty sums
    dwg = torch.full((5, K), 5.0, dtype=torch.bfloat16, device=DEV)
    dwu = torch.full((5, K), 5.0, dtype=torch.bfloat16, device=DEV)
    api.dual_gemv_backward(torch.zeros(0, K, dtype=torch.bfloat16, device=DEV),
                           torch.ones(5, K, dtype=torch.bfloat16, device=DEV),
                           torch.ones(5, K, dtype=torch.bfloat16, device=DEV),
                           torch.zeros(0, 5, dtype=torch.bfloat16, device=DEV),
                           dhidden=torch.zeros(0, K, dtype=torch.bfloat16, device=DEV), dgate_w=dwg, dup_w=dwu)
    torch.cuda.synchronize()
    assert (bits(dwg) == 0).all() and (bits(dwu) == 0).all()


def test_backward_gate_zero_closed_form():
    """Wg = 0: g = 0, so du = 0 (dWu = 0), dWg = bf16(sum_m (ds/2) h), dh = bf16(dg @ 0 + 0) = 0."""
    M, N, K = 4, 256, 512
    h, (_, wu), go = inputs.hidden(M, K, 75), inputs.weights(N, K, 75), inputs.grad_out(M, N, 75)
    wg = torch.zeros(N, K, dtype=torch.bfloat16)
    (dh, dwg, dwu), dg, du = run_backward(h, wg, wu, go)
    assert (bits(dwu) & 0x7FFF == 0).all() and (bits(dh) & 0x7FFF == 0).all()
    check_backward(h, wg, wu, go, (dh, dwg, dwu), dg, du, label="gate zero")


@pytest.mark.parametrize("M", [2, 160])
def test_autograd_function_matches_both_entry_points(M):
    """The autograd Function's forward is glu_dual_gemv and its gradients glu_dual_gemv_backward,
    at a decode batch and at a training micro-batch of more than 64 rows."""
    N, K = 700, 1024
    h, (wg, wu), go = inputs.hidden(M, K, 76), inputs.weights(N, K, 76), inputs.grad_out(M, N, 76)
    hd, gd, ud = (t.to(DEV).requires_grad_() for t in (h, wg, wu))
    out = autograd.dual_weight_glu(hd, gd, ud)
    out.backward(go.to(DEV))
    torch.cuda.synchronize()
    fwd = api.dual_gemv(h.to(DEV), wg.to(DEV), wu.to(DEV))
    ref = api.dual_gemv_backward(h.to(DEV), wg.to(DEV), wu.to(DEV), go.to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(fwd))
    for a, b in zip((hd.grad, gd.grad, ud.grad), ref):
        assert np.array_equal(bits(a), bits(b))


# one shape per way the backward runs: the one-pass kernel (M = 1), the K-split pass (M = 2,
# K = 4096), the 4-row kernel's fused first step before the contraction (M = 4) and before the
# matrix-core gradients (M = 12), the grouped GEMV with the separate elementwise kernel (M = 8 at
# K = 4104), the slice-major kernel's fused first step (M = 16, 40) and the tiled GEMM's (M = 100)
GRAPH_SHAPES = [(1, 1000, 1024, 2), (2, 500, 4096, 2), (4, 1000, 1024, 3), (8, 300, 4104, 4), (12, 1000, 1024, 5),
                (16, 1000, 2560, 5), (40, 300, 520, 5), (100, 1000, 520, 5)]


@pytest.mark.parametrize("M,N,K,launches", GRAPH_SHAPES)
def test_backward_graph_replays(M, N, K, launches):
    """A captured backward replays bitwise equal to an eager call, several times, with the outputs
    and the workspace clobbered and unrelated eager work between the replays."""
    assert api.backward_plan(M, N, K)["launches"] == launches
    say(f"[graph] backward M={M} N={N} K={K} launches={launches}")
    h, (wg, wu), go = inputs.hidden(M, K, 31), inputs.weights(N, K, 31), inputs.grad_out(M, N, 31)
    hd, gd, ud, od = h.to(DEV), wg.to(DEV), wu.to(DEV), go.to(DEV)
    ws = torch.empty(max(api.backward_workspace_bytes(M, N, K), 1), dtype=torch.uint8, device=DEV)
    outs = [torch.empty(M, K, dtype=torch.bfloat16, device=DEV), torch.empty(N, K, dtype=torch.bfloat16, device=DEV),
            torch.empty(N, K, dtype=torch.bfloat16, device=DEV)]
    api.dual_gemv_backward(hd, gd, ud, od, *outs, workspace=ws)
    torch.cuda.synchronize()
    eager = [bits(t) for t in outs] + [bits(ws[:4 * M * N].view(torch.bfloat16))]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        api.dual_gemv_backward(hd, gd, ud, od, *outs, workspace=ws)  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.dual_gemv_backward(hd, gd, ud, od, *outs, workspace=ws)
    for i in range(3):
        for t in outs:
            t.fill_(float("nan"))
        ws.fill_(0xA5)
        _ = (hd.float() * 3).sum()  # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        got = [bits(t) for t in outs] + [bits(ws[:4 * M * N].view(torch.bfloat16))]
        for name, a, b in zip(("dhidden", "dgate_w", "dup_w", "dg|du"), got, eager):
            assert np.array_equal(a, b), f"replay {i}: {name}"
