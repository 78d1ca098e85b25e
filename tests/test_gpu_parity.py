"""GPU parity: the HIP path through the C ABI against the oracle (needs an MI355X).

Bar (written out in oracle/check.py): every output within 2 bf16 ULP of the
oracle or inside its admissible interval (the bf16 values the oracle's epilogue
gives over every gate and up sum an fp32 accumulation of the kernel's depth can
reach, widened by 2 ULP; counted and reported, at any kappa), mean relative
error <= 0.3%, bit-exact fraction >= 99.9%.
Integer-exact properties (determinism, row consistency, exhaustive epilogue,
canaries) are checked bitwise.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import check
from glu_mlp_gemv_amd import api, inputs
from cases import EPILOGUE_PATHS, MFMA_SHAPES, MFMA_TUNINGS, SMALL

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_from_bits(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def say(*a):
    print(*a, flush=True)


def gpu_run(h, wg, wu, tuning=None):
    out = api.dual_gemv(h, wg, wu, tuning=tuning)
    torch.cuda.synchronize()
    return out


def parity(h_cpu, wg_cpu, wu_cpu, tuning=None, label=""):
    M, K = h_cpu.shape
    N = wg_cpu.shape[0]
    plan = api.plan(M, N, K, True, tuning)
    say(f"[parity] {label} M={M} N={N} K={K} plan={plan}")
    h, wg, wu = h_cpu.to(DEV), wg_cpu.to(DEV), wu_cpu.to(DEV)
    got = bits(gpu_run(h, wg, wu, tuning))
    ref = oracle.dual_gemv(bits(h_cpu), bits(wg_cpu), bits(wu_cpu), with_pre=True)
    rep = check.compare(got, ref, depth=plan["accum_depth"], k_len=K)
    say(f"[parity] {label}: {rep.summary()}")
    return rep, got, ref


# ---- the workloads at full size ---------------------------------------------

CASES = []
for name, w in inputs.WORKLOADS.items():
    if w.layers > 1:
        continue
    for M in w.Ms:
        for seed in w.seeds:
            CASES.append((name, M, seed))


@pytest.mark.parametrize("name,M,seed", CASES, ids=[f"{n}-M{m}-s{s}" for n, m, s in CASES])
def test_workload_parity(name, M, seed):
    h, wg, wu = inputs.case(name, M=M, seed=seed)
    rep, _, _ = parity(h, wg, wu, label=f"{name} seed {seed}")
    assert rep.ok, rep.summary()


def test_decode_stack_parity():
    """32 layers of K=2560 N=9216 in layer order; every layer's output against the oracle."""
    w = inputs.WORKLOADS["stack32_k2560_n9216"]
    hs = inputs.stack_hidden(0, w.layers, w.K)
    layers = inputs.stack_weights(0, w.layers, w.N, w.K, device=DEV)
    hs_dev = hs.to(DEV)
    outs = [api.dual_gemv(hs_dev[l:l + 1], *layers[l]) for l in range(w.layers)]
    torch.cuda.synchronize()
    depth = api.plan(1, w.N, w.K)["accum_depth"]
    worst = None
    for l in range(w.layers):
        wg, wu = (bits(t) for t in layers[l])
        ref = oracle.dual_gemv(bits(hs[l:l + 1]), wg, wu, with_pre=True)
        rep = check.compare(bits(outs[l]), ref, depth=depth, k_len=w.K)
        assert rep.ok, f"layer {l}: {rep.summary()}"
        if worst is None or rep.bit_exact_frac < worst.bit_exact_frac:
            worst = rep
    say(f"[stack] worst layer: {worst.summary()}")


# ---- ragged and small shapes, every kernel ------------------------------------



@pytest.mark.parametrize("dot", [0, 1])
@pytest.mark.parametrize("M,N,K", SMALL)
def test_small_valu(M, N, K, dot):
    """dot 0: the default (at M = 1 the matrix-core dot products), 1: fp32 FMAs at every M."""
    h, wg, wu = inputs.hidden(M, K, 3), *inputs.weights(N, K, 3)
    t = api.make_tuning(kernel=api.KERNEL_VALU, gemv_dot=dot)
    rep, _, _ = parity(h, wg, wu, tuning=t, label=f"valu dot {dot}")
    assert rep.ok, rep.summary()




@pytest.mark.parametrize("tn", range(len(MFMA_TUNINGS)))
@pytest.mark.parametrize("M,N,K", MFMA_SHAPES)
def test_small_mfma(M, N, K, tn):
    h, wg, wu = inputs.hidden(M, K, 4), *inputs.weights(N, K, 4)
    t = api.make_tuning(kernel=api.KERNEL_MFMA, **MFMA_TUNINGS[tn])
    rep, _, _ = parity(h, wg, wu, tuning=t, label=f"mfma {MFMA_TUNINGS[tn]}")
    assert rep.ok, rep.summary()


@pytest.mark.parametrize("M,N,K", [(1, 300, 1003), (3, 257, 77), (9, 100, 1), (20, 50, 130)])
def test_generic_k_not_multiple_of_8(M, N, K):
    h, wg, wu = inputs.hidden(M, K, 5), *inputs.weights(N, K, 5)
    rep, _, _ = parity(h, wg, wu, label="generic")
    assert rep.ok, rep.summary()


def test_generic_unaligned_pointers():
    M, N, K = 2, 500, 1024
    h, wg, wu = inputs.hidden(M, K, 6), *inputs.weights(N, K, 6)
    # views that start one element (2 bytes) into a larger buffer
    hb = torch.empty(M * K + 1, dtype=torch.bfloat16, device=DEV)[1:].view(M, K)
    gb = torch.empty(N * K + 1, dtype=torch.bfloat16, device=DEV)[1:].view(N, K)
    ub = torch.empty(N * K + 1, dtype=torch.bfloat16, device=DEV)[1:].view(N, K)
    hb.copy_(h); gb.copy_(wg); ub.copy_(wu)
    assert hb.data_ptr() % 16 != 0
    say("[unaligned] generic path")
    got = bits(gpu_run(hb, gb, ub))
    ref = oracle.dual_gemv(bits(h), bits(wg), bits(wu), with_pre=True)
    rep = check.compare(got, ref, depth=api.plan(M, N, K, False)["accum_depth"], k_len=K)
    assert rep.ok, rep.summary()


@pytest.mark.parametrize("kernel", [0, api.KERNEL_GENERIC])
def test_zero_and_empty_sizes(kernel):
    t = api.make_tuning(kernel=kernel) if kernel else None
    out = torch.full((3, 5), 7.0, dtype=torch.bfloat16, device=DEV)
    e = torch.empty(3, 0, dtype=torch.bfloat16, device=DEV)
    w = torch.empty(5, 0, dtype=torch.bfloat16, device=DEV)
    say("[zero] K=0")
    api.dual_gemv(e, w, w, out=out, tuning=t)
    torch.cuda.synchronize()
    assert np.all(bits(out) == 0), "K == 0 must give +0"
    o2 = torch.full((0, 5), 7.0, dtype=torch.bfloat16, device=DEV)
    api.dual_gemv(torch.empty(0, 8, dtype=torch.bfloat16, device=DEV),
                  torch.zeros(5, 8, dtype=torch.bfloat16, device=DEV),
                  torch.zeros(5, 8, dtype=torch.bfloat16, device=DEV), out=o2, tuning=t)
    torch.cuda.synchronize()


# ---- exhaustive epilogue through the public API ------------------------------

def _epilogue_case(u_bits: np.ndarray, tuning):
    """N = 65536 rows: gate row j holds g_j = pattern j at k = 0, so G = g_j exactly."""
    K = 32
    N = 1 << 16
    g_bits = np.arange(N, dtype=np.uint32).astype(np.uint16)
    wg = np.zeros((N, K), dtype=np.uint16)
    wu = np.zeros((N, K), dtype=np.uint16)
    wg[:, 0] = g_bits
    wu[:, 0] = u_bits
    h = np.zeros((1, K), dtype=np.uint16)
    h[0, 0] = 0x3F80  # 1.0
    ref = oracle.dual_gemv(h, wg, wu)
    got = bits(gpu_run(bf16_from_bits(h).to(DEV), bf16_from_bits(wg).to(DEV), bf16_from_bits(wu).to(DEV),
                       tuning))
    return got.ravel(), ref.ravel(), g_bits




@pytest.mark.parametrize("path", list(EPILOGUE_PATHS))
@pytest.mark.parametrize("up", ["one", "random"])
def test_exhaustive_epilogue(path, up):
    N = 1 << 16
    if up == "one":
        u = np.full(N, 0x3F80, dtype=np.uint16)
    else:
        u = np.random.default_rng(21).integers(0, 1 << 16, N).astype(np.uint16)
    say(f"[epilogue] path={path} up={up}")
    got, ref, g = _epilogue_case(u, api.make_tuning(**EPILOGUE_PATHS[path]))
    bad = check.compare_strict_bits(got, ref)
    if bad is not None:
        sample = [(hex(g[i]), hex(u[i]), hex(got[i]), hex(ref[i])) for i in bad[:12]]
        pytest.fail(f"{bad.size} of {N} differ (g, u, gpu, oracle): {sample}")


# ---- boundary semantics -------------------------------------------------------

def test_determinism_and_freshness():
    h, wg, wu = inputs.case("decode_k2560_n9216", seed=1)
    hd, gd, ud = h.to(DEV), wg.to(DEV), wu.to(DEV)
    a = bits(gpu_run(hd, gd, ud))
    for _ in range(3):
        assert np.array_equal(a, bits(gpu_run(hd, gd, ud))), "repeated calls must be bitwise equal"
    # in-place weight update: the next call must read the new weights
    gd.mul_(-1.0)
    fresh = bits(gpu_run(hd, gd, ud))
    ref = oracle.dual_gemv(bits(h), bits(gd.cpu()), bits(wu), with_pre=True)
    rep = check.compare(fresh, ref, depth=api.plan(1, 9216, 2560)["accum_depth"], k_len=2560)
    assert rep.ok, rep.summary()
    assert not np.array_equal(a, fresh)


@pytest.mark.parametrize("M", [2, 3, 4, 8])
def test_batched_rows_equal_single_row_valu(M):
    """VALU path with fp32 FMAs: row m of a batched call is bitwise the M=1 call on hidden row m."""
    h, wg, wu = inputs.case("batch_k4096_n12288", M=8, seed=1)
    h = h[:M].contiguous()
    hd, gd, ud = h.to(DEV), wg.to(DEV), wu.to(DEV)
    t = api.make_tuning(kernel=api.KERNEL_VALU, gemv_dot=1)
    batched = bits(gpu_run(hd, gd, ud, t))
    for m in range(M):
        single = bits(gpu_run(hd[m:m + 1].contiguous(), gd, ud, t))
        assert np.array_equal(single[0], batched[m]), f"row {m}"


@pytest.mark.parametrize("M", [2, 8, 16, 32])
def test_batched_rows_mfma_vs_single(M):
    """MFMA path: rows agree with the M=1 GEMV bit for bit except near rounding ties."""
    h, wg, wu = inputs.case("mfma_k5120_n17408", M=32, seed=1)
    h = h[:M].contiguous()
    hd, gd, ud = h.to(DEV), wg.to(DEV), wu.to(DEV)
    batched = bits(gpu_run(hd, gd, ud))
    worst = 0
    for m in sorted({0, M // 2, M - 1}):
        single = bits(gpu_run(hd[m:m + 1].contiguous(), gd, ud))[0]
        d = check.ulp_distance(single, batched[m])
        worst = max(worst, int(np.sort(d)[-5]))  # near-cancelled outputs may differ more
        assert np.mean(d == 0) > 0.998
    say(f"[mfma-vs-valu] 5th worst ULP {worst}")


def test_saturated_gate_scaling_is_exact():
    """With every gate saturated (G >= 17), out(2h) == 4 * out(h) bitwise."""
    M, N, K = 2, 1000, 1024
    h = torch.full((M, K), 0.5, dtype=torch.bfloat16)
    wg = (torch.rand(N, K, generator=torch.Generator().manual_seed(3)) * 0.1 + 0.05).to(torch.bfloat16)
    _, wu = inputs.weights(N, K, 9)
    hd, gd, ud = h.to(DEV), wg.to(DEV), wu.to(DEV)
    for tuning in (None, api.make_tuning(kernel=api.KERNEL_MFMA)):
        o1 = gpu_run(hd, gd, ud, tuning).float()
        o2 = gpu_run((hd.float() * 2).to(torch.bfloat16), gd, ud, tuning).float()
        assert torch.equal(o2, o1 * 4)


def test_nan_and_zero_gate():
    M, N, K = 1, 300, 512
    h, wg, wu = inputs.hidden(M, K, 7), *inputs.weights(N, K, 7)
    h[0, 10] = float("nan")
    got = bits(gpu_run(h.to(DEV), wg.to(DEV), wu.to(DEV)))
    assert check.is_nan_bits(got).all()
    z = bits(gpu_run(inputs.hidden(M, K, 7).to(DEV), torch.zeros(N, K, dtype=torch.bfloat16, device=DEV),
                     wu.to(DEV)))
    assert np.all((z & 0x7FFF) == 0)


@pytest.mark.parametrize("M,N,K,kernel", [(1, 1, 8, 0), (1, 65, 520, 0), (3, 3000, 1024, 0),
                                          (8, 130, 2560, 0), (20, 33, 512, 0), (1, 65, 520, api.KERNEL_MFMA),
                                          (2, 65, 1003, 0)])
def test_output_canaries(M, N, K, kernel):
    """Nothing is written outside out[M, N] (sentinels on both sides)."""
    pad = 4096
    buf = torch.full((M * N + 2 * pad,), -3.0, dtype=torch.bfloat16, device=DEV)
    out = buf[pad:pad + M * N].view(M, N)
    h, wg, wu = inputs.hidden(M, K, 8), *inputs.weights(N, K, 8)
    t = api.make_tuning(kernel=kernel) if kernel else None
    say(f"[canary] M={M} N={N} K={K}")
    api.dual_gemv(h.to(DEV), wg.to(DEV), wu.to(DEV), out=out, tuning=t)
    torch.cuda.synchronize()
    b = buf.float().cpu()
    assert torch.all(b[:pad] == -3.0) and torch.all(b[pad + M * N:] == -3.0)
    ref = oracle.dual_gemv(bits(h), bits(wg), bits(wu), with_pre=True)
    rep = check.compare(bits(out), ref, depth=api.plan(M, N, K, True, t)["accum_depth"], k_len=K)
    assert rep.ok, rep.summary()


def test_graph_capture_replays():
    """A captured call replays correctly several times with eager work between replays."""
    h, wg, wu = inputs.case("tail_k1024_n3000", seed=0)
    hd, gd, ud = h.to(DEV), wg.to(DEV), wu.to(DEV)
    out = torch.empty(1, 3000, dtype=torch.bfloat16, device=DEV)
    eager = bits(gpu_run(hd, gd, ud))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        api.dual_gemv(hd, gd, ud, out=out)  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.dual_gemv(hd, gd, ud, out=out)
    for i in range(4):
        out.fill_(1.0)
        _ = (hd.float() * 3).sum()  # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), eager), f"replay {i}"


# ---- the 8-row kernel's two K-walk orders -------------------------------------

PASS_SHAPES = [(9, 100, 512), (16, 1000, 1032), (17, 333, 2560), (32, 3000, 1024), (31, 64, 5120),
               (24, 2052, 5120), (32, 9, 64), (20, 7, 520)]


def mfma8_blocks(N):
    return -(-(-(-N // 8)) // 4)


@pytest.mark.parametrize("jb", [1, 2, 3])
@pytest.mark.parametrize("M,N,K", PASS_SHAPES)
def test_mfma8_slice_major_order(M, N, K, jb):
    """K walked once for up to three blocks of a workgroup: within the bar against the oracle,
    and bitwise equal to the block-by-block order (the per-lane summation order is the same)."""
    grid = -(-mfma8_blocks(N) // jb)
    h, wg, wu = inputs.hidden(M, K, 6), *inputs.weights(N, K, 6)
    t_pass = api.make_tuning(kernel=api.KERNEL_MFMA, rows_per_wave=8, mfma_order=2, grid=grid)
    t_blk = api.make_tuning(kernel=api.KERNEL_MFMA, rows_per_wave=8, mfma_order=1, mfma_segments=8,
                            mfma_depth=1, grid=grid)
    assert api.plan(M, N, K, True, t_pass)["kernel_symbol"].startswith("glu::mfma8_pass_kernel")
    rep, got, _ = parity(h, wg, wu, tuning=t_pass, label=f"mfma8 slice-major grid {grid}")
    assert rep.ok, rep.summary()
    ref = bits(gpu_run(h.to(DEV), wg.to(DEV), wu.to(DEV), t_blk))
    assert check.compare_strict_bits(got, ref) is None


PASS64_SHAPES = [(33, 100, 512), (40, 9, 64), (48, 1000, 1032), (57, 7, 520), (64, 3000, 1024),
                 (64, 2052, 5120), (65, 333, 2560), (100, 9216, 2560)]


@pytest.mark.parametrize("M,N,K", PASS64_SHAPES)
def test_mfma8_slice_major_64_rows(M, N, K):
    """Up to 64 rows of hidden per launch in the slice-major kernel (stages of 4 segments): within
    the bar against the oracle, and bitwise equal to the block-by-block order over launches of
    32 rows (each output's summation order does not depend on the hidden rows beside it)."""
    h, wg, wu = inputs.hidden(M, K, 7), *inputs.weights(N, K, 7)
    t_pass = api.make_tuning(kernel=api.KERNEL_MFMA, rows_per_wave=8, mfma_order=2, mfma_segments=4)
    t_blk = api.make_tuning(kernel=api.KERNEL_MFMA, rows_per_wave=8, mfma_order=1, mfma_segments=4)
    p = api.plan(M, N, K, True, t_pass)
    assert p["kernel_symbol"].startswith("glu::mfma8_pass_kernel") and p["m_per_launch"] == min(M, 64), p
    rep, got, _ = parity(h, wg, wu, tuning=t_pass, label="mfma8 slice-major 64 rows")
    assert rep.ok, rep.summary()
    ref = bits(gpu_run(h.to(DEV), wg.to(DEV), wu.to(DEV), t_blk))
    assert check.compare_strict_bits(got, ref) is None


@pytest.mark.parametrize("M,seed", [(64, 0), (48, 1)])
def test_mfma8_slice_major_64_rows_full_size_sampled(M, seed):
    """K=5120 N=17408 (1 % outlier weights) at the default plan for 33..64 rows of hidden: the
    whole output from the GPU, the oracle on a sample of rows (first, last and random)."""
    h, wg, wu = inputs.case("mfma_k5120_n17408", M=32, seed=seed)
    K = h.shape[1]
    hh = inputs.hidden(M, K, 60 + seed)
    hh[:32] = h
    plan = api.plan(M, wg.shape[0], K)
    assert plan["kernel_symbol"].startswith("glu::mfma8_pass_kernel<") and plan["launches"] == 1, plan
    say(f"[mfma8 64] full size M={M} plan={plan}")
    got = bits(api.dual_gemv(hh.to(DEV), wg.to(DEV), wu.to(DEV)))
    torch.cuda.synchronize()
    rows = sorted({0, 31, 32, M - 1, *np.random.default_rng(seed).integers(0, M, 3).tolist()})
    ref = oracle.dual_gemv(bits(hh[rows]), bits(wg), bits(wu), with_pre=True)
    rep = check.compare(got[rows], ref, depth=plan["accum_depth"], k_len=K)
    say(f"[mfma8 64] rows {rows}: {rep.summary()}")
    assert rep.ok, rep.summary()


def test_mfma8_slice_major_graph_replays():
    """The slice-major kernel at the M=32 K=5120 N=17408 workload, captured in a graph and replayed
    back to back with its inputs changing in place between replays: every replay matches the eager
    call on the same inputs bitwise."""
    M, N, K = 32, 17408, 5120
    t = api.make_tuning(kernel=api.KERNEL_MFMA, rows_per_wave=8, mfma_order=2)
    say(f"[graph] {api.plan(M, N, K, True, t)}")
    h0, wg, wu = inputs.case("mfma_k5120_n17408", M=M, seed=0)
    h, wg, wu = h0.to(DEV), wg.to(DEV), wu.to(DEV)
    out = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        api.dual_gemv(h, wg, wu, out=out, tuning=t)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(4):
            api.dual_gemv(h, wg, wu, out=out, tuning=t)
    torch.cuda.synchronize()
    for r in range(6):
        h.copy_((h0.float() * (1.0 + r / 8.0)).to(torch.bfloat16).to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = api.dual_gemv(h, wg, wu, tuning=t)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"replay {r}"


# ---- M = 1 with the dot products on the matrix cores ----------------------------

DOT_SHAPES = [s for s in SMALL if s[0] == 1] + [(1, 9216, 2560), (1, 12288, 4096), (1, 4000, 8192), (1, 70, 64)]


@pytest.mark.parametrize("rows", [1, 2])
@pytest.mark.parametrize("M,N,K", DOT_SHAPES)
def test_valu_matrix_core_dot(M, N, K, rows):
    """The M = 1 GEMV with each 512-element piece of a row dotted by one MFMA (the diagonal of D):
    within the bar against the oracle, ragged K and N tails included."""
    h, wg, wu = inputs.hidden(M, K, 9), *inputs.weights(N, K, 9)
    t = api.make_tuning(kernel=api.KERNEL_VALU, gemv_dot=2, rows_per_wave=rows)
    rep, _, _ = parity(h, wg, wu, tuning=t, label=f"valu matrix-core dot, {rows} rows per wave")
    assert rep.ok, rep.summary()


# one shape per forward kernel family (the M = 1 GEMV has its own test above) and three grouped calls
FWD_GRAPH_SHAPES = [(4, 1000, 1024, "glu::mfma_kernel<"), (7, 64, 40000, "glu::mfma_slice_kernel<"),
                    (16, 1000, 2560, "glu::mfma8_pass_kernel<"), (48, 1000, 2560, "glu::mfma8_pass_kernel<"),
                    (100, 1000, 520, "glu::gemm_kernel<")]


@pytest.mark.parametrize("M,N,K,sym", FWD_GRAPH_SHAPES)
def test_graph_replays_every_kernel(M, N, K, sym):
    """Each forward kernel family, captured in a graph, replays bitwise equal to an eager call."""
    assert api.plan(M, N, K)["kernel_symbol"].startswith(sym)
    say(f"[graph] forward M={M} N={N} K={K} {api.plan(M, N, K)['kernel_symbol']}")
    h, wg, wu = inputs.hidden(M, K, 41), *inputs.weights(N, K, 41)
    hd, gd, ud = h.to(DEV), wg.to(DEV), wu.to(DEV)
    out = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    api.dual_gemv(hd, gd, ud, out=out)
    torch.cuda.synchronize()
    eager = bits(out)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        api.dual_gemv(hd, gd, ud, out=out)  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.dual_gemv(hd, gd, ud, out=out)
    for i in range(3):
        out.fill_(float("nan"))
        _ = (hd.float() * 3).sum()  # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), eager), f"replay {i}"


@pytest.mark.parametrize("M", [1, 16, 48])
def test_grouped_graph_replays(M):
    """A grouped call of three projections (QKV-like row counts), captured and replayed."""
    K, Ns = 2560, (1024, 256, 256)
    h = inputs.hidden(M, K, 42).to(DEV)
    ws = [inputs.weights(n, K, 42 + i)[0].to(DEV) for i, n in enumerate(Ns)]
    outs = [torch.empty(M, n, dtype=torch.bfloat16, device=DEV) for n in Ns]
    api.grouped_gemv(h, ws, outs=outs)
    torch.cuda.synchronize()
    eager = [bits(o) for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        api.grouped_gemv(h, ws, outs=outs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.grouped_gemv(h, ws, outs=outs)
    for i in range(3):
        for o in outs:
            o.fill_(float("nan"))
        _ = (h.float() * 3).sum()
        g.replay()
        torch.cuda.synchronize()
        for j, o in enumerate(outs):
            assert np.array_equal(bits(o), eager[j]), f"replay {i}, projection {j}"
