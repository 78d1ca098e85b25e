"""Host-side planning over a sweep of shapes and tunings (no GPU).

Every plan entry point must return a status for every shape, never fault on
the host (a division by zero in the planner would kill the process, so the
sweep runs in a child process), and the backward's plans must cover their
rows and size the workspace for every partial sum they write.
"""
import math
import os
import subprocess
import sys
import textwrap

import pytest

from glu_mlp_gemv_amd import api



@pytest.fixture(scope="module", autouse=True)
def lib():
    import os
    if not os.path.exists(api.LIBRARY_PATH):
        pytest.fail("libglu_gemv.so is not built (run __graft_entry__.build())")
    return api.library()

SWEEP = textwrap.dedent("""
    import sys
    sys.path.insert(0, {root!r})
    from glu_mlp_gemv_amd import api
    n = 0
    tunings = [None] + [api.make_tuning(**kw) for kw in (
        dict(kernel=api.KERNEL_VALU), dict(kernel=api.KERNEL_MFMA), dict(kernel=api.KERNEL_GENERIC),
        dict(kernel=api.KERNEL_GEMM), dict(grid=1), dict(waves_per_block=1), dict(mfma_segments=2),
        dict(mfma_hidden=2), dict(mfma_hidden=3), dict(rows_per_wave=8), dict(gemm_tile_n=128))]
    for M in list(range(0, 12)) + [15, 16, 17, 31, 32, 33, 64, 65, 300]:
        for N in list(range(0, 10)) + [63, 64, 65, 1000]:
            for K in (0, 8, 16, 24, 64, 72, 520, 2560, 2568, 4104, 8200, 40000):
                for t in tunings:
                    for fast in (False, True):
                        for fn in (lambda: api.plan(M, N, K, fast, t),
                                   lambda: api.grouped_plan(M, K, N, fast, t, True),
                                   lambda: api.grouped_plan(M, K, N, fast, t, False)):
                            try:
                                fn()
                            except api.GluError:
                                pass
                            n += 1
                for fn in (lambda: api.backward_plan(M, N, K), lambda: api.backward_workspace_bytes(M, N, K)):
                    try:
                        fn()
                    except api.GluError:
                        pass
                    n += 1
    print(n)
""")


def test_every_plan_returns_a_status():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, "-c", SWEEP.format(root=root)], capture_output=True, text=True,
                         timeout=300)
    assert res.returncode == 0, (res.returncode, res.stderr[-2000:])
    assert int(res.stdout.split()[-1]) > 100_000


@pytest.mark.parametrize("M", list(range(1, 10)) + [16, 33, 64])
def test_backward_plans_cover_rows_and_partials(M):
    for N in (1, 2, 3, 63, 65, 255, 256, 257, 1000, 9216, 12288, 100000):
        for K in (8, 504, 520, 2560, 2568, 4096, 4104, 8192, 8200, 40000):
            p = api.backward_plan(M, N, K)
            ws = api.backward_workspace_bytes(M, N, K)
            gu = -(-(2 * M * N * 2) // 256) * 256   # dg and du at the workspace head, 256-byte aligned
            assert p["accum_depth"] >= 1
            if p["launches"] == 2:
                # one pass over the weights, one fp32 partial of dh per workgroup, then the reduction
                assert M <= 4 and p["grid"] >= 1
                assert ws == gu + p["grid"] * 2 * M * K * 4, (M, N, K)
                assert p["grid"] <= N
                if K >= 2568:
                    # K split over the lanes of the workgroup: at most two 16-byte chunks per lane
                    assert p["block"] % 64 == 0 and p["block"] <= 512
                    assert p["block"] * 8 * 2 >= K and (p["block"] * 8 >= K or M <= 3)
                    assert p["block"] - 64 < math.ceil(K / 8 / (1 if p["block"] * 8 >= K else 2))
            elif M > 8:
                # MFMA contractions: ranges of 32-row steps of the weights x 128-column tiles (up to
                # 64 rows of hidden), one fp32 partial of dh per range; zero-padded operand copies
                # before the partials
                ktiles = math.ceil(K / 128)
                # dg and du from the tiled GEMM or, where the forward runs it in one launch, the
                # slice-major 8-row kernel or (up to 16 rows) the 4-row kernel with hidden in LDS (the
                # elementwise step in their epilogues), else the grouped GEMV and the elementwise kernel
                gu_gemm = N % 4 == 0 and (M > 64 or (M > 32 and N % 8 != 0))
                f = api.plan(M, N, K)
                gu_pass = f["kernel_symbol"].startswith("glu::mfma8_pass_kernel") and f["launches"] == 1
                gu_mfma4 = (M <= 16 and f["kernel_symbol"].startswith("glu::mfma_kernel<")
                            and ", true, " in f["kernel_symbol"] and f["launches"] == 1)
                assert p["launches"] == (5 if gu_gemm or gu_pass or gu_mfma4 else 6) and p["grid"] % ktiles == 0
                splits = p["grid"] // ktiles
                jr = math.ceil(N / splits / 32) * 32 if splits > 1 else math.ceil(N / 32) * 32
                assert (splits - 1) * jr < N <= splits * jr or splits == 1
                mp16 = 16 if M <= 16 else (32 if M <= 32 else 64)
                mp32, np32 = math.ceil(M / 32) * 32, math.ceil(N / 32) * 32
                pad = lambda b: -(-b // 256) * 256
                copies = pad(2 * mp16 * np32 * 2) + pad(2 * N * mp32 * 2) + pad(K * mp32 * 2)
                assert ws == gu + copies + splits * 2 * M * K * 4, (M, N, K)
            else:
                nslabs = math.ceil(K / 512)
                assert p["grid"] % nslabs == 0
                nranges = p["grid"] // nslabs
                assert nranges <= N
                assert ws == gu + nranges * 2 * min(M, 8) * K * 4, (M, N, K)
                # dg and du from the forward's 4-row kernel with hidden in LDS (the elementwise step
                # as its epilogue) where the forward runs it in one launch, else the grouped GEMV and
                # the elementwise kernel
                f = api.plan(M, N, K)
                fused = f["kernel_symbol"].startswith("glu::mfma_kernel<") and ", true, " in f["kernel_symbol"] \
                    and f["launches"] == 1
                assert p["launches"] == (3 if fused else 4), (M, N, K)
