"""GPU parity of the grouped GEMV (n projections of one hidden) against the oracle's
plain projection, through the C ABI (needs an MI355X).

Each output is checked with the parity bar of oracle/check.py for a single
bf16 rounding (compare_linear): within 2 ULP or inside the admissible
interval, mean relative error <= 0.3 %, bit-exact >= 99.9 %.  Weight sets are
seeded synthetic N(0, 0.02^2) (the QKV-like and GDN-input-like shapes are
stand-ins: a wide projection next to narrower ones, and two 32-row ones).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import check
from glu_mlp_gemv_amd import api, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NAN = 0x7FC0
CANARY = 0x1234


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def weight_set(Ns, K, seed):
    out = []
    for i, N in enumerate(Ns):
        wg, _ = inputs.weights(N, K, seed * 100 + i)
        out.append(wg)
    return out


def check_all(h, ws, outs, tuning=None, fast=True, label=""):
    """Every output within the per-output bar and each projection's mean error within its bar; the
    bit-exact fraction over all outputs of the call."""
    M, K = h.shape
    rows = sum(w.shape[0] for w in ws)
    mult4 = all(w.shape[0] % 4 == 0 for w in ws)
    mult8 = all(w.shape[0] % 8 == 0 for w in ws)
    plan = api.grouped_plan(M, K, rows, fast, tuning, mult4, mult8)
    print(f"[grouped] {label} M={M} K={K} Ns={[w.shape[0] for w in ws]} plan={plan}", flush=True)
    reps = []
    for i, (w, o) in enumerate(zip(ws, outs)):
        ref = oracle.linear(bits(h), bits(w), with_pre=True)
        rep = check.compare_linear(bits(o), ref, depth=plan["accum_depth"], k_len=K)
        print(f"[grouped]   projection {i}: {rep.summary()}", flush=True)
        assert rep.failures == 0 and rep.mean_rel <= 3e-3, (i, rep.summary())
        reps.append(rep)
    n, inexact = sum(r.n for r in reps), sum(r.inexact for r in reps)
    print(f"[grouped]   call: {n - inexact} of {n} outputs bit-exact", flush=True)
    assert check.pooled_bit_exact_ok(reps), (inexact, n)


MFMA = api.KERNEL_MFMA
CASES = [
    ((4096, 1024, 1024), 2560, 1, {}),        # QKV-like triple at decode (VALU)
    ((4096, 1024, 1024), 2560, 4, {}),        # MFMA, hidden in LDS
    ((4096, 1024, 1024), 2560, 16, {}),       # MFMA, 80 KiB of hidden in LDS
    ((4096, 1024, 1024), 2560, 32, {}),       # MFMA, 160 KiB of hidden in LDS
    ((1024, 512), 4096, 32, {}),              # MFMA, hidden via L2
    ((2048, 1024, 32, 32), 2560, 1, {}),      # GDN-input-like quad
    ((2048, 1024, 32, 32), 2560, 2, {}),
    ((2048, 1024, 32, 32), 2560, 8, {}),
    ((1, 3, 300), 1024, 3, {}),               # ragged projection sizes: VALU
    ((7, 0, 64, 1, 129, 2, 33, 5), 512, 2, {}),  # eight projections, one empty: VALU
    ((8, 0, 64, 4, 128, 12, 32, 4), 512, 6, {}),  # eight projections, one empty: MFMA
    ((1000, 24), 8192, 1, {}),                # two stages per row (K/8 > 512)
    ((1000, 24), 8192, 3, {}),                # MFMA, K/8 = 1024 chunks in LDS
    ((640, 640), 4104, 5, {}),                # ragged K, padded LDS rows
    ((12, 4), 2056, 16, {}),                  # ragged K, hidden in LDS
    ((12, 4), 4104, 32, {}),                  # ragged K, hidden via L2
    ((300, 200), 1024, 9, {}),                # MFMA, three hidden tiles
    ((1024, 256), 1024, 33, {}),              # slices of 32 rows of hidden, then 1
    ((64, 65), 2048, 40, {}),                 # N % 4 != 0: VALU in slices of 8
    ((500, 77), 1024, 2, dict(kernel=api.KERNEL_GENERIC)),
    ((500, 77), 1024, 4, dict(kernel=api.KERNEL_VALU, rows_per_wave=1, waves_per_block=2, grid=5)),
    ((4096, 1024), 2560, 1, dict(kernel=MFMA)),
    ((500, 76), 1024, 4, dict(kernel=MFMA, mfma_hidden=2)),
    ((1024, 512), 4096, 8, dict(mfma_segments=4)),
    ((1024, 512), 4096, 7, dict(kernel=MFMA, mfma_segments=2, grid=3, waves_per_block=2)),
    ((256, 8), 2048, 12, dict(kernel=MFMA, grid=1000)),
    ((4096, 1024, 1024), 2560, 4, dict(kernel=api.KERNEL_VALU)),
    ((1, 1), 520, 2, {}),                     # fewer rows than one 4-row group, M >= 2
    ((2,), 520, 5, {}),
    ((3,), 64, 33, {}),
    # groups of 8 weight rows above 8 rows of hidden held in LDS (every N a multiple of 8)
    ((2048, 1024, 32, 32), 2560, 9, {}),      # two 8-row tiles, the second mostly padding
    ((1024, 256), 1024, 33 + 8, {}),          # 41 rows in one launch of 6 tiles of 8 rows
    ((8192, 4096, 32, 32), 2560, 32, {}),     # GDN-input-like quad
    ((4096, 1024, 1024), 2560, 17, {}),       # three 8-row tiles, the third mostly padding
    ((2048, 1024, 32, 32), 1024, 24, {}),
    ((1024, 512, 8), 2176, 32, {}),           # ragged stages (34 segments of 64 in stages of 8)
    ((1024, 512, 8), 2176, 20, dict(mfma_segments=5)),
    ((4096, 1024, 1024), 2560, 32, dict(rows_per_wave=4)),  # the 4-row layout on request
    ((1024, 1032), 2560, 32, {}),             # 1032 = 8 x 129 rows
    ((1024, 256), 1024, 40, {}),              # 40 rows in one launch: 5 tiles of 8 rows
    ((1024, 512), 2560, 12, dict(rows_per_wave=4)),  # 4-row layout, three tiles, 5 segments per stage
    ((2048, 1024, 32, 32), 2560, 12, dict(mfma_segments=5)),  # 8-row layout, 5 segments per stage
    ((9216, 9216), 2560, 12, {}),             # 2304 groups of 8 rows: three per wave on 192 workgroups
    ((9216, 9216), 2560, 16, dict(grid=384)),  # uneven: half the waves take two groups, half one
    # 8-row layout with K-slices of hidden streamed under the weights, one to three blocks per workgroup
    ((4096, 1024, 1024), 2560, 32, dict(mfma_hidden=3)),            # 192 blocks, one each
    ((4096, 1024, 1024), 2560, 32, dict(mfma_hidden=3, grid=64)),   # three blocks per workgroup
    ((8192, 4096, 32, 32), 2560, 32, dict(mfma_hidden=3, grid=193)),  # 386 blocks, two each
    ((8192, 4096, 32, 32), 2560, 24, dict(mfma_hidden=3, grid=129)),  # 3 tiles; three, three, ..., two
    ((2048, 1024, 32, 32), 2560, 9, dict(mfma_hidden=3)),           # two tiles, the second mostly padding
    ((1024, 512, 8), 2176, 32, dict(mfma_hidden=3)),                # ragged: 34 segments, stages of 8
    ((1024, 512, 8), 2176, 17, dict(mfma_hidden=3, grid=22)),       # 193 groups: a block of one group
    ((1024, 256), 1024, 40, dict(mfma_hidden=3)),                   # 40 rows: 5 tiles, one launch
    ((64, 8), 1024, 2, dict(mfma_hidden=3)),                        # nine groups: 3 blocks, 3 waves idle
    ((4096, 1024), 8192, 16, dict(mfma_hidden=3, grid=60)),         # 16 slices, blocks of three and two
    # up to 64 rows of hidden per launch: stages of 8 segments (a 128 KiB ring) or of 4 (64 KiB)
    ((4096, 1024, 1024), 2560, 64, {}),                             # QKV-like, 8 tiles
    ((4096, 1024, 1024), 2560, 64, dict(mfma_hidden=3, mfma_segments=4)),
    ((8192, 4096, 32, 32), 2560, 48, dict(mfma_hidden=3, grid=193)),  # GDN-like, two blocks each
    ((1024, 512, 8), 2176, 57, {}),                                 # ragged: 34 segments in stages of 8
    ((1024, 512, 8), 2176, 33, dict(mfma_hidden=3, mfma_segments=4, grid=22)),  # ragged, stages of 4
    ((1024, 256), 1024, 100, {}),                                   # launches of 64 and 36 rows
    ((64, 8), 1024, 64, dict(mfma_hidden=3)),                       # nine groups: 3 blocks, 3 waves idle
    ((4096, 1024), 8192, 64, dict(mfma_hidden=3, grid=60)),         # 32 slices, blocks of three and two
    ((4096, 1024), 8192, 40, dict(mfma_segments=4)),
]


@pytest.mark.parametrize("Ns,K,M,kw", CASES)
def test_grouped_parity(Ns, K, M, kw):
    h = inputs.hidden(M, K, 31)
    ws = weight_set(Ns, K, 31)
    t = api.make_tuning(**kw) if kw else None
    outs = api.grouped_gemv(h.to(DEV), [w.to(DEV) for w in ws], tuning=t)
    torch.cuda.synchronize()
    check_all(h, ws, [o.cpu() for o in outs], tuning=t, label=str(kw))


def test_grouped_generic_layouts():
    """K not a multiple of 8, and a hidden row stride that is not, take the generic kernel."""
    for K, pad in ((77, 0), (1024, 3)):
        M = 3
        h = inputs.hidden(M, K, 32)
        ws = weight_set((257, 9), K, 32)
        hbuf = torch.full((M, K + pad), NAN, dtype=torch.int16).view(torch.bfloat16)
        hbuf[:, :K] = h
        hv = hbuf.to(DEV)[:, :K]
        outs = api.grouped_gemv(hv, [w.to(DEV) for w in ws])
        torch.cuda.synchronize()
        check_all(h, ws, [o.cpu() for o in outs], fast=False, label=f"generic K={K} pad={pad}")


STRIDED = [((700, 130, 64), 4), ((700, 132, 64), 4), ((700, 132, 64), 16),
           ((704, 136, 64), 16), ((704, 136, 64), 32),  # every N a multiple of 8: the 8-row groups
           ((704, 136, 64), 48), ((704, 136, 64), 64)]  # 48 and 64 rows in one launch


@pytest.mark.parametrize("Ns,M", STRIDED)
def test_grouped_strided_views_and_canaries(Ns, M):
    """Weights as column slices of a wider block (NaN in the gaps), hidden rows padded with NaN,
    outputs into wider rows."""
    K = 2560
    h = inputs.hidden(M, K, 33)
    ws = weight_set(Ns, K, 33)
    hbuf = torch.full((M, K + 8), NAN, dtype=torch.int16).view(torch.bfloat16)
    hbuf[:, :K] = h
    hv = hbuf.to(DEV)[:, :K]
    views, bufs_out, outs = [], [], []
    for w in ws:
        buf = torch.full((w.shape[0], K + 24), NAN, dtype=torch.int16).view(torch.bfloat16)
        buf[:, :K] = w
        views.append(buf.to(DEV)[:, :K])
        ob = torch.full((M, w.shape[0] + 5), CANARY, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        bufs_out.append(ob)
        outs.append(ob[:, :w.shape[0]])
    api.grouped_gemv(hv, views, outs=outs)
    torch.cuda.synchronize()
    check_all(h, ws, [o.cpu() for o in outs], label="strided")
    for ob, w in zip(bufs_out, ws):
        assert (bits(ob)[:, w.shape[0]:] == CANARY).all(), "a write landed between output rows"
    packed = api.grouped_gemv(h.to(DEV), [w.to(DEV) for w in ws])
    torch.cuda.synchronize()
    for a, b in zip(packed, outs):
        assert np.array_equal(bits(a), bits(b)), "strided and packed runs differ"


@pytest.mark.parametrize("kernel", [api.KERNEL_VALU, api.KERNEL_MFMA])
def test_grouped_rows_independent_of_batch_and_group(kernel):
    """Within one kernel a row's result depends on nothing but its own hidden row and weight row:
    batched rows equal single-row calls bitwise, and a projection's output does not change with its
    companions.  (The VALU and MFMA kernels sum in different orders, so a batch and a single row
    are compared on the same kernel.)"""
    K = 2560
    t = api.make_tuning(kernel=kernel)
    h = inputs.hidden(6, K, 34).to(DEV)
    ws = [w.to(DEV) for w in weight_set((1500, 300, 32), K, 34)]
    plan6, plan1 = api.grouped_plan(6, K, 1832, tuning=t), api.grouped_plan(1, K, 1832, tuning=t)
    print(f"[grouped] rows: {plan6['kernel_symbol']} vs {plan1['kernel_symbol']}", flush=True)
    batched = api.grouped_gemv(h, ws, tuning=t)
    alone = api.grouped_gemv(h, ws[1:2], tuning=t)
    torch.cuda.synchronize()
    assert np.array_equal(bits(batched[1]), bits(alone[0]))
    for m in range(6):
        single = api.grouped_gemv(h[m], ws, tuning=t)
        torch.cuda.synchronize()
        for b, s in zip(batched, single):
            assert np.array_equal(bits(b[m]), bits(s)), m


def test_grouped_k_zero_and_determinism():
    h = torch.zeros(3, 0, dtype=torch.bfloat16, device=DEV)
    ws = [torch.zeros(5, 0, dtype=torch.bfloat16, device=DEV), torch.zeros(2, 0, dtype=torch.bfloat16, device=DEV)]
    outs = [torch.full((3, 5), 1.0, dtype=torch.bfloat16, device=DEV),
            torch.full((3, 2), 1.0, dtype=torch.bfloat16, device=DEV)]
    api.grouped_gemv(h, ws, outs=outs)
    torch.cuda.synchronize()
    assert all((bits(o) == 0).all() for o in outs)
    K = 1024
    hh = inputs.hidden(2, K, 35).to(DEV)
    ww = [w.to(DEV) for w in weight_set((900, 40), K, 35)]
    a = api.grouped_gemv(hh, ww)
    b = api.grouped_gemv(hh, ww)
    torch.cuda.synchronize()
    assert all(np.array_equal(bits(x), bits(y)) for x, y in zip(a, b))


@pytest.mark.parametrize("Ns,K,M,grid,seg", [((4096, 1024, 1024), 2560, 32, 0, 0), ((8192, 4096, 32, 32), 2560, 24, 129, 0),
                                             ((1024, 512, 8), 2176, 17, 22, 0), ((2048, 1024, 32, 32), 1024, 9, 0, 0),
                                             ((4096, 1024, 1024), 2560, 64, 0, 0), ((4096, 1024, 1024), 2560, 64, 0, 4),
                                             ((1024, 512, 8), 2176, 57, 22, 0), ((1024, 512, 8), 2176, 41, 0, 4)])
def test_grouped_slices_bitwise_equal_to_hidden_in_lds(Ns, K, M, grid, seg):
    """The K-slice walk adds every output's products in the order of the 8-row kernel with hidden
    whole in LDS (launches of at most 32 rows): the two agree bit for bit, also with 64 rows of
    hidden per launch of the slice walk."""
    print(f"grouped slices Ns={Ns} K={K} M={M} grid={grid} segments={seg}", flush=True)
    h = inputs.hidden(M, K, 33).to(DEV)
    ws = [w.to(DEV) for w in weight_set(Ns, K, 33)]
    a = api.grouped_gemv(h, ws, tuning=api.make_tuning(mfma_hidden=3, grid=grid, mfma_segments=seg))
    b = api.grouped_gemv(h, ws, tuning=api.make_tuning(rows_per_wave=8, mfma_hidden=1))
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
