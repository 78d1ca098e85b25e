"""GPU: row-strided operands through glu_dual_gemv_strided (needs an MI355X).

Every operand is placed in a wider buffer whose extra columns hold NaN, so a
kernel that reads past a row's K elements (or steps rows by K instead of the
real stride) poisons its outputs; the output rows are written into a wider
buffer whose extra columns hold a canary that must survive.  Results are
checked against the oracle on the packed rows, and, where the strided call
runs the same kernel as the packed one, bitwise against the packed call.
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


def widened(t: torch.Tensor, pad: int, fill: int) -> torch.Tensor:
    """A [R, C] view with row stride C + pad into a device buffer whose pad columns hold `fill`."""
    R, C = t.shape
    buf = torch.full((R, C + pad), fill, dtype=torch.int16).view(torch.bfloat16)
    buf[:, :C] = t
    return buf.to(DEV)[:, :C]


# (M, N, K, extra columns for hidden, gate_w, up_w, out, launch-shape override)
CASES = [
    (1, 3000, 2560, 0, 8, 24, 0, {}),                                    # VALU, wider weight rows
    (1, 300, 1024, 8, 16, 8, 5, dict(kernel=api.KERNEL_VALU)),           # VALU, out stride
    (3, 640, 2048, 8, 8, 16, 0, dict(kernel=api.KERNEL_VALU)),           # VALU, hidden in registers, M=3
    (8, 640, 8192, 16, 8, 8, 1, dict(kernel=api.KERNEL_VALU)),           # VALU, hidden staged in LDS
    (4, 1000, 1024, 8, 8, 16, 3, {}),                                    # MFMA, hidden in LDS
    (4, 1000, 1024, 16, 8, 8, 0, dict(kernel=api.KERNEL_MFMA, mfma_hidden=2)),  # MFMA, hidden via L2
    (8, 700, 5120, 8, 8, 8, 7, {}),                                      # 4-row K-slices
    (16, 700, 5120, 24, 8, 16, 0, {}),                                   # 8-row K-slices
    (32, 520, 5120, 8, 40, 8, 9, {}),                                    # 8-row K-slices, M = 32
    (40, 333, 1024, 8, 8, 8, 4, {}),                                     # one launch of 40 rows (5 tiles)
    (64, 700, 2560, 8, 16, 8, 3, {}),                                    # one launch of 64 rows (8 tiles)
    (70, 520, 1024, 8, 8, 16, 2, {}),                                    # tiled GEMM above 64 rows
    (3, 257, 77, 3, 5, 0, 2, {}),                                        # generic: K % 8 != 0
    (2, 300, 1024, 3, 0, 0, 0, {}),                                      # generic: hidden stride not a multiple of 8
]


@pytest.mark.parametrize("M,N,K,ph,pg,pu,po,kw", CASES)
def test_strided_rows(M, N, K, ph, pg, pu, po, kw):
    h, wg, wu = inputs.hidden(M, K, 21), *inputs.weights(N, K, 21)
    hs, gs, us = widened(h, ph, NAN), widened(wg, pg, NAN), widened(wu, pu, NAN)
    out_buf = torch.full((M, N + po), CANARY, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    out = out_buf[:, :N]
    t = api.make_tuning(**kw) if kw else None
    fast = K % 8 == 0 and ph % 8 == 0 and pg % 8 == 0 and pu % 8 == 0
    plan = api.plan(M, N, K, fast, t)
    print(f"[strided] M={M} N={N} K={K} pads=({ph},{pg},{pu},{po}) plan={plan}", flush=True)
    api.dual_gemv(hs, gs, us, out=out, tuning=t)
    torch.cuda.synchronize()
    got = bits(out)
    ref = oracle.dual_gemv(bits(h), bits(wg), bits(wu), with_pre=True)
    rep = check.compare(got, ref, depth=plan["accum_depth"], k_len=K)
    print(f"[strided] {rep.summary()}", flush=True)
    assert rep.ok, rep.summary()
    if po:
        assert (bits(out_buf)[:, N:] == CANARY).all(), "a write landed between output rows"
    if fast:
        packed = api.dual_gemv(h.to(DEV), wg.to(DEV), wu.to(DEV), tuning=t)
        torch.cuda.synchronize()
        assert np.array_equal(bits(packed), got), "strided and packed runs of one kernel differ"


def test_fused_block_column_slices():
    """Gate and up as column slices of one fused [N, 2K] block: each keeps the fused row stride."""
    M, N, K = 2, 2048, 2560
    h, wg, wu = inputs.hidden(M, K, 22), *inputs.weights(N, K, 22)
    fused = torch.cat([wg, wu], dim=1).to(DEV)
    gate, up = fused[:, :K], fused[:, K:]
    assert gate.stride(0) == 2 * K and up.stride(0) == 2 * K
    got = bits(api.dual_gemv(h.to(DEV), gate, up))
    packed = bits(api.dual_gemv(h.to(DEV), wg.to(DEV), wu.to(DEV)))
    torch.cuda.synchronize()
    assert np.array_equal(got, packed)


def test_transposed_weights_are_refused():
    h, wg, wu = inputs.hidden(1, 64, 23), *inputs.weights(64, 64, 23)
    with pytest.raises(ValueError):
        api.dual_gemv(h.to(DEV), wg.to(DEV).t(), wu.to(DEV))
