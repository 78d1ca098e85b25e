"""The streaming-read yardstick (glu_read_ceiling) on the GPU: it reads every row of both
matrices with the GEMV's launch shape.

The kernel XORs every 32-bit word a lane loads and stores to the sink only when the
result is one fixed value.  Planting that value in one word per lane of one row (every
other word zero) therefore makes exactly the lanes of the wave that owns the row write
it: a row the kernel skipped, or a chunk it did not load, leaves the sink untouched.
"""
import pytest
import torch

from glu_mlp_gemv_amd import api

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MAGIC = 0x7f3a5c91


@pytest.mark.parametrize("rows,K,row,fields", [
    (9216, 2560, 9215, {}),                      # the headline shape, last row
    (9216, 2560, 0, {}),
    (3000, 1024, 1717, {"rows_per_wave": 2}),
    (3001, 4096, 2999, {"rows_per_wave": 4}),   # the padded last group re-reads row 3000 (XOR cancels)
    (9216, 2560, 4711, {"xcd_bands": 1}),
    (9216, 2560, 8000, {"grid": 256, "waves_per_block": 4, "xcd_bands": 1}),
])
@pytest.mark.parametrize("in_b", [False, True])
def test_yardstick_reads_every_row_and_chunk(rows, K, row, fields, in_b):
    print(f"yardstick rows={rows} K={K} row={row} {fields} in_b={in_b}", flush=True)
    a = torch.zeros(rows, K, dtype=torch.bfloat16, device=DEV)
    b = torch.zeros(rows, K, dtype=torch.bfloat16, device=DEV)
    words = (b if in_b else a).view(torch.int32).view(rows, K // 2)
    # lane l reads 16-byte chunks l, l + 64, ...: plant the value in the first word of the
    # lane's last chunk of the row
    chunks = K // 8
    lanes = torch.arange(64, device=DEV)
    last = lanes + 64 * ((chunks - 1 - lanes) // 64)
    words[row, last * 4] = torch.tensor(MAGIC, dtype=torch.int32, device=DEV)
    sink = torch.zeros(64, dtype=torch.int32, device=DEV)
    api.read_ceiling(a, b, sink, tuning=api.make_tuning(**fields) if fields else None)
    torch.cuda.synchronize()
    assert (sink.cpu() == MAGIC).all()


def test_yardstick_leaves_the_sink_alone_on_plain_data():
    a = torch.ones(4608, 2560, dtype=torch.bfloat16, device=DEV)
    b = torch.full((4608, 2560), 2.0, dtype=torch.bfloat16, device=DEV)
    sink = torch.full((64,), 7, dtype=torch.int32, device=DEV)
    api.read_ceiling(a, b, sink)
    torch.cuda.synchronize()
    assert (sink.cpu() == 7).all()


@pytest.mark.parametrize("unit", [api.UNIT_MFMA_16X16X32_BF16, api.UNIT_MFMA_32X32X16_BF16, api.UNIT_LDS_READ_B128])
@pytest.mark.parametrize("waves", [1, 4, 16])
def test_unit_ceiling_runs_and_leaves_the_sink_alone(unit, waves):
    # the folded results never equal the fixed value for these operands, so the sink stays as it was
    print(f"unit ceiling unit={unit} waves={waves}", flush=True)
    sink = torch.full((64,), 7, dtype=torch.int32, device=DEV)
    api.unit_ceiling(unit, waves, 256, 50, sink)
    torch.cuda.synchronize()
    assert (sink.cpu() == 7).all()


@pytest.mark.parametrize("rows,K,fields", [(9216, 2560, {}), (3001, 1024, {"rows_per_wave": 2}), (77, 4096, {}),
                                           (12288, 4096, {"grid": 256, "waves_per_block": 4})])
def test_copy_ceiling_copies_every_row_and_nothing_else(rows, K, fields):
    print(f"copy ceiling rows={rows} K={K} {fields}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(rows + K)
    a = torch.randn(rows, K, generator=g).to(torch.bfloat16).to(DEV)
    b = torch.randn(rows, K, generator=g).to(torch.bfloat16).to(DEV)
    ca = torch.full((rows + 1, K), 7.0, dtype=torch.bfloat16, device=DEV)  # one canary row after the copy
    cb = torch.full((rows + 1, K), 7.0, dtype=torch.bfloat16, device=DEV)
    api.copy_ceiling(a, b, ca[:rows], cb[:rows], tuning=api.make_tuning(**fields) if fields else None)
    torch.cuda.synchronize()
    assert torch.equal(ca[:rows].view(torch.int16), a.view(torch.int16))
    assert torch.equal(cb[:rows].view(torch.int16), b.view(torch.int16))
    assert (ca[rows] == 7.0).all() and (cb[rows] == 7.0).all()
