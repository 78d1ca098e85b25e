"""The benchmark's rocprofv3 summarizers on small hand-written csv files (no GPU).

Kernel names in an anonymous namespace carry a parenthesis before the kernel's own name; the
summaries must keep the whole name and must not merge two kernels that share a grid size.
"""
import csv
import os

import bench


def write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_short_kernel_name():
    assert bench.short_kernel_name("void glu::(anonymous namespace)::copy_ceiling_kernel<5, 1>(int const*, int)") \
        == "glu::copy_ceiling_kernel<5, 1>"
    assert bench.short_kernel_name("void glu::dh_mfma_kernel<16>(glu::BwdArgs)") == "glu::dh_mfma_kernel<16>"


def test_trace_grid_keeps_kernels_apart(tmp_path):
    rows = []
    for name, t in (("void glu::(anonymous namespace)::copy_ceiling_kernel<5, 1>(int)", 100),
                    ("void glu::(anonymous namespace)::copy_ceiling_kernel<8, 1>(int)", 300),
                    ("void glu::(anonymous namespace)::copy_ceiling_kernel<8, 1>(int)", 500),
                    ("hipMemcpy something", 7)):
        rows.append({"Kernel_Name": name, "Grid_Size_X": 49152, "LDS_Block_Size": 0,
                     "Start_Timestamp": 1000, "End_Timestamp": 1000 + t})
    write_csv(str(tmp_path / "run" / "x_kernel_trace.csv"), rows)
    lines = bench.summarize_trace_grid(str(tmp_path)).splitlines()[2:]
    assert lines == ["| `glu::copy_ceiling_kernel<5, 1>` | 49152 | 0 | 1 | 100 | 100 | 100 |",
                     "| `glu::copy_ceiling_kernel<8, 1>` | 49152 | 0 | 2 | 400 | 500 | 300 |"]


def test_counter_table_keeps_kernels_apart(tmp_path):
    rows = []
    for disp, (name, v) in enumerate((("void glu::(anonymous namespace)::copy_ceiling_kernel<5, 1>(int)", 10.0),
                                      ("void glu::(anonymous namespace)::copy_ceiling_kernel<8, 1>(int)", 30.0),
                                      ("void glu::(anonymous namespace)::copy_ceiling_kernel<8, 1>(int)", 50.0))):
        # two rows of one counter in one dispatch are summed
        for part in (v / 2, v / 2):
            rows.append({"Kernel_Name": name, "Grid_Size": 49152, "Counter_Name": "FETCH_SIZE",
                         "Counter_Value": part, "Dispatch_Id": disp})
    write_csv(str(tmp_path / "run" / "x_counter_collection.csv"), rows)
    lines = bench.summarize_counter_table(str(tmp_path)).splitlines()[2:]
    assert lines == ["| `glu::copy_ceiling_kernel<5, 1>` | 49152 | FETCH_SIZE | 1 | 10.00 |",
                     "| `glu::copy_ceiling_kernel<8, 1>` | 49152 | FETCH_SIZE | 2 | 40.00 |"]
