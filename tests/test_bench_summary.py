"""Host logic of bench.py (CPU): the algorithmic work per body step that its rooflines divide by, and the
per-kernel table and busy time it builds from a rocprofv3 kernel trace (a small trace written here)."""
import os
import sqlite3

import pytest

import bench

DIMS = (2560, 4096, 9728)


def test_body_work_counts():
    w = bench.body_work(36)
    N = 262144
    # H accumulation: N n (n + 1) flops per H, one H per input dim and layer
    assert w["syrk"] == 36 * sum(float(N) * n * (n + 1) for n in DIMS) == 1113410141945856.0
    assert w["chol"] == pytest.approx(36 * sum(n ** 3 / 3.0 for n in DIMS))
    # the rotated finalize: S read mirrored, T fp64 written and read, H fp32 written
    assert w["finalize"] == 36 * 28.0 * sum(n * n for n in DIMS)
    # the weights' rotation: 8 bytes per weight of the 3 633 315 840
    assert w["rotate"] == 8.0 * 3633315840
    # pack and unpack move the same bytes: codes and scales one way, packed stream and scales the other
    assert w["pack"] == w["unpack"] == 4945674240.0


def _trace(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table kernels (name text, start integer, end integer)")
    con.executemany("insert into kernels values (?, ?, ?)", rows)
    con.commit()
    con.close()


def test_kernel_summary_table_and_busy_time(tmp_path):
    us = 1000  # trace times are in ns
    rows = [
        ("void wr::syrk_bf16_kernel(unsigned short const*)", 0, 1000 * us),
        ("void wr::chol_step_kernel(double*)", 500 * us, 600 * us),        # inside the first: no extra busy time
        ("void wr::syrk_bf16_kernel(unsigned short const*)", 2000 * us, 3000 * us),
        ("void wr::pack_vec_kernel<2>(unsigned char const*)", 2900 * us, 3100 * us),  # 100 us past the second
        ("at::native::some_torch_kernel", 0, 5000 * us),                  # not the library's: left out
    ]
    db = os.path.join(tmp_path, "run_results.db")
    _trace(db, rows)
    out = bench.kernel_summary(db, steps=2, layers=36)
    # 1000 + 100 + 1000 + 200 us of library kernel time; busy 1000 + 1000 + 100 us
    assert "2.30 ms of kernel time over 2 step(s) = 1.15 ms per step" in out
    assert "1.05 ms per step with at least one of them running" in out
    assert "| `syrk_bf16_kernel` | 2 | 2.00 | 1000.0 | 1.00 |" in out
    assert "| `pack_vec_kernel<2>` | 1 | 0.20 | 200.0 | 0.10 |" in out
    assert "some_torch_kernel" not in out
    # the SYRK roofline: one step's algorithmic flops over the SYRK's time per step (1.00 ms)
    tflops = bench.body_work(36)["syrk"] / 1e-3 / 1e12
    line = [l for l in out.splitlines() if l.startswith("| syrk |")][0]
    assert f"{tflops:.1f} TFLOP/s" in line and f"{tflops / bench.PEAK_BF16_TFLOPS:.3f}" in line
