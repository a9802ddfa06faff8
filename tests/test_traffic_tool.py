"""Host logic of the counter post-processing (no GPU): kernel classes, the
per-dispatch sums of a counter file, and the clock from GRBM_GUI_ACTIVE."""
from __future__ import annotations

import csv

import pytest

from lut_weight_quantized_amd import hbm_traffic as ht

COLS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
        "Start_Timestamp", "End_Timestamp"]


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(COLS, r)))


@pytest.mark.parametrize("name,cls", [
    ("void (anonymous namespace)::lut6_expanded_gemm_kernel<1, true, false>(GemmArgs)", "expanded_f16"),
    ("void (anonymous namespace)::lut6_tile256_kernel<2, false, true>(GemmArgs)", "fused_silu"),
    ("void (anonymous namespace)::lut6_stream_kernel<0, false, false, true>(GemmArgs)", "stream_f32"),
    ("void (anonymous namespace)::lut6_reduce_kernel<1>(float const*, void*, int, int, int, float)", "reduce"),
    ("void (anonymous namespace)::lut6_expand_kernel<2>(unsigned char const*, ...)", "expand"),
    ("__amd_rocclr_copyBuffer", None),
])
def test_classify(name, cls):
    assert ht.classify(name) == cls


def test_per_dispatch_sums_instances(tmp_path):
    # a counter is reported per instance (one row per XCD or channel); the
    # dispatch's value is the sum, dispatches in order
    p = tmp_path / "c.csv"
    _write(p, [(1, 2, "k2", "FETCH_SIZE", 10.0, 0, 5), (1, 2, "k2", "FETCH_SIZE", 5.5, 0, 5),
               (1, 1, "k1", "FETCH_SIZE", 3.0, 0, 5), (1, 1, "k1", "WRITE_SIZE", 99.0, 0, 5)])
    assert ht.per_dispatch(p, "FETCH_SIZE") == [("k1", 3.0), ("k2", 15.5)]


def test_per_dispatch_clock(tmp_path):
    # 8 XCDs each busy for 1,000 ns at 1.5 GHz: 8 * 1,500 cycles over 1,000 ns
    p = tmp_path / "g.csv"
    rows = [(1, 7, "gemm", "GRBM_GUI_ACTIVE", 1500.0, 1000, 2000) for _ in range(8)]
    rows.append((2, 8, "copy", "GRBM_GUI_ACTIVE", 8 * 2400.0, 0, 1000))
    _write(p, rows)
    got = ht.per_dispatch_clock(p)
    assert [n for n, _ in got] == ["gemm", "copy"]
    assert got[0][1] == pytest.approx(1.5)
    assert got[1][1] == pytest.approx(2.4)
