"""Host logic of the counter post-processing in gemm_counters.py (no GPU):
kernel classes, per-dispatch reductions of a counter file, the clock from
GRBM_GUI_ACTIVE and the grouping of dispatches into launches."""
from __future__ import annotations

import csv

import pytest

import gemm_counters as ht

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
    # GRBM_GUI_ACTIVE summed over the 8 XCDs, as one row per XCD or as one
    # aggregated row: 8 XCDs at 1.5 GHz for 1,000 ns, 8 x 2,400 cycles in 1,000 ns
    p = tmp_path / "g.csv"
    rows = [(1, 7, "gemm", "GRBM_GUI_ACTIVE", 1500.0, 1000, 2000) for _ in range(8)]
    rows.append((2, 8, "copy", "GRBM_GUI_ACTIVE", 8 * 2400.0, 0, 1000))
    _write(p, rows)
    got = ht.per_dispatch_clock(p)
    assert [n for n, _ in got] == ["gemm", "copy"]
    assert got[0][1] == pytest.approx(1.5)
    assert got[1][1] == pytest.approx(2.4)


def test_clock_beyond_the_chip_is_dropped():
    # a dispatch shorter than the counter window reads above the top clock
    assert ht.clock_or_none(1.5) == 1.5
    assert ht.clock_or_none(2.4) == 2.4
    assert ht.clock_or_none(3.0) is None


def test_group_launches():
    # an expanded launch is expansion + GEMM, a split one GEMM + reduction;
    # other kernels (copies, torch's) are not part of any launch
    names = ["at::fill", "lut6_expand_kernel<0>", "lut6_expanded_gemm_kernel<1, false, false>",
             "lut6_stream_kernel<0, false, false, true>", "lut6_tile256_kernel<1, true, true>",
             "lut6_reduce_kernel<1>", "__amd_rocclr_copyBuffer"]
    assert ht.group_launches(names) == [[1, 2], [3], [4, 5]]
