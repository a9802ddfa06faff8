"""GPU test of lut6_linear_noalloc, the entry point that allocates nothing.

It runs the same plan and kernels as lut6_linear with its scratch (the
expanded weight and the split-K partial sums) in the library's static
per-GPU array, so its output must equal lut6_linear's bit for bit, and both
must meet the oracle's criteria.  The calls run in a row from the largest
scratch use to the smallest, so every later call reads an array that still
holds an earlier call's contents.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from oracle import tolerance as tol

torch = pytest.importorskip("torch")
import lut_weight_quantized_amd as lq  # noqa: E402

pytestmark = pytest.mark.gpu

F32, F16, SILU = lq.EPI_STORE_F32, lq.EPI_STORE_F16, lq.EPI_SILU_MUL_F16

# (L, K, N, epilogue, in_scale, path): largest scratch first
CASES = [
    (2048, 4096, 4096, F16, 16.0, lq.PATH_EXPANDED),   # 34 MB expanded weight + 2 K slices
    (1536, 1024, 544, F16, 1.0, lq.PATH_EXPANDED),     # ragged N, expanded + 2 K slices
    (300, 1024, 96, F32, 1.0, lq.PATH_FUSED),          # fused, 2 K slices
    (100, 4096, 256, SILU, 2.0, lq.PATH_STREAM),       # streaming, K slices
    (70, 2048, 64, F32, 1.0, lq.PATH_STREAM),          # smallest last, 2 K slices
]


def _inputs(i, L, K, N):
    key = (90, i, 0)
    x = si.activations(L, K, 1.0, key)
    idx = si.indices(N, K, key)
    tab = si.tables(N, key, outlier_p=0.02)
    return x, idx, tab


def _raw(lib_fn, xd, pd, td, yd, L, K, N, s, epi):
    lib = lq.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    return getattr(lib, lib_fn)(xd.data_ptr(), pd.data_ptr(), td.data_ptr(), yd.data_ptr(),
                                L, K, N, float(s), int(epi), stream)


def test_noalloc_matches_linear_in_a_row(ora):
    torch.cuda.set_device(0)
    for i, (L, K, N, epi, s, path) in enumerate(CASES):
        print(f"[case] noalloc L={L} K={K} N={N} epi={epi} s={s}", flush=True)
        assert lq.linear_path(L, K, N, epi) == path
        x, idx, tab = _inputs(i, L, K, N)
        packed = lq.pack(idx)
        xd = torch.from_numpy(x).cuda()
        pd = torch.from_numpy(packed).cuda()
        td = torch.from_numpy(tab).cuda()
        n_out = N // 2 if epi == SILU else N
        dt = torch.float32 if epi == F32 else torch.float16
        # poison the outputs so an unwritten element cannot pass
        y_na = torch.full((L, n_out), float("nan"), dtype=dt, device="cuda")
        y_ref = torch.full((L, n_out), float("nan"), dtype=dt, device="cuda")
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        # through the C ABI: lut6_linear_noalloc, then lut6_linear
        assert _raw("lut6_linear_noalloc", xd, pd, td, y_na, L, K, N, s, epi) == 0
        torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info()[0]
        if i > 0:   # the first call may load the code object and its array
            assert free1 == free0, f"noalloc call changed free device memory by {free0 - free1} B"
        assert _raw("lut6_linear", xd, pd, td, y_ref, L, K, N, s, epi) == 0
        torch.cuda.synchronize()
        a = y_na.cpu().numpy()
        b = y_ref.cpu().numpy()
        assert np.array_equal(a.view(np.uint32 if epi == F32 else np.uint16),
                              b.view(np.uint32 if epi == F32 else np.uint16)), \
            "lut6_linear_noalloc differs from lut6_linear"
        # and the oracle's criteria on sampled rows
        rows = si.sample_rows(L, 48, (90, i, 1))
        S = tol.row_scale(x, tab, K, rows)
        pk = ora.pack(idx)
        yd = a[rows] if epi == F32 else a[rows].view(np.uint16)
        if epi == SILU:
            h, _ = ora.linear(x, pk, tab, epilogue=oracle.EPI_SILU_MUL_F16, in_scale=s, rows=rows)
            g, _ = ora.linear(x, pk, tab, epilogue=oracle.EPI_F32, in_scale=s, rows=rows)
            rep = tol.check(yd, h, S, fp16=True, S_elem=tol.silu_scale(g[:, :N // 2], g[:, N // 2:], S))
        else:
            ye, _ = ora.linear(x, pk, tab, epilogue=epi, in_scale=s, rows=rows)
            rep = tol.check(yd, ye, S, fp16=epi == F16)
        print(f"[case] noalloc L={L} K={K} N={N}: {rep}", flush=True)
        assert rep.ok, rep


def test_noalloc_refuses_oversized_scratch():
    # 65,536 channels at K = 4,096 and 2,048 tokens: a 545 MB expanded weight
    L, K, N = 2048, 4096, 65536
    x = torch.empty((L, K), dtype=torch.float16, device="cuda")
    p = torch.empty((N, K // 4 * 3), dtype=torch.uint8, device="cuda")
    t = torch.empty((N // 16, 64), dtype=torch.float16, device="cuda")
    y = torch.empty((L, N), dtype=torch.float16, device="cuda")
    with pytest.raises(lq.Lut6Error) as e:
        lq.linear_noalloc(x, p, t, y, epilogue=F16)
    assert e.value.status == "LUT6_E_SCRATCH"
