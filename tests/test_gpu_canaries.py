"""Output canaries: no entry point writes outside its output.

Every output tensor is a view into a larger device buffer filled with 0xFF
bytes (NaN as FP16 and FP32): 256 guard bytes before it and 4 KB after.
After each call the guards must be intact (no store before the first row or
past the last row, which in a contiguous [rows, cols] output is also where a
store past the last column of the last row would land), and no element of
the output may still hold the fill (every output element was written).
Each kernel path of every entry point is covered, with ragged shapes.
"""
from __future__ import annotations

import numpy as np
import pytest

import seeded_inputs as si

torch = pytest.importorskip("torch")
import lut_weight_quantized_amd as lq  # noqa: E402

pytestmark = pytest.mark.gpu

HEAD, TAIL = 256, 4096
F32, F16, SILU = lq.EPI_STORE_F32, lq.EPI_STORE_F16, lq.EPI_SILU_MUL_F16


def _say(*a):
    print("[case]", *a, flush=True)


def _guarded(shape, dtype):
    """(buffer, view): `view` is a contiguous `shape` tensor of `dtype` inside
    `buffer` (uint8, filled with 0xFF), 16-byte aligned."""
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    buf = torch.full((HEAD + n + TAIL,), 0xFF, dtype=torch.uint8, device="cuda")
    return buf, buf[HEAD:HEAD + n].view(dtype).view(shape)


def _check(buf, view, what):
    torch.cuda.synchronize()
    n = view.numel() * view.element_size()
    head = buf[:HEAD].cpu().numpy()
    tail = buf[HEAD + n:].cpu().numpy()
    assert np.all(head == 0xFF), f"{what}: {int(np.sum(head != 0xFF))} bytes written before the output"
    assert np.all(tail == 0xFF), f"{what}: {int(np.sum(tail != 0xFF))} bytes written past the output"
    if view.dtype in (torch.float16, torch.float32):
        unwritten = int(torch.isnan(view).sum())
        assert unwritten == 0, f"{what}: {unwritten} output elements never written"


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


# (L, K, N, epilogue, in_scale, expected path): every path with and without a K split
LINEAR_CASES = [
    (128, 256, 3104, F32, 1.0, lq.PATH_STREAM),       # 194 tiles: no split
    (100, 2048, 544, F16, 16.0, lq.PATH_STREAM),      # K split
    (77, 512, 96, SILU, 1.0, lq.PATH_STREAM),
    (700, 256, 16400, F16, 1.0, lq.PATH_FUSED),       # 195 tiles: no split
    (300, 1024, 96, F32, 2.0, lq.PATH_FUSED),         # K split
    (333, 512, 544, SILU, 1.0, lq.PATH_FUSED),
    (1600, 256, 8208, F16, 1.0, lq.PATH_EXPANDED),    # 231 tiles: no split
    (1536, 1024, 544, F32, 16.0, lq.PATH_EXPANDED),   # K split
    (1555, 512, 1056, SILU, 1.0, lq.PATH_EXPANDED),
]


@pytest.mark.parametrize("L,K,N,epi,s,path", LINEAR_CASES)
@pytest.mark.parametrize("entry", ["linear", "linear_noalloc"])
def test_linear_canaries(L, K, N, epi, s, path, entry):
    _say(entry, "canaries", L, K, N, epi, s)
    assert lq.linear_path(L, K, N, epi) == path
    key = (91, L, N)
    x = _dev(si.activations(L, K, 1.0, key))
    p = _dev(lq.pack(si.indices(N, K, key)))
    t = _dev(si.tables(N, key))
    n_out = N // 2 if epi == SILU else N
    buf, y = _guarded((L, n_out), torch.float32 if epi == F32 else torch.float16)
    if entry == "linear":
        lq.linear(x, p, t, epilogue=epi, in_scale=s, out=y)
    else:
        lq.linear_noalloc(x, p, t, y, epilogue=epi, in_scale=s)
    _check(buf, y, f"{entry} {L}x{K}x{N} epi {epi}")


@pytest.mark.parametrize("L,K,N,epi", [(100, 512, 96, F16), (150, 256, 64, SILU), (700, 512, 544, F32),
                                       (1600, 256, 160, SILU)])
def test_int8_linear_canaries(L, K, N, epi):
    _say("int8 canaries", L, K, N, epi)
    key = (92, L, N)
    x = _dev(si.activations(L, K, 1.0, key))
    q8, s8 = si.int8_weight(N, K, key)
    n_out = N // 2 if epi == SILU else N
    buf, y = _guarded((L, n_out), torch.float32 if epi == F32 else torch.float16)
    lq.int8_linear(x, _dev(q8), _dev(s8), epilogue=epi, out=y)
    _check(buf, y, f"int8 {L}x{K}x{N}")


@pytest.mark.parametrize("N,K", [(16, 64), (272, 576)])
def test_dequant_canaries(N, K):
    _say("dequant canaries", N, K)
    key = (93, N, K)
    buf, w = _guarded((N, K), torch.float16)
    lq.dequant(_dev(lq.pack(si.indices(N, K, key))), _dev(si.tables(N, key)), K, out=w)
    _check(buf, w, f"dequant {N}x{K}")


@pytest.mark.parametrize("L,Lk", [(1030, 1030), (40, 2000)])   # no key split; keys split over a long cache
def test_attention_canaries(L, Lk):
    _say("attention canaries", L, Lk)
    g = torch.Generator(device="cuda").manual_seed(L + Lk)
    qkv = torch.randn((Lk, 6144), generator=g, device="cuda").half()
    buf, o = _guarded((L, 4096), torch.float16)
    lq.attention(qkv[Lk - L:, :4096], qkv[:, 4096:5120], qkv[:, 5120:], n_heads=16, n_kv_heads=4, out=o)
    _check(buf, o, f"attention {L}/{Lk}")


@pytest.mark.parametrize("L", [40, 200])                     # token-sequential; chunked with a ragged chunk
def test_gated_delta_canaries(L):
    _say("gated delta canaries", L)
    g = torch.Generator(device="cuda").manual_seed(L)
    qkv = (torch.randn((L, 8192), generator=g, device="cuda") / 11.3).half()
    gl = -torch.rand((L, 32), generator=g, device="cuda") * 0.5
    be = torch.rand((L, 32), generator=g, device="cuda")
    sbuf, st = _guarded((32, 128, 128), torch.float32)
    st.zero_()
    obuf, o = _guarded((L, 4096), torch.float16)
    lq.gated_delta(qkv[:, :2048], qkv[:, 2048:4096], qkv[:, 4096:], gl, be, st, n_k_heads=16, n_v_heads=32,
                   out=o)
    _check(obuf, o, f"gated delta out L={L}")
    _check(sbuf, st, f"gated delta state L={L}")


def test_quantize_canaries():
    _say("quantize canaries")
    N, K = 48, 256
    w = _dev(si.weights(N, K, (94, 0, K)))
    pbuf, p = _guarded((N, K // 4 * 3), torch.uint8)
    tbuf, t = _guarded((N // 16, 64), torch.float16)
    lq.quantize(w, packed=p, tables=t)
    _check(pbuf, p, "quantize packed")
    _check(tbuf, t, "quantize tables")
