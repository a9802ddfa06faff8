"""CPU tests of the C ABI: the library loads, exports every declared symbol,
packs and unpacks exactly like the oracle, and refuses bad arguments with
the named status before touching the device.

No test here launches a kernel: arguments that pass validation are never
used, and the pointers are fake (aligned integers that are never read).
"""
from __future__ import annotations

import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

import lut_weight_quantized_amd as lq

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "lut6.h"


def _declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(lut6_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = lq.load_library()
    declared = _declared_functions()
    assert set(declared) == set(lq.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), f"{name} not exported"


def test_status_strings():
    for code, name in lq.STATUS.items():
        assert lq.status_string(code) == name
    assert lq.status_string(12345) == "LUT6_E_UNKNOWN"


def test_sizes():
    assert lq.packed_bytes(4096, 4096) == 4096 * 3072
    assert lq.table_bytes(4096) == 256 * 128
    assert lq.packed_bytes(16, 6) == 0 and lq.table_bytes(20) == 0 and lq.packed_bytes(-1, 4) == 0
    # bits per weight including tables: 6 + 64 / K
    assert (lq.packed_bytes(256, 4096) + lq.table_bytes(256)) * 8 / (256 * 4096) == 6 + 64 / 4096


def test_pack_matches_oracle_exhaustively(ora):
    t = np.arange(64 ** 4, dtype=np.uint32)
    idx = np.stack([(t // 64 ** i) % 64 for i in range(4)], axis=1).astype(np.uint8).reshape(64, -1)
    ours = lq.pack(idx)
    assert np.array_equal(ours, ora.pack(idx))
    assert np.array_equal(lq.unpack(ours, idx.shape[1]), idx)


def test_unpack_matches_oracle_on_every_byte_triple(ora):
    b = np.arange(2 ** 24, dtype=np.uint32)
    raw = np.stack([b % 256, (b // 256) % 256, b // 65536], axis=1).astype(np.uint8).reshape(16, -1)
    K = raw.shape[1] * 4 // 3
    assert np.array_equal(lq.unpack(raw, K), ora.unpack(raw, K))


def test_pack_refusals():
    bad = np.zeros((2, 8), np.uint8)
    bad[1, 5] = 64
    with pytest.raises(lq.Lut6Error) as e:
        lq.pack(bad)
    assert e.value.status == "LUT6_E_INDEX_RANGE"
    lib = lq.load_library()
    buf = np.zeros(64, np.uint8)
    assert lib.lut6_pack(buf.ctypes.data, buf.ctypes.data, 1, 6) == 2        # K % 4
    assert lib.lut6_pack(None, buf.ctypes.data, 1, 4) == 1
    assert lib.lut6_unpack(buf.ctypes.data, None, 1, 4) == 1
    assert lib.lut6_pack(buf.ctypes.data, buf.ctypes.data, 0, 4) == 2


# fake, 16-byte aligned, far-apart device addresses (never dereferenced)
X, P, T, Y = 0x10_0000_0000, 0x20_0000_0000, 0x30_0000_0000, 0x40_0000_0000


def _linear(x=X, p=P, t=T, y=Y, L=128, K=4096, N=4096, s=1.0, epi=1):
    return lq.load_library().lut6_linear(x, p, t, y, L, K, N, s, epi, None)


@pytest.mark.parametrize("kwargs, status", [
    (dict(x=None), 1), (dict(p=None), 1), (dict(t=None), 1), (dict(y=None), 1),
    (dict(L=-1), 2), (dict(K=0), 2), (dict(N=0), 2), (dict(K=4000), 2), (dict(K=100), 2),
    (dict(N=4008), 2), (dict(N=48, epi=2), 2), (dict(L=2 ** 31), 2),
    (dict(L=2 ** 18), 2), (dict(N=2 ** 20), 2),
    (dict(epi=3), 5), (dict(epi=-1), 5),
    (dict(s=3.0), 4), (dict(s=32.0), 4), (dict(s=0.5), 4), (dict(s=-1.0), 4),
    (dict(x=X + 8), 3), (dict(y=Y + 2), 3), (dict(p=P + 4), 3), (dict(t=T + 1), 3),
    (dict(y=X), 8), (dict(y=P + 16), 8), (dict(y=T), 8),
    (dict(L=0), 0),
])
def test_linear_validation(kwargs, status):
    assert _linear(**kwargs) == status


def test_linear_path():
    # few tokens stream the weight; mid-size L runs the fused kernel; from
    # 1536 tokens (3072 when K >= 8192) the weight is expanded once, unless
    # the expansion would not fit 31-bit offsets
    assert lq.linear_path(1, 4096, 4096) == lq.PATH_STREAM
    assert lq.linear_path(192, 12288, 4096) == lq.PATH_STREAM
    assert lq.linear_path(193, 4096, 4096) == lq.PATH_FUSED
    assert lq.linear_path(1535, 4096, 24576, lq.EPI_SILU_MUL_F16) == lq.PATH_FUSED
    assert lq.linear_path(1536, 4096, 4096) == lq.PATH_EXPANDED
    assert lq.linear_path(1536, 8128, 4096) == lq.PATH_EXPANDED
    assert lq.linear_path(3071, 8192, 4096) == lq.PATH_FUSED
    assert lq.linear_path(3072, 12288, 4096) == lq.PATH_EXPANDED
    assert lq.linear_path(16384, 12288, 4096) == lq.PATH_EXPANDED
    assert lq.linear_path(16384, 4096, 24576, lq.EPI_SILU_MUL_F16) == lq.PATH_EXPANDED
    # 8 * (K/64 + 1) * 4 KB per 256-channel tile: 2 GB at N = 96 * 256, K = 2^16
    assert lq.linear_path(4096, 65536, 96 * 256, lq.EPI_STORE_F32) == lq.PATH_FUSED
    with pytest.raises(lq.Lut6Error) as e:
        lq.linear_path(1024, 100, 4096)
    assert e.value.status == "LUT6_E_SHAPE"
    with pytest.raises(lq.Lut6Error) as e:
        lq.linear_path(1024, 4096, 4096, 7)
    assert e.value.status == "LUT6_E_EPILOGUE"


def test_dequant_validation():
    lib = lq.load_library()
    assert lib.lut6_dequant(None, T, Y, 32, 64, None) == 1
    assert lib.lut6_dequant(P, T, Y, 20, 64, None) == 2
    assert lib.lut6_dequant(P, T, Y, 32, 60, None) == 2
    assert lib.lut6_dequant(P + 4, T, Y, 32, 64, None) == 3
    assert lib.lut6_dequant(P, T, P, 32, 64, None) == 8


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.float16)
    with pytest.raises(TypeError):
        lq.linear(x, torch.zeros(16, 48, dtype=torch.uint8), torch.zeros(1, 64, dtype=torch.float16))


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(lq, "_lib", None)
    monkeypatch.setattr(lq, "LIB_PATH", tmp_path / "liblut6.so")
    with pytest.raises(RuntimeError, match="missing"):
        lq.load_library()


def _quantize(w=X, p=P, t=T, N=4096, K=4096):
    return lq.load_library().lut6_quantize(w, p, t, N, K, None)


@pytest.mark.parametrize("kwargs, status", [
    (dict(w=None), 1), (dict(p=None), 1), (dict(t=None), 1),
    (dict(N=0), 2), (dict(N=4008), 2), (dict(K=0), 2), (dict(K=100), 2), (dict(K=4032 + 32), 2),
    (dict(K=2 ** 18 + 64), 2), (dict(N=2 ** 32), 2),
    (dict(w=X + 2), 3), (dict(p=P + 4), 3), (dict(t=T + 8), 3),
    (dict(p=X), 8), (dict(t=X + 64), 8), (dict(t=P), 8),
])
def test_quantize_validation(kwargs, status):
    # refusals are decided on the host, before any device call
    assert _quantize(**kwargs) == status


Q, S = 0x50_0000_0000, 0x60_0000_0000


def _int8_quantize(w=X, q=Q, s=S, N=4096, K=4096):
    return lq.load_library().lut6_int8_quantize(w, q, s, N, K, None)


@pytest.mark.parametrize("kwargs, status", [
    (dict(w=None), 1), (dict(q=None), 1), (dict(s=None), 1),
    (dict(N=0), 2), (dict(K=0), 2), (dict(K=4016), 2), (dict(N=2 ** 62), 2), (dict(N=2 ** 40, K=32), 2),
    (dict(w=X + 2), 3), (dict(q=Q + 8), 3), (dict(s=S + 1), 3),
    (dict(q=X), 8), (dict(s=X + 64), 8), (dict(s=Q + 32), 8),
])
def test_int8_quantize_validation(kwargs, status):
    # refusals are decided on the host, before any device call
    assert _int8_quantize(**kwargs) == status


def _int8_linear(x=X, q=Q, s=S, y=Y, L=128, K=4096, N=4096, scale=1.0, epi=1):
    return lq.load_library().lut6_int8_linear(x, q, s, y, L, K, N, scale, epi, None)


@pytest.mark.parametrize("kwargs, status", [
    (dict(x=None), 1), (dict(q=None), 1), (dict(s=None), 1), (dict(y=None), 1),
    (dict(L=-1), 2), (dict(K=0), 2), (dict(K=4000), 2), (dict(K=4064), 2), (dict(N=4008), 2),
    (dict(N=48, epi=2), 2), (dict(L=2 ** 18), 2), (dict(N=2 ** 19), 2),
    (dict(epi=3), 5), (dict(scale=3.0), 4), (dict(scale=0.5), 4),
    (dict(x=X + 8), 3), (dict(q=Q + 8), 3), (dict(s=S + 2), 3), (dict(y=Y + 4), 3),
    (dict(y=X), 8), (dict(y=Q + 16), 8), (dict(y=S), 8),
    (dict(L=0), 0),
])
def test_int8_linear_validation(kwargs, status):
    # refusals are decided on the host, before any device call
    assert _int8_linear(**kwargs) == status


def _attention(q=X, ldq=4096, k=P, ldk=1024, v=T, ldv=1024, o=Y, ldo=4096, L=128, Lk=512,
               hq=16, hkv=4, d=256):
    return lq.load_library().lut6_attention(q, ldq, k, ldk, v, ldv, o, ldo, L, Lk, hq, hkv, d, None)


@pytest.mark.parametrize("kwargs, status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(d=128), 2), (dict(hkv=3), 2), (dict(hkv=0), 2), (dict(hq=0), 2), (dict(L=-1), 2),
    (dict(Lk=100), 2), (dict(ldq=4088), 2), (dict(ldk=1016), 2), (dict(ldo=256), 2),
    (dict(ldk=(1 << 24) + 8), 2), (dict(ldv=(1 << 24) + 8), 2),
    (dict(ldq=4100), 3), (dict(ldv=1028), 3), (dict(q=X + 8), 3), (dict(o=Y + 2), 3),
    (dict(o=X + 4096), 8), (dict(o=P), 8), (dict(o=T + 16), 8),
    (dict(L=0), 0), (dict(L=0, Lk=0), 0),
])
def test_attention_validation(kwargs, status):
    # refusals are decided on the host, before any device call
    assert _attention(**kwargs) == status


G, B, ST = 0x70_0000_0000, 0x80_0000_0000, 0x90_0000_0000


def _gated_delta(q=X, ldq=8192, k=X + 4096, ldk=8192, v=X + 8192, ldv=8192, g=G, be=B, ldg=32,
                 o=Y, ldo=4096, st=ST, L=64, hk=16, hv=32, dk=128, dv=128):
    return lq.load_library().lut6_gated_delta(q, ldq, k, ldk, v, ldv, g, be, ldg, o, ldo, st, L,
                                              hk, hv, dk, dv, None)


@pytest.mark.parametrize("kwargs, status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(g=None), 1), (dict(be=None), 1),
    (dict(o=None), 1), (dict(st=None), 1),
    (dict(dk=64), 2), (dict(dv=256), 2), (dict(hk=3), 2), (dict(hv=0), 2), (dict(L=-1), 2),
    (dict(ldq=2040), 2), (dict(ldv=4088), 2), (dict(ldo=4000), 2), (dict(ldg=31), 2),
    (dict(ldk=(1 << 24) + 8), 2), (dict(ldo=(1 << 24) + 8), 2),
    (dict(ldq=8196), 3), (dict(o=Y + 8), 3), (dict(g=G + 2), 3), (dict(st=ST + 1), 3),
    (dict(o=X + 64), 8), (dict(o=G), 8), (dict(st=X), 8), (dict(st=B + 4), 8), (dict(o=ST), 8),
    (dict(L=0), 0),
])
def test_gated_delta_validation(kwargs, status):
    # refusals are decided on the host, before any device call
    assert _gated_delta(**kwargs) == status


def _linear_noalloc(x=X, p=P, t=T, y=Y, L=128, K=4096, N=4096, s=1.0, epi=1):
    return lq.load_library().lut6_linear_noalloc(x, p, t, y, L, K, N, s, epi, None)


@pytest.mark.parametrize("kwargs, status", [
    (dict(x=None), 1), (dict(y=None), 1), (dict(L=-1), 2), (dict(K=100), 2), (dict(N=4008), 2),
    (dict(N=48, epi=2), 2), (dict(L=2 ** 18), 2), (dict(epi=3), 5), (dict(s=3.0), 4),
    (dict(x=X + 8), 3), (dict(y=X), 8), (dict(L=0), 0),
    # the expanded weight of 65,536 channels at K = 4,096 is 545 MB of scratch
    (dict(L=2048, N=65536), 9),
    # deep K (expanded from 3,072 tokens): 15 tiles x 8 x 1,025 chunks x 4 KB
    (dict(L=3072, K=65536, N=3840), 9),
])
def test_linear_noalloc_validation(kwargs, status):
    # the same host checks as lut6_linear, then LUT6_E_SCRATCH for shapes
    # whose scratch exceeds the static array; all before any device call
    assert _linear_noalloc(**kwargs) == status


def test_noalloc_scratch_size_is_declared():
    text = HEADER.read_text()
    m = re.search(r"#define LUT6_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == lq.NOALLOC_SCRATCH_BYTES


# ---------------------------------------------------------------------------
# the Python binding's own checks (meta tensors stand in for device memory;
# every mismatch must raise before the library is called)
# ---------------------------------------------------------------------------

@pytest.fixture
def meta_device(monkeypatch):
    import torch
    monkeypatch.setattr(lq, "_is_device", lambda t: isinstance(t, torch.Tensor))
    monkeypatch.setattr(lq, "_stream_handle", lambda stream: None)

    def make(shape, dtype):
        return torch.empty(shape, dtype=dtype, device="meta")
    return make


def test_binding_linear_shapes(meta_device):
    import torch
    f16, u8 = torch.float16, torch.uint8
    x, p, t = meta_device((8, 64), f16), meta_device((32, 48), u8), meta_device((2, 64), f16)
    with pytest.raises(TypeError):
        lq.linear(x, meta_device((32, 40), u8), t)
    with pytest.raises(TypeError):
        lq.linear(x, p, meta_device((1, 64), f16))
    with pytest.raises(TypeError):
        lq.linear(x, p, t, out=meta_device((8, 16), f16))
    with pytest.raises(TypeError):
        lq.linear_noalloc(x, p, t, None)
    with pytest.raises(TypeError):
        lq.linear_noalloc(x, p, t, meta_device((8, 32), torch.float32))
    # well-formed operands reach the library, which refuses the null
    # pointers of meta tensors without any device work
    with pytest.raises(lq.Lut6Error) as e:
        lq.linear(x, p, t)
    assert e.value.status == "LUT6_E_NULL"
    with pytest.raises(lq.Lut6Error) as e:
        lq.linear_noalloc(x, p, t, meta_device((8, 32), f16))
    assert e.value.status == "LUT6_E_NULL"


def test_binding_dequant_shapes(meta_device):
    import torch
    p, t = meta_device((32, 48), torch.uint8), meta_device((2, 64), torch.float16)
    with pytest.raises(ValueError):
        lq.dequant(p, t, 128)
    with pytest.raises(ValueError):
        lq.dequant(p, meta_device((3, 64), torch.float16), 64)
    with pytest.raises(ValueError):
        lq.dequant(p, t, 64, out=meta_device((32, 32), torch.float16))
    with pytest.raises(lq.Lut6Error):
        lq.dequant(p, t, 64)


def test_binding_int8_shapes(meta_device):
    import torch
    f16, i8 = torch.float16, torch.int8
    x, q, s = meta_device((8, 64), f16), meta_device((32, 64), i8), meta_device((32, 2), f16)
    with pytest.raises(ValueError):
        lq.int8_linear(x, meta_device((32, 128), i8), s)
    with pytest.raises(ValueError):
        lq.int8_linear(x, q, meta_device((32, 1), f16))
    with pytest.raises(ValueError):
        lq.int8_linear(x, q, meta_device((16, 2), f16))
    with pytest.raises(ValueError):
        lq.int8_linear(x, q, s, out=meta_device((8, 16), f16))
    with pytest.raises(lq.Lut6Error):
        lq.int8_linear(x, q, s)


def test_binding_attention_shapes(meta_device):
    import torch
    f16 = torch.float16
    q, k, v = meta_device((4, 1024), f16), meta_device((8, 256), f16), meta_device((8, 256), f16)
    with pytest.raises(ValueError):       # q narrower than its heads
        lq.attention(meta_device((4, 768), f16), k, v, n_heads=4, n_kv_heads=1)
    with pytest.raises(ValueError):       # v rows differ from k rows
        lq.attention(q, k, meta_device((7, 256), f16), n_heads=4, n_kv_heads=1)
    with pytest.raises(ValueError):       # k narrower than its heads
        lq.attention(q, k, v, n_heads=4, n_kv_heads=2)
    with pytest.raises(ValueError):       # out rows
        lq.attention(q, k, v, n_heads=4, n_kv_heads=1, out=meta_device((3, 1024), f16))
    with pytest.raises(TypeError):        # out dtype
        lq.attention(q, k, v, n_heads=4, n_kv_heads=1, out=meta_device((4, 1024), torch.float32))
    with pytest.raises(lq.Lut6Error):
        lq.attention(q, k, v, n_heads=4, n_kv_heads=1)


def test_binding_gated_delta_shapes(meta_device):
    import torch
    f16, f32 = torch.float16, torch.float32
    L = 5
    q, k, v = meta_device((L, 256), f16), meta_device((L, 256), f16), meta_device((L, 512), f16)
    g, b, st = meta_device((L, 4), f32), meta_device((L, 4), f32), meta_device((4, 128, 128), f32)
    kw = dict(n_k_heads=2, n_v_heads=4)
    with pytest.raises(ValueError):       # v narrower than its heads
        lq.gated_delta(q, k, meta_device((L, 384), f16), g, b, st, **kw)
    with pytest.raises(ValueError):       # g has too few rows
        lq.gated_delta(q, k, v, meta_device((L - 1, 4), f32), b, st, **kw)
    with pytest.raises(ValueError):       # beta narrower than the value heads
        lq.gated_delta(q, k, v, g, meta_device((L, 3), f32), st, **kw)
    with pytest.raises(ValueError):       # state too small
        lq.gated_delta(q, k, v, g, b, meta_device((3, 128, 128), f32), **kw)
    with pytest.raises(TypeError):        # out dtype
        lq.gated_delta(q, k, v, g, b, st, out=meta_device((L, 512), f32), **kw)
    with pytest.raises(ValueError):       # out rows
        lq.gated_delta(q, k, v, g, b, st, out=meta_device((L + 1, 512), f16), **kw)
    with pytest.raises(lq.Lut6Error):
        lq.gated_delta(q, k, v, g, b, st, **kw)


def test_binding_int8_quantize_shapes(meta_device):
    import torch
    w = meta_device((4, 64), torch.float16)
    with pytest.raises(ValueError):
        lq.int8_quantize(meta_device((4, 48), torch.float16))
    with pytest.raises(ValueError):
        lq.int8_quantize(w, q=meta_device((4, 32), torch.int8))
    with pytest.raises(ValueError):
        lq.int8_quantize(w, scales=meta_device((4, 1), torch.float16))
    with pytest.raises(TypeError):
        lq.int8_quantize(meta_device((4, 64), torch.float32))
    with pytest.raises(lq.Lut6Error):
        lq.int8_quantize(w)


def test_binding_quantize_shapes(meta_device):
    import torch
    w = meta_device((32, 64), torch.float16)
    with pytest.raises(ValueError):
        lq.quantize(meta_device((24, 64), torch.float16))
    with pytest.raises(ValueError):
        lq.quantize(w, packed=meta_device((32, 64), torch.uint8))
    with pytest.raises(ValueError):
        lq.quantize(w, tables=meta_device((1, 64), torch.float16))
    with pytest.raises(lq.Lut6Error):
        lq.quantize(w)
