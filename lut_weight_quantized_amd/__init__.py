"""LUT-6 weight-quantized linear layer on AMD Instinct MI355X (gfx950).

Thin ctypes binding of the C ABI in ``include/lut6.h`` (library
``liblut6.so`` in this package, built by ``lut_weight_quantized_amd.build``).
It only marshals arguments: every step of the computation runs in the HIP
kernels.  PyTorch is used for device memory and streams.  There is no CPU
fallback: if the library is missing, every call raises.

Format (page "Clef-Flash-ANE-LUT6", sections "Weight precision" and "LUT-6
text weights"): 6-bit indices along the input dimension of a row-major
[N, K] weight, four packed little-endian into three bytes, and one table of
64 FP16 values per 16 output channels.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import numpy as np

PKG = Path(__file__).resolve().parent
LIB_PATH = PKG / "liblut6.so"

EPI_STORE_F32 = 0
EPI_STORE_F16 = 1
EPI_SILU_MUL_F16 = 2

STATUS = {0: "LUT6_OK", 1: "LUT6_E_NULL", 2: "LUT6_E_SHAPE", 3: "LUT6_E_ALIGN",
          4: "LUT6_E_SCALE", 5: "LUT6_E_EPILOGUE", 6: "LUT6_E_INDEX_RANGE",
          7: "LUT6_E_DEVICE", 8: "LUT6_E_ALIAS", 9: "LUT6_E_SCRATCH"}

# bytes of the static per-GPU array behind lut6_linear_noalloc
NOALLOC_SCRATCH_BYTES = 256 << 20

EXPORTS = ("lut6_packed_bytes", "lut6_table_bytes", "lut6_pack", "lut6_unpack",
           "lut6_linear", "lut6_linear_path", "lut6_dequant", "lut6_int8_linear", "lut6_attention",
           "lut6_gated_delta",
           "lut6_quantize", "lut6_int8_quantize",
           "lut6_release",
           "lut6_status_string",
           "lut6_linear_noalloc")

# kernel paths of lut6_linear (lut6_linear_path)
PATH_STREAM = 0
PATH_FUSED = 1
PATH_EXPANDED = 2


class Lut6Error(RuntimeError):
    """A nonzero status from the library; ``.status`` is its name."""

    def __init__(self, status: int, where: str):
        self.code = int(status)
        self.status = STATUS.get(self.code, f"LUT6_E_UNKNOWN({status})")
        super().__init__(f"{where}: {self.status}")


_lib = None


def load_library() -> ctypes.CDLL:
    """Load ``liblut6.so``; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m lut_weight_quantized_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(str(LIB_PATH))
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    lib.lut6_packed_bytes.argtypes = [I64, I64]
    lib.lut6_packed_bytes.restype = ctypes.c_size_t
    lib.lut6_table_bytes.argtypes = [I64]
    lib.lut6_table_bytes.restype = ctypes.c_size_t
    lib.lut6_pack.argtypes = [P, P, I64, I64]
    lib.lut6_pack.restype = ctypes.c_int
    lib.lut6_unpack.argtypes = [P, P, I64, I64]
    lib.lut6_unpack.restype = ctypes.c_int
    lib.lut6_linear.argtypes = [P, P, P, P, I64, I64, I64, ctypes.c_float, ctypes.c_int, P]
    lib.lut6_linear.restype = ctypes.c_int
    lib.lut6_linear_noalloc.argtypes = [P, P, P, P, I64, I64, I64, ctypes.c_float, ctypes.c_int, P]
    lib.lut6_linear_noalloc.restype = ctypes.c_int
    lib.lut6_linear_path.argtypes = [I64, I64, I64, ctypes.c_int]
    lib.lut6_linear_path.restype = ctypes.c_int
    lib.lut6_dequant.argtypes = [P, P, P, I64, I64, P]
    lib.lut6_dequant.restype = ctypes.c_int
    lib.lut6_int8_linear.argtypes = [P, P, P, P, I64, I64, I64, ctypes.c_float, ctypes.c_int, P]
    lib.lut6_int8_linear.restype = ctypes.c_int
    lib.lut6_attention.argtypes = [P, I64, P, I64, P, I64, P, I64, I64, I64, I64, I64, I64, P]
    lib.lut6_attention.restype = ctypes.c_int
    lib.lut6_gated_delta.argtypes = [P, I64, P, I64, P, I64, P, P, I64, P, I64, P, I64, I64, I64, I64,
                                     I64, P]
    lib.lut6_gated_delta.restype = ctypes.c_int
    lib.lut6_quantize.argtypes = [P, P, P, I64, I64, P]
    lib.lut6_quantize.restype = ctypes.c_int
    lib.lut6_int8_quantize.argtypes = [P, P, P, I64, I64, P]
    lib.lut6_int8_quantize.restype = ctypes.c_int
    lib.lut6_release.argtypes = []
    lib.lut6_release.restype = ctypes.c_int
    lib.lut6_status_string.argtypes = [ctypes.c_int]
    lib.lut6_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise Lut6Error(status, where)


def status_string(status: int) -> str:
    return load_library().lut6_status_string(int(status)).decode()


def packed_bytes(N: int, K: int) -> int:
    return int(load_library().lut6_packed_bytes(N, K))


def table_bytes(N: int) -> int:
    return int(load_library().lut6_table_bytes(N))


# ---------------------------------------------------------------------------
# host format functions (numpy in, numpy out)
# ---------------------------------------------------------------------------

def pack(idx: np.ndarray) -> np.ndarray:
    """uint8 indices [N, K] (each 0..63) -> packed bytes [N, 3K/4]."""
    idx = np.ascontiguousarray(idx)
    if idx.dtype != np.uint8 or idx.ndim != 2:
        raise TypeError("idx must be a 2-D uint8 array")
    N, K = idx.shape
    out = np.empty((N, 3 * K // 4 if K % 4 == 0 else 0), np.uint8)
    _check(load_library().lut6_pack(idx.ctypes.data, out.ctypes.data, N, K), "lut6_pack")
    return out


def unpack(packed: np.ndarray, K: int) -> np.ndarray:
    """packed bytes [N, 3K/4] -> uint8 indices [N, K]."""
    packed = np.ascontiguousarray(packed)
    if packed.dtype != np.uint8 or packed.ndim != 2 or packed.shape[1] * 4 != 3 * K:
        raise TypeError("packed must be a uint8 [N, 3K/4] array")
    out = np.empty((packed.shape[0], K), np.uint8)
    _check(load_library().lut6_unpack(packed.ctypes.data, out.ctypes.data, packed.shape[0], K),
           "lut6_unpack")
    return out


# ---------------------------------------------------------------------------
# device functions (torch tensors on the current HIP device)
# ---------------------------------------------------------------------------

def _stream_handle(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _same_device(*ts):
    dev = ts[0].device
    for t in ts[1:]:
        if t.device != dev:
            raise ValueError(f"tensors on different devices: {dev} and {t.device}")


def _is_device(t) -> bool:
    import torch
    return isinstance(t, torch.Tensor) and t.is_cuda


def _require(t, dtype, name):
    if not _is_device(t):
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise TypeError(f"{name} must be contiguous")


def _linear_operands(x, packed, tables, epilogue, out):
    """Check linear's operands; returns (L, K, N, out), allocating out if None."""
    import torch
    _require(x, torch.float16, "x")
    _require(packed, torch.uint8, "packed")
    _require(tables, torch.float16, "tables")
    if x.dim() != 2 or packed.dim() != 2:
        raise TypeError("x and packed must be 2-D")
    L, K = x.shape
    N = packed.shape[0]
    if packed.shape[1] * 4 != 3 * K or tables.numel() * 16 != N * 64:
        raise TypeError("packed / tables do not match x's K and packed's N")
    _same_device(x, packed, tables)
    n_out = N // 2 if epilogue == EPI_SILU_MUL_F16 else N
    dt = torch.float32 if epilogue == EPI_STORE_F32 else torch.float16
    if out is None:
        out = torch.empty((L, n_out), dtype=dt, device=x.device)
    else:
        _require(out, dt, "out")
        if tuple(out.shape) != (L, n_out):
            raise TypeError(f"out must be [{L}, {n_out}]")
        _same_device(x, out)
    return L, K, N, out


def linear(x, packed, tables, *, epilogue: int = EPI_STORE_F16, in_scale: float = 1.0,
           out=None, stream=None):
    """y = epilogue((fp16(x * in_scale) @ W^T) / in_scale) on the GPU.

    x: float16 [L, K]; packed: uint8 [N, 3K/4]; tables: float16 [N/16, 64];
    returns float32 [L, N] (EPI_STORE_F32), float16 [L, N] (EPI_STORE_F16) or
    float16 [L, N/2] (EPI_SILU_MUL_F16: rows [0, N/2) of W gate, the rest up).
    """
    L, K, N, out = _linear_operands(x, packed, tables, epilogue, out)
    st = load_library().lut6_linear(x.data_ptr(), packed.data_ptr(), tables.data_ptr(),
                                    out.data_ptr(), L, K, N, float(in_scale), int(epilogue),
                                    _stream_handle(stream))
    _check(st, "lut6_linear")
    return out


def linear_noalloc(x, packed, tables, out, *, epilogue: int = EPI_STORE_F16,
                   in_scale: float = 1.0, stream=None):
    """``linear`` without any device allocation: ``out`` must be given, and
    the library's scratch is its static per-GPU array (NOALLOC_SCRATCH_BYTES).
    Calls on one GPU must not overlap in time."""
    if out is None:
        raise TypeError("linear_noalloc needs a caller-allocated out")
    L, K, N, out = _linear_operands(x, packed, tables, epilogue, out)
    st = load_library().lut6_linear_noalloc(x.data_ptr(), packed.data_ptr(), tables.data_ptr(),
                                            out.data_ptr(), L, K, N, float(in_scale),
                                            int(epilogue), _stream_handle(stream))
    _check(st, "lut6_linear_noalloc")
    return out


def linear_path(L: int, K: int, N: int, epilogue: int = EPI_STORE_F16) -> int:
    """Which kernels lut6_linear runs for these sizes (PATH_*); raises on
    sizes it would refuse."""
    r = int(load_library().lut6_linear_path(L, K, N, int(epilogue)))
    if r < 0:
        raise Lut6Error(-r, "lut6_linear_path")
    return r


def dequant(packed, tables, K: int, *, out=None, stream=None):
    """FP16 weight [N, K] with w[n, k] = tables[n/16][index(n, k)] (bit copy)."""
    import torch
    _require(packed, torch.uint8, "packed")
    _require(tables, torch.float16, "tables")
    if packed.dim() != 2 or packed.shape[1] * 4 != 3 * K:
        raise ValueError(f"packed must be [N, {3 * K // 4}] for K = {K}")
    N = packed.shape[0]
    if tables.numel() * 16 != N * 64:
        raise ValueError(f"tables must hold {N // 16} x 64 entries for N = {N}")
    _same_device(packed, tables)
    if out is None:
        out = torch.empty((N, K), dtype=torch.float16, device=packed.device)
    else:
        _require(out, torch.float16, "out")
        if tuple(out.shape) != (N, K):
            raise ValueError(f"out must be [{N}, {K}]")
        _same_device(packed, out)
    st = load_library().lut6_dequant(packed.data_ptr(), tables.data_ptr(), out.data_ptr(),
                                     N, K, _stream_handle(stream))
    _check(st, "lut6_dequant")
    return out


def int8_linear(x, q, scales, *, epilogue: int = EPI_STORE_F16, in_scale: float = 1.0,
                out=None, stream=None):
    """y = epilogue((fp16(x * in_scale) @ W^T) / in_scale) for an int8 weight:
    W = fp16(q * scales[:, k // 32]); q int8 [N, K], scales float16 [N, K/32]."""
    import torch
    _require(x, torch.float16, "x")
    _require(q, torch.int8, "q")
    _require(scales, torch.float16, "scales")
    if x.dim() != 2 or q.dim() != 2:
        raise ValueError("x and q must be 2-D")
    L, K = x.shape
    N = q.shape[0]
    if q.shape[1] != K:
        raise ValueError(f"q must be [N, {K}] to match x's K")
    if K % 32 or tuple(scales.shape) != (N, K // 32):
        raise ValueError(f"scales must be [{N}, K/32] with K % 32 == 0 (K = {K})")
    _same_device(x, q, scales)
    n_out = N // 2 if epilogue == EPI_SILU_MUL_F16 else N
    dtype = torch.float32 if epilogue == EPI_STORE_F32 else torch.float16
    if out is None:
        out = torch.empty((L, n_out), dtype=dtype, device=x.device)
    else:
        _require(out, dtype, "out")
        if tuple(out.shape) != (L, n_out):
            raise ValueError(f"out must be [{L}, {n_out}]")
        _same_device(x, out)
    st = load_library().lut6_int8_linear(x.data_ptr(), q.data_ptr(), scales.data_ptr(), out.data_ptr(),
                                         L, K, N, float(in_scale), int(epilogue), _stream_handle(stream))
    _check(st, "lut6_int8_linear")
    return out


def _rows(t, name, dtype, rows, min_cols):
    """A 2-D device tensor of `rows` rows, unit column stride (row stride free)
    and at least `min_cols` columns: what the kernels read from each row."""
    if not _is_device(t):
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype or t.dim() != 2 or t.stride(1) != 1:
        raise TypeError(f"{name} must be 2-D {dtype} with unit column stride")
    if t.shape[0] != rows:
        raise ValueError(f"{name} must have {rows} rows, got {t.shape[0]}")
    if t.shape[1] < min_cols:
        raise ValueError(f"{name} must have at least {min_cols} columns, got {t.shape[1]}")
    if t.shape[0] > 1 and t.stride(0) < min_cols:
        raise ValueError(f"{name}'s rows overlap (row stride {t.stride(0)} < {min_cols})")


def _ld(t):
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def attention(q, k, v, *, n_heads: int, n_kv_heads: int, head_dim: int = 256, out=None,
              stream=None):
    """Causal grouped-query attention of the last L of Lk positions.

    q: float16 [L, >= n_heads*head_dim] (2-D, rows may be strided views such
    as columns of the Q|K|V projection output), k, v: float16 [Lk, >=
    n_kv_heads*head_dim]; returns o float16 [L, n_heads * head_dim]."""
    import torch
    if n_heads <= 0 or n_kv_heads <= 0 or head_dim <= 0:
        raise ValueError("head counts and head_dim must be positive")
    L, Lk = q.shape[0], k.shape[0]
    _rows(q, "q", torch.float16, L, n_heads * head_dim)
    _rows(k, "k", torch.float16, Lk, n_kv_heads * head_dim)
    _rows(v, "v", torch.float16, Lk, n_kv_heads * head_dim)
    _same_device(q, k, v)
    if out is None:
        out = torch.empty((L, n_heads * head_dim), dtype=torch.float16, device=q.device)
    else:
        _rows(out, "out", torch.float16, L, n_heads * head_dim)
        _same_device(q, out)
    st = load_library().lut6_attention(q.data_ptr(), _ld(q), k.data_ptr(), _ld(k), v.data_ptr(), _ld(v),
                                       out.data_ptr(), _ld(out), L, Lk, n_heads, n_kv_heads, head_dim,
                                       _stream_handle(stream))
    _check(st, "lut6_attention")
    return out


def gated_delta(q, k, v, g, beta, state, *, n_k_heads: int, n_v_heads: int, out=None,
                stream=None):
    """Gated delta rule over the L rows (tokens) of q, k, v; updates `state`
    (float32 [n_v_heads, 128, 128], in place) and returns o float16
    [L, n_v_heads * 128].  q, k: float16 [L, >= n_k_heads*128]; v float16
    [L, >= n_v_heads*128] (row strides allowed, unit column stride); g, beta:
    float32 [L, >= n_v_heads] with the same row stride."""
    import torch
    if n_k_heads <= 0 or n_v_heads <= 0:
        raise ValueError("head counts must be positive")
    L = q.shape[0]
    _rows(q, "q", torch.float16, L, n_k_heads * 128)
    _rows(k, "k", torch.float16, L, n_k_heads * 128)
    _rows(v, "v", torch.float16, L, n_v_heads * 128)
    _rows(g, "g", torch.float32, L, n_v_heads)
    _rows(beta, "beta", torch.float32, L, n_v_heads)
    if L > 1 and g.stride(0) != beta.stride(0):
        raise ValueError("g and beta must have the same row stride")
    _require(state, torch.float32, "state")
    if state.numel() != n_v_heads * 128 * 128:
        raise ValueError(f"state must hold [{n_v_heads}, 128, 128] floats")
    _same_device(q, k, v, g, beta, state)
    if out is None:
        out = torch.empty((L, n_v_heads * 128), dtype=torch.float16, device=q.device)
    else:
        _rows(out, "out", torch.float16, L, n_v_heads * 128)
        _same_device(q, out)
    st = load_library().lut6_gated_delta(q.data_ptr(), _ld(q), k.data_ptr(), _ld(k), v.data_ptr(), _ld(v),
                                         g.data_ptr(), beta.data_ptr(), _ld(g), out.data_ptr(), _ld(out),
                                         state.data_ptr(), L, n_k_heads, n_v_heads, 128, 128,
                                         _stream_handle(stream))
    _check(st, "lut6_gated_delta")
    return out


def quantize(w, *, packed=None, tables=None, stream=None):
    """Fit LUT-6 tables to an FP16 weight [N, K] (40 rounds of 1-D k-means per
    16 rows) and pack its indices; returns (packed uint8 [N, 3K/4], tables
    float16 [N/16, 64]), both on w's device."""
    import torch
    _require(w, torch.float16, "w")
    if w.dim() != 2:
        raise ValueError("w must be 2-D [N, K]")
    N, K = w.shape
    if K % 4 or N % 16:
        raise ValueError(f"w must be [N, K] with N % 16 == 0 and K % 4 == 0, got [{N}, {K}]")
    if packed is None:
        packed = torch.empty((N, K // 4 * 3), dtype=torch.uint8, device=w.device)
    else:
        _require(packed, torch.uint8, "packed")
        if tuple(packed.shape) != (N, K // 4 * 3):
            raise ValueError(f"packed must be [{N}, {K // 4 * 3}]")
    if tables is None:
        tables = torch.empty((N // 16, 64), dtype=torch.float16, device=w.device)
    else:
        _require(tables, torch.float16, "tables")
        if tuple(tables.shape) != (N // 16, 64):
            raise ValueError(f"tables must be [{N // 16}, 64]")
    _same_device(w, packed, tables)
    st = load_library().lut6_quantize(w.data_ptr(), packed.data_ptr(), tables.data_ptr(),
                                      N, K, _stream_handle(stream))
    _check(st, "lut6_quantize")
    return packed, tables


def int8_quantize(w, *, q=None, scales=None, stream=None):
    """int8 codes of an FP16 weight [N, K] for int8_linear: symmetric per
    block of 32 inputs (scale = largest magnitude / 127 in FP16, codes
    rounded and clamped to -127..127); returns (q int8 [N, K], scales
    float16 [N, K/32]), both on w's device."""
    import torch
    _require(w, torch.float16, "w")
    if w.dim() != 2:
        raise ValueError("w must be 2-D [N, K]")
    N, K = w.shape
    if K % 32 or N == 0:
        raise ValueError(f"w must be [N, K] with N > 0 and K % 32 == 0, got [{N}, {K}]")
    if q is None:
        q = torch.empty((N, K), dtype=torch.int8, device=w.device)
    else:
        _require(q, torch.int8, "q")
        if tuple(q.shape) != (N, K):
            raise ValueError(f"q must be [{N}, {K}]")
    if scales is None:
        scales = torch.empty((N, K // 32), dtype=torch.float16, device=w.device)
    else:
        _require(scales, torch.float16, "scales")
        if tuple(scales.shape) != (N, K // 32):
            raise ValueError(f"scales must be [{N}, {K // 32}]")
    _same_device(w, q, scales)
    st = load_library().lut6_int8_quantize(w.data_ptr(), q.data_ptr(), scales.data_ptr(), N, K,
                                           _stream_handle(stream))
    _check(st, "lut6_int8_quantize")
    return q, scales


def release() -> None:
    _check(load_library().lut6_release(), "lut6_release")
