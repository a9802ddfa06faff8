"""CPU oracle of the LUT-6 linear layer -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  The product library never does, and this
package imports nothing from it.

The arithmetic lives in ``lut6_oracle.c`` (plain C, FP64 accumulation, its
own FP16 codec and unpack; see the header of that file for the passages of
page "Clef-Flash-ANE-LUT6" it follows).  This module compiles it with gcc and
marshals numpy arrays into it through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SRC = HERE / "lut6_oracle.c"
LIB = HERE / "liblut6_oracle.so"

EPI_F32, EPI_F16, EPI_SILU_MUL_F16 = 0, 1, 2
OK, E_NULL, E_SHAPE, E_SCALE, E_EPILOGUE, E_INDEX_RANGE, E_ROWS, E_NOMEM = 0, 1, 2, 4, 5, 6, 8, 9

CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
          "-Wall", "-Wextra"]


class OracleError(RuntimeError):
    pass


def build(out: Path | None = None, mutant: int = 0) -> Path:
    """Compile the oracle (``mutant`` > 0 plants a known mistake; tests only)."""
    out = Path(out) if out is not None else LIB
    cmd = ["gcc", *CFLAGS, f"-DORA_MUTANT={int(mutant)}", "-o", str(out), str(SRC), "-lm"]
    tmp = out.with_suffix(out.suffix + f".tmp{os.getpid()}")
    cmd[cmd.index(str(out))] = str(tmp)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_P = ctypes.c_void_p
_I64 = ctypes.c_int64


class Oracle:
    """ctypes view of one build of the oracle library."""

    def __init__(self, path: Path):
        lib = ctypes.CDLL(str(path))
        lib.ora_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.ora_f16_to_f64.restype = ctypes.c_double
        lib.ora_f64_to_f16.argtypes = [ctypes.c_double]
        lib.ora_f64_to_f16.restype = ctypes.c_uint16
        lib.ora_f16_decode_array.argtypes = [_P, _P, _I64]
        lib.ora_f16_decode_array.restype = None
        lib.ora_f16_encode_array.argtypes = [_P, _P, _I64]
        lib.ora_f16_encode_array.restype = None
        for name in ("ora_pack", "ora_unpack"):
            getattr(lib, name).argtypes = [_P, _P, _I64, _I64]
            getattr(lib, name).restype = ctypes.c_int
        lib.ora_dequant.argtypes = [_P, _P, _P, _I64, _I64]
        lib.ora_dequant.restype = ctypes.c_int
        lib.ora_linear.argtypes = [_P, _P, _P, _I64, _I64, _I64, ctypes.c_double,
                                   ctypes.c_int, _P, _I64, ctypes.c_int, _P, _P]
        lib.ora_linear.restype = ctypes.c_int
        lib.ora_int8_linear.argtypes = [_P, _P, _P, _I64, _I64, _I64, ctypes.c_double,
                                        ctypes.c_int, _P, _I64, ctypes.c_int, _P, _P]
        lib.ora_int8_linear.restype = ctypes.c_int
        lib.ora_int8_dequant.argtypes = [_P, _P, _P, _I64, _I64]
        lib.ora_int8_dequant.restype = ctypes.c_int
        lib.ora_int8_quantize.argtypes = [_P, _P, _P, _I64, _I64]
        lib.ora_int8_quantize.restype = ctypes.c_int
        lib.ora_attention.argtypes = [_P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _I64, _I64,
                                      _P, _I64, ctypes.c_int, _P, _P, _P, _P]
        lib.ora_attention.restype = ctypes.c_int
        lib.ora_gated_delta.argtypes = [_P, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _I64, _I64, _I64,
                                        _I64, _I64, _P, ctypes.c_int, _P, _P, _P, _P]
        lib.ora_gated_delta.restype = ctypes.c_int
        lib.ora_quantize.argtypes = [_P, _P, _P, _I64, _I64, _I64, _I64, _P]
        lib.ora_quantize.restype = ctypes.c_int
        lib.ora_km_centres.argtypes = [_P, _I64, _I64, _I64, ctypes.c_int, _P]
        lib.ora_km_centres.restype = ctypes.c_int
        lib.ora_packed_bytes.argtypes = [_I64, _I64]
        lib.ora_packed_bytes.restype = _I64
        lib.ora_table_bytes.argtypes = [_I64]
        lib.ora_table_bytes.restype = _I64
        self.lib = lib
        self.path = path

    # -- FP16 codec ------------------------------------------------------
    def f16_to_f64(self, bits: np.ndarray) -> np.ndarray:
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, np.float64)
        self.lib.ora_f16_decode_array(bits.ctypes.data, out.ctypes.data, bits.size)
        return out

    def f64_to_f16(self, v: np.ndarray) -> np.ndarray:
        v = np.ascontiguousarray(v, dtype=np.float64)
        out = np.empty(v.shape, np.uint16)
        self.lib.ora_f16_encode_array(v.ctypes.data, out.ctypes.data, v.size)
        return out

    # -- format ------------------------------------------------------------
    def pack(self, idx: np.ndarray) -> np.ndarray:
        idx = np.ascontiguousarray(idx, dtype=np.uint8)
        n, k = idx.shape
        out = np.empty((n, 3 * k // 4), np.uint8)
        st = self.lib.ora_pack(idx.ctypes.data, out.ctypes.data, n, k)
        if st != OK:
            raise OracleError(f"ora_pack status {st}")
        return out

    def unpack(self, packed: np.ndarray, k: int) -> np.ndarray:
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        n = packed.shape[0]
        out = np.empty((n, k), np.uint8)
        st = self.lib.ora_unpack(packed.ctypes.data, out.ctypes.data, n, k)
        if st != OK:
            raise OracleError(f"ora_unpack status {st}")
        return out

    def packed_bytes(self, n: int, k: int) -> int:
        return int(self.lib.ora_packed_bytes(n, k))

    def table_bytes(self, n: int) -> int:
        return int(self.lib.ora_table_bytes(n))

    # -- dequant / linear --------------------------------------------------
    def dequant(self, packed: np.ndarray, tables: np.ndarray, k: int) -> np.ndarray:
        """FP16 bits [N, K] of the dequantized weight."""
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        tables = np.ascontiguousarray(tables).view(np.uint16)
        n = packed.shape[0]
        out = np.empty((n, k), np.uint16)
        st = self.lib.ora_dequant(packed.ctypes.data, tables.ctypes.data, out.ctypes.data, n, k)
        if st != OK:
            raise OracleError(f"ora_dequant status {st}")
        return out

    def linear(self, x: np.ndarray, packed: np.ndarray, tables: np.ndarray, *,
               epilogue: int, in_scale: float = 1.0, rows=None, threads: int | None = None):
        """Return (y_exact float64, y_out) for the listed token rows.

        ``x`` is FP16 [L, K] (float16 or uint16 bits), ``packed`` [N, 3K/4] bytes,
        ``tables`` FP16 [N/16, 64].  ``y_out`` is float32 for EPI_F32 and FP16
        bits (uint16) otherwise; its width is N, or N/2 for EPI_SILU_MUL_F16.
        """
        x = np.ascontiguousarray(x).view(np.uint16)
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        tables = np.ascontiguousarray(tables).view(np.uint16)
        L, K = x.shape
        N = packed.shape[0]
        if packed.shape[1] * 4 != 3 * K:
            raise OracleError("packed width does not match K")
        if rows is None:
            rows_arr, n_rows, rows_ptr = None, L, None
        else:
            rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
            n_rows = rows_arr.size
            rows_ptr = rows_arr.ctypes.data
        n_out = N // 2 if epilogue == EPI_SILU_MUL_F16 else N
        y_exact = np.empty((n_rows, n_out), np.float64)
        y_out = np.empty((n_rows, n_out), np.float32 if epilogue == EPI_F32 else np.uint16)
        if threads is None:
            threads = len(os.sched_getaffinity(0))
        st = self.lib.ora_linear(x.ctypes.data, packed.ctypes.data, tables.ctypes.data,
                                 L, K, N, float(in_scale), int(epilogue), rows_ptr, n_rows,
                                 int(threads), y_exact.ctypes.data, y_out.ctypes.data)
        if st != OK:
            raise OracleError(f"ora_linear status {st}")
        return y_exact, y_out


    # -- int8 weight-only variant -------------------------------------------
    def int8_linear(self, x: np.ndarray, q: np.ndarray, scales: np.ndarray, *,
                    epilogue: int, in_scale: float = 1.0, rows=None, threads: int | None = None):
        """As linear(), for an int8 weight q [N, K] with FP16 scales [N, K/32]."""
        x = np.ascontiguousarray(x).view(np.uint16)
        q = np.ascontiguousarray(q).view(np.int8)
        scales = np.ascontiguousarray(scales).view(np.uint16)
        L, K = x.shape
        N = q.shape[0]
        if q.shape[1] != K or scales.shape != (N, K // 32):
            raise OracleError("q / scales shapes do not match x")
        if rows is None:
            rows_arr, n_rows, rows_ptr = None, L, None
        else:
            rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
            n_rows = rows_arr.size
            rows_ptr = rows_arr.ctypes.data
        n_out = N // 2 if epilogue == EPI_SILU_MUL_F16 else N
        y_exact = np.empty((n_rows, n_out), np.float64)
        y_out = np.empty((n_rows, n_out), np.float32 if epilogue == EPI_F32 else np.uint16)
        if threads is None:
            threads = len(os.sched_getaffinity(0))
        st = self.lib.ora_int8_linear(x.ctypes.data, q.ctypes.data, scales.ctypes.data,
                                      L, K, N, float(in_scale), int(epilogue), rows_ptr, n_rows,
                                      int(threads), y_exact.ctypes.data, y_out.ctypes.data)
        if st != OK:
            raise OracleError(f"ora_int8_linear status {st}")
        return y_exact, y_out

    def int8_dequant(self, q: np.ndarray, scales: np.ndarray) -> np.ndarray:
        """FP16 bits [N, K]: the weight nearest to q * scale."""
        q = np.ascontiguousarray(q).view(np.int8)
        scales = np.ascontiguousarray(scales).view(np.uint16)
        n, k = q.shape
        w = np.empty((n, k), np.uint16)
        st = self.lib.ora_int8_dequant(q.ctypes.data, scales.ctypes.data, w.ctypes.data, n, k)
        if st != OK:
            raise OracleError(f"ora_int8_dequant status {st}")
        return w

    def int8_quantize(self, w16: np.ndarray):
        """Codes int8 [N, K] and FP16 scale bits [N, K/32] of an FP16 weight
        (symmetric per block of 32, codes clamped to -127..127)."""
        w = np.ascontiguousarray(w16).view(np.uint16)
        n, k = w.shape
        q = np.empty((n, k), np.int8)
        qs = np.empty((n, max(k // 32, 1)), np.uint16)
        st = self.lib.ora_int8_quantize(w.ctypes.data, q.ctypes.data, qs.ctypes.data, n, k)
        if st != OK:
            raise OracleError(f"ora_int8_quantize status {st}")
        return q, qs

    # -- full attention -----------------------------------------------------
    def attention(self, q: np.ndarray, k: np.ndarray, v: np.ndarray, *, n_heads: int,
                  n_kv_heads: int, head_dim: int, rows=None, threads: int | None = None,
                  with_bounds: bool = False):
        """Causal GQA softmax attention of the last L of Lk positions.

        q: FP16 [L, ldq] (head h at columns h*D..), k, v: FP16 [Lk, ld] (head
        g at columns g*D..).  Returns (o_exact float64, o_out FP16 bits), each
        [n_rows, n_heads*head_dim], plus (o_abs, v_abs) when with_bounds."""
        q = np.ascontiguousarray(q).view(np.uint16)
        k = np.ascontiguousarray(k).view(np.uint16)
        v = np.ascontiguousarray(v).view(np.uint16)
        L, Lk = q.shape[0], k.shape[0]
        if v.shape[0] != Lk:
            raise OracleError("k and v lengths differ")
        if rows is None:
            rows_arr, n_rows, rows_ptr = None, L, None
        else:
            rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
            n_rows, rows_ptr = rows_arr.size, rows_arr.ctypes.data
        W = n_heads * head_dim
        oe = np.empty((n_rows, W), np.float64)
        oo = np.empty((n_rows, W), np.uint16)
        oa = np.empty((n_rows, W), np.float64) if with_bounds else None
        va = np.empty((n_rows, W), np.float64) if with_bounds else None
        if threads is None:
            threads = len(os.sched_getaffinity(0))
        st = self.lib.ora_attention(q.ctypes.data, q.shape[1], k.ctypes.data, k.shape[1],
                                    v.ctypes.data, v.shape[1], L, Lk, n_heads, n_kv_heads, head_dim,
                                    rows_ptr, n_rows, int(threads), oe.ctypes.data, oo.ctypes.data,
                                    oa.ctypes.data if with_bounds else None,
                                    va.ctypes.data if with_bounds else None)
        if st != OK:
            raise OracleError(f"ora_attention status {st}")
        return (oe, oo, oa, va) if with_bounds else (oe, oo)

    # -- Gated DeltaNet recurrence ---------------------------------------------
    def gated_delta(self, q, k, v, g, beta, *, n_k_heads: int, n_v_heads: int, dk: int = 128,
                    dv: int = 128, state=None, threads: int | None = None):
        """Gated delta rule over L tokens (see ora_gated_delta).

        q, k: FP16 [L, ld] (key head at columns kh*dk ..), v: FP16 [L, ld]
        (value head at h*dv ..), g, beta: float32 [L, n_v_heads], state:
        float32 [n_v_heads, dk, dv] or None.  Returns (o_exact, o_out bits,
        o_abs) [L, n_v_heads*dv] and the final state (float64)."""
        q = np.ascontiguousarray(q).view(np.uint16)
        k = np.ascontiguousarray(k).view(np.uint16)
        v = np.ascontiguousarray(v).view(np.uint16)
        g = np.ascontiguousarray(g, dtype=np.float32)
        beta = np.ascontiguousarray(beta, dtype=np.float32)
        L = q.shape[0]
        if k.shape[0] != L or v.shape[0] != L or g.shape != beta.shape or g.shape[0] != L:
            raise OracleError("q, k, v, g, beta lengths differ")
        st_in = None if state is None else np.ascontiguousarray(state, dtype=np.float32)
        W = n_v_heads * dv
        oe = np.empty((L, W), np.float64)
        oo = np.empty((L, W), np.uint16)
        oa = np.empty((L, W), np.float64)
        so = np.empty((n_v_heads, dk, dv), np.float64)
        if threads is None:
            threads = len(os.sched_getaffinity(0))
        st = self.lib.ora_gated_delta(q.ctypes.data, q.shape[1], k.ctypes.data, k.shape[1],
                                      v.ctypes.data, v.shape[1], g.ctypes.data, beta.ctypes.data,
                                      g.shape[1], L, n_k_heads, n_v_heads, dk, dv,
                                      None if st_in is None else st_in.ctypes.data, int(threads),
                                      oe.ctypes.data, oo.ctypes.data, oa.ctypes.data, so.ctypes.data)
        if st != OK:
            raise OracleError(f"ora_gated_delta status {st}")
        return oe, oo, oa, so

    # -- table fitting ---------------------------------------------------
    def quantize(self, w16: np.ndarray, groups=None, with_sse: bool = False):
        """1-D k-means tables and packed indices of an FP16 weight [N, K].

        Returns (packed uint8 [N, 3K/4], tables uint16 [N/16, 64]), and the
        first group's squared errors when with_sse (before round 1 and after
        every round: as many values as the oracle ran rounds, plus one); with
        ``groups`` = (g0, g1) only those groups' rows and tables are computed
        (the rest are zero)."""
        w = np.ascontiguousarray(np.asarray(w16).view(np.uint16))
        n, k = w.shape
        g0, g1 = (0, n // 16) if groups is None else groups
        packed = np.zeros((n, 3 * k // 4), np.uint8)
        tables = np.zeros((n // 16, 64), np.uint16)
        sse = np.full(64, np.nan, np.float64)
        st = self.lib.ora_quantize(w.ctypes.data, packed.ctypes.data, tables.ctypes.data, n, k,
                                   int(g0), int(g1), sse.ctypes.data if with_sse else None)
        if st != OK:
            raise OracleError(f"ora_quantize status {st}")
        return (packed, tables, sse[~np.isnan(sse)]) if with_sse else (packed, tables)

    def km_centres(self, w16: np.ndarray, group: int, rounds: int) -> np.ndarray:
        """Group `group`'s 64 FP64 centres after `rounds` Lloyd rounds (0: the
        starting centres), as ora_quantize computes them."""
        w = np.ascontiguousarray(np.asarray(w16).view(np.uint16))
        n, k = w.shape
        c = np.zeros(64, np.float64)
        st = self.lib.ora_km_centres(w.ctypes.data, n, k, int(group), int(rounds), c.ctypes.data)
        if st != OK:
            raise OracleError(f"ora_km_centres status {st}")
        return c


_default: Oracle | None = None


def load(rebuild: bool = False) -> Oracle:
    """The default (unmutated) oracle, built on first use."""
    global _default
    if _default is None or rebuild:
        if rebuild or not LIB.exists() or LIB.stat().st_mtime < SRC.stat().st_mtime:
            build()
        _default = Oracle(LIB)
    return _default
