"""Parity criteria between a device result and the oracle -- test
infrastructure only (used by the tests, the smoke check and the benchmark's
parity sample).

Criteria, fixed before any device run:
  * dequantized weights: bit-exact (a lookup has exactly one right answer);
  * every output: |y - y_ref| <= B_row with
        B_row = 2e-3 * ||x_row||_2 * max|table| * sqrt(K) / 64
    where x_row is the unscaled input row, max|table| the largest magnitude
    over all tables of the weight, and y_ref the oracle's unrounded value.
    The bound is on the FP32 result: an FP16 output also carries its own
    rounding to FP16, up to half an FP16 ulp, which even fp16(y_ref) has
    (for short K and small tables that half ulp exceeds B_row), so for FP16
    outputs the allowance is B_row + ulp16(y_ref) / 2;
  * FP16 outputs: at most 1 unit in the last place from fp16(y_ref)
    (distance between the ordered bit patterns, +0 == -0).  Near zero the
    FP16 ulp falls below the FP32 summation noise of any correct FP32-
    accumulating kernel, so where |y_ref| < tau_row = 2^-8 * S_row
    (S_row = B_row / 2e-3, the natural scale of the row) the allowance is
    the absolute ulp16(tau_row) instead.  An FP32 sum of exact FP16
    products, added 16 at a time, has errors up to about 2^-20.5 S_row on
    the full-size workloads (K = 4,096 and 12,288, 262,144 outputs each):
    up to 1.4 ulp16(2^-10 S_row), and 0.36 ulp16(2^-8 S_row);
  * SiLU(gate) * up: the bound propagates through h = silu(g) * u as
        B_h = (1.1 |u_ref| + |silu(g_ref)|) * B_row     (|silu'| <= 1.1)
    with the same ulp rule on S_h = B_h / 2e-3.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

REL = 2e-3
TAU_REL = 2.0 ** -8                # the near-zero floor, as a fraction of S_row


def row_scale(x16: np.ndarray, tables16: np.ndarray, K: int, rows=None) -> np.ndarray:
    """S_row = ||x_row||_2 * max|table| * sqrt(K) / 64 for the listed rows."""
    x = np.asarray(x16).view(np.float16)
    if rows is not None:
        x = x[np.asarray(rows)]
    xn = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=1))
    tmax = float(np.max(np.abs(np.asarray(tables16).view(np.float16).astype(np.float64))))
    return xn * tmax * np.sqrt(K) / 64.0


def _ordered(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp16(v: np.ndarray) -> np.ndarray:
    """Spacing of FP16 numbers at |v| (2^-24 below the normal range)."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


@dataclass
class Report:
    ok: bool
    n: int
    max_abs_err: float
    max_err_over_bound: float
    max_ulp: int
    strict_ulp_violations: int       # beyond 1 ulp, counted without the floor (diagnostic)
    floor_cases: int
    failures: int
    floor_max_ratio: float = 0.0     # largest |y - fp16(y_ref)| / ulp16(tau) in the floor (<= 1 passes)

    def __str__(self):
        return (f"ok={self.ok} n={self.n} max|err|={self.max_abs_err:.3g} "
                f"max err/bound={self.max_err_over_bound:.3g} max_ulp={self.max_ulp} "
                f"strict>1ulp={self.strict_ulp_violations} floor={self.floor_cases} "
                f"floor max/allow={self.floor_max_ratio:.3g} failures={self.failures}")


def check(y_dev: np.ndarray, y_exact: np.ndarray, S_row: np.ndarray, *, fp16: bool,
          S_elem: np.ndarray | None = None) -> Report:
    """Compare device outputs with the oracle's unrounded values.

    y_dev: float32 array, or FP16 (float16 / uint16 bits) when fp16=True.
    S_row: per-row scale [rows]; S_elem (optional, SiLU) per-element scale.
    """
    y_exact = np.asarray(y_exact, np.float64)
    S = np.asarray(S_elem, np.float64) if S_elem is not None else np.asarray(S_row, np.float64)[:, None]
    S = np.broadcast_to(S, y_exact.shape)
    bound = REL * S
    if fp16:
        bits = np.asarray(y_dev).view(np.uint16)
        val = bits.view(np.float16).astype(np.float64)
        with np.errstate(invalid="ignore"):
            bound = bound + 0.5 * ulp16(np.where(np.isfinite(y_exact), y_exact, 0.0))
    else:
        val = np.asarray(y_dev, np.float32).astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        err = np.abs(val - y_exact)
        same_inf = np.isinf(val) & np.isinf(y_exact) & (np.sign(val) == np.sign(y_exact))
        both_nan = np.isnan(val) & np.isnan(y_exact)
        special = same_inf | both_nan
        err = np.where(special, 0.0, err)
        bad = ~(err <= bound)
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    max_ulp = 0
    strict = 0
    floor_cases = 0
    if fp16:
        with np.errstate(over="ignore"):
            ref_bits = y_exact.astype(np.float16).view(np.uint16)
        d = np.abs(_ordered(bits) - _ordered(ref_bits))
        d = np.where(special, 0, d)
        tau = TAU_REL * S
        floor = np.abs(y_exact) < tau
        ref16 = ref_bits.view(np.float16).astype(np.float64)
        with np.errstate(invalid="ignore"):
            floor_dev = np.abs(val - ref16) / ulp16(tau)
            floor_ok = floor_dev <= 1.0
        ulp_bad = np.where(floor, ~floor_ok, d > 1)
        floor_max = float(np.max(floor_dev[floor])) if np.any(floor) else 0.0
        bad = bad | ulp_bad
        max_ulp = int(d[~floor].max()) if np.any(~floor) else 0
        strict = int(np.sum(d > 1))
        floor_cases = int(np.sum(floor))
    return Report(ok=not bool(np.any(bad)), n=int(y_exact.size),
                  max_abs_err=float(np.max(err)) if err.size else 0.0,
                  max_err_over_bound=float(np.max(ratio)) if ratio.size else 0.0,
                  max_ulp=max_ulp, strict_ulp_violations=strict, floor_cases=floor_cases,
                  failures=int(np.sum(bad)), floor_max_ratio=floor_max if fp16 else 0.0)


def silu_scale(g_exact: np.ndarray, u_exact: np.ndarray, S_row: np.ndarray) -> np.ndarray:
    """Per-element S_h = (1.1 |u| + |silu(g)|) * S_row for h = silu(g) * u."""
    g = np.asarray(g_exact, np.float64)
    u = np.asarray(u_exact, np.float64)
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(-g))
    return (1.1 * np.abs(u) + np.abs(silu)) * np.asarray(S_row, np.float64)[:, None]


# -- full attention ------------------------------------------------------------
#
# The device computes o = (sum_j fp16(16 p_j) v_j) / (16 l) with p_j, l in
# FP32 against the running maximum.  Against the exact o = sum_j P_j v_j
# (P the exact softmax) the error is bounded, per output element, by
#   A * (2^-11 + eps_s + eps_acc) + 2^-29 * V + ulp16(o) / 2 + 2^-23 |o|
# with A = sum_j P_j |v_j| and V = sum_j |v_j| over the visible keys:
#   * 2^-11: fp16(16 p) of a normal value is within a relative 2^-11;
#   * 2^-29 V: a subnormal 16 p is within 2^-25 absolutely, and after the
#     division by 16 l (l >= 1) each key adds at most 2^-29 |v_j|;
#   * eps_s = 2^-22 (1.1 S1 + 1): a score is a 256-term FP32 sum (two
#     levels of at most 16 additions: 32 * 2^-24 relative to
#     S1 = max_j sum_d |q_d k_jd|); p_j = exp((s_j - s_max) / 16) moves by
#     the errors of both scores over 16, plus the base-2 exponential's error;
#   * eps_acc = (16 nkb + 320) 2^-24, nkb = key blocks of 64: the FP32
#     accumulation chains of o (4 products of 16 per block) and l, and the
#     per-block rescales, which o and l share, so they only perturb the
#     weights of the average (a device that takes keys in blocks of 32 has
#     the same chains per 64 keys and at most one more rescale, within the
#     16 counted per block);
#   * the FP16 rounding of o, and the FP32 product by 1 / (16 l).
# S1 is bounded by ||q_row,head||_1 * max|k|.

def attention_bound(o_exact, o_abs, v_abs, s1, nkb: int) -> np.ndarray:
    o_exact = np.asarray(o_exact, np.float64)
    eps = 2.0 ** -11 + 2.0 ** -22 * (1.1 * np.asarray(s1, np.float64) + 1.0) + (16 * nkb + 320) * 2.0 ** -24
    return (np.asarray(o_abs, np.float64) * eps + 2.0 ** -29 * np.asarray(v_abs, np.float64)
            + 0.5 * ulp16(o_exact) + 2.0 ** -23 * np.abs(o_exact))


def check_attention(o_dev16, o_exact, o_abs, v_abs, s1, nkb: int):
    """(ok, failures, max error / bound) of FP16 device outputs."""
    val = np.asarray(o_dev16).view(np.float16).astype(np.float64)
    bound = attention_bound(o_exact, o_abs, v_abs, s1, nkb)
    err = np.abs(val - np.asarray(o_exact, np.float64))
    bad = ~(err <= bound)
    return (not bool(np.any(bad)), int(np.sum(bad)),
            float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0)


# -- Gated DeltaNet recurrence ---------------------------------------------------
#
# The device keeps the state in FP32 and reproduces the gated delta rule
# token by token.  Each token adds rounding of a few FP32 ulps to every state
# entry (the decay product, one fused update, and the 128-term dot product
# S^T k behind d: 8 sequential terms and a 4-level tree), and the token map
# S -> exp(g) S (I - beta k k^T) does not expand errors for beta |k|^2 in
# [0, 2].  Taking the per-token roundings as independent, the state error
# after t tokens grows like sqrt(t); with a wide margin:
#   |o_t - o_ref| <= ulp16(o_ref) / 2
#                    + 2^-18 sqrt(t + 1) (A_t + ||q_t||_1 / sqrt(128) * s_rms)
# A_t = sum_i |S_ij q_i| / sqrt(128) (the oracle returns it) and s_rms the
# root mean square of the head's final state, a floor for entries near zero.

def gated_delta_bound(o_exact, o_abs, q_l1, s_rms, t) -> np.ndarray:
    eps = 2.0 ** -18 * np.sqrt(np.asarray(t, np.float64) + 1.0)
    o_exact = np.asarray(o_exact, np.float64)
    return (0.5 * ulp16(o_exact)
            + eps * (np.asarray(o_abs, np.float64) + np.asarray(q_l1, np.float64) / np.sqrt(128.0) * s_rms))


def check_gated_delta(o_dev16, o_exact, o_abs, q_l1, s_rms, t):
    val = np.asarray(o_dev16).view(np.float16).astype(np.float64)
    bound = gated_delta_bound(o_exact, o_abs, q_l1, s_rms, t)
    err = np.abs(val - np.asarray(o_exact, np.float64))
    bad = ~(err <= bound)
    return (not bool(np.any(bad)), int(np.sum(bad)),
            float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0)
