"""Seeded synthetic inputs for the LUT-6 linear layer.

Shared by the tests, the benchmark and the smoke check, and by both the GPU
path and the CPU oracle.  It holds none of the method's arithmetic: it draws
raw 6-bit indices, FP16 tables and FP16 activations and nothing else
(packing, lookup and the product live on each side separately).

Shapes follow page "Clef-Flash-ANE-LUT6", section "Model architecture"
(hidden 4,096, MLP 12,288, 24 Gated DeltaNet layers with 16 key and 32 value
heads of 128, 8 full-attention layers with 16 query and 4 key-value heads of
256, context up to 16,384 tokens processed 128 per call).  Distributions:
activations ~N(0, sigma) rounded to FP16; indices uniform on 0..63; each
16-channel group's 64 table entries ~N(0, 0.02) (the second argument is the
standard deviation), optionally with a fraction of entries drawn at 8x that
scale, rounded to FP16 and sorted ascending -- a stand-in for the k-means
tables of section "LUT-6 text weights", whose trained weights are not here.

Every stream comes from ``numpy.random.default_rng([2026, cfg, layer, proj,
tensor])`` (PCG64) with tensor 0 = x, 1 = a second activation, 2 = indices,
3 = tables, 4 = outlier mask, 5 = sampled rows, 6 = an FP16 weight to fit
tables to, 7 = int8 weight codes, 8 = their per-block scales.  Weights are keyed by
(cfg, layer, projection); activations are shared by every GEMM of a workload
that reads the same stream at the same width, keyed by (cfg, 0, K): the
hidden state x, a stand-in `a` for an attention / recurrence output, and a
stand-in for the MLP down-projection input (its own seeded stream, so every
GEMM is checked on inputs that come from the generator alone).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

T_X, T_A, T_IDX, T_TAB, T_OUTLIER, T_ROWS, T_W, T_Q, T_QS = 0, 1, 2, 3, 4, 5, 6, 7, 8
EPI_F32, EPI_F16, EPI_SILU_MUL_F16 = 0, 1, 2


def rng(cfg: int, layer: int, proj: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng([2026, cfg, layer, proj, tensor])


def activations(L: int, K: int, sigma: float, key: tuple[int, int, int], tensor: int = T_X) -> np.ndarray:
    """FP16 [L, K] ~ N(0, sigma): float32 normals, scaled, rounded to nearest even."""
    g = rng(*key, tensor)
    return (g.standard_normal((L, K), dtype=np.float32) * np.float32(sigma)).astype(np.float16)


def indices(N: int, K: int, key: tuple[int, int, int]) -> np.ndarray:
    """uint8 [N, K], uniform on 0..63 (the low 6 bits of uniform random bytes)."""
    g = rng(*key, T_IDX)
    return (np.frombuffer(g.bytes(N * K), np.uint8) & np.uint8(63)).reshape(N, K)


def tables(N: int, key: tuple[int, int, int], sigma: float = 0.02,
           outlier_p: float = 0.0, outlier_scale: float = 8.0) -> np.ndarray:
    """FP16 [N/16, 64], each row sorted ascending."""
    g = rng(*key, T_TAB)
    t = g.standard_normal((N // 16, 64), dtype=np.float64) * sigma
    if outlier_p > 0:
        m = rng(*key, T_OUTLIER).random((N // 16, 64)) < outlier_p
        t = np.where(m, t * outlier_scale, t)
    return np.sort(t.astype(np.float16), axis=1)


def weights(N: int, K: int, key: tuple[int, int, int], sigma: float = 0.02,
            outlier_p: float = 0.02, outlier_scale: float = 8.0) -> np.ndarray:
    """FP16 weight [N, K] for table fitting: N(0, sigma) with a fraction
    outlier_p of the entries scaled by outlier_scale (the spread the tables
    of the workloads model)."""
    g = rng(*key, T_W)
    w = g.standard_normal((N, K), dtype=np.float32) * np.float32(sigma)
    m = g.random((N, K), dtype=np.float32) < outlier_p
    return np.where(m, w * np.float32(outlier_scale), w).astype(np.float16)


def int8_weight(N: int, K: int, key: tuple[int, int, int], sigma: float = 0.02):
    """int8 codes [N, K] uniform on -127..127 and FP16 scales [N, K/32],
    each sigma * 2.5 / 127 times a log-normal factor (spread 0.25): the
    shapes of a weight kept as int8 per block of 32 along K."""
    q = rng(*key, T_Q).integers(-127, 128, size=(N, K), dtype=np.int16).astype(np.int8)
    f = np.exp(rng(*key, T_QS).standard_normal((N, K // 32)) * 0.25)
    return q, (f * (sigma * 2.5 / 127.0)).astype(np.float16)


def sample_rows(L: int, count: int, key: tuple[int, int, int]) -> np.ndarray:
    """Rows 0 and L-1 plus (count-2) distinct seeded rows, sorted."""
    if count >= L:
        return np.arange(L, dtype=np.int64)
    g = rng(*key, T_ROWS)
    inner = g.choice(np.arange(1, L - 1), size=count - 2, replace=False)
    return np.sort(np.concatenate([[0, L - 1], inner]).astype(np.int64))


def sha256(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


# ---------------------------------------------------------------------------
# The workloads.  Each GEMM is (L, K, N, epilogue, in_scale, x sigma, table
# outlier fraction); N of a fused gate/up launch counts both halves.
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Gemm:
    name: str
    L: int
    K: int
    N: int
    epilogue: int
    in_scale: float = 1.0
    x_sigma: float = 1.0
    outlier_p: float = 0.0
    x_tensor: int = T_X      # which activation stream feeds it

    @property
    def n_out(self) -> int:
        return self.N // 2 if self.epilogue == EPI_SILU_MUL_F16 else self.N

    @property
    def flops(self) -> int:
        return 2 * self.L * self.K * self.N

    @property
    def bytes(self) -> int:
        """Algorithmic HBM bytes: packed + tables + x + y, each moved once."""
        out_elt = 4 if self.epilogue == EPI_F32 else 2
        return (self.N * 3 * self.K // 4 + self.N // 16 * 128 + self.L * self.K * 2
                + self.L * self.n_out * out_elt)


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    description: str
    layers: tuple = field(default_factory=tuple)   # tuple of tuples of Gemm

    @property
    def flops(self) -> int:
        return sum(g.flops for layer in self.layers for g in layer)

    @property
    def bytes(self) -> int:
        return sum(g.bytes for layer in self.layers for g in layer)

    def gemms(self):
        for li, layer in enumerate(self.layers):
            for pi, g in enumerate(layer):
                yield li, pi, g


HIDDEN, MLP = 4096, 12288
DN_QKV = 16 * 128 * 2 + 32 * 128          # 8,192: Gated DeltaNet q, k (16 heads) and v (32 heads)
DN_Z = 32 * 128                           # 4,096
FA_Q, FA_KV = 16 * 256, 4 * 256           # 4,096 and 1,024


def _deltanet_layer(L: int) -> tuple:
    return (Gemm("qkv|z", L, HIDDEN, DN_QKV + DN_Z, EPI_F16),
            Gemm("out", L, HIDDEN, HIDDEN, EPI_F16, x_tensor=T_A),
            Gemm("gate|up", L, HIDDEN, 2 * MLP, EPI_SILU_MUL_F16),
            Gemm("down", L, MLP, HIDDEN, EPI_F16, in_scale=16.0, x_sigma=0.5, x_tensor=T_A))


def _attention_layer(L: int) -> tuple:
    return (Gemm("q|k|v", L, HIDDEN, FA_Q + 2 * FA_KV, EPI_F16),
            Gemm("o", L, HIDDEN, HIDDEN, EPI_F16, x_tensor=T_A),
            Gemm("gate|up", L, HIDDEN, 2 * MLP, EPI_SILU_MUL_F16),
            Gemm("down", L, MLP, HIDDEN, EPI_F16, in_scale=16.0, x_sigma=0.5, x_tensor=T_A))


def _sweep_layers(L: int) -> tuple:
    # full attention every fourth layer: layers 3, 7, ..., 31
    return tuple(_attention_layer(L) if i % 4 == 3 else _deltanet_layer(L) for i in range(32))


WORKLOADS = {
    "o_proj_l128": Workload(
        1, "o_proj_l128",
        "one LUT-6 linear, L=128, K=4096 -> N=4096, fp32 out",
        ((Gemm("o", 128, HIDDEN, HIDDEN, EPI_F32),),)),
    "mlp_gate_up_l512": Workload(
        2, "mlp_gate_up_l512",
        "MLP gate|up fused, L=512, K=4096 -> 2x12288, SiLU(gate)*up to fp16",
        ((Gemm("gate|up", 512, HIDDEN, 2 * MLP, EPI_SILU_MUL_F16, outlier_p=0.02),),)),
    "mlp_down_l1024": Workload(
        3, "mlp_down_l1024",
        "MLP down, L=1024, K=12288 -> 4096, x~N(0,0.5), in_scale 16, fp16 out",
        ((Gemm("down", 1024, MLP, HIDDEN, EPI_F16, in_scale=16.0, x_sigma=0.5),),)),
    "hybrid_block_l4096": Workload(
        4, "hybrid_block_l4096",
        "one hybrid block's projections at L=4096: qkv|z, q|k|v, out, fp16 out",
        ((Gemm("qkv|z", 4096, HIDDEN, DN_QKV + DN_Z, EPI_F16),
          Gemm("q|k|v", 4096, HIDDEN, FA_Q + 2 * FA_KV, EPI_F16),
          Gemm("out", 4096, HIDDEN, HIDDEN, EPI_F16, x_tensor=T_A)),)),
    "hybrid_block_l4096_six": Workload(
        4, "hybrid_block_l4096_six",
        "the same block's projections as six launches: qkv, z, out, q, k, v, fp16 out",
        ((Gemm("qkv", 4096, HIDDEN, DN_QKV, EPI_F16),
          Gemm("z", 4096, HIDDEN, DN_Z, EPI_F16),
          Gemm("out", 4096, HIDDEN, HIDDEN, EPI_F16, x_tensor=T_A),
          Gemm("q", 4096, HIDDEN, FA_Q, EPI_F16),
          Gemm("k", 4096, HIDDEN, FA_KV, EPI_F16),
          Gemm("v", 4096, HIDDEN, FA_KV, EPI_F16)),)),
    "prefill_sweep_l16384": Workload(
        5, "prefill_sweep_l16384",
        "all 32 layers' LUT-6 projections and MLPs at L=16384, fp16 out",
        _sweep_layers(16384)),
}


def gemm_activation(cfg: int, g: Gemm) -> np.ndarray:
    """The activation a GEMM of workload `cfg` reads (shared across layers)."""
    return activations(g.L, g.K, g.x_sigma, (cfg, 0, g.K), g.x_tensor)


def gemm_weight(cfg: int, layer: int, proj: int, g: Gemm):
    """(idx uint8 [N,K], tables fp16 [N/16,64]) of one GEMM."""
    key = (cfg, layer, proj)
    return indices(g.N, g.K, key), tables(g.N, key, outlier_p=g.outlier_p)


def gemm_inputs(cfg: int, layer: int, proj: int, g: Gemm):
    """(x fp16 [L,K], idx uint8 [N,K], tables fp16 [N/16,64]) for one GEMM."""
    idx, tab = gemm_weight(cfg, layer, proj, g)
    return gemm_activation(cfg, g), idx, tab
