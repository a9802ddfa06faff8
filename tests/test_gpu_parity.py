"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every input is seeded and synthetic (seeded_inputs.py).  The oracle gets its
own packing of the raw indices; the device gets the library's packing.  The
criteria are those of oracle/tolerance.py: bit-exact dequantization, the
float bound on every output, 1 FP16 ulp (with the near-zero floor) on FP16
outputs.  Full-size workloads are checked on every row when the oracle can
afford it and on seeded sampled rows otherwise.
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


def _say(*a):
    print("[case]", *a, flush=True)


def _dev(a: np.ndarray, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to("cuda")


def gpu_linear(x16, idx, tab16, epi, s, packed=None):
    packed = lq.pack(idx) if packed is None else packed
    y = lq.linear(_dev(x16), _dev(packed), _dev(tab16), epilogue=epi, in_scale=s)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    return y.view(np.uint16) if epi != F32 else y


def oracle_check(ora, x16, idx, tab16, epi, s, y_dev, rows=None, packer=None, gathered=False):
    """Report whether the device output (all rows, or `rows`) meets the criteria.

    The oracle computes from the raw indices packed by `packer` (an oracle;
    itself by default).  With `gathered`, y_dev holds only the rows `rows`."""
    K = x16.shape[1]
    N = idx.shape[0]
    packed = (packer or ora).pack(idx)
    S = tol.row_scale(x16, tab16, K, rows)
    yd = y_dev if rows is None or gathered else y_dev[np.asarray(rows)]
    if epi == SILU:
        h_exact, _ = ora.linear(x16, packed, tab16, epilogue=oracle.EPI_SILU_MUL_F16, in_scale=s, rows=rows)
        a_exact, _ = ora.linear(x16, packed, tab16, epilogue=oracle.EPI_F32, in_scale=s, rows=rows)
        Se = tol.silu_scale(a_exact[:, : N // 2], a_exact[:, N // 2:], S)
        rep = tol.check(yd, h_exact, S, fp16=True, S_elem=Se)
    else:
        y_exact, _ = ora.linear(x16, packed, tab16, epilogue=epi, in_scale=s, rows=rows)
        rep = tol.check(yd, y_exact, S, fp16=(epi == F16))
    return rep


def _problem(L, K, N, seed, *, sigma=1.0, outliers=0.02, subnormal=False):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((L, K)) * sigma).astype(np.float16)
    if subnormal:
        flat = x.reshape(-1)
        flat[::13] = (g.integers(1, 1024, size=flat[::13].size) * 2.0 ** -24 *
                      g.choice([-1, 1], size=flat[::13].size)).astype(np.float16)
    idx = g.integers(0, 64, size=(N, K), dtype=np.uint8)
    t = g.standard_normal((N // 16, 64)) * 0.02
    m = g.random((N // 16, 64)) < outliers
    tab = np.sort(np.where(m, t * 8, t).astype(np.float16), axis=1)
    return x, idx, tab


# ---------------------------------------------------------------------------
# dequantization: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(16, 64), (48, 192), (272, 576), (96, 12288), (4096, 4096)])
def test_dequant_bit_exact(ora, N, K):
    _say("dequant", N, K)
    _, idx, tab = _problem(1, K, N, 7 + N + K)
    w = lq.dequant(_dev(lq.pack(idx)), _dev(tab), K)
    torch.cuda.synchronize()
    got = w.cpu().numpy().view(np.uint16)
    want = ora.dequant(ora.pack(idx), tab, K)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------
# identity readout: x = I_K gives y = W^T bit for bit (one product per output)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("s", [1.0, 16.0])
@pytest.mark.parametrize("K", [64, 256, 1024])
def test_identity_readout(ora, K, s):
    _say("identity", K, s)
    N = 96
    _, idx, tab = _problem(1, K, N, 3)
    eye = np.eye(K, dtype=np.float16)
    y = gpu_linear(eye, idx, tab, F16, s)
    W = ora.dequant(ora.pack(idx), tab, K)
    assert np.array_equal(y, W.T)


# ---------------------------------------------------------------------------
# small and ragged shapes, every epilogue, both regimes
# ---------------------------------------------------------------------------

SHAPES = [(1, 64, 32), (3, 128, 32), (17, 192, 64), (64, 64, 96), (100, 256, 288),
          (128, 576, 64), (129, 128, 128), (193, 320, 160), (256, 128, 544),
          (300, 192, 288), (513, 256, 320), (777, 128, 96), (300, 1024, 96),
          (513, 2048, 160), (260, 4096, 544), (192, 12288, 96), (160, 3072, 1056),
          (128, 1024, 2080), (1024, 64, 32), (1029, 256, 160), (1535, 576, 544),
          (1280, 12288, 64)]


@pytest.mark.parametrize("L,K,N", SHAPES)
@pytest.mark.parametrize("epi,s", [(F32, 1.0), (F16, 1.0), (F16, 16.0), (SILU, 1.0), (SILU, 4.0)])
def test_linear_small(ora, L, K, N, epi, s):
    _say("small", L, K, N, epi, s)
    assert lq.linear_path(L, K, N, epi) in (lq.PATH_STREAM, lq.PATH_FUSED)
    x, idx, tab = _problem(L, K, N, L * 7 + K + N, sigma=0.5 if s > 1 else 1.0,
                           subnormal=(L % 2 == 1))
    y = gpu_linear(x, idx, tab, epi, s)
    rep = oracle_check(ora, x, idx, tab, epi, s, y)
    assert rep.ok, str(rep)


# few tokens over a whole 4096-wide K slice per wave group: the streaming
# kernel's variant that loads every chunk's packed words up front (enough
# tiles: no K split; 64 tokens and 4,096 channels at K = 8,192: two slices);
# ragged L, every epilogue and scale
SHAPES_STREAM16 = [(128, 4096, 4096), (40, 4096, 6144), (64, 8192, 4096)]


@pytest.mark.parametrize("L,K,N", SHAPES_STREAM16)
@pytest.mark.parametrize("epi,s", [(F32, 1.0), (F16, 1.0), (F16, 16.0), (SILU, 1.0), (SILU, 4.0)])
def test_linear_stream_whole_slices(ora, L, K, N, epi, s):
    _say("stream16", L, K, N, epi, s)
    assert lq.linear_path(L, K, N, epi) == lq.PATH_STREAM
    x, idx, tab = _problem(L, K, N, L * 11 + K + N, sigma=0.5 if s > 1 else 1.0,
                           subnormal=(L % 2 == 1))
    y = gpu_linear(x, idx, tab, epi, s)
    rep = oracle_check(ora, x, idx, tab, epi, s, y)
    assert rep.ok, str(rep)


# many tokens: the weight is expanded once and the GEMM reads FP16 tiles;
# ragged L and N, split K (few tiles), every epilogue and scale
SHAPES_MANY = [(1536, 64, 32), (1541, 256, 160), (1600, 576, 544), (2047, 128, 96),
               (1536, 1024, 288), (3072, 8192, 64)]


@pytest.mark.parametrize("L,K,N", SHAPES_MANY)
@pytest.mark.parametrize("epi,s", [(F32, 1.0), (F16, 1.0), (F16, 16.0), (SILU, 1.0), (SILU, 4.0)])
def test_linear_many_tokens(ora, L, K, N, epi, s):
    _say("many", L, K, N, epi, s)
    assert lq.linear_path(L, K, N, epi) == lq.PATH_EXPANDED
    x, idx, tab = _problem(L, K, N, L * 5 + K + N, sigma=0.5 if s > 1 else 1.0,
                           subnormal=(L % 2 == 1))
    y = gpu_linear(x, idx, tab, epi, s)
    rep = oracle_check(ora, x, idx, tab, epi, s, y)
    assert rep.ok, str(rep)


# Cold activations, warm weight: every call's activations are evicted from
# the caches (a 512 MB copy) and the packed weight is read back just before
# the call.  Copies of the activations into LDS are then slow and loads of the
# weight into registers fast, so a wait that assumed loads complete in issue
# order (all but the youngest outstanding) lets a barrier pass before the
# copies land; this checks that no path relies on that.
SHAPES_COLD = [(128, 4096, 4096, F16), (40, 1024, 2080, F32), (513, 2048, 160, F16),
               (1536, 1024, 288, F16), (3072, 8192, 64, F32)]


@pytest.mark.parametrize("L,K,N,epi", SHAPES_COLD)
def test_cold_activation_calls(ora, L, K, N, epi):
    _say("cold", L, K, N, epi)
    big = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    big2 = torch.empty_like(big)
    _, idx, tab = _problem(1, K, N, L + 11 * K + N)
    packed = lq.pack(idx)
    pd, td = _dev(packed), _dev(tab)
    for trial in range(3):
        x = _problem(L, K, 16, 1000 * trial + L + K)[0]
        xd = _dev(x)
        big2.copy_(big)
        pd.sum()
        torch.cuda.synchronize()
        y = lq.linear(xd, pd, td, epilogue=epi)
        torch.cuda.synchronize()
        y = y.cpu().numpy()
        rep = oracle_check(ora, x, idx, tab, epi, 1.0, y.view(np.uint16) if epi != F32 else y)
        assert rep.ok, f"trial {trial}: {rep}"


def test_workspaces_grow_per_stream_and_after_release(ora):
    # Each call below needs a larger workspace than the stream's previous one
    # (expanded weight at L >= 1,536, split-K partials at L = 40).  The calls
    # alternate between two streams and are enqueued with no host wait in
    # between: a stream's workspace grows in stream order (the smaller buffer
    # freed behind the work already on it).  After lut6_release they are made
    # again.  Every result meets the criteria on sampled rows.
    _say("workspaces")
    shapes = [(1536, 256, 256, F16), (40, 1024, 2080, F32), (1536, 512, 512, F16),
              (40, 2048, 4160, F32), (1536, 1024, 1024, F16)]
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()

    def run_all():
        done = []
        for i, (L, K, N, epi) in enumerate(shapes):
            x, idx, tab = _problem(L, K, N, 900 + i)
            st = side if i % 2 else main
            with torch.cuda.stream(st):
                y = lq.linear(_dev(x), _dev(lq.pack(idx)), _dev(tab), epilogue=epi, stream=st)
            done.append((x, idx, tab, epi, y))
        torch.cuda.synchronize()
        for x, idx, tab, epi, y in done:
            L = x.shape[0]
            yh = y.cpu().numpy()
            yh = yh.view(np.uint16) if epi != F32 else yh
            rows = np.unique(np.concatenate([np.arange(0, L, max(1, L // 24)), [L - 1]]))
            rep = oracle_check(ora, x, idx, tab, epi, 1.0, yh, rows=rows)
            assert rep.ok, str(rep)

    run_all()
    lq.release()
    run_all()


def test_non_aligned_n_tiles(ora):
    # N = 16 * odd so the last channel tile is partial in both regimes
    for L in (64, 384, 1088):
        _say("ragged-n", L)
        x, idx, tab = _problem(L, 128, 16 * 37, 91 + L)
        y = gpu_linear(x, idx, tab, F16, 1.0)
        rep = oracle_check(ora, x, idx, tab, F16, 1.0, y)
        assert rep.ok, str(rep)


# ---------------------------------------------------------------------------
# the five workloads at full size, in the launch configuration the benchmark uses
# ---------------------------------------------------------------------------

_ACTS = {}     # (cfg, L, K, stream) -> (host, device) activations of the current workload


def _workload_gemm_check(ora, cfg, layer, proj, g, n_rows):
    """One GEMM of a workload at full size on the GPU, in the launch the
    benchmark makes; all rows (n_rows None) or seeded sampled rows (rows 0
    and L - 1 among them) against the oracle, gathered on the device."""
    key = (cfg, g.L, g.K, g.x_tensor)
    if key not in _ACTS:
        if any(k[0] != cfg for k in _ACTS):
            _ACTS.clear()
        xh = si.gemm_activation(cfg, g)
        _ACTS[key] = (xh, _dev(xh))
    x = _ACTS[key][0]
    idx, tab = si.gemm_weight(cfg, layer, proj, g)
    rows = None if n_rows is None else si.sample_rows(g.L, n_rows, (cfg, layer, proj))
    y = lq.linear(_ACTS[key][1], _dev(lq.pack(idx)), _dev(tab), epilogue=g.epilogue, in_scale=g.in_scale)
    if rows is not None:
        y = y[torch.from_numpy(rows).to(y.device)]
    y = y.cpu().numpy()
    y = y.view(np.uint16) if g.epilogue != F32 else y
    rep = oracle_check(ora, x, idx, tab, g.epilogue, g.in_scale, y, rows, gathered=True)
    assert rep.ok, f"{g.name}: {rep}"
    return rep


@pytest.mark.parametrize("name,n_rows", [("o_proj_l128", None), ("mlp_gate_up_l512", None),
                                         ("mlp_down_l1024", None), ("hybrid_block_l4096", 256),
                                         ("hybrid_block_l4096_six", 256)])
def test_workload(ora, name, n_rows):
    # L = 128, 512 and 1,024 on every row; each projection of the L = 4,096
    # block on 256 sampled rows
    w = si.WORKLOADS[name]
    for li, pi, g in w.gemms():
        _say(name, g.name, g.L, g.K, g.N)
        rep = _workload_gemm_check(ora, w.cfg, li, pi, g, n_rows)
        _say(name, g.name, rep)


@pytest.mark.parametrize("layer", range(32))
def test_prefill_sweep_layer(ora, layer):
    # every layer of the 32-layer sweep (24 Gated DeltaNet, 8 full
    # attention), every projection, at L = 16,384 on 64 sampled rows
    w = si.WORKLOADS["prefill_sweep_l16384"]
    for pi, g in enumerate(w.layers[layer]):
        _say("sweep", layer, g.name)
        _workload_gemm_check(ora, w.cfg, layer, pi, g, 64)


# ---------------------------------------------------------------------------
# properties
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("L,K,N,epi", [(128, 4096, 4096, F32), (1024, 512, 1024, F16),
                                       (96, 256, 128, SILU), (1500, 768, 160, F32)])
def test_deterministic(L, K, N, epi):
    _say("determinism", L, K, N, epi)
    x, idx, tab = _problem(L, K, N, 5)
    xs, ps, ts = _dev(x), _dev(lq.pack(idx)), _dev(tab)
    outs = []
    for _ in range(3):
        outs.append(lq.linear(xs, ps, ts, epilogue=epi).cpu().numpy().tobytes())
    assert outs[0] == outs[1] == outs[2]


@pytest.mark.parametrize("epi", [F32, F16, SILU])
@pytest.mark.parametrize("L", [64, 640, 1024])
def test_scale_invariance(L, epi):
    # power-of-two scaling commutes with rounding when nothing overflows
    _say("scale-invariance", L, epi)
    x, idx, tab = _problem(L, 256, 256, 8)
    y1 = gpu_linear(x, idx, tab, epi, 1.0)
    for s in (2.0, 16.0):
        assert gpu_linear(x, idx, tab, epi, s).tobytes() == y1.tobytes()


@pytest.mark.parametrize("L", [32, 512, 1024])
def test_overflow_gives_inf(ora, L):
    _say("overflow", L)
    x, idx, _ = _problem(L, 128, 64, 2)
    x[:, 3] = np.float16(4096.0)         # 4096 * 16 = 65536 overflows FP16
    tab = np.full((4, 64), 0.5, np.float16)
    for epi in (F32, F16):
        y = gpu_linear(x, idx, tab, epi, 16.0)
        yv = y if epi == F32 else y.view(np.float16)
        _, ref = ora.linear(x, ora.pack(idx), tab, epilogue=epi, in_scale=16.0)
        rv = ref if epi == F32 else ref.view(np.float16)
        assert np.all(np.isposinf(yv)) and np.all(np.isposinf(rv))


def test_concatenation_invariance():
    # [W1; W2] gives [y1 | y2] bit for bit: tables belong to 16-row groups
    L, K = 2048, 256
    _say("concat", L, K)
    x, idx1, tab1 = _problem(L, K, 4096, 10)
    _, idx2, tab2 = _problem(1, K, 2048, 11)
    y1 = gpu_linear(x, idx1, tab1, F16, 1.0)
    y2 = gpu_linear(x, idx2, tab2, F16, 1.0)
    y12 = gpu_linear(x, np.concatenate([idx1, idx2]), np.concatenate([tab1, tab2]), F16, 1.0)
    assert np.array_equal(y12, np.concatenate([y1, y2], axis=1))


# ---------------------------------------------------------------------------
# the checks see the layout: the device result must FAIL against oracles with
# a planted mistake (big-endian packing, wrong table group, gate/up swapped,
# scale not undone)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mutant,epi,s", [(1, F16, 1.0), (2, F16, 1.0), (3, F16, 1.0),
                                          (4, F16, 16.0), (5, SILU, 1.0)])
def test_mutation_controls(tmp_path, ora, mutant, epi, s):
    _say("mutation", mutant)
    x, idx, tab = _problem(64, 256, 128, 12, sigma=0.5)
    y = gpu_linear(x, idx, tab, epi, s)
    assert oracle_check(ora, x, idx, tab, epi, s, y).ok
    bad = oracle.Oracle(oracle.build(tmp_path / f"m{mutant}.so", mutant=mutant))
    # the mutant reads bytes packed by the correct oracle
    assert not oracle_check(bad, x, idx, tab, epi, s, y, packer=ora).ok


# ---------------------------------------------------------------------------
# table fitting: lut6_quantize against the oracle, bit for bit (tables and
# packed indices)
# ---------------------------------------------------------------------------

def _q_weights(N, K, seed, kind):
    g = np.random.default_rng(seed)
    if kind == "normal":
        w = g.standard_normal((N, K)) * 0.02
        w[g.random((N, K)) < 0.02] *= 8.0
        return w.astype(np.float16)
    if kind == "edge":
        # groups of their own kind: constant, two values, zeros of both signs
        # with subnormals, few distinct values, huge range
        w = (g.standard_normal((N, K)) * 0.02).astype(np.float16)
        groups = N // 16
        for gi in range(groups):
            blk = w[16 * gi:16 * gi + 16]
            mode = gi % 5
            if mode == 0:
                blk[:] = np.float16(-1.5)
            elif mode == 1:
                blk[:] = np.where(g.random(blk.shape) < 0.5, np.float16(0.25), np.float16(-0.0078))
            elif mode == 2:
                bits = g.integers(0, 1024, size=blk.shape).astype(np.uint16)
                bits[g.random(blk.shape) < 0.3] = 0
                bits |= (g.random(blk.shape) < 0.5).astype(np.uint16) << 15
                blk[:] = bits.view(np.float16)
            elif mode == 3:
                blk[:] = g.choice(np.array([-2.0, -0.5, 0.0, 0.125, 3.0], np.float16), size=blk.shape)
            else:
                blk[:] = (g.standard_normal(blk.shape) * 100.0).astype(np.float16)
        return w
    raise ValueError(kind)


def _gpu_quantize(w16):
    p, t = lq.quantize(_dev(w16))
    torch.cuda.synchronize()
    return p.cpu().numpy(), t.cpu().numpy().view(np.uint16)


# The "edge" weights include groups whose new centres come out of the sort's
# order in some rounds (equal zeros of opposite sign: the oracle re-sorts in 2
# rounds of the 80 x 128 weight and 4 of the 160 x 64 one), so both the
# kernel's in-order shortcut and its full rank sort are compared.
@pytest.mark.parametrize("N,K,kind", [(16, 64, "normal"), (32, 256, "normal"), (48, 1024, "normal"),
                                      (80, 128, "edge"), (160, 64, "edge"), (64, 4096, "normal"),
                                      (16, 12288, "normal")])
def test_quantize_matches_oracle(ora, N, K, kind):
    _say("quantize", N, K, kind)
    w = _q_weights(N, K, N + K, kind)
    p_gpu, t_gpu = _gpu_quantize(w)
    p_ora, t_ora = ora.quantize(w)
    assert np.array_equal(t_gpu, t_ora), "tables"
    assert np.array_equal(p_gpu, p_ora), "packed indices"


def test_quantize_full_layer_sampled_groups(ora):
    # a 4,096 x 4,096 weight (256 groups, 256 workgroups): four groups
    # against the oracle, every group twice on the GPU (same bytes)
    _say("quantize full", 4096, 4096)
    w = _q_weights(4096, 4096, 77, "normal")
    wd = _dev(w)
    p1, t1 = lq.quantize(wd)
    p2, t2 = lq.quantize(wd)
    torch.cuda.synchronize()
    p1, t1 = p1.cpu().numpy(), t1.cpu().numpy().view(np.uint16)
    assert np.array_equal(p1, p2.cpu().numpy()) and np.array_equal(t1, t2.cpu().numpy().view(np.uint16))
    for g in (0, 1, 137, 255):
        p_ora, t_ora = ora.quantize(w, groups=(g, g + 1))
        assert np.array_equal(t1[g], t_ora[g]), f"table of group {g}"
        assert np.array_equal(p1[16 * g:16 * g + 16], p_ora[16 * g:16 * g + 16]), f"indices of group {g}"
    # the fitted tables reproduce the weight to about 6-bit precision
    back = ora.dequant(p1[:64], t1[:4], 4096).view(np.float16).astype(np.float64)
    ref = w[:64].astype(np.float64)
    assert np.sqrt(np.mean((back - ref) ** 2)) < 0.05 * np.sqrt(np.mean(ref ** 2))


# ---------------------------------------------------------------------------
# int8 weight-only variant: int8 codes, one FP16 scale per row and 32 k
# ---------------------------------------------------------------------------

def _gpu_int8(x16, q, s16, epi, s):
    y = lq.int8_linear(_dev(x16), _dev(q), _dev(s16), epilogue=epi, in_scale=s)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    return y.view(np.uint16) if epi != F32 else y


def _int8_check(ora, x16, q, s16, epi, s, y_dev, rows=None):
    w = ora.int8_dequant(q, s16).view(np.float16)
    N = q.shape[0]
    S = tol.row_scale(x16, w, x16.shape[1], rows)
    yd = y_dev if rows is None else y_dev[np.asarray(rows)]
    if epi == SILU:
        h_exact, _ = ora.int8_linear(x16, q, s16, epilogue=oracle.EPI_SILU_MUL_F16, in_scale=s, rows=rows)
        a_exact, _ = ora.int8_linear(x16, q, s16, epilogue=oracle.EPI_F32, in_scale=s, rows=rows)
        return tol.check(yd, h_exact, S, fp16=True,
                         S_elem=tol.silu_scale(a_exact[:, : N // 2], a_exact[:, N // 2:], S))
    y_exact, _ = ora.int8_linear(x16, q, s16, epilogue=epi, in_scale=s, rows=rows)
    return tol.check(yd, y_exact, S, fp16=(epi == F16))


@pytest.mark.parametrize("s", [1.0, 16.0])
@pytest.mark.parametrize("K,N", [(64, 32), (256, 96), (1024, 272)])
def test_int8_identity_readout(ora, K, N, s):
    # x = I_K: each output is one product, so y = W^T bit for bit, W the
    # oracle's dequantized int8 weight (including the FP16 rounding of q * s)
    _say("int8 identity", K, N, s)
    q, sc = si.int8_weight(N, K, (11, K, N))
    sc = sc.copy()
    sc[0, 0] = np.float16(6e-8)                      # subnormal weights
    y = _gpu_int8(np.eye(K, dtype=np.float16), q, sc, F16, s)
    assert np.array_equal(y, ora.int8_dequant(q, sc).T)


# K = 4,160 is 65 chunks of 64: for L <= 192 three waves take 16 chunks and one
# takes 17 (pairs, then an odd last chunk); K = 64, 192 and 256 give one chunk
# per busy wave, K = 512 two.
INT8_SHAPES = [(1, 64, 32), (17, 192, 64), (100, 256, 288), (130, 64, 48), (192, 512, 4112),
               (150, 4160, 96), (257, 576, 544), (513, 1024, 160), (1029, 4096, 96), (2048, 128, 4128),
               (64, 12288, 64)]


@pytest.mark.parametrize("L,K,N", INT8_SHAPES)
@pytest.mark.parametrize("epi,s", [(F32, 1.0), (F16, 1.0), (F16, 16.0), (SILU, 1.0), (SILU, 4.0)])
def test_int8_linear(ora, L, K, N, epi, s):
    _say("int8", L, K, N, epi, s)
    q, sc = si.int8_weight(N, K, (11, L, K))
    x = si.activations(L, K, 1.0, (11, L, N))
    if epi == SILU and N % 32:
        with pytest.raises(lq.Lut6Error):                  # gate and up halves need N % 32 == 0
            _gpu_int8(x, q, sc, epi, s)
        return
    rep = _int8_check(ora, x, q, sc, epi, s, _gpu_int8(x, q, sc, epi, s))
    assert rep.ok, rep


@pytest.mark.parametrize("L,K,N,epi", [(4096, 4096, 4096, F16), (4096, 4096, 24576, SILU),
                                       (128, 12288, 4096, F16)])
def test_int8_full_layer_sampled_rows(ora, L, K, N, epi):
    _say("int8 full", L, K, N, epi)
    q, sc = si.int8_weight(N, K, (12, L, N))
    x = si.activations(L, K, 1.0, (12, L, K))
    rows = si.sample_rows(L, 12, (12, L, N))
    rep = _int8_check(ora, x, q, sc, epi, 1.0, _gpu_int8(x, q, sc, epi, 1.0), rows=rows)
    assert rep.ok, rep


# int8 code selection: codes and scales bit-exact against the oracle

@pytest.mark.parametrize("N,K", [(1, 32), (16, 96), (96, 4096), (4096, 4096), (24576, 4096)])
def test_int8_quantize_matches_oracle(ora, N, K):
    _say("int8 quantize", N, K)
    w = si.weights(N, K, (13, N, K))
    q, sc = lq.int8_quantize(_dev(w))
    torch.cuda.synchronize()
    qo, so = ora.int8_quantize(w)
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), so)


def test_int8_quantize_every_block_maximum(ora):
    # one block per finite positive FP16 magnitude a (a, -a and 30 seeded
    # fractions of it) and two zero blocks: every rounding of the scale,
    # subnormal scales and the clamp included, decided on the device as in
    # the oracle
    _say("int8 quantize every maximum")
    a = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    g = np.random.default_rng(14)
    f = g.uniform(-1.0, 1.0, size=(a.size, 30))
    w = np.concatenate([a[:, None], -a[:, None], a[:, None] * f], axis=1).astype(np.float16)
    w = np.concatenate([w, np.zeros((2, 32), np.float16)], axis=0)
    q, sc = lq.int8_quantize(_dev(w))
    torch.cuda.synchronize()
    qo, so = ora.int8_quantize(w)
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), so)
    assert np.array_equal(q.cpu().numpy(), qo)


def test_int8_quantize_feeds_int8_linear(ora):
    # the device's codes and scales drive int8_linear to the oracle's result
    _say("int8 quantize then linear")
    L, K, N = 64, 1024, 256
    w = si.weights(N, K, (15, N, K))
    q, sc = lq.int8_quantize(_dev(w))
    x = si.activations(L, K, 1.0, (15, L, N))
    y = lq.int8_linear(_dev(x), q, sc, epilogue=F16)
    torch.cuda.synchronize()
    qo, so = ora.int8_quantize(w)
    rep = _int8_check(ora, x, qo, so.view(np.float16), F16, 1.0, y.cpu().numpy().view(np.uint16))
    assert rep.ok, rep


# ---------------------------------------------------------------------------
# full attention: FP16 probabilities x 16, against the exact softmax
# ---------------------------------------------------------------------------

def _att_s1(q16, k16, rows, Hq, Hkv, D):
    """Per (row, head) bound on sum_d |q_d k_d|, broadcast over the head's D outputs."""
    q = np.abs(q16[np.asarray(rows)][:, : Hq * D].astype(np.float64)).reshape(len(rows), Hq, D)
    kmax = float(np.max(np.abs(k16[:, : Hkv * D].astype(np.float64))))
    return np.repeat(q.sum(axis=2) * kmax, D, axis=1)


def _att_case(ora, q, k, v, Hq, Hkv, rows=None, D=256):
    """Run the device on torch views q, k, v and check `rows` against the oracle."""
    L, Lk = q.shape[0], k.shape[0]
    o = lq.attention(q, k, v, n_heads=Hq, n_kv_heads=Hkv)
    torch.cuda.synchronize()
    rows = np.arange(L) if rows is None else np.asarray(rows)
    qn, kn, vn = (t.cpu().numpy() for t in (q, k, v))
    oe, _, oa, va = ora.attention(qn, kn, vn, n_heads=Hq, n_kv_heads=Hkv, head_dim=D, rows=rows,
                                  with_bounds=True)
    od = o.cpu().numpy()[rows].view(np.uint16)
    nkb = (Lk - L + int(rows.max())) // 64 + 1
    return tol.check_attention(od, oe, oa, va, _att_s1(qn, kn, rows, Hq, Hkv, D), nkb), o


def _att_inputs(L, Lk, Hq, Hkv, seed, scale=1.0):
    g = np.random.default_rng(seed)
    D = 256
    q = (g.standard_normal((L, Hq * D)) * scale).astype(np.float16)
    k = (g.standard_normal((Lk, Hkv * D)) * scale).astype(np.float16)
    v = g.standard_normal((Lk, Hkv * D)).astype(np.float16)
    return _dev(q), _dev(k), _dev(v)


ATT_SHAPES = [(1, 1, 16, 4), (5, 5, 2, 1), (37, 37, 4, 4), (128, 128, 16, 4), (130, 200, 4, 2),
              (300, 1000, 16, 4), (64, 4096, 16, 4), (1024, 1024, 16, 4), (129, 129, 1, 1),
              (1, 4096, 16, 4), (1, 65, 2, 1)]


@pytest.mark.parametrize("L,Lk,Hq,Hkv", ATT_SHAPES)
def test_attention(ora, L, Lk, Hq, Hkv):
    _say("attention", L, Lk, Hq, Hkv)
    q, k, v = _att_inputs(L, Lk, Hq, Hkv, L * 7 + Lk)
    (ok, bad, ratio), _ = _att_case(ora, q, k, v, Hq, Hkv)
    assert ok, (bad, ratio)


@pytest.mark.parametrize("scale", [0.25, 2.0])
def test_attention_sharp_and_flat_scores(ora, scale):
    # scale 2: scores of ~64, so one or two keys carry each row; 0.25: near-uniform
    _say("attention scale", scale)
    q, k, v = _att_inputs(200, 700, 8, 2, 11, scale=scale)
    (ok, bad, ratio), _ = _att_case(ora, q, k, v, 8, 2)
    assert ok, (bad, ratio)


def test_attention_reads_fused_qkv_rows(ora):
    # q, k, v as column ranges of one [L, 6144] projection output
    _say("attention fused qkv")
    L = 300
    g = np.random.default_rng(5)
    y = _dev(g.standard_normal((L, 6144)).astype(np.float16))
    q, k, v = y[:, :4096], y[:, 4096:5120], y[:, 5120:]
    (ok, bad, ratio), o = _att_case(ora, q, k, v, 16, 4)
    assert ok, (bad, ratio)
    # the same values in separate contiguous tensors give the same bits
    o2 = lq.attention(q.contiguous(), k.contiguous(), v.contiguous(), n_heads=16, n_kv_heads=4)
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))


def test_attention_tiny_probabilities_keep_their_mass(ora):
    # key 0 dominates every row: the other 4,095 keys have p = 1.5 * 2^-24
    # each (16 p = 24 * 2^-24, exact in FP16) and carry the value 1, key 0
    # the value 0, so the output is their summed mass.  Unscaled, each p is
    # an FP16 tie between 2^-24 and 2^-23 and loses a third of itself, far
    # beyond the bound's 2^-29 V term; scaled by 16 it is kept.
    _say("attention tiny probabilities")
    Lk, D = 4096, 256
    q = np.ones((1, D), np.float16)
    k = np.zeros((Lk, D), np.float16)
    k[0, :255] = 1.0
    k[0, 255] = np.float16(16 * (24 * np.log(2) - np.log(1.5)) - 255)   # score gap 259.68
    v = np.ones((Lk, D), np.float16)
    v[0] = 0
    (ok, bad, ratio), o = _att_case(ora, _dev(q), _dev(k), _dev(v), 1, 1)
    assert ok, (bad, ratio)


@pytest.mark.parametrize("L,Lk", [(16384, 16384), (128, 16384), (6200, 6200), (6208, 7000)])
def test_attention_full_size_sampled_rows(ora, L, Lk):
    # the attention layers at the longest context: the whole prefill, and
    # the last 128-token chunk over the full cache; q|k|v in one buffer.
    # 16,384 and the two shapes of about 6,200 queries (784 workgroups, a
    # ragged last query block, one over a longer cache) take 32-key blocks
    # with two workgroups per CU; 128 queries split the keys
    _say("attention full", L, Lk)
    g = np.random.default_rng(L)
    kv = _dev(g.standard_normal((Lk, 2048)).astype(np.float16))
    q = _dev(g.standard_normal((L, 4096)).astype(np.float16))
    rows = si.sample_rows(L, 8, (14, L, Lk))
    (ok, bad, ratio), _ = _att_case(ora, q, kv[:, :1024], kv[:, 1024:], 16, 4, rows=rows)
    assert ok, (bad, ratio)


def test_attention_deterministic():
    q, k, v = _att_inputs(500, 900, 16, 4, 3)
    a = lq.attention(q, k, v, n_heads=16, n_kv_heads=4)
    b = lq.attention(q, k, v, n_heads=16, n_kv_heads=4)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---------------------------------------------------------------------------
# Gated DeltaNet recurrence: FP32 state, against the FP64 sequential rule
# ---------------------------------------------------------------------------

def _gdn_problem(L, Hk, Hv, seed, with_state=True):
    """q|k|v in one [L, 2*Hk*128 + Hv*128] buffer (the projection's layout),
    g in (-0.5, 0], beta in [0, 1), an optional random initial state."""
    g = np.random.default_rng(seed)
    d = 128
    qkv = np.concatenate([g.standard_normal((L, 2 * Hk * d)) / np.sqrt(d),
                          g.standard_normal((L, Hv * d))], axis=1).astype(np.float16)
    gl = (-g.random((L, Hv)) * 0.5).astype(np.float32)
    be = g.random((L, Hv)).astype(np.float32)
    s0 = (g.standard_normal((Hv, d, d)) * 0.1).astype(np.float32) if with_state else np.zeros((Hv, d, d), np.float32)
    return qkv, gl, be, s0


def _gdn_run(qkv, gl, be, s0, Hk, Hv):
    d = 128
    y = _dev(qkv)
    st = _dev(s0)
    o = lq.gated_delta(y[:, : Hk * d], y[:, Hk * d: 2 * Hk * d], y[:, 2 * Hk * d:], _dev(gl), _dev(be), st,
                       n_k_heads=Hk, n_v_heads=Hv)
    torch.cuda.synchronize()
    return o.cpu().numpy().view(np.uint16), st.cpu().numpy()


def _gdn_check(ora, qkv, gl, be, s0, Hk, Hv, o_dev, s_dev):
    d = 128
    q, k, v = qkv[:, : Hk * d], qkv[:, Hk * d: 2 * Hk * d], qkv[:, 2 * Hk * d:]
    oe, _, oa, so = ora.gated_delta(q, k, v, gl, be, n_k_heads=Hk, n_v_heads=Hv, state=s0)
    L = qkv.shape[0]
    s_rms = np.repeat(np.sqrt(np.mean(so.reshape(Hv, -1) ** 2, axis=1)), d)[None, :]
    ql1 = np.abs(q.astype(np.float64)).reshape(L, Hk, d).sum(axis=2)
    ql1 = np.repeat(np.repeat(ql1, Hv // Hk, axis=1), d, axis=1)
    t = np.arange(L)[:, None]
    rep = tol.check_gated_delta(o_dev, oe, oa, ql1, s_rms, t)
    # the final state, entry by entry, within the same allowance at t = L - 1
    s_err = np.abs(s_dev.astype(np.float64) - so)
    s_bound = 2.0 ** -18 * np.sqrt(L) * (np.abs(so) + s_rms.reshape(Hv, d)[:, :1, None])
    return rep, bool(np.all(s_err <= s_bound))


# below 64 tokens the token-sequential kernel runs, from 64 the chunked one
# (64-position chunks; ragged last chunks at 65, 129, 200 and 1,000)
GDN_SHAPES = [(1, 1, 1), (5, 2, 4), (63, 1, 2), (64, 2, 2), (65, 16, 32), (128, 2, 4), (129, 1, 1),
              (200, 16, 32), (1000, 4, 8)]


@pytest.mark.parametrize("L,Hk,Hv", GDN_SHAPES)
def test_gated_delta(ora, L, Hk, Hv):
    _say("gated delta", L, Hk, Hv)
    qkv, gl, be, s0 = _gdn_problem(L, Hk, Hv, L + 31 * Hv)
    o, s = _gdn_run(qkv, gl, be, s0, Hk, Hv)
    (ok, bad, ratio), s_ok = _gdn_check(ora, qkv, gl, be, s0, Hk, Hv, o, s)
    print(f"[case] gated delta L={L}: failures={bad} max err/bound={ratio:.3f} state ok={s_ok}", flush=True)
    assert ok and s_ok, (bad, ratio, s_ok)


def test_gated_delta_zero_state_and_unit_keys(ora):
    # beta = 1 and k_t = e_i: row i of the state becomes v_t, which q = e_i
    # reads back: o_t = fp16(v_t / sqrt(128)) for every token
    _say("gated delta unit keys")
    L, Hk, Hv, d = 300, 2, 4, 128
    qkv, gl, be, s0 = _gdn_problem(L, Hk, Hv, 5, with_state=False)
    kq = np.zeros((L, Hk * d), np.float16)
    for t in range(L):
        for kh in range(Hk):
            kq[t, kh * d + (7 * t + kh) % d] = 1.0
    qkv[:, : Hk * d] = kq
    qkv[:, Hk * d: 2 * Hk * d] = kq
    o, s = _gdn_run(qkv, gl, np.ones_like(be), s0, Hk, Hv)
    want = (qkv[:, 2 * Hk * d:].astype(np.float64) / np.sqrt(d)).astype(np.float16).view(np.uint16)
    d_ulp = np.abs(o.astype(np.int32) - want.astype(np.int32))
    assert int(d_ulp.max()) <= 1


@pytest.mark.parametrize("L,a", [(60, 23), (333, 128)])
def test_gated_delta_carried_state_is_exact(L, a):
    # two calls with the state carried between them give the bits of one
    # call: on the token-sequential path at any split, on the chunked path
    # when the split falls on a chunk boundary (the chunks are counted from
    # each call's first token)
    _say("gated delta carried state", L, a)
    Hk, Hv = 16, 32
    qkv, gl, be, s0 = _gdn_problem(L, Hk, Hv, 9)
    o_all, s_all = _gdn_run(qkv, gl, be, s0, Hk, Hv)
    o1, s1 = _gdn_run(qkv[:a], gl[:a], be[:a], s0, Hk, Hv)
    o2, s2 = _gdn_run(qkv[a:], gl[a:], be[a:], s1, Hk, Hv)
    assert np.array_equal(np.concatenate([o1, o2]), o_all)
    assert np.array_equal(s2, s_all)


def test_gated_delta_carried_state_any_split(ora):
    # a split off the chunk grid changes the evaluation order, not the
    # result: both calls together meet the criteria of one
    _say("gated delta carried state, unaligned split")
    L, Hk, Hv, a = 333, 16, 32, 130
    qkv, gl, be, s0 = _gdn_problem(L, Hk, Hv, 9)
    o1, s1 = _gdn_run(qkv[:a], gl[:a], be[:a], s0, Hk, Hv)
    o2, s2 = _gdn_run(qkv[a:], gl[a:], be[a:], s1, Hk, Hv)
    (ok, bad, ratio), s_ok = _gdn_check(ora, qkv, gl, be, s0, Hk, Hv, np.concatenate([o1, o2]), s2)
    assert ok and s_ok, (bad, ratio, s_ok)


@pytest.mark.parametrize("L", [4096, 16384])
def test_gated_delta_layer_full_size(ora, L):
    # one linear-attention layer's recurrence: 16 key and 32 value heads over
    # a 4,096-token prefill chunk and over the whole 16,384-token context,
    # q|k|v read in place from the projection; every output and the final
    # state against the FP64 sequential rule
    _say("gated delta full", L)
    qkv, gl, be, s0 = _gdn_problem(L, 16, 32, 17)
    o, s = _gdn_run(qkv, gl, be, s0, 16, 32)
    (ok, bad, ratio), s_ok = _gdn_check(ora, qkv, gl, be, s0, 16, 32, o, s)
    print(f"[case] gated delta L={L}: failures={bad} max err/bound={ratio:.3f} state ok={s_ok}", flush=True)
    assert ok and s_ok, (bad, ratio, s_ok)


@pytest.mark.parametrize("L", [32, 512])
def test_int8_overflow_gives_inf(ora, L):
    # x * 16 = 65536 overflows FP16 in one column: with every weight
    # positive, every output is +inf on both int8 paths, as in the oracle
    _say("int8 overflow", L)
    g = np.random.default_rng(3)
    x = (g.random((L, 128)) * 0.5).astype(np.float16)
    x[:, 3] = np.float16(4096.0)
    q = g.integers(1, 128, size=(64, 128)).astype(np.int8)
    sc = np.full((64, 4), 0.01, np.float16)
    for epi in (F32, F16):
        y = _gpu_int8(x, q, sc, epi, 16.0)
        yv = y if epi == F32 else y.view(np.float16)
        _, ref = ora.int8_linear(x, q, sc, epilogue=epi, in_scale=16.0)
        rv = ref if epi == F32 else ref.view(np.float16)
        assert np.all(np.isposinf(yv)) and np.all(np.isposinf(rv))
