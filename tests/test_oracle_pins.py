"""Pins of the CPU oracle against what the pages and the mathematics fix.

The oracle is the plain definition of the LUT-6 linear layer (page
"Clef-Flash-ANE-LUT6", sections "Weight precision" and "LUT-6 text
weights").  Nothing here re-types its C code: each pin compares it with
something independent of it --

  * hand-worked packing examples (tests/golden/pack_worked_examples.txt) and
    the exhaustive bijection over all 2^24 index tuples / byte triples;
  * the page's storage figure of about 6.02 bits per weight at K = 4,096
    (tests/golden/storage_bits_per_weight.txt);
  * numpy's IEEE binary16 conversions, exhaustively and on every tie;
  * exact rational (Python integer) brute force on tiny GEMMs;
  * closed forms: constant, zero, per-group and ramp tables, identity and
    one-hot activations, the scale invariance of power-of-two in_scale;
  * the SiLU epilogue against torch's silu in float64.

``test_pins_catch_planted_mistakes`` rebuilds the oracle with each of a list
of plausible mistakes planted (ORA_MUTANT) and checks that at least one pin
fails for every one of them.
"""
from __future__ import annotations

from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest

import oracle
import seeded_inputs as si

GOLDEN = Path(__file__).resolve().parent / "golden"


# ---------------------------------------------------------------------------
# independent helpers (exact arithmetic; no oracle code)
# ---------------------------------------------------------------------------

def _frac(v) -> Fraction:
    return Fraction(float(v))


def _round_exact(q: Fraction, dtype) -> np.ndarray:
    """Correctly rounded (nearest, ties to even) value of the rational q."""
    c = np.array([float(q)]).astype(dtype)[0]          # within one ulp of the answer
    cands = [c, np.nextafter(c, dtype(-np.inf)), np.nextafter(c, dtype(np.inf))]
    cands = [v for v in cands if np.isfinite(v)]
    best = min(cands, key=lambda v: (abs(_frac(v) - q),
                                     int(np.array([v], dtype=dtype).view(
                                         np.uint16 if dtype == np.float16 else np.uint32)[0]) & 1))
    return np.array([best], dtype=dtype)


def _small_problem(L, K, N, seed, *, x_scale=1.0, subnormal_x=False):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((L, K)) * x_scale).astype(np.float16)
    if subnormal_x:
        x.reshape(-1)[:: 7] = (g.integers(1, 1024, size=x.size)[:: 7] * 2.0 ** -24).astype(np.float16)
    idx = g.integers(0, 64, size=(N, K), dtype=np.uint8)
    tab = np.sort((g.standard_normal((N // 16, 64)) * 0.02).astype(np.float16), axis=1)
    return x, idx, tab


def _exact_acc(x, idx, tab, s):
    """Exact sum_k fp16(x*s)[l,k] * T[n//16][idx[n,k]] / s as Fractions."""
    L, K = x.shape
    N = idx.shape[0]
    xs = [[_frac(v) * Fraction(s) for v in row] for row in x]     # exact: s = 2^e, no overflow
    out = [[None] * N for _ in range(L)]
    mag = [[None] * N for _ in range(L)]
    for n in range(N):
        w = [_frac(tab[n // 16][i]) for i in idx[n]]
        for l in range(L):
            terms = [a * b for a, b in zip(xs[l], w)]
            out[l][n] = sum(terms, Fraction(0)) / Fraction(s)
            mag[l][n] = sum((abs(t) for t in terms), Fraction(0)) / Fraction(s)
    return out, mag


# ---------------------------------------------------------------------------
# pins: each takes an Oracle and raises AssertionError on a mismatch
# ---------------------------------------------------------------------------

def _pack_examples():
    rows = []
    for line in (GOLDEN / "pack_worked_examples.txt").read_text().splitlines():
        if not line.strip() or line.lstrip().startswith("#"):
            continue
        left, right = line.split(":")
        rows.append(([int(v) for v in left.split()], bytes(int(b, 16) for b in right.split())))
    return rows


def pin_pack_worked_examples(ora):
    ex = _pack_examples()
    assert len(ex) >= 10
    idx = np.array([e[0] for e in ex], np.uint8).reshape(1, -1)
    packed = ora.pack(idx)
    want = b"".join(e[1] for e in ex)
    assert packed.tobytes() == want, "packing differs from the hand-worked examples"
    back = ora.unpack(np.frombuffer(want, np.uint8).reshape(1, -1), idx.shape[1])
    assert np.array_equal(back, idx), "unpacking differs from the hand-worked examples"


def pin_pack_exhaustive(ora):
    # every 4-tuple of 6-bit indices packs to a distinct 3-byte group and back
    t = np.arange(64 ** 4, dtype=np.uint32)
    idx = np.stack([(t // 64 ** i) % 64 for i in range(4)], axis=1).astype(np.uint8).reshape(1, -1)
    packed = ora.pack(idx)
    assert packed.size == 3 * 64 ** 4
    tri = packed.reshape(-1, 3).astype(np.uint32)
    code = tri[:, 0] + 256 * tri[:, 1] + 65536 * tri[:, 2]
    assert np.unique(code).size == 2 ** 24, "packing is not injective"
    assert np.array_equal(ora.unpack(packed, idx.shape[1]), idx), "round trip idx->bytes->idx"
    # and every byte triple is the packing of exactly one tuple
    allb = np.arange(2 ** 24, dtype=np.uint32)
    raw = np.stack([allb % 256, (allb // 256) % 256, allb // 65536], axis=1).astype(np.uint8).reshape(1, -1)
    again = ora.pack(ora.unpack(raw, 4 * 2 ** 24))
    assert np.array_equal(again, raw), "round trip bytes->idx->bytes"


def pin_storage(ora):
    want = {}
    for line in (GOLDEN / "storage_bits_per_weight.txt").read_text().splitlines():
        if line.strip() and not line.lstrip().startswith("#"):
            k, v = line.split(":")
            want[int(k)] = float(v)
    for K, printed in want.items():
        N = 256
        idx = np.zeros((N, K), np.uint8)
        total = ora.pack(idx).nbytes + ora.table_bytes(N)
        assert ora.packed_bytes(N, K) == ora.pack(idx).nbytes
        bpw = total * 8 / (N * K)
        assert bpw == 6 + 64 / K
        assert round(bpw, 2) == printed, f"{bpw} bits/weight vs the page's {printed}"


def pin_f16_decode(ora):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = ora.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(ours, ref, equal_nan=True), "binary16 decode"
    assert np.array_equal(np.signbit(ours), np.signbit(ref))


def pin_f16_encode(ora):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    pos = np.sort(vals[np.isfinite(vals) & (vals >= 0)])
    mids = (pos[:-1] + pos[1:]) / 2                          # exact ties
    up = np.nextafter(mids, np.inf)
    dn = np.nextafter(mids, -np.inf)
    g = np.random.default_rng(7)
    rnd = g.standard_normal(200_000) * 10.0 ** g.uniform(-9, 5, 200_000)
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 65504.0, 65519.99, 65520.0,
                        65536.0, 1e10, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
                        2.0 ** -14 - 2.0 ** -25, 1 + 2.0 ** -11 + 2.0 ** -40])
    v = np.concatenate([vals[np.isfinite(vals)], mids, -mids, up, dn, -up, rnd, special])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    ours = ora.f64_to_f16(v)
    nan = np.isnan(v)
    assert np.array_equal(ours[~nan], ref[~nan]), "binary16 encode (round to nearest even)"
    assert np.all((ours[nan] & 0x7c00) == 0x7c00) and np.all((ours[nan] & 0x3ff) != 0)


def pin_dequant(ora):
    x, idx, tab = _small_problem(1, 192, 96, 11)
    w = ora.dequant(ora.pack(idx), tab, 192)
    ref = tab.view(np.uint16)[np.arange(96)[:, None] // 16, idx]
    assert np.array_equal(w, ref), "dequantized weight != T[n//16][idx]"


def pin_linear_bruteforce(ora):
    for i, (L, K, N) in enumerate([(1, 64, 16), (3, 128, 32), (5, 64, 96), (9, 192, 48)]):
        x, idx, tab = _small_problem(L, K, N, 100 + i, subnormal_x=(i % 2 == 1))
        packed = ora.pack(idx)
        for s in (1.0, 16.0):
            exact, mag = _exact_acc(x, idx, tab, s)
            for epi in (oracle.EPI_F32, oracle.EPI_F16):
                ye, yo = ora.linear(x, packed, tab, epilogue=epi, in_scale=s, threads=2)
                for l in range(L):
                    for n in range(N):
                        q = exact[l][n]
                        assert abs(_frac(ye[l, n]) - q) <= Fraction(1, 10 ** 12) * mag[l][n] + Fraction(1, 2 ** 80)
                        dt = np.float32 if epi == oracle.EPI_F32 else np.float16
                        got = yo[l:l + 1, n] if epi == oracle.EPI_F32 else yo[l:l + 1, n].view(np.float16)
                        want = _round_exact(q, dt)
                        assert got.tobytes() == want.tobytes(), (L, K, N, s, epi, l, n)


def pin_linear_silu(ora):
    import torch
    # One-hot activations read single table entries: a_gate[l, n] = T0[l],
    # a_up[l, n] = T1[l]; the epilogue must give silu(T0[l]) * T1[l].
    probes = np.array([0, 0.5, -0.5, 1, -1, 2, -2, 8, -8, 20, -20, 100, -100,
                       1000, -1000, 0.001, -0.001, 3.14, -3.14], np.float16)
    ups = np.array([1, 1, 1, 0.5, 0.5, 1, 1, -2, -2, 1, 1, 0.25, 0.25,
                    1, 1, 3, 3, 1, 1], np.float16)
    L, K, N = probes.size, 64, 32
    tab = np.zeros((2, 64), np.float16)
    tab[0, :L] = probes
    tab[1, :L] = ups
    idx = np.tile(np.arange(K, dtype=np.uint8) % 64, (N, 1))
    x = np.zeros((L, K), np.float16)
    x[np.arange(L), np.arange(L)] = 1.0
    ye, yo = ora.linear(x, ora.pack(idx), tab, epilogue=oracle.EPI_SILU_MUL_F16, threads=1)
    g = torch.tensor(probes.astype(np.float64))
    ref = (torch.nn.functional.silu(g) * torch.tensor(ups.astype(np.float64))).numpy()
    for n in range(N // 2):
        assert np.allclose(ye[:, n], ref, rtol=1e-14, atol=0), "silu(gate) * up"
        assert np.array_equal(yo[:, n], ref.astype(np.float16).view(np.uint16))
    # silu(g) - silu(-g) = g and silu(g) ~ g for large g
    pair = {float(p): ye[i, 0] / float(ups[i]) for i, p in enumerate(probes)}
    for p in (0.5, 1, 2, 8, 20, 100, 3.14):
        p16 = float(np.float16(p))
        assert abs(pair[p16] - pair[-p16] - p16) <= 1e-12 * max(1.0, p16)
    assert pair[1000.0] == 1000.0 and pair[0.0] == 0.0


def pin_special_tables(ora):
    g = np.random.default_rng(5)
    L, K, N = 4, 256, 64
    x = g.standard_normal((L, K)).astype(np.float16)
    idx = g.integers(0, 64, size=(N, K), dtype=np.uint8)
    packed = ora.pack(idx)
    xsum = [sum((_frac(v) for v in row), Fraction(0)) for row in x]
    # constant tables c = 2^-3: y = c * sum_k x
    tab = np.full((N // 16, 64), 0.125, np.float16)
    _, yo = ora.linear(x, packed, tab, epilogue=oracle.EPI_F32, threads=3)
    for l in range(L):
        assert np.all(yo[l] == np.float32(float(xsum[l] / 8))), "constant table"
    # zero tables: +0 everywhere, for every epilogue
    tab = np.zeros((N // 16, 64), np.float16)
    for epi in (oracle.EPI_F32, oracle.EPI_F16, oracle.EPI_SILU_MUL_F16):
        _, yo = ora.linear(x, packed, tab, epilogue=epi, threads=1)
        assert np.all(yo.view(np.uint32 if epi == oracle.EPI_F32 else np.uint16) == 0)
    # per-group constant tables T[g][:] = g + 1: y[l, n] = (n // 16 + 1) * sum_k x
    tab = np.repeat(np.arange(1, N // 16 + 1, dtype=np.float16)[:, None], 64, axis=1)
    _, yo = ora.linear(x, packed, tab, epilogue=oracle.EPI_F32, threads=2)
    for l in range(L):
        want = np.array([float(xsum[l] * (n // 16 + 1)) for n in range(N)], np.float32)
        assert np.array_equal(yo[l], want), "per-group tables"
    # ramp tables T[g][j] = j/64 with x = 1: y[l, n] = sum_k idx[n, k] / 64 (raw indices)
    tab = np.tile((np.arange(64) / 64).astype(np.float16), (N // 16, 1))
    ones = np.ones((2, K), np.float16)
    _, yo = ora.linear(ones, packed, tab, epilogue=oracle.EPI_F32, threads=2)
    want = (idx.astype(np.int64).sum(axis=1) / 64).astype(np.float32)
    assert np.array_equal(yo[0], want) and np.array_equal(yo[1], want), "ramp tables"


def pin_identity_readout(ora):
    # x = I_K: y[l, n] = W[n, l] bit for bit (one product per output), any s
    K, N = 64, 48
    _, idx, tab = _small_problem(1, K, N, 21)
    W = tab.view(np.uint16)[np.arange(N)[:, None] // 16, idx]
    eye = np.eye(K, dtype=np.float16)
    for s in (1.0, 16.0):
        _, yo = ora.linear(eye, ora.pack(idx), tab, epilogue=oracle.EPI_F16, in_scale=s, threads=2)
        assert np.array_equal(yo, W.T), "identity readout"
    # the smallest subnormal activation times 1024 is exactly 2^-14
    x = np.zeros((1, K), np.float16)
    x[0, 5] = np.float16(2.0 ** -24)
    tab1 = np.full((N // 16, 64), 1024, np.float16)
    _, yo = ora.linear(x, ora.pack(idx), tab1, epilogue=oracle.EPI_F32, threads=1)
    assert np.all(yo == np.float32(2.0 ** -14)), "subnormal activation"


def pin_in_scale(ora):
    g = np.random.default_rng(9)
    L, K, N = 6, 128, 64
    x = g.standard_normal((L, K)).astype(np.float16)
    idx = g.integers(0, 64, size=(N, K), dtype=np.uint8)
    tab = np.sort((g.standard_normal((N // 16, 64)) * 0.02).astype(np.float16), axis=1)
    packed = ora.pack(idx)
    for epi in (oracle.EPI_F32, oracle.EPI_F16, oracle.EPI_SILU_MUL_F16):
        _, y1 = ora.linear(x, packed, tab, epilogue=epi, in_scale=1.0, threads=2)
        for s in (2.0, 4.0, 8.0, 16.0):
            _, ys = ora.linear(x, packed, tab, epilogue=epi, in_scale=s, threads=2)
            assert y1.tobytes() == ys.tobytes(), f"power-of-two in_scale {s} changed the result"
    # overflow: 4096 * 16 = 65536 is beyond FP16, so the scaled input is +inf
    xo = np.zeros((1, K), np.float16)
    xo[0, 0] = 4096
    pos = np.full((N // 16, 64), 0.5, np.float16)
    _, yf = ora.linear(xo, packed, pos, epilogue=oracle.EPI_F32, in_scale=16.0, threads=1)
    assert np.all(np.isposinf(yf)), "overflowing scaled input"
    _, yh = ora.linear(xo, packed, pos, epilogue=oracle.EPI_F16, in_scale=8.0, threads=1)
    assert np.all(yh.view(np.float16) == np.float16(2048.0)), "largest in-range scale"


# -- int8 weight-only variant ------------------------------------------------

def pin_int8_dequant(ora):
    # the product q * scale is exact in double, so numpy's double -> half
    # conversion (round to nearest even, overflow to inf) is the definition
    q, s = si.int8_weight(32, 256, (9, 0, 0))
    s = s.copy()
    s[0, 0] = np.float16(600.0)                       # 127 * 600 overflows FP16
    s[1, 1] = np.float16(6e-8)                        # subnormal products
    q[0, :32] = np.arange(-128, 128, 8, dtype=np.int16).astype(np.int8)
    with np.errstate(over="ignore"):
        want = (q.astype(np.float64) * np.repeat(s.astype(np.float64), 32, axis=1)).astype(np.float16)
    got = ora.int8_dequant(q, s)
    assert np.array_equal(got, want.view(np.uint16))
    assert np.isinf(want[0, 31]) and want[0, 16] == 0.0


def pin_int8_as_lut6(ora):
    # codes -32..31 with one power-of-two scale per 16 rows are exactly a
    # 64-entry table (entry i = (i - 32) * scale): both variants must give
    # the same bits, so the LUT-6 pins carry over to the int8 reading
    N, K, L = 64, 256, 9
    g = np.random.default_rng(5)
    idx = g.integers(0, 64, size=(N, K), dtype=np.uint8)
    e = g.integers(-10, -4, size=N // 16)
    tab = ((np.arange(64)[None, :] - 32) * np.exp2(e)[:, None]).astype(np.float16)
    q = (idx.astype(np.int16) - 32).astype(np.int8)
    s = np.repeat(np.exp2(e), 16)[:, None].repeat(K // 32, axis=1).astype(np.float16)
    x = si.activations(L, K, 1.0, (9, 0, 1))
    for epi in (0, 1, 2):
        for sc in (1.0, 8.0):
            ya, oa = ora.linear(x, ora.pack(idx), tab, epilogue=epi, in_scale=sc)
            yb, ob = ora.int8_linear(x, q, s, epilogue=epi, in_scale=sc)
            assert np.array_equal(ya, yb) and np.array_equal(oa, ob)


def pin_int8_block_scale(ora):
    # doubling one block's scale (exact) adds exactly that block's part of
    # the dot product once more, for every token row
    N, K, L = 16, 128, 5
    q, s = si.int8_weight(N, K, (9, 1, 0))
    x = si.activations(L, K, 1.0, (9, 1, 1))
    y0, _ = ora.int8_linear(x, q, s, epilogue=0)
    s2 = s.copy()
    s2[3, 2] = s2[3, 2] * np.float16(2)
    y1, _ = ora.int8_linear(x, q, s2, epilogue=0)
    w = q[3, 64:96].astype(np.float64) * np.float64(s[3, 2])
    part = x[:, 64:96].astype(np.float64) @ np.array([np.float64(np.float16(v)) for v in w])
    assert np.allclose(y1[:, 3] - y0[:, 3], part, rtol=0, atol=1e-12)
    assert np.array_equal(np.delete(y1, 3, axis=1), np.delete(y0, 3, axis=1))


# -- full attention ------------------------------------------------------------

def _att_inputs(L, Lk, Hq, Hkv, D, seed, extra=0):
    g = np.random.default_rng(seed)
    q = (g.standard_normal((L, Hq * D + extra)) * 0.5).astype(np.float16)
    k = (g.standard_normal((Lk, Hkv * D + extra)) * 0.5).astype(np.float16)
    v = g.standard_normal((Lk, Hkv * D + extra)).astype(np.float16)
    return q, k, v


def pin_attention_sdpa(ora):
    # torch's float64 scaled_dot_product_attention with an explicit mask (the
    # L queries are the last L of Lk positions) and the key-value heads
    # repeated for their query heads; strided rows (extra columns) included
    import torch
    for L, Lk, Hq, Hkv, D in ((5, 9, 4, 2, 16), (7, 7, 3, 1, 8), (1, 12, 2, 2, 32)):
        q, k, v = _att_inputs(L, Lk, Hq, Hkv, D, L * 100 + Lk, extra=3)
        oe, _ = ora.attention(q, k, v, n_heads=Hq, n_kv_heads=Hkv, head_dim=D)
        tq = torch.from_numpy(q[:, :Hq * D].astype(np.float64)).view(L, Hq, D).transpose(0, 1)
        tk = torch.from_numpy(k[:, :Hkv * D].astype(np.float64)).view(Lk, Hkv, D).transpose(0, 1)
        tv = torch.from_numpy(v[:, :Hkv * D].astype(np.float64)).view(Lk, Hkv, D).transpose(0, 1)
        tk = tk.repeat_interleave(Hq // Hkv, dim=0)
        tv = tv.repeat_interleave(Hq // Hkv, dim=0)
        mask = torch.arange(Lk)[None, :] <= (Lk - L + torch.arange(L))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
        ref = ref.transpose(0, 1).reshape(L, Hq * D).numpy()
        assert np.allclose(oe, ref, rtol=1e-12, atol=1e-13), "attention against torch sdpa"


def pin_attention_closed_forms(ora):
    L, Hq, Hkv, D = 6, 4, 2, 16
    q, k, v = _att_inputs(L, L, Hq, Hkv, D, 3)
    oe, oo, oa, va = ora.attention(q, k, v, n_heads=Hq, n_kv_heads=Hkv, head_dim=D, with_bounds=True)
    # the first query sees one key: its output is that key's value row
    want0 = np.repeat(v[0].reshape(Hkv, D), Hq // Hkv, axis=0).reshape(-1)
    assert np.array_equal(oo[0], want0.view(np.uint16)), "single visible key"
    # zero queries: every visible key equally likely, the mean of the values
    z = np.zeros_like(q)
    ez, _ = ora.attention(z, k, v, n_heads=Hq, n_kv_heads=Hkv, head_dim=D)
    vv = v.astype(np.float64).reshape(L, Hkv, D)
    for i in range(L):
        mean = np.repeat(vv[: i + 1].mean(axis=0), Hq // Hkv, axis=0).reshape(-1)
        assert np.allclose(ez[i], mean, rtol=1e-13, atol=1e-15), "uniform weights"
    # bounds: sum p |v| between |o| and max |v|; sum |v| over the visible rows
    assert np.all(oa >= np.abs(oe) - 1e-15)
    va_want = np.repeat(np.cumsum(np.abs(vv), axis=0), Hq // Hkv, axis=1).reshape(L, -1)
    assert np.allclose(va, va_want, rtol=1e-14)
    # softmax shift invariance: a constant added to every score changes
    # nothing; q scaled so that one key dominates gives that key's value
    q2 = np.zeros_like(q)
    q2[:, :D] = (k[1, :D].astype(np.float32) * 64).astype(np.float16)   # head 0 -> kv head 0
    e2, _ = ora.attention(q2, k, v, n_heads=Hq, n_kv_heads=Hkv, head_dim=D)
    s = (q2[3, :D].astype(np.float64) @ k[:4, :D].astype(np.float64).T) / np.sqrt(D)
    if np.argmax(s) == 1 and np.sort(s)[-1] - np.sort(s)[-2] > 60:
        assert np.allclose(e2[3, :D], v[1, :D].astype(np.float64), rtol=0, atol=1e-20 + 1e-12)


# -- Gated DeltaNet recurrence ---------------------------------------------------

def _gdn_inputs(L, Hk, Hv, d, seed):
    g = np.random.default_rng(seed)
    q = (g.standard_normal((L, Hk * d)) / np.sqrt(d)).astype(np.float16)
    k = (g.standard_normal((L, Hk * d)) / np.sqrt(d)).astype(np.float16)
    v = g.standard_normal((L, Hv * d)).astype(np.float16)
    gl = (-g.random((L, Hv)) * 0.5).astype(np.float32)
    be = g.random((L, Hv)).astype(np.float32)
    s0 = (g.standard_normal((Hv, d, d)) * 0.1).astype(np.float32)
    return q, k, v, gl, be, s0


def pin_gated_delta_frozen_state(ora):
    # beta = 0, g = 0: the state never changes, o_t = S0^T q_t / sqrt(dk)
    L, Hk, Hv, d = 5, 2, 4, 8
    q, k, v, gl, be, s0 = _gdn_inputs(L, Hk, Hv, d, 1)
    oe, _, _, so = ora.gated_delta(q, k, v, np.zeros_like(gl), np.zeros_like(be), n_k_heads=Hk,
                                   n_v_heads=Hv, dk=d, dv=d, state=s0)
    qf = q.astype(np.float64).reshape(L, Hk, d)
    for h in range(Hv):
        want = qf[:, h // 2] @ s0[h].astype(np.float64) / np.sqrt(d)
        assert np.allclose(oe[:, h * d:(h + 1) * d], want, rtol=1e-13, atol=1e-15), "frozen state"
    assert np.array_equal(so, s0.astype(np.float64))


def pin_gated_delta_decay_only(ora):
    # beta = 0: S_t = exp(g_1 + .. + g_t) S0
    L, Hk, Hv, d = 6, 1, 2, 8
    q, k, v, gl, be, s0 = _gdn_inputs(L, Hk, Hv, d, 2)
    _, _, _, so = ora.gated_delta(q, k, v, gl, np.zeros_like(be), n_k_heads=Hk, n_v_heads=Hv,
                                  dk=d, dv=d, state=s0)
    for h in range(Hv):
        f = np.exp(np.sum(gl[:, h].astype(np.float64)))
        assert np.allclose(so[h], f * s0[h], rtol=1e-12), "decay"


def pin_gated_delta_overwrites_unit_keys(ora):
    # beta = 1 and k_t = e_i: the update replaces row i of the (decayed)
    # state by v_t, so reading with q = e_i right after gives v_t / sqrt(dk);
    # every other row only decays
    L, Hk, Hv, d = 7, 2, 4, 8
    q, k, v, gl, be, s0 = _gdn_inputs(L, Hk, Hv, d, 3)
    rows = np.arange(L) % d
    k = np.zeros_like(k)
    for t in range(L):
        for kh in range(Hk):
            k[t, kh * d + (rows[t] + kh) % d] = 1.0
    q = k.copy()
    oe, _, _, so = ora.gated_delta(q, k, v, gl, np.ones_like(be), n_k_heads=Hk, n_v_heads=Hv,
                                   dk=d, dv=d, state=s0)
    vf = v.astype(np.float64)
    assert np.allclose(oe, vf / np.sqrt(d), rtol=1e-13, atol=1e-15), "delta rule overwrite"
    for h in range(Hv):
        kh = h // 2
        last = {}
        for t in range(L):
            last[(rows[t] + kh) % d] = t
        decay = np.exp(np.cumsum(gl[::-1, h].astype(np.float64))[::-1])   # exp(g_t + .. + g_{L-1})
        for i in range(d):
            if i in last:
                t = last[i]
                want = vf[t, h * d:(h + 1) * d] * (decay[t + 1] if t + 1 < L else 1.0)
            else:
                want = s0[h, i].astype(np.float64) * decay[0]
            assert np.allclose(so[h, i], want, rtol=1e-12, atol=1e-14), "row kept or decayed"


def pin_gated_delta_split_sequence(ora):
    # running [0, a) then [a, L) from the carried state equals one run
    L, Hk, Hv, d, a = 9, 2, 4, 8, 4
    q, k, v, gl, be, s0 = _gdn_inputs(L, Hk, Hv, d, 4)
    oe, _, _, so = ora.gated_delta(q, k, v, gl, be, n_k_heads=Hk, n_v_heads=Hv, dk=d, dv=d, state=s0)
    o1, _, _, s1 = ora.gated_delta(q[:a], k[:a], v[:a], gl[:a], be[:a], n_k_heads=Hk, n_v_heads=Hv,
                                   dk=d, dv=d, state=s0)
    o2, _, _, s2 = ora.gated_delta(q[a:], k[a:], v[a:], gl[a:], be[a:], n_k_heads=Hk, n_v_heads=Hv,
                                   dk=d, dv=d, state=s1.astype(np.float32))
    assert np.array_equal(o1, oe[:a])
    assert np.allclose(o2, oe[a:], rtol=1e-6, atol=1e-7)    # the carried state is rounded to FP32


# ---------------------------------------------------------------------------
# table fitting: what the page fixes (page "Clef-Flash-ANE-LUT6", section
# "LUT-6 text weights": 40 rounds of one-dimensional k-means per 16-channel
# group, half of the starting values at quantiles and half spread evenly
# from the group's minimum to its maximum).  The Lloyd rounds are recomputed
# here independently: values as exact integers in 2^-24 units (numpy's FP16
# conversion), cluster boundaries as exact rational midpoints, means as
# correctly rounded rationals.
# ---------------------------------------------------------------------------

def _units(w16) -> np.ndarray:
    """FP16 values as exact integers in units of 2^-24."""
    return (np.asarray(w16, np.float16).astype(np.float64) * 2.0 ** 24).astype(np.int64)


def _km_assign(u: np.ndarray, c) -> np.ndarray:
    """Nearest of the sorted centres c for values u (2^-24 units), the lower
    of two equally near ones: u goes below the exact midpoint m of c_i and
    c_(i+1) when u <= m, i.e. u <= floor((c_i + c_(i+1)) * 2^23)."""
    t = np.array([(Fraction(c[i]) + Fraction(c[i + 1])) * 2 ** 23 for i in range(len(c) - 1)])
    t = np.array([int(v.numerator // v.denominator) for v in t], dtype=np.int64)
    return np.searchsorted(t, u, side="left")


def _km_step(u_sorted: np.ndarray, c) -> list:
    """One Lloyd round: each centre becomes its cluster's mean (rounded once
    to the nearest double), an empty cluster keeps its centre, then sort."""
    cl = _km_assign(u_sorted, c)
    cnt = np.bincount(cl, minlength=len(c))
    pref = np.concatenate([[0], np.cumsum(u_sorted)])
    ends = np.cumsum(cnt)
    new = []
    for q in range(len(c)):
        if cnt[q]:
            tot = int(pref[ends[q]] - pref[ends[q] - cnt[q]])
            new.append(float(Fraction(tot, int(cnt[q]))) * 2.0 ** -24)
        else:
            new.append(float(c[q]))
    return sorted(new)


def _block_group():
    """A 16 x 64 group of 32 distinct FP16 values, 32 copies each (shuffled),
    the two ends far out: every quantile inside one of the 32 equal shares of
    the sorted values is that share's value, whatever rank is taken."""
    q = np.concatenate([[-0.5], (np.arange(30) - 14.5) * 0.003, [0.75]]).astype(np.float16)
    assert np.all(np.diff(q.astype(np.float64)) > 0)
    vals = np.repeat(q, 32)[np.random.default_rng(11).permutation(1024)]
    return vals.reshape(16, 64), q.astype(np.float64)


def _slow_group(K=1024, seed=12):
    """N(0, 0.02) with 2% outliers at 8x: k-means is still moving at round 40."""
    g = np.random.default_rng(seed)
    w = g.standard_normal((16, K)) * 0.02
    w[g.random((16, K)) < 0.02] *= 8.0
    return w.astype(np.float16)


def pin_quantize_starts(ora):
    w, q = _block_group()
    c0 = ora.km_centres(w, 0, 0)
    lo, hi = q[0], q[-1]
    even = lo + (hi - lo) * np.arange(32) / 31.0
    want = np.sort(np.concatenate([q, even]))
    # 32 quantiles (one per share) and 32 even steps from min to max, both
    # ends included; the tolerance only covers the evaluation order
    assert np.allclose(c0, want, rtol=0, atol=2.0 ** -50), "starting centres"
    assert c0[0] == lo and c0[-1] == hi
    # the squared error before the first round, and one value per round
    _, _, sse = ora.quantize(w, with_sse=True)
    assert len(sse) == 41, f"{len(sse) - 1} rounds instead of 40"
    vals = np.repeat(q, 32)
    d = np.min(np.abs(vals[:, None] - want[None, :]), axis=1)
    assert abs(sse[0] - float(np.sum(d * d))) <= 1e-12 * float(np.sum(d * d))


def pin_quantize_lloyd_step(ora):
    for w in (_block_group()[0], _slow_group(K=256, seed=13)):
        u = np.sort(_units(w).reshape(-1))
        for r in (0, 1, 6):
            c = ora.km_centres(w, 0, r)
            nxt = ora.km_centres(w, 0, r + 1)
            assert list(nxt) == _km_step(u, list(c)), f"Lloyd round {r + 1}"


def pin_quantize_forty_rounds(ora):
    w = _slow_group()
    K = w.shape[1]
    u = np.sort(_units(w).reshape(-1))
    c = list(ora.km_centres(w, 0, 0))          # the starts, pinned above
    hist = [c]
    for _ in range(40):
        c = _km_step(u, c)
        hist.append(c)

    def table(cs):
        return np.sort(np.asarray(cs, np.float64).astype(np.float16).astype(np.float64))
    t39, t40 = table(hist[39]), table(hist[40])
    assert not np.array_equal(t39, t40), "the group must still move at round 40"
    packed, tables = ora.quantize(w)
    got = tables[0].view(np.float16).astype(np.float64)
    assert np.array_equal(got, t40), "table = the 40th round's centres rounded to FP16"
    idx = ora.unpack(packed, K).astype(np.int64)
    want = _km_assign(_units(w).reshape(-1), list(t40)).reshape(16, K)
    assert np.array_equal(idx, want), "index = nearest entry, the lower on a tie"


# ---------------------------------------------------------------------------
# int8 code selection (page "clef-flash — Core AI", section "Precision": int8
# per block of 32, symmetric with clipping).  Closed-form blocks: the scale is
# the largest magnitude over 127 rounded once to FP16, codes are w / s rounded
# to nearest even and clamped to -127..127.
# ---------------------------------------------------------------------------

def _i8_block_rows(blocks):
    """Rows of FP16 values, one 32-wide block per row (zero padded)."""
    w = np.zeros((len(blocks), 32), np.float16)
    for r, b in enumerate(blocks):
        w[r, :len(b)] = np.asarray(b, np.float64).astype(np.float16)
    return w


def pin_int8_quantize_grid(ora):
    # largest magnitude 127 * 2^-7: the scale is 2^-7 exactly and every
    # multiple j * 2^-7 (|j| <= 127) is coded as j; only element 0 holds the
    # maximum, so halves of a block would get other scales
    g = np.random.default_rng(31)
    j = g.integers(-126, 127, size=(6, 64))
    j[:, 0] = np.array([127, -127, 127, -127, 127, -127])
    j[:, 32] = -j[:, 0]
    w = (j * 2.0 ** -7).astype(np.float16)
    q, qs = ora.int8_quantize(w)
    assert np.array_equal(q.astype(np.int64), j), "codes of an exact grid"
    assert np.all(qs == np.float16(2.0 ** -7).view(np.uint16)), "scale = max / 127"


def pin_int8_quantize_ties(ora):
    # scale 1 (largest magnitude 127): halves go to the even neighbour
    w = _i8_block_rows([[127.0, 2.5, -2.5, 3.5, 0.5, -0.5, 1.5, -126.5, 126.5]])
    q, qs = ora.int8_quantize(w)
    assert qs[0, 0] == np.float16(1.0).view(np.uint16)
    assert list(q[0, :9]) == [127, 2, -2, 4, 0, 0, 2, -126, 126], list(q[0, :9])


def pin_int8_quantize_clamp_and_fp16_scale(ora):
    # largest magnitude 2^-17: 2^-17 / 127 = 2^-24 * 128/127 rounds to the
    # FP16 subnormal 2^-24, so the maximum's quotient is exactly 128 and is
    # clamped to 127 (and -128 to -127: symmetric).  100 * 2^-24 is coded
    # 100 against the FP16 scale (99.2 against the unrounded one)
    t = 2.0 ** -24
    w = _i8_block_rows([[2.0 ** -17, 100 * t, -3 * t], [-(2.0 ** -17), -100 * t, 3 * t]])
    q, qs = ora.int8_quantize(w)
    assert np.all(qs[:, 0] == 1), "scale 2^-24 (FP16 bits 0x0001)"
    assert list(q[0, :3]) == [127, 100, -3] and list(q[1, :3]) == [-127, -100, 3], (q[0, :3], q[1, :3])


def pin_int8_quantize_zero_scales(ora):
    # an all-zero block and one whose scale rounds to zero (2^-24 / 127)
    w = _i8_block_rows([[0.0], [2.0 ** -24, -(2.0 ** -24)]])
    q, qs = ora.int8_quantize(w)
    assert np.all(qs == 0) and np.all(q == 0)


def pin_int8_quantize_round_trip(ora):
    # any block: the weight the layer uses, fp16(q * s), is within half a
    # step of w (plus its own FP16 rounding) unless the code was clamped, and
    # a code is clamped only where |w| is at least 126.5 steps (a scale that
    # is an FP16 subnormal can be rounded far down); a block whose scale is
    # an FP16 normal codes its largest magnitude as +-127; q(-w) = -q(w)
    g = np.random.default_rng(32)
    w = (g.standard_normal((24, 256)) * 0.02).astype(np.float16)
    w[3] *= np.float16(1e-3)                                   # a row of tiny blocks
    q, qs = ora.int8_quantize(w)
    s = qs.view(np.float16).astype(np.float64).repeat(32, axis=1)
    wq = ora.int8_dequant(q, qs).view(np.float16).astype(np.float64)
    wd = w.astype(np.float64)
    ulp = np.spacing(np.abs(wd).astype(np.float16)).astype(np.float64)
    inner = np.abs(q.astype(np.int64)) < 127
    assert np.all((np.abs(wq - wd) <= s / 2 + ulp + 1e-30)[inner]), "within half a step"
    assert np.all((np.abs(wd) >= 126.5 * s)[~inner]), "clamped only past 126.5 steps"
    assert np.any(~inner & (np.abs(wd) > 127.5 * s)), "the tiny row has a clamped code"
    normal = qs.view(np.float16).astype(np.float64) >= 2.0 ** -14
    top = np.abs(q.astype(np.int64)).reshape(24, -1, 32).max(axis=2)
    assert np.all(top[normal] == 127), "the largest magnitude codes as 127"
    qn, qsn = ora.int8_quantize(-w)
    assert np.array_equal(qn.astype(np.int64), -q.astype(np.int64)) and np.array_equal(qsn, qs)


def test_int8_scale_is_one_rounding_in_fp32():
    # the device takes fp16(fp32(a) / 127) for the block scale, two roundings;
    # for every finite FP16 magnitude it equals the single rounding of a / 127
    # (through FP64, whose 53 bits cannot land on an FP16 midpoint here), so
    # oracle and device agree on every scale
    a = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16)
    f32 = (a.astype(np.float32) / np.float32(127)).astype(np.float16)
    f64 = (a.astype(np.float64) / 127.0).astype(np.float16)
    assert np.array_equal(f32.view(np.uint16), f64.view(np.uint16))


PINS = [pin_pack_worked_examples, pin_pack_exhaustive, pin_storage, pin_f16_decode,
        pin_f16_encode, pin_dequant, pin_linear_bruteforce, pin_linear_silu,
        pin_special_tables, pin_identity_readout, pin_in_scale, pin_int8_dequant,
        pin_int8_as_lut6, pin_int8_block_scale, pin_attention_sdpa, pin_attention_closed_forms,
        pin_gated_delta_frozen_state, pin_gated_delta_decay_only, pin_gated_delta_overwrites_unit_keys,
        pin_gated_delta_split_sequence, pin_quantize_starts, pin_quantize_lloyd_step,
        pin_quantize_forty_rounds, pin_int8_quantize_grid, pin_int8_quantize_ties,
        pin_int8_quantize_clamp_and_fp16_scale, pin_int8_quantize_zero_scales,
        pin_int8_quantize_round_trip]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(ora, pin):
    pin(ora)


def test_oracle_refusals(ora):
    with pytest.raises(oracle.OracleError):
        ora.pack(np.full((1, 4), 64, np.uint8))                  # index out of range
    with pytest.raises(oracle.OracleError):
        ora.pack(np.zeros((1, 6), np.uint8))                     # K not a multiple of 4
    x = np.zeros((2, 64), np.float16)
    idx = np.zeros((16, 64), np.uint8)
    tab = np.zeros((1, 64), np.float16)
    with pytest.raises(oracle.OracleError):                      # SiLU split needs N % 32
        ora.linear(x, ora.pack(idx), tab, epilogue=oracle.EPI_SILU_MUL_F16)
    with pytest.raises(oracle.OracleError):
        ora.linear(x, ora.pack(idx), tab, epilogue=oracle.EPI_F16, rows=[2])


def test_oracle_row_subset(ora):
    x, idx, tab = _small_problem(9, 128, 64, 3)
    packed = ora.pack(idx)
    full_e, full_o = ora.linear(x, packed, tab, epilogue=oracle.EPI_F16)
    rows = [0, 4, 8]
    sub_e, sub_o = ora.linear(x, packed, tab, epilogue=oracle.EPI_F16, rows=rows)
    assert np.array_equal(sub_o, full_o[rows]) and np.array_equal(sub_e, full_e[rows])


def test_oracle_threads_do_not_change_result(ora):
    x, idx, tab = _small_problem(7, 256, 96, 4)
    packed = ora.pack(idx)
    a = ora.linear(x, packed, tab, epilogue=oracle.EPI_F32, threads=1)
    b = ora.linear(x, packed, tab, epilogue=oracle.EPI_F32, threads=5)
    assert a[0].tobytes() == b[0].tobytes()


MUTANTS = {1: "big-endian byte order", 2: "index order reversed", 3: "one table per 32 channels",
           4: "no scale-back", 5: "gate and up halves swapped", 6: "SiLU sign error",
           7: "last input column dropped", 8: "ties rounded away from zero",
           9: "subnormal decode off by 2x", 10: "activations read transposed",
           11: "f32 output truncated", 12: "int8 scale per block of 16",
           13: "int8 code read unsigned", 14: "int8 product truncated to FP16",
           15: "attention sum off by one", 16: "attention heads interleaved",
           17: "attention mask one key short", 18: "attention scaled by 1 over D",
           19: "delta rule heads interleaved", 20: "delta rule beta ignored", 21: "delta rule unscaled",
           22: "k-means 39 rounds", 23: "k-means starts all quantiles",
           24: "k-means even starts miss min and max", 25: "int8 codes not clamped",
           26: "int8 scale over 128", 27: "int8 quotient on the unrounded scale",
           28: "int8 ties away from zero", 29: "int8 codes per block of 16",
           30: "int8 clamp asymmetric"}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: MUTANTS[m].replace(" ", "_"))
def test_pins_catch_planted_mistakes(mutant, tmp_path):
    lib = oracle.build(tmp_path / f"liblut6_oracle_m{mutant}.so", mutant=mutant)
    bad = oracle.Oracle(lib)
    caught = []
    for pin in PINS:
        try:
            pin(bad)
        except (AssertionError, oracle.OracleError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught planted mistake {mutant} ({MUTANTS[mutant]})"


def test_seeded_inputs_are_reproducible():
    a = si.gemm_inputs(1, 0, 0, si.Gemm("t", 8, 64, 32, si.EPI_F16))
    b = si.gemm_inputs(1, 0, 0, si.Gemm("t", 8, 64, 32, si.EPI_F16))
    assert all(np.array_equal(u, v) for u, v in zip(a, b))
    tab = a[2]
    assert np.all(np.diff(tab.astype(np.float64), axis=1) >= 0), "tables sorted"
    assert a[1].max() <= 63


# ---------------------------------------------------------------------------
# the parity criterion itself: the exactly rounded oracle passes, a result one
# rounding step or more beyond it does not
# ---------------------------------------------------------------------------

def test_floor_admits_fp32_accumulation(ora):
    # an FP32-accumulating kernel (exact FP16 products, FP32 sums of 16 at a
    # time in k order) meets the FP16 criterion, near-zero floor included,
    # at the deepest K of the workloads (the down projection, K = 12,288,
    # input scaled by 16); an FP16 output 3 floor allowances off fails
    from oracle import tolerance as tol
    L, K, N, s = 48, 12288, 256, 16.0
    g = np.random.default_rng(21)
    x = (g.standard_normal((L, K)) * 0.5).astype(np.float16)
    idx = g.integers(0, 64, size=(N, K), dtype=np.uint8)
    tab = np.sort((g.standard_normal((N // 16, 64)) * 0.02).astype(np.float16), axis=1)
    packed = ora.pack(idx)
    y, _ = ora.linear(x, packed, tab, epilogue=oracle.EPI_F32, in_scale=s)
    y = np.asarray(y, np.float64)
    W = ora.dequant(packed, tab, K).view(np.float16).astype(np.float64)
    xs = (x.astype(np.float64) * s).astype(np.float16).astype(np.float64)
    acc = np.zeros((L, N), np.float32)
    for k0 in range(0, K, 16):
        acc = (acc + (xs[:, k0:k0 + 16] @ W[:, k0:k0 + 16].T).astype(np.float32)).astype(np.float32)
    y16 = (acc.astype(np.float64) / s).astype(np.float16)
    S = tol.row_scale(x, tab, K)
    rep = tol.check(y16, y, S, fp16=True)
    assert rep.ok and rep.floor_cases > 0, str(rep)
    # the FP32 error itself stays well inside the floor's allowance (the
    # FP16 roundings of y and y_ref add at most one step of their own)
    tau = tol.TAU_REL * S
    err32 = np.abs(acc.astype(np.float64) / s - y)
    assert float(np.max(err32 / tol.ulp16(tau)[:, None])) < 0.5
    # one floor output moved 3 allowances away fails
    i, j = np.argwhere(np.abs(y) < tau[:, None])[0]
    bad = y16.copy()
    bad[i, j] = np.float16(float(y16[i, j]) + 3 * tol.ulp16(tau[i]))
    assert not tol.check(bad, y, S, fp16=True).ok


def test_tolerance_accepts_rounded_oracle_and_rejects_drift(ora):
    from oracle import tolerance as tol
    # K = 64 and no table outliers: half an FP16 ulp of the largest outputs
    # exceeds 2e-3 * S_row, the tightest case of the criterion
    for (L, K, N, seed) in [(256, 64, 32, 11), (64, 4096, 64, 12)]:
        x, idx, tab = _small_problem(L, K, N, seed)
        packed = ora.pack(idx)
        S = tol.row_scale(x, tab, K)
        y, _ = ora.linear(x, packed, tab, epilogue=oracle.EPI_F32)
        y = np.asarray(y, np.float64)
        r16 = y.astype(np.float16)
        assert tol.check(r16, y, S, fp16=True).ok
        assert tol.check(y.astype(np.float32), y, S, fp16=False).ok
        # pick the element with the largest |y| relative to its row scale
        i, j = np.unravel_index(np.argmax(np.abs(y) / S[:, None]), y.shape)
        # FP32: one bound beyond fails
        bad32 = y.astype(np.float32)
        bad32[i, j] = y[i, j] + 1.01 * 2e-3 * S[i] * np.sign(y[i, j])
        assert not tol.check(bad32, y, S, fp16=False).ok
        # FP16: the neighbours of fp16(y_ref) away from y_ref, one and two
        # ulps out: two always fail (ulp rule), one fails where the FP32
        # bound is below half an ulp (error >= 1 ulp > bound + ulp / 2)
        away = np.float16(np.inf if r16[i, j] >= y[i, j] else -np.inf)
        for steps in (2, 1):
            v = r16[i, j]
            for _ in range(steps):
                v = np.nextafter(v, away)
            bad16 = r16.copy()
            bad16[i, j] = v
            rep = tol.check(bad16, y, S, fp16=True)
            if steps == 2 or 2e-3 * S[i] < 0.5 * tol.ulp16(y[i, j]):
                assert not rep.ok, (L, K, N, steps, str(rep))
    # SiLU(gate) * up rounded once to FP16 passes
    x, idx, tab = _small_problem(128, 64, 64, 13)
    packed = ora.pack(idx)
    S = tol.row_scale(x, tab, 64)
    h, _ = ora.linear(x, packed, tab, epilogue=oracle.EPI_SILU_MUL_F16)
    a, _ = ora.linear(x, packed, tab, epilogue=oracle.EPI_F32)
    Se = tol.silu_scale(a[:, :32], a[:, 32:], S)
    assert tol.check(np.asarray(h, np.float64).astype(np.float16), h, S, fp16=True, S_elem=Se).ok


# ---------------------------------------------------------------------------
# table fitting (1-D k-means, page "Clef-Flash-ANE-LUT6", section "LUT-6 text
# weights").  The page fixes the round count (40) and the starting mix (32
# quantiles, 32 even steps from the group's minimum to its maximum); the pins
# above check both.  The tests below are properties that hold for k-means
# whatever its remaining details.
# ---------------------------------------------------------------------------

def _q_values(tables_u16: np.ndarray) -> np.ndarray:
    return tables_u16.view(np.float16).astype(np.float64)


def _q_weights(N, K, seed, kind="normal"):
    g = np.random.default_rng(seed)
    if kind == "normal":
        w = g.standard_normal((N, K)) * 0.02
        w[g.random((N, K)) < 0.02] *= 8.0                  # outliers, as in the workloads
    elif kind == "positive":
        w = 0.01 + np.abs(g.standard_normal((N, K))) * 0.02  # normal FP16 range only
    else:
        raise ValueError(kind)
    return w.astype(np.float16)


def test_quantize_sse_never_increases_and_tables_sorted(ora):
    w = _q_weights(32, 256, 1)
    packed, tables, sse = ora.quantize(w, with_sse=True)
    assert np.all(np.diff(sse) <= 0.0), "a Lloyd round never raises the squared error"
    assert sse[-1] < sse[0]
    tv = _q_values(tables)
    assert np.all(np.diff(tv, axis=1) >= 0), "tables ascending"
    assert np.all(np.isfinite(tv))


def test_quantize_indices_are_nearest_entries(ora):
    w = _q_weights(48, 128, 2)
    packed, tables = ora.quantize(w)
    idx = ora.unpack(packed, 128).astype(np.int64)
    tv = _q_values(tables)
    wv = w.astype(np.float64)
    for g in range(3):
        d = np.abs(wv[16 * g:16 * g + 16, :, None] - tv[g][None, None, :])
        best = d.min(axis=2)
        chosen = np.take_along_axis(d, idx[16 * g:16 * g + 16, :, None], axis=2)[..., 0]
        assert np.array_equal(chosen, best), "every index picks a nearest entry"
        # on a tie the lower index: no lower entry is as near
        lower_as_near = (d <= best[..., None]) & (np.arange(64)[None, None, :] < idx[16 * g:16 * g + 16, :, None])
        assert not lower_as_near.any()


def test_quantize_two_values_and_constant_group_are_exact(ora):
    g = np.random.default_rng(3)
    a, b = np.float16(-0.03125), np.float16(0.0478)
    w = np.where(g.random((16, 64)) < 0.3, a, b).astype(np.float16)
    c = np.full((16, 64), np.float16(0.0123), np.float16)
    w2 = np.concatenate([w, c])
    packed, tables = ora.quantize(w2)
    back = ora.dequant(packed, tables, 64).view(np.float16)
    assert np.array_equal(back.view(np.uint16), w2.view(np.uint16)), "reconstruction is exact"
    assert set(_q_values(tables)[1]) == {float(np.float16(0.0123))}


def test_quantize_scale_and_permutation(ora):
    w = _q_weights(16, 128, 4, kind="positive")
    p1, t1 = ora.quantize(w)
    # scaling by two is exact for normal FP16 values, and k-means commutes with it
    p2, t2 = ora.quantize((w.astype(np.float64) * 2).astype(np.float16))
    assert np.array_equal(p1, p2)
    assert np.array_equal(_q_values(t2), 2 * _q_values(t1))
    # the table depends on the multiset of values only; indices follow their weights
    g = np.random.default_rng(5)
    perm = g.permutation(16 * 128)
    wp = w.reshape(-1)[perm].reshape(16, 128)
    p3, t3 = ora.quantize(wp)
    assert np.array_equal(t3, t1)
    i1 = ora.unpack(p1, 128).reshape(-1)
    i3 = ora.unpack(p3, 128).reshape(-1)
    assert np.array_equal(i3, i1[perm])


def test_quantize_group_subset_and_refusals(ora):
    w = _q_weights(64, 64, 6)
    pa, ta = ora.quantize(w)
    pb, tb = ora.quantize(w, groups=(1, 3))
    assert np.array_equal(pb[16:48], pa[16:48]) and np.array_equal(tb[1:3], ta[1:3])
    bad = w.copy()
    bad.view(np.uint16)[0, 0] = 0x7C00                      # +inf
    with pytest.raises(oracle.OracleError):
        ora.quantize(bad)
    with pytest.raises(oracle.OracleError):
        ora.quantize(w[:8])                                   # N % 16

