"""Benchmark of the LUT-6 dequant-GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of every LUT-6 linear layer of a 32-layer hybrid prefill
at L = 16,384 tokens (page "Clef-Flash-ANE-LUT6", section "Model
architecture": 24 Gated DeltaNet layers with qkv|z, out, gate|up and down
projections, 8 full-attention layers with q|k|v, o, gate|up and down; hidden
4,096, MLP 12,288), 128 launches of lut6_linear over seeded synthetic weights
(per-layer seeds) and activations that are resident in HBM before timing
starts.  The line printed is throughput in TFLOP/s, with

  * roofline: the dominant launch class's algorithmic FLOPs per lut6_linear
    call over the call's average time (HIP events around the call on its
    stream, so for the many-token path the weight expansion and the GEMM
    together), against the FP16 dense MFMA peak (2,516.6 TFLOP/s); its HBM
    traffic, the shader clock and the MFMA busy share during it come from the
    rocprofv3 counter record in profiles/ (gemm_counters.py) when that record
    was taken on the current kernel source, else null;
  * l128_stream: the L = 128 single projection (4,096 -> 4,096, FP32 out) in
    algorithmic HBM GB/s over back-to-back launches, rotating over enough
    weight sets that the 256 MB last-level cache cannot hold them;
  * per_config: the other workloads (L = 512 gate|up, L = 1,024 down, one
    L = 4,096 block's projections as three launches and as six), each timed
    over back-to-back launches that rotate through enough buffer copies (at
    least 512 MB) that the last-level cache cannot hold them: TFLOP/s and
    algorithmic GB/s against the FP16 peak and HBM bandwidth; and, labelled
    warm, the same passes on one buffer set;
  * quantize: lut6_quantize (table fitting by 1-D k-means) on a 4,096 x 4,096
    and a 4,096 x 12,288 seeded FP16 weight: time per call, weights per
    second and algorithmic GB/s, with the oracle on one 16-row group beside;
  * int8_variant: the int8 weight-only variant (int8 codes, one FP16 scale
    per 32 k) beside LUT-6 on the same shapes (L = 128 and 4,096);
  * attention: the attention layers' full attention (FP16, probabilities
    x 16) at L = Lk = 16,384 and 4,096, and a 128-query chunk over 16,384
    keys, in TFLOP/s against the FP16 peak;
  * gated_delta: one linear-attention layer's Gated DeltaNet recurrence
    (32 value heads, FP32 state) over 4,096 and 16,384 tokens;
  * int8_quantize: lut6_int8_quantize (int8 codes per block of 32) on the
    24,576 x 4,096 gate|up weight and a 4,096 x 4,096 one, in algorithmic
    GB/s against HBM;
  * cpu_baseline: the CPU oracle timed on a bounded sample of the same step
    (64 sampled token rows of every GEMM of all 32 layers), on this host's
    cores;
  * parity_sample: those sampled rows of the GPU result against the oracle.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "LUT-6 GEMM TFLOP/s + % FP16 MFMA peak at L>=1024; HBM GB/s at L=128"
PEAK_FP16_TFLOPS = 2516.6          # 256 CUs x 2.4 GHz x 4,096 FLOP/clk (dense FP16 MFMA)
PEAK_HBM_GBS = 8000.0              # HBM3E
STEP_WORKLOAD = "prefill_sweep_l16384"
STREAM_WORKLOAD = "o_proj_l128"
OTHER_WORKLOADS = ("mlp_gate_up_l512", "mlp_down_l1024", "hybrid_block_l4096", "hybrid_block_l4096_six")
ROTATE_BYTES = 512 << 20           # at least twice the 256 MB last-level cache
COUNTER_FILE = ROOT / "profiles" / "gemm_counters.json"
KERNEL_SOURCES = [ROOT / "lut_weight_quantized_amd" / "csrc" / "lut6_linear.hip"]
COUNTER_LAYERS = (0, 3)            # one Gated DeltaNet and one full-attention layer
COUNTER_WORKLOADS = ("o_proj_l128", "mlp_gate_up_l512", "mlp_down_l1024")
COPY_BYTES = 256 << 20             # calibration copy for the HBM byte counters


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(p.read_bytes())
    return h.hexdigest()


def kernel_class(g) -> str:
    """Which kernels lut6_linear launches for this GEMM (path and epilogue)."""
    import lut_weight_quantized_amd as lq
    regime = {lq.PATH_STREAM: "stream", lq.PATH_FUSED: "fused",
              lq.PATH_EXPANDED: "expanded"}[lq.linear_path(g.L, g.K, g.N, g.epilogue)]
    epi = {0: "f32", 1: "f16", 2: "silu"}[g.epilogue]
    return f"{regime}_{epi}"


# the kernels one lut6_linear call of each path runs (for the roofline record)
PATH_KERNELS = {"stream": ["lut6_stream_kernel", "lut6_reduce_kernel (only when K is split)"],
                "fused": ["lut6_tile256_kernel"],
                "expanded": ["lut6_expand_kernel", "lut6_expanded_gemm_kernel"]}


def cpu_threads() -> int:
    """Threads for the CPU oracle: every core this process may run on, or
    OMP_NUM_THREADS if that is lower (a shared host's CPU share)."""
    env = os.environ.get("OMP_NUM_THREADS")
    n = len(os.sched_getaffinity(0))
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, n)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_workload(lq, si, torch, stream, name: str, launches: int = 20) -> dict:
    """Median time of one pass over a workload's GEMMs (one launch each),
    over back-to-back passes that rotate through copies of every buffer
    (at least ROTATE_BYTES in all), so each launch reads from HBM."""
    w = si.WORKLOADS[name]
    gemms = [g for _, _, g in w.gemms()]
    per_set = sum(g.bytes for g in gemms)
    sets = max(2, -(-ROTATE_BYTES // per_set))
    base = []
    for li, pi, g in w.gemms():
        idx, tab = si.gemm_weight(w.cfg, li, pi, g)
        base.append((torch.from_numpy(lq.pack(idx)).to("cuda"), torch.from_numpy(tab).to("cuda"),
                     torch.from_numpy(si.gemm_activation(w.cfg, g)).to("cuda")))
        del idx
    bufs = []
    for _ in range(sets):
        bufs.append([(p.clone(), t.clone(), x.clone(),
                      torch.empty((g.L, g.n_out), device="cuda",
                                  dtype=torch.float32 if g.epilogue == 0 else torch.float16))
                     for (p, t, x), g in zip(base, gemms)])
    del base

    def one_pass(i):
        for (p, t, x, y), g in zip(bufs[i % sets], gemms):
            lq.linear(x, p, t, epilogue=g.epilogue, in_scale=g.in_scale, out=y, stream=stream)

    for i in range(2 * sets):
        one_pass(i)
    torch.cuda.synchronize()
    reps = []
    for r in range(3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(launches):
            one_pass(i)
        e1.record(stream)
        torch.cuda.synchronize()
        reps.append(e0.elapsed_time(e1) * 1e3 / launches)
    us = sorted(reps)[1]
    # warm: the same buffer set every pass (resident in the last-level cache)
    warm = []
    for r in range(3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(launches):
            one_pass(0)
        e1.record(stream)
        torch.cuda.synchronize()
        warm.append(e0.elapsed_time(e1) * 1e3 / launches)
    us_warm = sorted(warm)[1]
    del bufs
    torch.cuda.empty_cache()
    tf = w.flops / (us * 1e-6) / 1e12
    gbs = w.bytes / (us * 1e-6) / 1e9
    tf_warm = w.flops / (us_warm * 1e-6) / 1e12
    return {"workload": name, "gemms": [f"{g.name} L={g.L} K={g.K} N={g.N}" for g in gemms],
            "paths": [{lq.PATH_STREAM: "stream", lq.PATH_FUSED: "fused", lq.PATH_EXPANDED: "expanded"}[
                lq.linear_path(g.L, g.K, g.N, g.epilogue)] for g in gemms],
            "us_per_pass": round(us, 2), "tflop_s": round(tf, 1),
            "frac_fp16_peak": round(tf / PEAK_FP16_TFLOPS, 4), "gb_s": round(gbs, 1),
            "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "flops": w.flops, "algorithmic_bytes": w.bytes,
            "buffer_sets_rotated": sets, "warm_us_per_pass": round(us_warm, 2),
            "warm_tflop_s": round(tf_warm, 1), "warm_frac_fp16_peak": round(tf_warm / PEAK_FP16_TFLOPS, 4)}


QUANT_SHAPES = (("o_proj", 4096, 4096), ("down", 4096, 12288))


def time_quantize(lq, si, torch, stream, no_cpu: bool) -> list:
    """lut6_quantize (table fitting) on two seeded weights: median of 3 runs
    of 5 back-to-back calls; algorithmic bytes = the FP16 weight read once
    plus the packed indices and tables written.  Beside it, the oracle on
    one 16-row group, scaled to the whole weight."""
    out = []
    for name, N, K in QUANT_SHAPES:
        w16 = si.weights(N, K, (9, 0, K))
        w = torch.from_numpy(w16).to("cuda")
        packed = torch.empty((N, K // 4 * 3), dtype=torch.uint8, device="cuda")
        tables = torch.empty((N // 16, 64), dtype=torch.float16, device="cuda")
        for _ in range(2):
            lq.quantize(w, packed=packed, tables=tables, stream=stream)
        torch.cuda.synchronize()
        reps = []
        for r in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(5):
                lq.quantize(w, packed=packed, tables=tables, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            reps.append(e0.elapsed_time(e1) * 1e3 / 5)
        us = sorted(reps)[1]
        nbytes = N * K * 2 + N * K // 4 * 3 + N // 16 * 128
        rec = {"weight": f"{name} N={N} K={K}", "us_per_call": round(us, 1),
               "gweights_per_s": round(N * K / (us * 1e-6) / 1e9, 2),
               "gb_s": round(nbytes / (us * 1e-6) / 1e9, 1),
               "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
               "algorithmic_bytes": nbytes, "groups": N // 16}
        if not no_cpu:
            import oracle
            ora = oracle.load()
            t0 = time.perf_counter()
            ora.quantize(w16, groups=(0, 1))
            cpu_s = time.perf_counter() - t0
            rec["cpu_oracle"] = {"s_per_group": round(cpu_s, 3), "cores": 1, "kind": "oracle",
                                 "us_per_call_scaled": round(cpu_s * (N // 16) * 1e6, 0),
                                 "sample": "one 16-row group, single thread, scaled to all groups"}
        out.append(rec)
        del w, packed, tables
    torch.cuda.empty_cache()
    return out


INT8_SHAPES = (("o_proj", 128, 4096, 4096), ("o_proj", 4096, 4096, 4096), ("down", 4096, 12288, 4096))


INT8_QUANT_SHAPES = (("gate|up", 24576, 4096), ("o_proj", 4096, 4096))


def time_int8_quantize(lq, si, torch, stream) -> list:
    """lut6_int8_quantize (int8 codes and scales per block of 32) on seeded
    FP16 weights: median of 3 runs of 5 back-to-back calls; algorithmic
    bytes = the weight read once, the codes and the scales written.  The
    gate|up weight (201 MB read, 101 MB written) exceeds the last-level
    cache, so its rate is HBM's."""
    out = []
    for name, N, K in INT8_QUANT_SHAPES:
        w = torch.from_numpy(si.weights(N, K, (16, N, K))).to("cuda")
        q = torch.empty((N, K), dtype=torch.int8, device="cuda")
        sc = torch.empty((N, K // 32), dtype=torch.float16, device="cuda")
        us = _median_us(lambda: lq.int8_quantize(w, q=q, scales=sc, stream=stream), torch, stream)
        nbytes = N * K * 2 + N * K + N * (K // 32) * 2
        out.append({"weight": f"{name} N={N} K={K}", "us_per_call": round(us, 1),
                    "gb_s": round(nbytes / (us * 1e-6) / 1e9, 1),
                    "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                    "algorithmic_bytes": nbytes})
        del w, q, sc
    torch.cuda.empty_cache()
    return out


def _median_us(fn, torch, stream, calls: int = 5) -> float:
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    reps = []
    for _ in range(3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(calls):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        reps.append(e0.elapsed_time(e1) * 1e3 / calls)
    return sorted(reps)[1]


def time_int8(lq, si, torch, stream) -> list:
    """The int8 weight-only variant (int8 codes, one FP16 scale per 32 k)
    beside LUT-6 on the same shapes, FP16 output: median of 3 runs of 5
    back-to-back calls each.  The int8 path expands the weight and runs the
    FP16 GEMM at every token count."""
    out = []
    for name, L, K, N in INT8_SHAPES:
        x = torch.from_numpy(si.activations(L, K, 1.0, (13, 0, K))).to("cuda")
        q8, s8 = si.int8_weight(N, K, (13, 1, K))
        q = torch.from_numpy(q8).to("cuda")
        sc = torch.from_numpy(s8).to("cuda")
        packed = torch.from_numpy(lq.pack(si.indices(N, K, (13, 2, K)))).to("cuda")
        tab = torch.from_numpy(si.tables(N, (13, 2, K))).to("cuda")
        y = torch.empty((L, N), dtype=torch.float16, device="cuda")
        us8 = _median_us(lambda: lq.int8_linear(x, q, sc, epilogue=lq.EPI_STORE_F16, out=y, stream=stream),
                         torch, stream)
        us6 = _median_us(lambda: lq.linear(x, packed, tab, epilogue=lq.EPI_STORE_F16, out=y, stream=stream),
                         torch, stream)
        flops = 2.0 * L * K * N
        b8 = L * K * 2 + N * K + N * (K // 32) * 2 + L * N * 2
        b6 = L * K * 2 + N * K // 4 * 3 + N // 16 * 128 + L * N * 2
        out.append({"gemm": f"{name} L={L} K={K} N={N} f16", "int8_us_per_call": round(us8, 2),
                    "lut6_us_per_call": round(us6, 2), "int8_over_lut6_time": round(us8 / us6, 3),
                    "int8_tflop_s": round(flops / (us8 * 1e-6) / 1e12, 1),
                    "lut6_tflop_s": round(flops / (us6 * 1e-6) / 1e12, 1),
                    "int8_algorithmic_bytes": b8, "lut6_algorithmic_bytes": b6,
                    "int8_frac_hbm": round(b8 / (us8 * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                    "lut6_frac_hbm": round(b6 / (us6 * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)})
        del x, q, sc, packed, tab, y
    torch.cuda.empty_cache()
    return out


ATT_SHAPES = ((16384, 16384), (4096, 4096), (128, 16384))


def time_attention(lq, torch, stream) -> list:
    """Full attention of one attention layer (16 query, 4 key-value heads of
    256; causal, the L queries the last L of Lk positions), reading q, k, v
    in place from one fused [L, 6144] projection output: median of 3 runs
    of 5 back-to-back calls.  FLOPs = 4 * 256 * 16 * (visible keys summed
    over the queries)."""
    out = []
    g = torch.Generator(device="cuda").manual_seed(2026)
    for L, Lk in ATT_SHAPES:
        qkv = torch.randn((Lk, 6144), generator=g, device="cuda", dtype=torch.float32).to(torch.float16)
        q = qkv[Lk - L:, :4096]
        k, v = qkv[:, 4096:5120], qkv[:, 5120:]
        o = torch.empty((L, 4096), dtype=torch.float16, device="cuda")
        us = _median_us(lambda: lq.attention(q, k, v, n_heads=16, n_kv_heads=4, out=o, stream=stream),
                        torch, stream)
        visible = L * (Lk - L) + L * (L + 1) // 2
        flops = 4.0 * 256 * 16 * visible
        tf = flops / (us * 1e-6) / 1e12
        out.append({"shape": f"L={L} Lk={Lk} heads 16/4 x 256", "us_per_call": round(us, 1),
                    "tflop_s": round(tf, 1), "frac_fp16_peak": round(tf / PEAK_FP16_TFLOPS, 4),
                    "flops": flops})
        del qkv, o
    torch.cuda.empty_cache()
    return out


GDN_LENGTHS = (4096, 16384)


def time_gated_delta(lq, torch, stream) -> list:
    """Gated DeltaNet recurrence of one linear-attention layer (16 key and
    32 value heads of 128, state [32, 128, 128] FP32), q|k|v read in place
    from one fused [L, 8192] projection output: median of 3 runs of 5
    back-to-back calls.  FLOPs per token and value head: 7 * 128 * 128
    (decay, S^T k, the rank-one update, S^T q)."""
    out = []
    g = torch.Generator(device="cuda").manual_seed(2027)
    for L in GDN_LENGTHS:
        qkv = (torch.randn((L, 8192), generator=g, device="cuda", dtype=torch.float32) / 11.3).to(torch.float16)
        gl = -torch.rand((L, 32), generator=g, device="cuda", dtype=torch.float32) * 0.5
        be = torch.rand((L, 32), generator=g, device="cuda", dtype=torch.float32)
        st = torch.zeros((32, 128, 128), dtype=torch.float32, device="cuda")
        o = torch.empty((L, 4096), dtype=torch.float16, device="cuda")
        q, k, v = qkv[:, :2048], qkv[:, 2048:4096], qkv[:, 4096:]
        us = _median_us(lambda: lq.gated_delta(q, k, v, gl, be, st, n_k_heads=16, n_v_heads=32, out=o,
                                               stream=stream), torch, stream)
        flops = 7.0 * 128 * 128 * 32 * L
        out.append({"shape": f"L={L} heads 16/32 x 128", "us_per_call": round(us, 1),
                    "tokens_per_s": round(L / (us * 1e-6), 0),
                    "gflop_s": round(flops / (us * 1e-6) / 1e9, 1), "flops": flops,
                    "note": "chunked form (64 positions) on the matrix cores"})
        del qkv, gl, be, st, o
    torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--cpu-rows", type=int, default=64,
                    help="sampled token rows per GEMM (every GEMM of every layer) in the "
                         "parity sample and the CPU-oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stream-iters", type=int, default=200)
    ap.add_argument("--counter-run", action="store_true",
                    help="launch the GEMMs of sweep layers 0 and 3 once each, then the L = 128, 512 "
                         "and 1,024 workloads, then a 256 MiB copy, and exit (the workload "
                         "gemm_counters.py runs under rocprofv3 --pmc)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run it with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    import lut_weight_quantized_amd as lq
    import seeded_inputs as si

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    lq.load_library()
    stream = torch.cuda.current_stream()

    w = si.WORKLOADS[STEP_WORKLOAD]
    L = w.layers[0][0].L

    # ---------------- inputs, resident in HBM ----------------
    t0 = time.time()
    acts, acts_host = {}, {}
    for _, _, g in w.gemms():
        key = (g.K, g.x_tensor)
        if key not in acts:
            acts_host[key] = si.gemm_activation(w.cfg, g)
            acts[key] = torch.from_numpy(acts_host[key]).to("cuda")
    weights = []
    for li, layer in enumerate(w.layers):
        lw = []
        for pi, g in enumerate(layer):
            idx, tab = si.gemm_weight(w.cfg, li, pi, g)
            lw.append((torch.from_numpy(lq.pack(idx)).to("cuda"), torch.from_numpy(tab).to("cuda")))
            del idx
        weights.append(lw)
        if li % 8 == 7:
            log(f"weights for layers 0..{li} resident ({time.time() - t0:.1f} s)")
    outs = {}
    for _, pi, g in w.gemms():
        key = (g.name, g.n_out)
        if key not in outs:
            outs[key] = torch.empty((g.L, g.n_out), dtype=torch.float16, device="cuda")
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s")

    plan = [(li, pi, g, acts[(g.K, g.x_tensor)], weights[li][pi], outs[(g.name, g.n_out)])
            for li, pi, g in w.gemms()]

    if args.counter_run:
        # one launch per GEMM of layers 0 (Gated DeltaNet) and 3 (full attention),
        # in that order, then one of each smaller workload, then the calibration
        # copy: 256 MiB read, 256 MiB written
        for li, pi, g, x, (p, t), y in plan:
            if li in COUNTER_LAYERS:
                lq.linear(x, p, t, epilogue=g.epilogue, in_scale=g.in_scale, out=y, stream=stream)
        for name in COUNTER_WORKLOADS:
            cw = si.WORKLOADS[name]
            for li, pi, g in cw.gemms():
                idx, tab = si.gemm_weight(cw.cfg, li, pi, g)
                xs = torch.from_numpy(si.gemm_activation(cw.cfg, g)).to("cuda")
                ys = torch.empty((g.L, g.n_out), device="cuda",
                                 dtype=torch.float32 if g.epilogue == 0 else torch.float16)
                pw, tw = torch.from_numpy(lq.pack(idx)).to("cuda"), torch.from_numpy(tab).to("cuda")
                torch.cuda.synchronize()
                lq.linear(xs, pw, tw, epilogue=g.epilogue, in_scale=g.in_scale, out=ys, stream=stream)
                torch.cuda.synchronize()
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("counter run done")
        return 0

    def step(events=None):
        for li, pi, g, x, (p, t), y in plan:
            if events is not None:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            lq.linear(x, p, t, epilogue=g.epilogue, in_scale=g.in_scale, out=y, stream=stream)
            if events is not None:
                e1.record(stream)
                events.append((g, e0, e1))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = []
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step(events)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    ms_per_step = t_total * 1e3 / args.steps

    # per kernel class: launches, total time, algorithmic FLOPs
    per = {}
    for g, e0, e1 in events:
        c = per.setdefault(kernel_class(g), {"n": 0, "ms": 0.0, "flops": 0, "bytes": 0})
        c["n"] += 1
        c["ms"] += e0.elapsed_time(e1)
        c["flops"] += g.flops
        c["bytes"] += g.bytes
    dom_name = max(per, key=lambda k: per[k]["ms"])
    dom = per[dom_name]
    avg_ms = dom["ms"] / dom["n"]
    flops_per_launch = dom["flops"] / dom["n"]
    achieved = flops_per_launch / (avg_ms * 1e-3) / 1e12
    kernels_ms = sum(c["ms"] for c in per.values()) / args.steps
    value = w.flops / (ms_per_step * 1e-3) / 1e12
    log(f"step {ms_per_step:.3f} ms, kernels {kernels_ms:.3f} ms, {value:.1f} TFLOP/s; "
        + ", ".join(f"{k}: {v['n'] // args.steps}/step {v['ms'] / v['n'] * 1e3:.1f} us avg "
                    f"{v['flops'] / v['n'] / (v['ms'] / v['n'] * 1e-3) / 1e12:.1f} TFLOP/s"
                    for k, v in sorted(per.items())))

    # counter record (gemm_counters.py), only while taken on this kernel source
    counters = {}
    if COUNTER_FILE.exists():
        rec = json.loads(COUNTER_FILE.read_text())
        if rec.get("kernel_source_sha256") == kernel_source_sha():
            counters = rec.get("per_class", {})
    dom_c = counters.get(dom_name, {})
    traffic = dom_c.get("hbm_bytes_per_launch")
    sclk = dom_c.get("sclk_ghz")

    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
                "traffic": traffic, "kernel": dom_name,
                "kernels_per_launch": PATH_KERNELS[dom_name.split("_")[0]],
                "avg_launch_us": round(avg_ms * 1e3, 2),
                "flops_per_launch": flops_per_launch, "launches_per_step": dom["n"] // args.steps,
                "timing": "HIP events around each lut6_linear call on its stream (all its kernels)"}
    if sclk:
        # the board runs below its 2.4 GHz peak clock under this load: the
        # fraction of the dense peak at the clock the counter pass measured
        roofline["sclk_ghz"] = sclk
        roofline["frac_at_sclk"] = round(achieved / (PEAK_FP16_TFLOPS * sclk / 2.4), 4)
    if dom_c:
        roofline["mfma_busy_frac"] = dom_c.get("mfma_busy_frac")
        roofline["mfma_f16_flops_per_launch_counted"] = dom_c.get("mfma_f16_flops_per_launch")
        roofline["counters"] = "profiles/gemm_counters.json (rocprofv3 --pmc, this kernel source)"

    # ---------------- parity sample + CPU baseline (oracle) ----------------
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        from oracle import tolerance as tol
        ora = oracle.load()
        threads = cpu_threads()
        cpu_s, cpu_flops, worst, n_checked, all_ok, n_gemms = 0.0, 0, 0.0, 0, True, 0
        for li, pi, g, xd, (p, t), _ in plan:
            # each GEMM once more into a fresh output, its sampled rows
            # gathered on the device, against the oracle on the same rows
            x = acts_host[(g.K, g.x_tensor)]
            idx, tab = si.gemm_weight(w.cfg, li, pi, g)
            rows = si.sample_rows(g.L, args.cpu_rows, (w.cfg, li, pi))
            y = torch.empty((g.L, g.n_out), dtype=torch.float16, device="cuda")
            lq.linear(xd, p, t, epilogue=g.epilogue, in_scale=g.in_scale, out=y, stream=stream)
            yd = y[torch.from_numpy(rows).to("cuda")].cpu().numpy().view(np.uint16)
            del y
            packed = ora.pack(idx)
            del idx
            tc = time.perf_counter()
            ye, _ = ora.linear(x, packed, tab, epilogue=g.epilogue, in_scale=g.in_scale,
                               rows=rows, threads=threads)
            cpu_s += time.perf_counter() - tc
            cpu_flops += 2 * len(rows) * g.K * g.N
            S = tol.row_scale(x, tab, g.K, rows)
            if g.epilogue == si.EPI_SILU_MUL_F16:
                a, _ = ora.linear(x, packed, tab, epilogue=si.EPI_F32, in_scale=g.in_scale,
                                  rows=rows, threads=threads)
                rep = tol.check(yd, ye, S, fp16=True,
                                S_elem=tol.silu_scale(a[:, :g.N // 2], a[:, g.N // 2:], S))
            else:
                rep = tol.check(yd, ye, S, fp16=True)
            all_ok &= rep.ok
            worst = max(worst, rep.max_err_over_bound)
            n_checked += rep.n
            n_gemms += 1
            if not rep.ok or pi == 0:
                log(f"layer {li} {g.name}: {rep}")
        cpu_value = cpu_flops / cpu_s / 1e12
        cpu = {"value": round(cpu_value, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
               "sample": (f"{args.cpu_rows} sampled token rows (rows 0 and L-1 among them) of each of "
                          f"the {n_gemms} GEMMs of all {len(w.layers)} layers "
                          f"({cpu_flops / 1e9:.1f} GFLOP in {cpu_s:.1f} s, FP64 oracle, "
                          f"{threads} threads: this process's CPU affinity, capped by OMP_NUM_THREADS "
                          f"when set; {cpu_model()})")}
        parity = {"ok": bool(all_ok), "outputs_checked": n_checked, "gemms": n_gemms,
                  "layers": len(w.layers), "rows_per_gemm": args.cpu_rows,
                  "max_err_over_bound": round(worst, 4)}

    # ---------------- L = 128 weight-streaming projection ----------------
    sw = si.WORKLOADS[STREAM_WORKLOAD]
    sg = sw.layers[0][0]
    sets = 40      # 40 x 15.8 MB working sets > 256 MB last-level cache
    x128 = torch.from_numpy(si.gemm_activation(sw.cfg, sg)).to("cuda")
    sets_w = []
    for i in range(sets):
        idx, tab = si.gemm_weight(sw.cfg, i, 0, sg)
        sets_w.append((torch.from_numpy(lq.pack(idx)).to("cuda"), torch.from_numpy(tab).to("cuda"),
                       x128.clone(), torch.empty((sg.L, sg.N), dtype=torch.float32, device="cuda")))
    for i in range(2 * sets):
        p, t, x, y = sets_w[i % sets]
        lq.linear(x, p, t, epilogue=sg.epilogue, out=y, stream=stream)
    torch.cuda.synchronize()
    # back-to-back launches between one event pair: the per-launch time
    # includes every kernel of a call and the gaps between calls, and none
    # of the host's launch latency
    reps = []
    for r in range(3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.stream_iters):
            p, t, x, y = sets_w[i % sets]
            lq.linear(x, p, t, epilogue=sg.epilogue, out=y, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        reps.append(e0.elapsed_time(e1) * 1e3 / args.stream_iters)
    us_med = sorted(reps)[1]
    gbs = sg.bytes / (us_med * 1e-6) / 1e9
    stream_rec = {"workload": STREAM_WORKLOAD, "us_per_launch": round(us_med, 2),
                  "gb_s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                  "tflop_s": round(sg.flops / (us_med * 1e-6) / 1e12, 1),
                  "algorithmic_bytes": sg.bytes, "weight_sets_rotated": sets,
                  "note": (f"median of 3 runs of {args.stream_iters} back-to-back launches; "
                           "spans each call's kernels and the gaps between calls")}
    sc = counters.get(kernel_class(sg), {})
    if sc:
        stream_rec.update(traffic=sc.get("hbm_bytes_per_launch"), mfma_busy_frac=sc.get("mfma_busy_frac"),
                          sclk_ghz=sc.get("sclk_ghz"))
    log(f"L=128 stream: {us_med:.2f} us, {gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS:.1%} of HBM)")
    del sets_w

    # ---------------- the other workloads ----------------
    quant = time_quantize(lq, si, torch, stream, args.no_cpu_baseline)
    i8q = time_int8_quantize(lq, si, torch, stream)
    int8 = time_int8(lq, si, torch, stream)
    att = time_attention(lq, torch, stream)
    gdn = time_gated_delta(lq, torch, stream)

    per_config = []
    for name in OTHER_WORKLOADS:
        rec = time_workload(lq, si, torch, stream, name)
        if name in COUNTER_WORKLOADS:
            gc = counters.get(kernel_class(si.WORKLOADS[name].layers[0][0]), {})
            if gc:
                rec.update(traffic=gc.get("hbm_bytes_per_launch"), mfma_busy_frac=gc.get("mfma_busy_frac"),
                           sclk_ghz=gc.get("sclk_ghz"))
        per_config.append(rec)
        log(f"{name}: {rec['us_per_pass']:.1f} us, {rec['tflop_s']:.0f} TFLOP/s "
            f"({rec['frac_fp16_peak']:.1%} of FP16 peak)")

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": STEP_WORKLOAD, "L": L, "layers": len(w.layers),
                   "launches_per_step": len(plan), "flops_per_step": w.flops,
                   "algorithmic_bytes_per_step": w.bytes,
                   "frac_fp16_peak": round(value / PEAK_FP16_TFLOPS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "l128_stream": stream_rec,
        "per_config": per_config,
        "quantize": quant,
        "int8_variant": int8,
        "attention": att,
        "gated_delta": gdn,
        "int8_quantize": i8q,
        "parity_sample": parity,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
