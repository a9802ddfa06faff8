"""HBM bytes per LUT-6 GEMM launch from hardware counters.

    python -m lut_weight_quantized_amd.hbm_traffic

Runs ``bench.py --traffic-run`` (one launch of every GEMM of one Gated
DeltaNet layer and one full-attention layer of the L = 16,384 prefill sweep,
then a 256 MiB device copy) three times under ``rocprofv3 --pmc``: for
FETCH_SIZE, for WRITE_SIZE (both in KiB per dispatch) and for
GRBM_GUI_ACTIVE.  The copy moves a known number of bytes, so the counter it
reads gives the factor that turns counter units into bytes.  Per kernel
class (the same classes bench.py uses) the result is the average HBM bytes
per launch of that class over one sweep step (24 Gated DeltaNet layers and 8
full-attention layers), and the shader clock during that class's GEMM
dispatches: GRBM_GUI_ACTIVE, which counts busy GPU cycles summed over the 8
XCDs, divided by 8 and by the dispatch's duration.

Writes gemm_hbm_traffic.json (read by bench.py from profiles/, which
reports the bytes only while the kernel source hash still matches) and
gemm_hbm_traffic_prefill_sweep_l16384.md into the raw-output folder (OUT)
and, with --install, into profiles/.  ``--from-csv`` skips the runs and re-reads
the counter files of an earlier run.  This process never touches the GPU
itself; the profiled runs are child processes.
"""
from __future__ import annotations

import csv
import hashlib
import json
import shutil
import subprocess
import sys
import time
from collections import defaultdict
from pathlib import Path

ROOT = Path(__file__).resolve().parent.parent
OUT = ROOT / "gpurun_out" / "hbm_traffic"
PROFILES = ROOT / "profiles"
KERNEL_SOURCES = [ROOT / "lut_weight_quantized_amd" / "csrc" / "lut6_linear.hip"]
COPY_BYTES = 256 << 20
NUM_XCD = 8
LAYER_WEIGHTS = {0: 24, 3: 8}       # layer seen in the run -> layers of its kind per step
PASS_TIMEOUT_S = 240


def source_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(p.read_bytes())
    return h.hexdigest()


def classify(name: str) -> str | None:
    """bench.py's kernel class of a LUT-6 kernel name, None for anything else.

    "reduce" (a split-K reduction, after its GEMM) and "expand" (the weight
    expansion, before its GEMM) belong to the neighbouring GEMM's launch."""
    if "lut6_reduce_kernel" in name:
        return "reduce"
    if "lut6_expand_kernel" in name:
        return "expand"
    for kind, regime in (("lut6_expanded_gemm_kernel<", "expanded"), ("lut6_tile256_kernel<", "fused"),
                         ("lut6_stream_kernel<", "stream")):
        if kind in name:
            epi = name.split(kind, 1)[1].split(",", 1)[0].strip()
            return f"{regime}_" + {"0": "f32", "1": "f16", "2": "silu"}[epi]
    return None


def run_pass(counter: str) -> Path:
    d = OUT / counter
    if d.exists():
        shutil.rmtree(d)
    d.mkdir(parents=True)
    cmd = ["rocprofv3", "--pmc", counter, "--output-format", "csv", "-d", str(d), "-o", "run",
           "--", sys.executable, str(ROOT / "bench.py"), "--traffic-run"]
    print("[traffic]", " ".join(cmd), flush=True)
    with open(d / "log.txt", "w") as logf:
        proc = subprocess.Popen(cmd, stdout=logf, stderr=subprocess.STDOUT, cwd=ROOT)
        try:
            rc = proc.wait(timeout=PASS_TIMEOUT_S)
        except subprocess.TimeoutExpired:
            proc.kill()
            proc.wait()
            raise RuntimeError(f"{counter} pass timed out")
    found = list(d.rglob("*counter_collection.csv"))
    # rocprofv3 may end with a segmentation fault after the program finished
    # and wrote its results; the results are then whole
    if not found:
        raise RuntimeError(f"{counter} pass failed (rc={rc}); see {d / 'log.txt'}")
    print(f"[traffic] {counter} pass rc={rc}", flush=True)
    return found[0]


def per_dispatch(path: Path, counter: str) -> list[tuple[str, float]]:
    """(kernel name, counter value in KiB) per dispatch, in dispatch order."""
    vals: dict[int, float] = defaultdict(float)
    names: dict[int, str] = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        vals[d] += float(r["Counter_Value"])
        names[d] = r["Kernel_Name"]
    return [(names[d], vals[d]) for d in sorted(vals)]


def per_dispatch_clock(path: Path) -> list[tuple[str, float]]:
    """(kernel name, shader clock in GHz) per dispatch, in dispatch order,
    from a GRBM_GUI_ACTIVE pass (the counter file carries each dispatch's
    start and end in ns)."""
    cyc: dict[int, float] = defaultdict(float)
    dur: dict[int, int] = {}
    names: dict[int, str] = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != "GRBM_GUI_ACTIVE":
            continue
        d = int(r["Dispatch_Id"])
        cyc[d] += float(r["Counter_Value"])
        dur[d] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        names[d] = r["Kernel_Name"]
    return [(names[d], cyc[d] / NUM_XCD / max(dur[d], 1)) for d in sorted(cyc)]


def existing(counter: str) -> Path:
    found = list((OUT / counter).rglob("*counter_collection.csv"))
    if not found:
        raise RuntimeError(f"no {counter} counter file under {OUT / counter}")
    return found[0]


def main() -> int:
    args = set(sys.argv[1:])
    get = existing if "--from-csv" in args else run_pass
    fetch = per_dispatch(get("FETCH_SIZE"), "FETCH_SIZE")
    write = per_dispatch(get("WRITE_SIZE"), "WRITE_SIZE")
    if len(fetch) != len(write):
        raise RuntimeError("the two passes saw different dispatch lists")

    # the calibration copy is the last dispatch
    copy_name = fetch[-1][0]
    fetch_factor = COPY_BYTES / (fetch[-1][1] * 1024)
    write_factor = COPY_BYTES / (write[-1][1] * 1024)

    # LUT-6 dispatches: layer 0's launches first, then layer 3's; a GEMM, the
    # weight expansion before it and the reduction after it (if any) are
    # consecutive dispatches
    lut = [(n, f * 1024 * fetch_factor, w * 1024 * write_factor)
           for (n, f), (_, w) in zip(fetch[:-1], write[:-1]) if classify(n) is not None]
    launches = []                      # [class, bytes read, bytes written]
    pending = [0.0, 0.0]               # an expansion waiting for its GEMM
    for n, rb, wb in lut:
        c = classify(n)
        if c == "reduce":
            launches[-1][1] += rb
            launches[-1][2] += wb
        elif c == "expand":
            pending = [pending[0] + rb, pending[1] + wb]
        else:
            launches.append([c, rb + pending[0], wb + pending[1]])
            pending = [0.0, 0.0]
    if len(launches) != 8:
        raise RuntimeError(f"expected 8 GEMM launches (4 per layer), saw {len(launches)}")
    per_class: dict[str, dict] = {}
    for i, (c, rb, wb) in enumerate(launches):
        weight = LAYER_WEIGHTS[0] if i < 4 else LAYER_WEIGHTS[3]
        e = per_class.setdefault(c, {"launches_per_step": 0, "read": 0.0, "written": 0.0})
        e["launches_per_step"] += weight
        e["read"] += weight * rb
        e["written"] += weight * wb
    for e in per_class.values():
        n = e["launches_per_step"]
        e["read_bytes_per_launch"] = round(e.pop("read") / n)
        e["write_bytes_per_launch"] = round(e.pop("written") / n)
        e["hbm_bytes_per_launch"] = e["read_bytes_per_launch"] + e["write_bytes_per_launch"]
    dominant = max(per_class, key=lambda c: per_class[c]["launches_per_step"])

    # shader clock per class, over its GEMM dispatches (expansions and
    # reductions excluded), weighted like the bytes
    clock = [(n, ghz) for n, ghz in per_dispatch_clock(get("GRBM_GUI_ACTIVE"))
             if classify(n) not in (None, "reduce", "expand")]
    if len(clock) != 8:
        raise RuntimeError(f"expected 8 GEMM dispatches in the clock pass, saw {len(clock)}")
    sums: dict[str, list] = {}
    for i, (n, ghz) in enumerate(clock):
        weight = LAYER_WEIGHTS[0] if i < 4 else LAYER_WEIGHTS[3]
        acc = sums.setdefault(classify(n), [0.0, 0])
        acc[0] += weight * ghz
        acc[1] += weight
    for c, (tot, n) in sums.items():
        per_class[c]["sclk_ghz"] = round(tot / n, 3)

    cmd = "python3 -m lut_weight_quantized_amd.hbm_traffic"
    rec = {
        "kernel_source_sha256": source_sha(),
        "kernel_class": dominant,
        "hbm_bytes_per_launch": per_class[dominant]["hbm_bytes_per_launch"],
        "sclk_ghz": per_class[dominant].get("sclk_ghz"),
        "per_class": per_class,
        "calibration": {"kernel": copy_name, "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                        "fetch_factor": round(fetch_factor, 4), "write_factor": round(write_factor, 4)},
        "command": cmd,
        "counter_runs": ["rocprofv3 --pmc FETCH_SIZE -- python3 bench.py --traffic-run",
                         "rocprofv3 --pmc WRITE_SIZE -- python3 bench.py --traffic-run",
                         "rocprofv3 --pmc GRBM_GUI_ACTIVE -- python3 bench.py --traffic-run"],
        "date": time.strftime("%Y-%m-%d"),
    }
    dests = [OUT] + ([PROFILES] if "--install" in args else [])
    for d in dests:
        d.mkdir(parents=True, exist_ok=True)
        (d / "gemm_hbm_traffic.json").write_text(json.dumps(rec, indent=1) + "\n")

    lines = ["# HBM traffic and shader clock per LUT-6 GEMM launch, prefill sweep at L = 16,384", "",
             f"Command: `{cmd}` (three counter passes:",
             "`rocprofv3 --pmc FETCH_SIZE -- python3 bench.py --traffic-run`, then the same with",
             "`WRITE_SIZE` and with `GRBM_GUI_ACTIVE`).  Layers 0 and 3 weighted 24 : 8 as in one",
             "sweep step.", "",
             f"Calibration: `{copy_name[:60]}` copying {COPY_BYTES >> 20} MiB reads "
             f"{fetch[-1][1]:.0f} KiB (FETCH_SIZE) and writes {write[-1][1]:.0f} KiB (WRITE_SIZE): "
             f"factors {fetch_factor:.4f} and {write_factor:.4f} bytes per counted byte.", "",
             "Shader clock: `rocprofv3 --pmc GRBM_GUI_ACTIVE -- python3 bench.py --traffic-run`; the",
             "counter (busy cycles summed over the 8 XCDs) / 8 / each GEMM dispatch's duration.", "",
             "| class | launches/step | read MB/launch | written MB/launch | HBM MB/launch | clock GHz |",
             "|---|---|---|---|---|---|"]
    for c, e in sorted(per_class.items()):
        lines.append(f"| {c} | {e['launches_per_step']} | {e['read_bytes_per_launch'] / 1e6:.1f} | "
                     f"{e['write_bytes_per_launch'] / 1e6:.1f} | {e['hbm_bytes_per_launch'] / 1e6:.1f} | "
                     f"{e.get('sclk_ghz', float('nan')):.3f} |")
    lines += ["", "Per dispatch (KiB, raw counters):", "", "| kernel | FETCH_SIZE | WRITE_SIZE |",
              "|---|---|---|"]
    for (n, f), (_, w) in zip(fetch, write):
        lines.append(f"| {n[:70]} | {f:.0f} | {w:.0f} |")
    lines += ["", f"Kernel source sha256: {rec['kernel_source_sha256']}", ""]
    for d in dests:
        (d / "gemm_hbm_traffic_prefill_sweep_l16384.md").write_text("\n".join(lines))
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
