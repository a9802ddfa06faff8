"""Hardware counters of the LUT-6 GEMM launches: HBM bytes, shader clock and
the matrix-core (MFMA) busy share.

    python gemm_counters.py [--install] [--from-csv]

Runs ``bench.py --counter-run`` under ``rocprofv3 --pmc``, one pass per
counter group (rocprofv3 does not split counters over passes):

  1. FETCH_SIZE, 2. WRITE_SIZE (KiB per dispatch), 3. GRBM_GUI_ACTIVE,
  4. SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_F16 and GRBM_GUI_ACTIVE.

The counter run launches once every GEMM of one Gated DeltaNet layer (0)
and one full-attention layer (3) of the L = 16,384 prefill sweep, then the
L = 128 projection, the L = 512 gate|up and the L = 1,024 down projection,
then a 256 MiB device copy.  The copy moves a known number of bytes, so
what the byte counters read for it gives the factor that turns counter
units into bytes.  Per kernel class (the classes bench.py uses: path and
epilogue) the record holds, for one launch of that class (its weight
expansion and split-K reduction included for the bytes; the GEMM dispatch
alone for clock and MFMA):

  * HBM bytes read and written;
  * the shader clock: GRBM_GUI_ACTIVE (busy cycles, summed over the 8
    XCDs) / 8 over the dispatch's duration;
  * the MFMA busy share, rocprofv3's MfmaUtil: SQ_VALU_MFMA_BUSY_CYCLES
    summed over the chip over (GRBM_GUI_ACTIVE / 8 x 1,024 SIMDs);
  * the FP16 MFMA FLOPs the hardware counted: SQ_INSTS_VALU_MFMA_MOPS_F16
    x 512.

Sweep launches are weighted 24 : 8 (layers of each kind in one step).
Writes gemm_counters.json (bench.py reads it from profiles/ and reports it
only while the kernel source hash still matches) and gemm_counters.md into
the raw-output folder (OUT) and, with --install, into profiles/.
``--from-csv`` re-reads the counter files of an earlier run.  This process
never touches the GPU itself; the profiled runs are child processes.
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

ROOT = Path(__file__).resolve().parent
OUT = ROOT / "gpurun_out" / "gemm_counters"
PROFILES = ROOT / "profiles"
KERNEL_SOURCES = [ROOT / "lut_weight_quantized_amd" / "csrc" / "lut6_linear.hip"]
COPY_BYTES = 256 << 20
NUM_XCD = 8
NUM_SIMD = 256 * 4
PASS_TIMEOUT_S = 240
# the GEMM launches of the counter run, in order: (label, weight per step)
LAUNCHES = ([("sweep layer 0", 24)] * 4 + [("sweep layer 3", 8)] * 4
            + [("o_proj_l128", 1), ("mlp_gate_up_l512", 1), ("mlp_down_l1024", 1)])
PASSES = {"fetch": ["FETCH_SIZE"], "write": ["WRITE_SIZE"], "clock": ["GRBM_GUI_ACTIVE"],
          "mfma": ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F16", "GRBM_GUI_ACTIVE"]}


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


def run_pass(tag: str) -> Path:
    d = OUT / tag
    if d.exists():
        shutil.rmtree(d)
    d.mkdir(parents=True)
    cmd = ["rocprofv3", "--pmc", *PASSES[tag], "--output-format", "csv", "-d", str(d), "-o", "run",
           "--", sys.executable, str(ROOT / "bench.py"), "--counter-run"]
    print("[counters]", " ".join(cmd), flush=True)
    with open(d / "log.txt", "w") as logf:
        proc = subprocess.Popen(cmd, stdout=logf, stderr=subprocess.STDOUT, cwd=ROOT)
        try:
            rc = proc.wait(timeout=PASS_TIMEOUT_S)
        except subprocess.TimeoutExpired:
            proc.kill()
            proc.wait()
            raise RuntimeError(f"{tag} pass timed out")
    found = list(d.rglob("*counter_collection.csv"))
    # rocprofv3 may end with a segmentation fault after the program finished
    # and wrote its results; the results are then whole
    if not found:
        raise RuntimeError(f"{tag} pass failed (rc={rc}); see {d / 'log.txt'}")
    print(f"[counters] {tag} pass rc={rc}", flush=True)
    return found[0]


def per_dispatch(path: Path, counter: str, how: str = "sum") -> list[tuple[str, float]]:
    """(kernel name, counter value) per dispatch, in dispatch order: the sum
    (or the largest, how="max") over the counter's instances."""
    vals: dict[int, float] = {}
    names: dict[int, str] = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        v = float(r["Counter_Value"])
        vals[d] = (vals.get(d, 0.0) + v) if how == "sum" else max(vals.get(d, v), v)
        names[d] = r["Kernel_Name"]
    return [(names[d], vals[d]) for d in sorted(vals)]


def durations(path: Path) -> list[int]:
    """Each dispatch's duration in ns, in dispatch order."""
    dur: dict[int, int] = {}
    for r in csv.DictReader(open(path)):
        dur[int(r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return [dur[d] for d in sorted(dur)]


def per_dispatch_clock(path: Path) -> list[tuple[str, float]]:
    """(kernel name, shader clock in GHz) per dispatch, from a pass holding
    GRBM_GUI_ACTIVE (busy cycles summed over the 8 XCDs, whether reported as
    one row or one per XCD): cycles per XCD over the dispatch's duration."""
    return [(n, cyc / NUM_XCD / max(ns, 1))
            for (n, cyc), ns in zip(per_dispatch(path, "GRBM_GUI_ACTIVE"), durations(path))]


MAX_SCLK_GHZ = 2.4    # the MI355X's highest shader clock


def clock_or_none(ghz: float) -> float | None:
    """The clock estimate, or None where it exceeds the chip's highest clock:
    for a dispatch shorter than rocprofv3's counter window, GRBM_GUI_ACTIVE
    also counts busy cycles outside the dispatch, so neither the clock nor
    the MFMA busy share (whose denominator it is) means anything."""
    return ghz if ghz <= MAX_SCLK_GHZ * 1.01 else None


def existing(tag: str) -> Path:
    found = list((OUT / tag).rglob("*counter_collection.csv"))
    if not found:
        raise RuntimeError(f"no {tag} counter file under {OUT / tag}")
    return found[0]


def group_launches(names: list[str]) -> list[list[int]]:
    """Dispatch indices of each GEMM launch: its expansion, the GEMM, its
    reduction; dispatches of other kernels are left out."""
    launches, pending = [], []
    for i, n in enumerate(names):
        c = classify(n)
        if c is None:
            continue
        if c == "reduce":
            launches[-1].append(i)
        elif c == "expand":
            pending.append(i)
        else:
            launches.append(pending + [i])
            pending = []
    return launches


def fmt(x: float | None) -> str:
    return "—" if x is None else f"{x:.3f}"


def main() -> int:
    args = set(sys.argv[1:])
    get = existing if "--from-csv" in args else run_pass
    fetch = per_dispatch(get("fetch"), "FETCH_SIZE")
    write = per_dispatch(get("write"), "WRITE_SIZE")
    clock = per_dispatch_clock(get("clock"))
    mpath = get("mfma")
    busy = per_dispatch(mpath, "SQ_VALU_MFMA_BUSY_CYCLES")
    mops = per_dispatch(mpath, "SQ_INSTS_VALU_MFMA_MOPS_F16")
    gui = per_dispatch(mpath, "GRBM_GUI_ACTIVE")          # summed over the 8 XCDs
    names = [n for n, _ in fetch]
    for other in (write, clock, busy, mops, gui):
        if [n for n, _ in other] != names:
            raise RuntimeError("the passes saw different dispatch lists")

    # the calibration copy is the last dispatch
    copy_name = names[-1]
    fetch_factor = COPY_BYTES / (fetch[-1][1] * 1024)
    write_factor = COPY_BYTES / (write[-1][1] * 1024)

    launches = group_launches(names)
    if len(launches) != len(LAUNCHES):
        raise RuntimeError(f"expected {len(LAUNCHES)} GEMM launches, saw {len(launches)}")
    per_class: dict[str, dict] = {}
    for (label, weight), idx in zip(LAUNCHES, launches):
        gemm = [i for i in idx if classify(names[i]) not in ("reduce", "expand")][0]
        c = classify(names[gemm])
        e = per_class.setdefault(c, {"launches_per_step": 0, "workload": label, "_w": 0, "read": 0.0,
                                     "written": 0.0, "clock": 0.0, "busy": 0.0, "flops": 0.0, "window": True})
        e["launches_per_step"] += weight if label.startswith("sweep") else 0
        e["_w"] += weight
        e["read"] += weight * sum(fetch[i][1] for i in idx) * 1024 * fetch_factor
        e["written"] += weight * sum(write[i][1] for i in idx) * 1024 * write_factor
        e["clock"] += weight * clock[gemm][1]
        e["window"] = e["window"] and clock_or_none(clock[gemm][1]) is not None
        e["busy"] += weight * busy[gemm][1] / (gui[gemm][1] / NUM_XCD * NUM_SIMD)
        e["flops"] += weight * mops[gemm][1] * 512
    for e in per_class.values():
        w = e.pop("_w")
        e["read_bytes_per_launch"] = round(e.pop("read") / w)
        e["write_bytes_per_launch"] = round(e.pop("written") / w)
        e["hbm_bytes_per_launch"] = e["read_bytes_per_launch"] + e["write_bytes_per_launch"]
        ok = e.pop("window")
        e["sclk_ghz"] = round(e.pop("clock") / w, 3) if ok else None
        e["mfma_busy_frac"] = round(e.pop("busy") / w, 4) if ok else None
        if not ok:
            e["note"] = "dispatch shorter than the counter window: no clock or MFMA busy share"
        e["mfma_f16_flops_per_launch"] = round(e.pop("flops") / w)
    sweep = {c: e for c, e in per_class.items() if e["launches_per_step"]}
    dominant = max(sweep, key=lambda c: sweep[c]["launches_per_step"])

    cmd = "python3 gemm_counters.py --install"
    runs = [f"rocprofv3 --pmc {' '.join(v)} -- python3 bench.py --counter-run" for v in PASSES.values()]
    rec = {
        "kernel_source_sha256": source_sha(),
        "kernel_class": dominant,
        "hbm_bytes_per_launch": per_class[dominant]["hbm_bytes_per_launch"],
        "sclk_ghz": per_class[dominant]["sclk_ghz"],
        "mfma_busy_frac": per_class[dominant]["mfma_busy_frac"],
        "per_class": per_class,
        "calibration": {"kernel": copy_name, "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                        "fetch_factor": round(fetch_factor, 4), "write_factor": round(write_factor, 4)},
        "command": cmd,
        "counter_runs": runs,
        "date": time.strftime("%Y-%m-%d"),
    }
    dests = [OUT] + ([PROFILES] if "--install" in args else [])
    for d in dests:
        d.mkdir(parents=True, exist_ok=True)
        (d / "gemm_counters.json").write_text(json.dumps(rec, indent=1) + "\n")

    lines = ["# LUT-6 GEMM launches: HBM bytes, shader clock and MFMA busy share (rocprofv3 counters)", "",
             f"Command: `{cmd}`, four counter passes of `python3 bench.py --counter-run` (one launch of",
             "every GEMM of sweep layers 0 and 3 at L = 16,384, then the L = 128, 512 and 1,024",
             "workloads, then a 256 MiB copy):", ""]
    lines += [f"- `{r}`" for r in runs]
    lines += ["", f"Calibration: `{copy_name[:60]}` copying {COPY_BYTES >> 20} MiB reads "
              f"{fetch[-1][1]:.0f} KiB (FETCH_SIZE) and writes {write[-1][1]:.0f} KiB (WRITE_SIZE): "
              f"factors {fetch_factor:.4f} and {write_factor:.4f} bytes per counted byte.", "",
              "Clock: GRBM_GUI_ACTIVE (summed over the 8 XCDs) / 8 over the GEMM dispatch's duration.",
              "MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES (all SIMDs) / (GRBM_GUI_ACTIVE / 8 x 1,024 SIMDs), rocprofv3's",
              "MfmaUtil.  MFMA FLOPs: SQ_INSTS_VALU_MFMA_MOPS_F16 x 512.  Sweep classes are weighted",
              "24 : 8 as in one step.", "",
              "| class | workload | launches/step | read MB | written MB | HBM MB | clock GHz | MFMA busy | MFMA GFLOP |",
              "|---|---|---|---|---|---|---|---|---|"]
    for c, e in sorted(per_class.items()):
        lines.append(f"| {c} | {e['workload']} | {e['launches_per_step']} | {e['read_bytes_per_launch'] / 1e6:.1f} | "
                     f"{e['write_bytes_per_launch'] / 1e6:.1f} | {e['hbm_bytes_per_launch'] / 1e6:.1f} | "
                     f"{fmt(e['sclk_ghz'])} | {fmt(e['mfma_busy_frac'])} | "
                     f"{e['mfma_f16_flops_per_launch'] / 1e9:.1f} |")
    lines += ["", "Per dispatch (raw counters; bytes in KiB, cycles as counted):", "",
              "| kernel | FETCH_SIZE | WRITE_SIZE | clock GHz | MFMA busy cycles | MOPS_F16 |",
              "|---|---|---|---|---|---|"]
    for i, n in enumerate(names):
        lines.append(f"| {n[:70]} | {fetch[i][1]:.0f} | {write[i][1]:.0f} | {fmt(clock_or_none(clock[i][1]))} | "
                     f"{busy[i][1]:.0f} | {mops[i][1]:.0f} |")
    lines += ["", "A dash: the estimate exceeded the chip's 2.4 GHz, because the dispatch is shorter than the",
              "counter window (GRBM_GUI_ACTIVE then also counts cycles outside it); its MFMA busy share is",
              "not given either.", "", f"Kernel source sha256: {rec['kernel_source_sha256']}", ""]
    for d in dests:
        (d / "gemm_counters.md").write_text("\n".join(lines))
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
