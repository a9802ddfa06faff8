"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's host format code (lut6_format.cpp: pack, unpack, sizes,
status names) and the whole CPU oracle (oracle/lut6_oracle.c) are built with
gcc/g++ -fsanitize=address,undefined and driven by tests/sanitize/driver.c,
which allocates every buffer at its exact size.  A control build reads one
byte past a buffer and must be reported, so a silently disabled sanitizer
cannot pass.  CPU only; no device code is involved.
"""
from __future__ import annotations

import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
DRIVER = ROOT / "tests" / "sanitize" / "driver.c"
ORACLE_C = ROOT / "oracle" / "lut6_oracle.c"
FORMAT_CPP = ROOT / "lut_weight_quantized_amd" / "csrc" / "lut6_format.cpp"
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _build(tmp: Path, control: bool) -> Path:
    if not shutil.which("gcc") or not shutil.which("g++"):
        pytest.skip("gcc/g++ not available")
    objs = []
    for src, cc, std, extra in ((ORACLE_C, "gcc", "-std=c99", ["-ffp-contract=off", "-pthread"]),
                                (DRIVER, "gcc", "-std=c99", ["-DSANITIZE_CONTROL"] if control else []),
                                (FORMAT_CPP, "g++", "-std=c++17",
                                 ["-D__HIP_PLATFORM_AMD__", f"-I{ROOT / 'include'}", "-I/opt/rocm/include"])):
        obj = tmp / (src.stem + ".o")
        subprocess.run([cc, std, *SAN, *extra, "-c", str(src), "-o", str(obj)], check=True)
        objs.append(str(obj))
    exe = tmp / ("driver_control" if control else "driver")
    subprocess.run(["g++", *SAN, "-pthread", *objs, "-lm", "-o", str(exe)], check=True)
    return exe


def test_host_code_is_clean_under_sanitizers(tmp_path):
    exe = _build(tmp_path, control=False)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "sanitize driver ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr


def test_sanitizer_reports_a_planted_overflow(tmp_path):
    exe = _build(tmp_path, control=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr
