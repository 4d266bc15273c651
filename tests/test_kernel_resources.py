"""Register budget of the d = 256 streaming kernels (CPU only: a compile).

The d = 256 quantize and dequantize kernels hold half a vector per lane (two
lanes per vector), which must fit the registers of two waves per SIMD with
nothing spilled to scratch memory.  Every d = 256 quantize / dequantize
translation unit is compiled for gfx950 with the compiler's resource-usage
report, and every kernel instance in it must report no spill and two waves per SIMD.
(The paired SRFT organisation keeps one lane per vector at d = 256 and is
not covered.)"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_quantization_srft_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# rotation selectors: 0 SRFT (real-input), 2 SRHT, 3 none; 1, the paired SRFT
# organisation, keeps the one-lane kernel at d = 256 and is not checked here
UNITS = [f"k_{part}_d256_r{r}" for part in ("quantize", "dequantize") for r in (0, 2, 3)]


def _report(unit, out_dir):
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "--cuda-device-only", "-c", os.path.join(CSRC, unit + ".hip"), "-o", os.path.join(out_dir, unit + ".o"),
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=1200)
    assert r.returncode == 0, r.stderr[-2000:]
    rows, cur = [], None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            rows.append(cur)
            continue
        m = re.search(r"remark:\s+(ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|VGPRs Spill): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1)] = int(m.group(2))
    return unit, rows


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("python3") is None, reason="needs hipcc")
def test_d256_streaming_kernels_do_not_spill(tmp_path):
    with ThreadPoolExecutor(max_workers=min(len(UNITS), os.cpu_count() or 4)) as ex:
        reports = list(ex.map(lambda u: _report(u, str(tmp_path)), UNITS))
    checked = 0
    for unit, rows in reports:
        kernels = [r for r in rows if "quantize" in r["name"]]
        assert kernels, unit
        for r in kernels:
            assert r.get("ScratchSize [bytes/lane]", 0) == 0, (unit, r)
            assert r.get("VGPRs Spill", 0) == 0, (unit, r)
            assert r.get("Occupancy [waves/SIMD]", 0) >= 2, (unit, r)
            checked += 1
    assert checked >= 6 * 24
