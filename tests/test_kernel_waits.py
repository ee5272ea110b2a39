"""The grouped-GEMM kernels fill LDS with direct global->LDS loads one or
two chunks ahead of the MFMAs that read the current chunk.  The compiler
guards an LDS read it cannot tell apart from the stage such a load is
filling with a wait for every outstanding vector-memory operation, which
also waits for the chunks in flight and turns the pipeline into load
latency plus compute (an 8-byte operand read did this in the MXFP6 and the
E2M1 small-batch paths).  Built here for gfx950 (assembly only, no GPU):
no vector-memory wait may directly precede an LDS read in these kernels."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "expert_ffn_execution_router_amd", "csrc")
SOURCES = ["gemm_pf.hip", "gemm_pf8.hip", "gemm_dec.hip", "gemv.hip"]


def _asm(src, out):
    from expert_ffn_execution_router_amd.build import HIP_FLAGS
    flags = [f for f in HIP_FLAGS if f != "-fPIC"]
    subprocess.run(["hipcc", *flags, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out], check=True,
                   capture_output=True, text=True)
    return open(out).read().splitlines()


def _waits_before_lds_reads(lines):
    bad = []
    for i, line in enumerate(lines):
        if "s_waitcnt" not in line or "vmcnt" not in line:
            continue
        j = i + 1
        while j < len(lines) and (not lines[j].strip() or lines[j].strip()[0] in ";."):
            j += 1
        if j < len(lines) and lines[j].strip().startswith("ds_read"):
            bad.append((i, line.strip(), lines[j].strip()))
    return bad


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="needs hipcc")
def test_no_wait_for_in_flight_loads_before_lds_reads(tmp_path):
    outs = [str(tmp_path / (s + ".s")) for s in SOURCES]
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        asm = list(ex.map(_asm, SOURCES, outs))
    for src, lines in zip(SOURCES, asm):
        assert sum("s_endpgm" in l for l in lines) >= 4, src      # the kernels were built
        bad = _waits_before_lds_reads(lines)
        assert not bad, (src, bad[:5])
