"""ThreadSanitizer run of the host FFN thread pool (the host branch's
resident pool): two threads submit jobs to one pool at once, as a
synchronous decode call and a HIP host callback can, then one thread submits
jobs after idle gaps on both sides of the workers' polling window; no data
race may be reported and every result must equal the job run alone.  Host code only,
compiled here with g++ (no GPU code is involved)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "expert_ffn_execution_router_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_pool_is_race_free_under_tsan(tmp_path):
    exe = str(tmp_path / "host_pool_stress")
    cmd = ["g++", "-std=c++20", "-O1", "-g", "-fsanitize=thread", "-march=x86-64-v3", "-pthread", "-I" + CSRC,
           os.path.join(ROOT, "tests", "host_pool_stress.cpp"), os.path.join(CSRC, "host_ffn.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 exitcode=66")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert "ThreadSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr[-2000:])
