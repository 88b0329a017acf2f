"""Host code of the library under the host compiler's address and
undefined-behaviour sanitizers (CPU only: the sanitizers instrument host
code, and nothing here launches a kernel)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dynamic_kv_cache_amd", "csrc")


def test_host_entry_points_under_asan_ubsan(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
    if hipcc is None:
        pytest.skip("hipcc not found")
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    exe = str(tmp_path / "host_checks")
    objs = [str(tmp_path / f) for f in ("checks.o", "api.o", "kernels.o")]
    hip_common = [hipcc, "-O1", "-g", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
                  "-packed-fp32-ops", "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    steps = [
        # the C driver: host code only
        [cc, "-std=c99", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-I", os.path.join(ROOT, "include"), "-c", os.path.join(ROOT, "tests", "c_abi", "host_checks.c"),
         "-o", objs[0]],
        # the library: sanitizers on its host code, none on device code
        hip_common + san + ["-c", os.path.join(CSRC, "fastocr_api.cpp"), "-o", objs[1]],
        hip_common + san + ["-c", os.path.join(CSRC, "kernels.hip"), "-o", objs[2]],
        [hipcc, "--offload-arch=gfx950", "-Wno-unused-command-line-argument"] + san + objs + ["-o", exe],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, (" ".join(cmd), r.stderr[-3000:])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "host checks ok" in r.stdout
