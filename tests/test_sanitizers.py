"""AddressSanitizer / UndefinedBehaviorSanitizer builds of the host code
(CPU only, no GPU involved):

* the oracle (oracle/mxq_oracle.c), driven by tests/sanitize/oracle_asan.c
  over small and edge-case shapes of every entry point and its rejected
  inputs;
* the library's C-ABI layer and the MXFP4 unit's host code, driven by
  tests/sanitize/api_asan.cpp: every entry point with arguments its checks
  must reject, and well-formed ones that must stop at the device gate.

Any sanitizer report fails the run (-fno-sanitize-recover)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-Wno-unknown-pragmas", os.path.join(ROOT, "oracle", "mxq_oracle.c"),
         os.path.join(ROOT, "tests", "sanitize", "oracle_asan.c"), "-o", exe, "-lm"])
    r = run([exe])
    assert r.stdout.strip() == "ok"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_abi_validation_under_asan_ubsan(tmp_path):
    objs = []
    common = ["--offload-arch=gfx950", "-std=c++17", "-g", "-O1", *SAN_HOST]
    for src in ("mxq_api.hip", "qdq_mxfp4.hip"):
        obj = str(tmp_path / (src + ".o"))
        run([HIPCC, *common, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-c",
             os.path.join(ROOT, "moe_grouped_gemm_mxq_amd", "csrc", src), "-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "api_drv.o")
    run([HIPCC, *common, "-x", "hip", "-c", os.path.join(ROOT, "tests", "sanitize", "api_asan.cpp"), "-o", drv])
    exe = str(tmp_path / "api_asan")
    run([HIPCC, "--offload-arch=gfx950", "-fsanitize=address,undefined", *objs, drv, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", HIP_VISIBLE_DEVICES="")
    r = run([exe], env=env)
    assert r.stdout.strip() == "ok"
