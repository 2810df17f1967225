"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only): the library's sources are rebuilt with the sanitizers on their host
side (device code unchanged), linked with tests/host_sanitize.cpp -- every
C-ABI entry point's argument checks, the block manager on a seeded random
workload with its invariants, SHA-256 on the FIPS examples -- and run, once
with the SHA extensions and once on the portable SHA-256 path."""

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_84_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed:\n{r.stdout}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="ROCm compilers not found")
@pytest.mark.skipif(_gpu_visible(), reason="the argument checks run where no GPU is visible")
def test_host_code_under_sanitizers(tmp_path):
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["-O1", "-g", "-std=c++17", "-I", INCLUDE, "-I", CSRC]
    hip_flags = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
                 "-packed-fp32-ops"]
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=8) as pool:
        for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
            obj = str(tmp_path / (os.path.basename(src) + ".o"))
            jobs.append(pool.submit(_run, [HIPCC] + common + hip_flags + host_san +
                                    ["-c", src, "-o", obj], str(tmp_path)))
        # host-only C++ (no .hip file on these lines): clang with its sanitizers
        clang_san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
        for src, extra in ((os.path.join(CSRC, "block_manager.cpp"), []),
                           (os.path.join(ROOT, "tests", "host_sanitize.cpp"),
                            ["-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"])):
            obj = str(tmp_path / (os.path.basename(src) + ".o"))
            jobs.append(pool.submit(_run, [CLANG] + common + clang_san + extra +
                                    ["-c", src, "-o", obj], str(tmp_path)))
        for j in jobs:
            j.result()
    exe = str(tmp_path / "host_sanitize")
    objs = sorted(glob.glob(str(tmp_path / "*.o")))
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined"] + objs + ["-o", exe], str(tmp_path))
    for env in ({}, {"PKV_SHA256_PORTABLE": "1"}):
        r = subprocess.run([exe], capture_output=True, text=True,
                           env={**os.environ, **env}, timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr[-4000:]
        assert "all checks passed" in r.stdout
