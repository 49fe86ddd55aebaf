"""The native host code (block manager, metadata builders) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer, driven by tests/c_abi_host.c (host
entry points only, including a long allocate / append / release stress).  CPU only:
no GPU code is built here."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_319_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="needs gcc/g++")
def test_host_code_under_asan_ubsan(tmp_path):
    inc = f"-I{os.path.join(ROOT, 'include')}"
    objs = []
    for src in ("block_manager.cpp", "prepare.cpp"):
        obj = tmp_path / (src + ".o")
        res = subprocess.run(["g++", "-std=c++17", "-O1", "-g", *SAN, inc, "-c",
                              os.path.join(CSRC, src), "-o", str(obj)],
                             capture_output=True, text=True)
        assert res.returncode == 0, res.stderr
        objs.append(str(obj))
    drv = tmp_path / "driver.o"
    res = subprocess.run(["gcc", "-std=c99", "-O1", "-g", "-DNV_HOST_ONLY", *SAN, inc, "-c",
                          os.path.join(ROOT, "tests", "c_abi_host.c"), "-o", str(drv)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    exe = tmp_path / "host_san"
    res = subprocess.run(["g++", *SAN, str(drv), *objs, "-o", str(exe)],
                         capture_output=True, text=True)
    if res.returncode != 0 and "asan" in res.stderr.lower():
        pytest.skip("sanitizer runtime not installed")
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.strip() == "c abi ok"
