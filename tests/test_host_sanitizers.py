"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every library source is compiled for gfx950 with the sanitizers on the host
side only (device code is built as usual), linked with the C driver in
host_validation/driver.c, and run here without a GPU.  The driver sweeps a
seeded set of edge-valued problems through moe_validate, the workspace size
functions and every entry point's pointer, alignment and size checks; none of
its calls reaches a kernel launch.  Any sanitizer report fails the run.
"""
import concurrent.futures
import importlib.util
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _build_module():
    spec = importlib.util.spec_from_file_location("_moe_build", os.path.join(ROOT, "sparse_moe_layer_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(" ".join(cmd) + "\n" + r.stdout + r.stderr)


@pytest.mark.timeout(600)
@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not present")
def test_host_code_under_asan_and_ubsan(tmp_path):
    b = _build_module()
    # the library's own flags with -O3 traded for -O1 -g (readable reports)
    flags = [f for f in b.FLAGS if f != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer"] + SAN

    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        _run([HIPCC] + flags + lang + ["-c", os.path.join(b.CSRC, src), "-o", obj])
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, b.SOURCES))
    drv_o = str(tmp_path / "driver.o")
    # the driver is plain C11: the header must stay usable from C
    _run([CLANG, "-std=c11", "-Wall", "-Werror", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"),
          "-c", os.path.join(ROOT, "tests", "host_validation", "driver.c"), "-o", drv_o])
    exe = str(tmp_path / "driver")
    _run([HIPCC, "--offload-arch=gfx950"] + SAN + [drv_o] + objs + ["-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    assert "failures 0" in r.stdout
