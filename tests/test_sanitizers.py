"""CPU runs under AddressSanitizer and UndefinedBehaviorSanitizer:

* the oracle (plain C) built with -fsanitize=address,undefined, driven through
  routing and the forward pass in every mode, and every codec entry point
  (tests/sanitize/oracle_driver.c);
* the library's host code (argument checks, workspace sizing and layout,
  error strings) built with the sanitizers on its host pass only, driven with
  arguments that every entry point refuses before touching a device
  (tests/sanitize/abi_driver.c).

No GPU is used; a sanitizer finding aborts the driver and fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1")


def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_driver"
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-ffp-contract=off", os.path.join(HERE, "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", str(exe), "-lm"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=dict(ENV, ASAN_OPTIONS="detect_leaks=1"),
                       timeout=600)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs hipcc and ROCm clang")
def test_library_host_code_under_sanitizers(tmp_path):
    src = os.path.join(ROOT, "skew_aware_grouped_amd", "csrc")
    inc = os.path.join(ROOT, "include")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Xclang",
             "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", inc, "-I", src,
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all"]
    procs, objs = [], []
    from skew_aware_grouped_amd import build
    for name in build.SOURCES:
        obj = str(tmp_path / name.replace(".hip", ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, *flags, "-c", os.path.join(src, name), "-o", obj],
                                      stdout=subprocess.DEVNULL, stderr=subprocess.PIPE, text=True))
    for p in procs:
        _, err = p.communicate(timeout=900)
        assert p.returncode == 0, err[-2000:]
    lib = str(tmp_path / "libmoe_asan.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", *objs, "-o", lib], check=True,
                   stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    exe = str(tmp_path / "abi_driver")
    subprocess.run([CLANG, "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-I", inc,
                    os.path.join(HERE, "abi_driver.c"), lib, f"-Wl,-rpath,{tmp_path}", "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr
