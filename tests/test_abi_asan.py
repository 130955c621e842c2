"""The C ABI's host-side validation layer under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only: the device code is not
instrumented). api.cpp is compiled with the sanitizers on its host pass,
linked with the library's other objects and a C driver that calls every
entry point with arguments it must refuse before any launch
(tests/asan/abi_driver.c). No GPU is needed: nothing is enqueued."""
import os
import shutil
import subprocess

import pytest

from long_context_prefill_attn_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.timeout(300)
def test_abi_validation_under_sanitizers(tmp_path):
    if not (os.path.exists(B.HIPCC) and shutil.which("gcc") and shutil.which("g++")):
        pytest.skip("hipcc and gcc are needed for the sanitizer build")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
    objs = []
    for src in B.SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        extra = san if src == "api.cpp" else []
        r = subprocess.run([B.HIPCC, *B.FLAGS, *extra, "-x", "hip", "-c", os.path.join(B.CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    drv = str(tmp_path / "abi_driver.o")
    r = subprocess.run(["gcc", "-std=c99", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                        "-I", os.path.join(ROOT, "include"), "-c", os.path.join(HERE, "asan", "abi_driver.c"),
                        "-o", drv], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "abi_driver")
    r = subprocess.run(["g++", "-fsanitize=address,undefined", drv, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                        "-Wl,-rpath,/opt/rocm/lib", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "0 failures" in r.stdout
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
