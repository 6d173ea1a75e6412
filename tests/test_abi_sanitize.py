"""The C ABI's argument validation under host AddressSanitizer and
UndefinedBehaviorSanitizer.

Builds every library source with the sanitizers on host code only (device code
is compiled as usual and never runs: there is no GPU here, so every call stops
at its argument checks or at the device check) together with
tests/abi_sanitize_driver.cpp, a sweep of null, misaligned, out-of-range and
extreme arguments over every entry point, and runs it.  Any out-of-bounds
access, signed overflow or other undefined behaviour in the validation aborts
the run."""

import os
import shutil
import subprocess
import tempfile

import pytest

from nested_int_matmul_amd import build as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "abi_sanitize_driver.cpp")

# sanitizers on the host side of each translation unit only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def sanitized_binary():
    try:
        cc = b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    tmp = tempfile.mkdtemp(prefix="mq_san_")
    flags = [f for f in b.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"] + HOST_SAN
    objs, procs = [], []
    for src in b.SOURCES:
        o = os.path.join(tmp, src + ".o")
        objs.append(o)
        procs.append(subprocess.Popen([cc, *flags, "-c", os.path.join(b.CSRC, src), "-o", o],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    drv = os.path.join(tmp, "driver.o")
    procs.append(subprocess.Popen([cc, *flags, "-x", "hip", "-c", DRIVER, "-o", drv],
                                  stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out[-4000:]
    exe = os.path.join(tmp, "abi_sweep")
    subprocess.run([cc, "--offload-arch=gfx950", *HOST_SAN, *objs, drv, "-o", exe], check=True)
    yield exe
    shutil.rmtree(tmp, ignore_errors=True)


def test_abi_validation_under_asan_and_ubsan(sanitized_binary):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="")
    p = subprocess.run([sanitized_binary], env=env, capture_output=True, text=True, timeout=300)
    out = p.stdout + p.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert p.returncode == 0, out[-4000:]
    assert "0 unexpected" in out
