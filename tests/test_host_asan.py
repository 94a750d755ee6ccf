"""The host code of the C ABI under AddressSanitizer.

The library sources are compiled host-only (relocatable device code mode, no device code is
generated) with the sanitizer on the host compilation and linked with small C drivers:
tests/asan/abi_host_checks.c runs every entry point's argument checks with host structs
allocated at exactly their size and must end with every status code as documented and no
sanitizer report; tests/asan/planted_overread.c hands moe_fused a parameter block one field
short and must draw the report, which shows that the library's host code is instrumented.
Device pointers in the drivers are placeholders, so this runs only where no GPU is visible."""
import os
import shlex
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_moe_expert_sort_amd", "csrc")
DRIVERS = os.path.join(ROOT, "tests", "asan")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/lib/llvm/bin/clang"
INC = ["-I", CSRC, "-I", os.path.join(ROOT, "include")]

# the sanitizer is applied to the host compilation only
HOST_ASAN = "-Xarch_host -fsanitize=address -fno-omit-frame-pointer -g -O1"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86")

pytestmark = [
    pytest.mark.skipif(torch.cuda.is_available(), reason="placeholder device pointers: CPU-only checks"),
    pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not found"),
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stderr[-3000:]


@pytest.fixture(scope="module")
def asan_objects(tmp_path_factory):
    d = tmp_path_factory.mktemp("asan")
    objs = []
    for name in sorted(os.listdir(CSRC)):
        if name.endswith(".hip"):
            obj = str(d / (name + ".o"))
            _run([HIPCC, "--cuda-host-only", "-fgpu-rdc", "-std=c++17", "-fPIC", *shlex.split(HOST_ASAN), *INC,
                  "-c", os.path.join(CSRC, name), "-o", obj])
            objs.append(obj)
    return d, objs


def _driver(asan_objects, name):
    d, objs = asan_objects
    drv = str(d / (name + ".o"))
    _run([CLANG, "-std=c11", "-fsanitize=address", "-fno-omit-frame-pointer", "-g", "-O1", *INC,
          "-c", os.path.join(DRIVERS, name + ".c"), "-o", drv])
    exe = str(d / name)
    _run([HIPCC, "--offload-arch=gfx950", "--cuda-host-only", "-fgpu-rdc", *shlex.split(HOST_ASAN), *objs, drv,
          "-o", exe])
    return subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=120)


def test_abi_host_checks_under_address_sanitizer(asan_objects):
    r = _driver(asan_objects, "abi_host_checks")
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "all passed" in r.stdout


def test_address_sanitizer_reports_a_planted_overread(asan_objects):
    r = _driver(asan_objects, "planted_overread")
    assert r.returncode == 86, r.stdout[-2000:] + r.stderr[-4000:]
    assert "heap-buffer-overflow" in r.stderr
    assert "fused_call" in r.stderr            # reported inside the library's host code
