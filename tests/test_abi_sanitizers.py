"""The C ABI's host-side validation under AddressSanitizer and UBSan (CPU only).

``sdpa_api.cpp`` holds every check the library makes before its first HIP
call.  It is compiled again here with the host sanitizers (each ``-fsanitize``
flag reaches the host compilation only, through ``-Xarch_host``; the device
code is untouched) and linked with the in-tree kernel objects into a separate
library.  Two drivers then run against that library, with the sanitizers set
to stop at the first report:

* the C program of ``test_header_c.py``, built with clang and the same
  sanitizers;
* the ctypes validation tests of ``test_abi.py``, in a Python process with the
  sanitizer runtime preloaded and the binding pointed at the sanitized library.

No GPU is needed: validation returns before any HIP call.
"""

import glob
import os
import subprocess
import sys

import pytest

from tests.test_header_c import C_PROGRAM
from transformer_attention_sdpa_amd import build_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


@pytest.fixture(scope="module")
def san_lib(tmp_path_factory):
    objs = [o for o in glob.glob(os.path.join(build_lib.BUILD, "*.o"))
            if os.path.basename(o) != "sdpa_api.o"]
    if len(objs) != len(build_lib.SOURCES) - 1 or not os.path.exists(CLANG):
        pytest.skip("the library's kernel objects are not built, or clang is missing")
    d = tmp_path_factory.mktemp("san")
    api = str(d / "sdpa_api_san.o")
    flags = [f for f in build_lib.FLAGS if f not in ("-O3",)] + ["-O1", "-g"]
    r = subprocess.run([build_lib.HIPCC, *flags, *HOST_SAN, "-c",
                        os.path.join(build_lib.CSRC, "sdpa_api.cpp"), "-o", api],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    lib = str(d / "libsdpa_san.so")
    r = subprocess.run([build_lib.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", api, *objs,
                        "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return d, lib


def test_c_program_under_sanitizers(san_lib):
    d, lib = san_lib
    src = d / "abi.c"
    src.write_text(C_PROGRAM)
    exe = str(d / "abi_san")
    r = subprocess.run([CLANG, "-std=c99", "-g", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", f"-I{os.path.join(ROOT, 'include')}", str(src),
                        lib, f"-Wl,-rpath,{d}", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120,
                         env={**os.environ, **SAN_ENV})
    assert run.returncode == 0 and "c abi ok" in run.stdout, run.stdout + run.stderr


DRIVER = r"""
import sys
import pytest
from transformer_attention_sdpa_amd import _lib
_lib.LIB_PATH = sys.argv[1]
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu",
                      "-k", "validation or exported or constants or version or workspace_size",
                      sys.argv[2]]))
"""


def test_ctypes_validation_under_sanitizers(san_lib):
    d, lib = san_lib
    rt = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True).stdout.strip()
    if not os.path.exists(rt):
        pytest.skip("no shared AddressSanitizer runtime")
    run = subprocess.run([sys.executable, "-c", DRIVER, lib, os.path.join(ROOT, "tests", "test_abi.py")],
                         capture_output=True, text=True, timeout=600, cwd=ROOT,
                         env={**os.environ, **SAN_ENV, "LD_PRELOAD": rt})
    tail = (run.stdout + run.stderr)[-4000:]
    assert run.returncode == 0, tail
    assert "passed" in run.stdout and "Sanitizer" not in run.stdout + run.stderr, tail
