"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer runs (no GPU).

Two instrumented builds, each exercised by the existing CPU tests in a child
process with its sanitizer runtime preloaded:

* the oracle and the input generator (oracle/oracle.c, synth/synth.c), built
  with gcc -fsanitize=address,undefined, under tests/test_oracle_pins.py;
* the library's argument-validation layer (csrc/api.cpp, which runs before
  any HIP call), built with the sanitizers on its host code only and linked
  with the kernels' objects of the regular build, under tests/test_abi.py and
  tests/test_binding_validation.py (no call there reaches a kernel).

Any sanitizer report ends the child with an error; the test also checks that
the child really mapped the instrumented library.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from helpers import ROOT

pytestmark = pytest.mark.slow

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CSRC = os.path.join(ROOT, "ulysses_sp_attention_amd", "csrc")
OBJ_DIR = os.path.join(ROOT, "ulysses_sp_attention_amd", "_build")
SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=0:exitcode=86",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=87",
}


def run_child(tests, env_extra, must_map):
    """Run pytest on `tests` in a child with the given environment; check that
    it passed and that it mapped `must_map`."""
    env = dict(os.environ, **SAN_ENV, **env_extra)
    probe = ("import os, runpy, sys; import pytest; "
             f"rc = pytest.main(['-x', '-q', '-p', 'no:cacheprovider', *{tests!r}]); "
             "maps = open('/proc/self/maps').read(); "
             f"sys.exit(rc if {must_map!r} in maps else 99)")
    r = subprocess.run([sys.executable, "-c", probe], cwd=os.path.join(ROOT, "tests"), env=env,
                       capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.returncode, r.stdout[-3000:], r.stderr[-3000:])


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    return tmp_path_factory.mktemp("sanitized")


def test_oracle_and_generator_under_asan_ubsan(workdir):
    libs = {}
    for name, src in (("oracle", os.path.join(ROOT, "oracle", "oracle.c")),
                      ("synth", os.path.join(ROOT, "synth", "synth.c"))):
        out = os.path.join(workdir, f"lib{name}_san.so")
        subprocess.run(["gcc", "-O1", "-g", "-fPIC", "-shared", "-fopenmp", "-std=c11",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-fno-omit-frame-pointer", src, "-o", out, "-lm"], check=True)
        libs[name] = out
    runtime = subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True,
                             capture_output=True, text=True).stdout.strip()
    run_child(["test_oracle_pins.py"],
              {"ULYSSES_ORACLE_LIB": libs["oracle"], "ULYSSES_SYNTH_LIB": libs["synth"],
               "LD_PRELOAD": runtime}, "liboracle_san.so")


def test_abi_validation_under_asan_ubsan(workdir):
    objs = sorted(glob.glob(os.path.join(OBJ_DIR, "*.o")))
    if not any(o.endswith("attn_fwd.o") for o in objs):
        from ulysses_sp_attention_amd import _build
        _build.build_lib()
        objs = sorted(glob.glob(os.path.join(OBJ_DIR, "*.o")))
    api_o = os.path.join(workdir, "api_san.o")
    # Sanitizers on the host pass only (each flag right after -Xarch_host).
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.run([HIPCC, "-O1", "-g", "-fPIC", "-std=c++17", "-I", os.path.join(ROOT, "include"),
                    "-I", CSRC, *san, "-c", os.path.join(CSRC, "api.cpp"), "-o", api_o],
                   check=True, capture_output=True)
    lib = os.path.join(workdir, "libulysses_san.so")
    kernels = [o for o in objs if not o.endswith(os.sep + "api.o")]
    subprocess.run([HIPCC, "-shared", "-fPIC", *san, "-shared-libsan", api_o, *kernels, "-o", lib],
                   check=True, capture_output=True)
    runtime = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], check=True,
                             capture_output=True, text=True).stdout.strip()
    assert os.path.exists(runtime), runtime
    run_child(["test_abi.py", "test_binding_validation.py"],
              {"ULYSSES_LIB": lib, "LD_PRELOAD": runtime}, "libulysses_san.so")
