"""CPU-only AddressSanitizer / UndefinedBehaviorSanitizer runs: the oracle
(oracle/moe_oracle.c, gcc) and the host code of the HIP library (argument
validation, sizes and workspace layouts of every C-ABI entry point; hipcc
with the sanitizers on the host side only) are rebuilt with ASan and UBSan
into a temporary directory, and the tests that exercise them without a GPU
-- the oracle's pins and the ABI checks -- run against those builds in a
child process that preloads the matching sanitizer runtime.  Any report
(out-of-bounds access, use after free, signed overflow, misaligned or null
dereference, ...) fails the child and so this test.  No GPU is used: the ABI
tests only reach the host-side checks."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _runtime(cmd):
    out = subprocess.run(cmd, capture_output=True, text=True).stdout.strip()
    return out if out and os.path.isabs(out) and os.path.exists(out) else None


def _child(tests, env_extra, timeout=600):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", *tests, "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    assert r.returncode == 0, (r.stdout[-4000:] + r.stderr[-4000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, r.stderr[-4000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    asan = _runtime(["gcc", "-print-file-name=libasan.so"])
    if asan is None:
        pytest.skip("gcc's ASan runtime not found")
    lib = tmp_path / "libmoe_oracle_san.so"
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", str(lib), "-lm"])
    _child(["tests/test_oracle_pins.py", "tests/test_oracle_bwd_pins.py"],
           {"LD_PRELOAD": asan, "MOE_ORACLE_LIB": str(lib)})


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_library_host_code_under_asan_ubsan(tmp_path):
    asan = _runtime([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"])
    if asan is None:
        pytest.skip("clang's ASan runtime not found")
    src = os.path.join(ROOT, "mixture_experts_layer_topkrouter_amd", "csrc")
    hips = sorted(f for f in os.listdir(src) if f.endswith(".hip"))
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Wno-unused-function",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-I", os.path.join(ROOT, "include")]

    def compile_one(f):
        obj = tmp_path / (f + ".o")
        r = subprocess.run([HIPCC, *flags, "-c", os.path.join(src, f), "-o", str(obj)], capture_output=True,
                           text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return str(obj)

    with ThreadPoolExecutor(max_workers=min(8, len(hips))) as ex:
        objs = list(ex.map(compile_one, hips))
    lib = tmp_path / "libmoe_san.so"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", str(lib)])
    _child(["tests/test_abi.py"], {"LD_PRELOAD": asan, "MOE_HIP_LIB": str(lib)})
