"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The ClikaRT "conv_transpose" API page (Throws) makes every inconsistent argument an error
the caller sees; here the library's host code (attribute resolver, stride-phase planner,
dispatcher, argument validation of every entry point) and the fp64 oracle are rebuilt
with ASan + UBSan and run through the same host-only checks as the normal builds:

* the library's host tests (test_library_host.py: every exported symbol, the resolver
  against the oracle's on 3000 random attribute sets, validation that launches nothing,
  dispatcher choices, the no-allocation entry point's size check) with a host-sanitized
  libconvtranspose.so (device code is unchanged; nothing is launched);
* every oracle pin (test_oracle_pins.py) with a sanitized oracle.

Each runs in a child process with the sanitizer runtime preloaded; any sanitizer report
fails the test (UBSan reports are fatal, leaks are not checked: the HIP runtime and
PyTorch keep allocations for the process's lifetime).
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transposed_convolution_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# host-side sanitizers only: each -fsanitize= goes to the host compilation
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer", "SUMMARY: UndefinedBehavior")


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _gcc_runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p) else None


def _run_child(env_extra, args):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] + args,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    found = [s for s in REPORTS if s in out]
    assert r.returncode == 0 and not found, f"sanitized run failed ({found}):\n{out[-6000:]}"
    return out


@pytest.fixture(scope="module")
def sanitized_library():
    if not os.path.exists(HIPCC) or not _clang_asan_runtime():
        pytest.skip("hipcc or its AddressSanitizer runtime is not available")
    os.makedirs(OUT, exist_ok=True)
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-w"] + HOST_SAN
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))

    def compile_one(src):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        r = subprocess.run([HIPCC] + flags + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, f"hipcc failed on {src}:\n{r.stderr[-3000:]}"
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = os.path.join(OUT, "libconvtranspose_san.so")
    r = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950"] + HOST_SAN + ["-o", lib] + objs,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return lib


@pytest.fixture(scope="module")
def sanitized_oracle():
    asan = _gcc_runtime("libasan.so")
    if not shutil.which("gcc") or not asan:
        pytest.skip("gcc's AddressSanitizer runtime is not available")
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "libctoracle_san.so")
    r = subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-shared", "-fPIC", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                        os.path.join(ROOT, "oracle", "ct_oracle.c"), "-o", lib, "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return lib, asan


def test_library_host_code_under_sanitizers(sanitized_library):
    out = _run_child({"LD_PRELOAD": _clang_asan_runtime(), "CT_LIBRARY_PATH": sanitized_library},
                     ["tests/test_library_host.py"])
    assert " passed" in out


def test_oracle_pins_under_sanitizers(sanitized_oracle):
    lib, asan = sanitized_oracle
    out = _run_child({"LD_PRELOAD": asan, "CT_ORACLE_LIB": lib}, ["tests/test_oracle_pins.py"])
    assert " passed" in out
