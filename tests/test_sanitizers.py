"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds of the same sources, made here in _build/sanitize/:
  * the fp64 oracle (oracle/titans_oracle.c) with gcc -fsanitize=address,undefined;
  * the HIP library with the sanitizers on its host code only (the C ABI's validation,
    workspace sizing and dispatch); its gfx950 device code is compiled as usual and never
    runs here.
Each is then loaded by the existing tests in a child process with the matching
sanitizer runtime preloaded (gcc's for the oracle, clang's for the library): the oracle
pins and planted-mistake tests, and every C-ABI argument test.  Any report (a memory error
or, as UBSan is built not to recover, undefined behaviour) fails the child process.
"""
import concurrent.futures
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CSRC = os.path.join(ROOT, "sequence_models_amd", "csrc")

pytestmark = pytest.mark.timeout(900)


def _have(tool):
    return subprocess.run(["bash", "-c", f"command -v {tool}"], capture_output=True).returncode == 0


def _runtime(compiler, name):
    path = subprocess.run([compiler, f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _child(env_extra, args):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True,
                          text=True)


PROBE = ("import sys; sys.path.insert(0, '.'); import {mod}; {load}; "
         "maps = open('/proc/self/maps').read(); "
         "print('sanitizer runtime mapped:', 'asan' in maps); "
         "print('library:', {path})")


@pytest.mark.skipif(not _have("gcc"), reason="gcc not available")
def test_oracle_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "liboracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "titans_oracle.c"),
                           "-o", lib, "-lm"])
    rt = _runtime("gcc", "libasan.so")
    assert rt, "gcc's libasan.so not found"
    env = {"LD_PRELOAD": rt, "TITANS_ORACLE_LIB": lib}
    probe = _child(env, ["-c", PROBE.format(mod="oracle", load="oracle._load()", path="oracle._LIB")])
    assert probe.returncode == 0, probe.stderr[-3000:]
    assert "sanitizer runtime mapped: True" in probe.stdout and lib in probe.stdout, probe.stdout
    r = _child(env, ["-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                     "tests/test_oracle_pins.py", "tests/test_oracle_mutations.py",
                     "tests/test_oracle_grad_pins.py"])
    print(r.stdout[-2000:])
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def _compile_host_sanitized(src):
    obj = os.path.join(OUT, os.path.splitext(os.path.basename(src))[0] + ".o")
    # sanitizers on the host side only (-Xarch_host before each flag); device code as usual
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address,undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libasan",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return obj


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_validation_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile_host_sanitized, srcs))
    lib = os.path.join(OUT, "libtitans_mem_san.so")
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                           "-Xarch_host", "-fsanitize=address,undefined",
                           "-Xarch_host", "-shared-libasan", *objs, "-o", lib])
    rt = _runtime(os.path.join(os.path.dirname(HIPCC), "..", "llvm", "bin", "clang"),
                  "libclang_rt.asan-x86_64.so")
    assert rt, "clang's ASan runtime not found"
    env = {"LD_PRELOAD": rt, "TITANS_MEM_LIB": lib}
    probe = _child(env, ["-c", PROBE.format(mod="sequence_models_amd", load="None",
                                            path="sequence_models_amd.LIB_PATH")])
    assert probe.returncode == 0, probe.stderr[-3000:]
    assert "sanitizer runtime mapped: True" in probe.stdout and lib in probe.stdout, probe.stdout
    r = _child(env, ["-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "tests/test_abi_cpu.py"])
    print(r.stdout[-2000:])
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr
