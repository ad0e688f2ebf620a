"""The CPU test tier against AddressSanitizer + UndefinedBehaviorSanitizer
builds (CPU only, no GPU):

* the oracle (oracle.c) built with -fsanitize=address,undefined;
* libmoe's host code (the C ABI's validation, planning and argument checks in
  api.cpp, the profiler) built the same way and linked with the unchanged
  device objects of the regular build.

Each is loaded in a fresh Python process (ASan's runtime preloaded, any
sanitizer report fatal) through ORACLE_LIBRARY_PATH / MOE_LIBRARY_PATH, and
the oracle pins, the oracle backward and the ABI tests run against them.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparsely_gated_mixture_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


pytestmark = pytest.mark.skipif(
    shutil.which("gcc") is None or shutil.which("g++") is None or _runtime("libasan.so") is None
    or not os.path.isdir("/opt/rocm/include"),
    reason="needs gcc/g++ with the sanitizer runtimes and the ROCm headers")


def _sh(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}{r.stderr[-3000:]}"


@pytest.fixture(scope="module")
def san_env(tmp_path_factory):
    out = tmp_path_factory.mktemp("san")
    ora = str(out / "liboracle_san.so")
    _sh(["gcc"] + SAN + ["-fPIC", "-shared", "-fopenmp", "-std=c11", "-o", ora,
                         os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    dev = sorted(os.path.join(BUILD, f) for f in os.listdir(BUILD) if f.endswith(".hip.o")) \
        if os.path.isdir(BUILD) else []
    if not dev:
        pytest.skip("the regular build's device objects (_build/*.hip.o) are missing")
    host = []
    for src in ("api.cpp", "profile.cpp"):
        obj = str(out / (src + ".o"))
        _sh(["g++"] + SAN + ["-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I",
                             "/opt/rocm/include", "-I", CSRC, "-I", os.path.join(ROOT, "include"),
                             "-c", os.path.join(CSRC, src), "-o", obj])
        host.append(obj)
    moe = str(out / "libmoe_san.so")
    _sh(["g++", "-shared", "-fsanitize=address,undefined", "-o", moe] + dev + host +
        ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    env = dict(os.environ)
    env.update(LD_PRELOAD=_runtime("libasan.so"), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", ORACLE_LIBRARY_PATH=ora,
               MOE_LIBRARY_PATH=moe, PYTHONPATH=ROOT + os.pathsep + env.get("PYTHONPATH", ""))
    return env, ora, moe


def test_sanitized_builds_are_the_ones_loaded(san_env):
    env, ora, moe = san_env
    code = ("import oracle, sparsely_gated_mixture_amd as m; oracle.lib(); m.load_library(); "
            "print(open('/proc/self/maps').read())")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       cwd=ROOT, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert ora in r.stdout and moe in r.stdout
    assert "libasan" in r.stdout


def test_cpu_tier_under_sanitizers(san_env):
    env, _, _ = san_env
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", "tests/test_oracle_pins.py", "tests/test_oracle_backward.py",
                        "tests/test_abi.py"], env=env, capture_output=True, text=True, cwd=ROOT,
                       timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail
