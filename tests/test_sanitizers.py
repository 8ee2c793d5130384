"""AddressSanitizer and UndefinedBehaviorSanitizer runs of the host code (CPU only).

* The C-ABI layer (``csrc/api.cpp``) is built for the host with the kernel
  launches replaced by stand-ins (``tests/sanitize/launch_stubs.cpp``) that
  read and write every byte the kernels of each launch would, and a driver
  (``tests/sanitize/abi_driver.cpp``) calls every entry point with buffers of
  exactly the sizes the header states. A workspace sized or carved wrongly, a
  pointer offset past its buffer or undefined behaviour in the host
  arithmetic aborts the run.
* The C oracle (``oracle/deltanet_oracle.c``) is built with the same
  sanitizers and the oracle's own test module runs against that build.

Each run has a planted-mistake twin that must fail, so the sanitizers are
known to be watching: a workspace formula one block short in a copy of
``api.cpp``, and a read one element past a state row in a copy of the oracle.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunkwise_delta_rule_amd", "csrc")
SAN_DIR = os.path.join(ROOT, "tests", "sanitize")
ORACLE_SRC = os.path.join(ROOT, "oracle", "deltanet_oracle.c")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0", "UBSAN_OPTIONS": "print_stacktrace=1"}

needs_clang = pytest.mark.skipif(not os.path.exists(CLANGXX), reason="ROCm clang++ not found")


def build_abi_driver(out_dir, api_src):
    exe = os.path.join(out_dir, "abi_driver")
    cmd = [CLANGXX, "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, api_src,
           os.path.join(SAN_DIR, "launch_stubs.cpp"), os.path.join(SAN_DIR, "abi_driver.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def run(cmd, extra_env=None, timeout=600):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(extra_env or {})
    return subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout, cwd=ROOT)


@needs_clang
def test_host_abi_under_sanitizers(tmp_path):
    exe = build_abi_driver(str(tmp_path), os.path.join(CSRC, "api.cpp"))
    r = run([exe])
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert " 0 failures" in r.stdout
    print(r.stdout.splitlines()[-1])


@needs_clang
def test_host_abi_sanitizer_catches_a_short_workspace(tmp_path):
    src = open(os.path.join(CSRC, "api.cpp")).read()
    good = "((size_t)dk * dk + 2 * (size_t)dv * dk) * sizeof(float)"
    assert good in src
    bad_src = tmp_path / "api_short.cpp"
    # one state block short: the carved ws_S region runs past the caller's buffer
    bad_src.write_text(src.replace(good, "((size_t)dk * dk + (size_t)dv * dk) * sizeof(float)", 1)
                       .replace('#include "../../include/deltanet.h"', '#include "deltanet.h"'))
    exe = build_abi_driver(str(tmp_path), str(bad_src))
    r = run([exe])
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stdout[-1000:]


def build_oracle(out, src):
    cmd = ["gcc", "-std=c99", "-fopenmp", "-fPIC", "-shared", *SAN, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


def libasan():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(libasan() is None, reason="gcc's libasan not found")
def test_oracle_under_sanitizers(tmp_path):
    lib = build_oracle(str(tmp_path / "liboracle_san.so"), ORACLE_SRC)
    env = {"LD_PRELOAD": libasan(), "DELTANET_ORACLE_LIB": lib}
    # the sanitized build is the one the oracle module loads
    probe = run([sys.executable, "-c", "import oracle; print(oracle.load()._name)"], env)
    assert probe.returncode == 0 and probe.stdout.strip() == lib, probe.stderr[-2000:]
    r = run([sys.executable, "-m", "pytest", "tests/test_oracle.py", "-q", "-x", "-p", "no:cacheprovider"], env,
            timeout=1200)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    print(r.stdout.strip().splitlines()[-1])


@pytest.mark.skipif(libasan() is None, reason="gcc's libasan not found")
def test_oracle_sanitizer_catches_an_overrun(tmp_path):
    src = open(ORACLE_SRC).read()
    good = "for (int j = 0; j < dk; ++j) acc += Si[j] * kt[j];"
    assert good in src
    bad = tmp_path / "oracle_overrun.c"
    bad.write_text(src.replace(good, "for (int j = 0; j <= dk; ++j) acc += Si[j] * kt[j];", 1))
    lib = build_oracle(str(tmp_path / "liboracle_bad.so"), str(bad))
    code = ("import numpy as np, oracle\n"
            "r = np.random.default_rng(0)\n"
            "x = lambda *s: r.standard_normal(s)\n"
            "oracle.deltanet_fwd(x(1, 5, 1, 8), x(1, 5, 1, 8), x(1, 5, 1, 8), x(1, 5, 1))\n")
    r = run([sys.executable, "-c", code], {"LD_PRELOAD": libasan(), "DELTANET_ORACLE_LIB": lib})
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-2000:]
