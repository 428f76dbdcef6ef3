"""Address and undefined-behaviour sanitizers on the CPU side.

- Both oracles built with gcc -fsanitize=address,undefined run every pin.
- The library's host code (argument validation, planning) built with
  address and undefined-behaviour sanitizers on its host pass only runs the
  C-ABI tests (no GPU: every call there fails validation before a launch).

Each runs in a child process with the sanitizer runtime preloaded (the
Python interpreter itself is not instrumented); any report aborts it.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from oracle import build as oracle_build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run(code, preload, timeout):
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV)
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=timeout)


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's address-sanitizer runtime is not installed")
    san = ("-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all")
    rec = oracle_build.build(oracle_build.SRC, str(tmp_path / "liboracle_san.so"), extra=san)
    pre = oracle_build.build(oracle_build.PRE_SRC, str(tmp_path / "libpre_san.so"), extra=san)
    code = (
        "import sys, functools\n"
        f"sys.path[:0] = [{ROOT!r}, {HERE!r}]\n"
        "import oracle, oracle_pins\n"
        "from oracle_pre_pins import ALL_PRE_PINS\n"
        f"run = functools.partial(oracle.run, lib_path={rec!r}, threads=4)\n"
        "for p in oracle_pins.ALL_PINS: p(run)\n"
        f"for p in ALL_PRE_PINS: p({pre!r})\n"
        "print('PINS_OK', len(oracle_pins.ALL_PINS), len(ALL_PRE_PINS))\n"
    )
    out = _run(code, asan, 300)
    assert out.returncode == 0 and "PINS_OK" in out.stdout, out.stdout[-2000:] + out.stderr[-4000:]


def test_host_code_under_asan_ubsan(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    runtimes = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not shutil.which(hipcc) and not os.path.exists(hipcc):
        pytest.skip("hipcc is not installed")
    if not runtimes:
        pytest.skip("the compiler's address-sanitizer runtime is not installed")
    from linear_attention_recurrence_gated_amd import build as lib_build
    flags = list(lib_build.FLAGS)
    flags[flags.index("-O3")] = "-O1"
    san = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
           "-Xarch_host -fno-sanitize-recover=all -Xarch_host -shared-libsan").split()
    procs, objs = [], []
    for src in lib_build.sources():
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([hipcc, *flags, "-g", *san, "-c", src, "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p in procs:
        _, err = p.communicate(timeout=600)
        assert p.returncode == 0, err[-2000:]
    lib = str(tmp_path / "libgdn_san.so")
    link = subprocess.run([hipcc, f"--offload-arch={lib_build.ARCH}", "-shared", "-fPIC", *san, *objs, "-o", lib],
                          capture_output=True, text=True, timeout=600)
    assert link.returncode == 0, link.stderr[-2000:]
    code = (
        "import sys\n"
        f"sys.path[:0] = [{ROOT!r}, {HERE!r}]\n"
        "from linear_attention_recurrence_gated_amd import gdn\n"
        f"gdn.LIB_PATH = {lib!r}\n"
        "import pytest\n"
        f"rc = pytest.main(['-q', '-p', 'no:cacheprovider', {os.path.join(HERE, 'test_abi.py')!r}])\n"
        "print('ABI_RC', int(rc))\n"
    )
    out = _run(code, runtimes[-1], 600)
    assert out.returncode == 0 and "ABI_RC 0" in out.stdout, out.stdout[-3000:] + out.stderr[-4000:]
