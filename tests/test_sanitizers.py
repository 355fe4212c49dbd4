"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds are made in a temporary directory and the CPU tests that exercise them run in a child
process with the sanitizer runtime preloaded:

* the fp64 oracle (``oracle/oracle.c``) built by gcc with ``-fsanitize=address,undefined``, under
  the oracle's pin tests;
* the library with its host code (argument checks, planning, workspace layout, launch set-up)
  sanitized by clang, under the ABI tests.  The device code is built as usual.

Each configuration first runs a positive control: a few lines with a heap overflow and a signed
overflow, built the same way, must be reported.  A sanitizer report in the real run fails the
test (``halt_on_error``).  Skipped where a GPU is visible (the child runs host-only tests).
"""
import glob
import os
import subprocess
import sys
import textwrap

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="host sanitizer runs are made without a GPU")

SAN_ENV = dict(ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")

CONTROL_C = textwrap.dedent("""
    #include <stdlib.h>
    #include <limits.h>
    int heap_overflow(int i) { int* p = (int*)malloc(4 * sizeof(int)); int v = p[i]; free(p); return v; }
    int signed_overflow(int x) { return x + INT_MAX; }
""")


def _child(env_extra, args, timeout=900):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(env_extra)
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=timeout)


def _control(lib, preload):
    """Load `lib` under the runtime and call its two planted faults in separate children."""
    out = {}
    for fn, arg in (("heap_overflow", 6), ("signed_overflow", 5)):
        code = f"import ctypes; ctypes.CDLL({lib!r}).{fn}({arg})"
        res = _child({"LD_PRELOAD": preload}, ["-c", code], timeout=120)
        # (UBSan's object-size check may see the overflowing load before ASan does)
        out[fn] = (res.returncode,
                   "AddressSanitizer" in res.stderr or "runtime error" in res.stderr)
    return out


def _sanitizer_clean(res):
    text = res.stdout + res.stderr
    return res.returncode == 0 and "AddressSanitizer" not in text and "runtime error" not in text


def test_oracle_under_asan_and_ubsan(tmp_path):
    flags = ["-O1", "-g", "-fPIC", "-shared", "-pthread", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    preload = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    ctrl_src = tmp_path / "control.c"
    ctrl_src.write_text(CONTROL_C)
    ctrl = str(tmp_path / "libcontrol_gcc.so")
    subprocess.run(["gcc", *flags, str(ctrl_src), "-o", ctrl], check=True)
    for fn, (rc, reported) in _control(ctrl, preload).items():
        assert rc != 0 and reported, f"gcc sanitizer control {fn} was not reported"

    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", *flags, "-std=c11", os.path.join(ROOT, "oracle", "oracle.c"), "-o",
                    lib, "-lm"], check=True)
    res = _child({"LD_PRELOAD": preload, "ORACLE_LIBRARY": lib},
                 ["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_oracle.py",
                  "tests/test_oracle_decay.py", "tests/test_oracle_layer.py"])
    assert _sanitizer_clean(res), res.stdout[-3000:] + res.stderr[-3000:]
    assert " passed" in res.stdout


def test_library_host_code_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from long_context_hybrid_amd import build as lib_build

    runtimes = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not runtimes:
        pytest.skip("clang's ASan runtime is not installed")
    preload = runtimes[0]
    host = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
              "-shared-libsan"):
        host += ["-Xarch_host", f]

    ctrl_src = tmp_path / "control.cpp"
    ctrl_src.write_text('extern "C" {\n' + CONTROL_C + "}\n")
    ctrl = str(tmp_path / "libcontrol_clang.so")
    subprocess.run(["/opt/rocm/llvm/bin/clang++", "-O1", "-g", "-fPIC", "-shared",
                    "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-shared-libsan", str(ctrl_src), "-o",
                    ctrl], check=True)
    for fn, (rc, reported) in _control(ctrl, preload).items():
        assert rc != 0 and reported, f"clang sanitizer control {fn} was not reported"

    lib = str(tmp_path / "liblightning_san.so")
    lib_build.build(out=lib, extra=["-g", "-fno-omit-frame-pointer", *host], link_extra=host)
    res = _child({"LD_PRELOAD": preload, "LIGHTNING_LIBRARY": lib},
                 ["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_abi.py"])
    assert _sanitizer_clean(res), res.stdout[-3000:] + res.stderr[-3000:]
    assert " passed" in res.stdout
