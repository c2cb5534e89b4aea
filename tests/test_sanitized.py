"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* The oracle (oracle_gemm.c) is rebuilt with -fsanitize=address,undefined and
  every pin of tests/oracle_pins.py runs against it in a child interpreter
  with the sanitizer runtime preloaded: any out-of-bounds access, use after
  free or undefined operation in the oracle fails the test.
* The C ABI's host side (gemm_api.hip and the launchers, host pass only:
  the GPU code is built as usual) is rebuilt the same way and the
  argument-checking paths that need no GPU (every entry point's argument
  errors, the dispatch query, the status strings) run under it.
"""
import glob
import json
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "OMP_NUM_THREADS": "2"}


def runtime(path):
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("sanitizer runtime not found: %s" % path)
    return path


def run_child(code, preload):
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV)
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          timeout=600, env=env)
    report = proc.stdout[-4000:] + proc.stderr[-4000:]
    assert "AddressSanitizer" not in proc.stderr, report
    assert "runtime error" not in proc.stderr, report
    assert proc.returncode == 0, report
    return proc


def test_oracle_pins_under_sanitizers(tmp_path):
    asan = runtime(subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                                  text=True, check=True).stdout.strip())
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                    "-Wall", "-Werror", oracle.SOURCE, "-o", lib, "-lm"], check=True)
    code = ("import sys; sys.path[:0] = [%r, %r]; import oracle_pins; "
            "oracle_pins.main(%r, %r)" % (HERE, ROOT, lib,
                                          os.path.join(HERE, "golden", "worked_2x2.txt")))
    proc = run_child(code, asan)
    line = [l for l in proc.stdout.splitlines() if l.startswith("PIN_FAILURES ")]
    assert line and json.loads(line[-1][len("PIN_FAILURES "):]) == []


def test_sanitizer_catches_a_planted_overrun(tmp_path):
    """The check has teeth: a copy of the oracle whose vector sum reads one
    element past the end (planted here, on the CPU) is reported."""
    asan = runtime(subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                                  text=True, check=True).stdout.strip())
    text = open(oracle.SOURCE).read()
    planted = text.replace("for (int64_t i = 0; i < n; ++i) {\n        s += (double)x[i];",
                           "for (int64_t i = 0; i <= n; ++i) {\n        s += (double)x[i];")
    assert planted != text
    src = tmp_path / "oracle_overrun.c"
    src.write_text(planted)
    lib = str(tmp_path / "liboracle_overrun.so")
    subprocess.run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fopenmp", "-fPIC",
                    "-shared", "-std=c11", str(src), "-o", lib, "-lm"], check=True)
    code = ("import sys; sys.path.insert(0, %r); import numpy as np; from oracle import Oracle; "
            "Oracle(%r).sum_f32(np.ones(1000, dtype=np.float32))" % (ROOT, lib))
    env = dict(os.environ, LD_PRELOAD=asan, **SAN_ENV)
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          timeout=300, env=env)
    assert proc.returncode != 0
    assert "heap-buffer-overflow" in proc.stderr, proc.stderr[-3000:]


SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def sanitized_library():
    """libgemm.so with its host pass built under the sanitizers, cached in
    the package's _build/ folder until a source or the flags change."""
    import hashlib
    from roofline_driven_optimisation_amd import build as b
    if not os.path.exists(b.HIPCC):
        pytest.skip("hipcc not found")
    h = hashlib.sha256(" ".join(b.CFLAGS + SAN_FLAGS).encode())
    for path in b.sources() + glob.glob(os.path.join(b.CSRC, "*.h")) + [
            os.path.join(b.INCLUDE, "gemm.h")]:
        h.update(open(path, "rb").read())
    out_dir = os.path.join(b.BUILD_DIR, "host_sanitized")
    lib = os.path.join(out_dir, "libgemm_sanitized.so")
    stamp = os.path.join(out_dir, "sources.sha256")
    if not (os.path.exists(lib) and os.path.exists(stamp) and
            open(stamp).read() == h.hexdigest()):
        b.build(extra=SAN_FLAGS, lib=lib, build_dir=out_dir, check_load=False)
        with open(stamp, "w") as f:
            f.write(h.hexdigest())
    return lib


def test_c_abi_host_paths_under_sanitizers():
    clang_rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not clang_rt:
        pytest.skip("clang's AddressSanitizer runtime not found")
    lib = sanitized_library()
    # the C-ABI tests that need no GPU, against the sanitized build (the
    # exported-symbol list is left out: instrumentation adds runtime hooks)
    code = ("import sys; sys.path[:0] = [%r, %r]\n"
            "from roofline_driven_optimisation_amd import binding\n"
            "binding.library_path = lambda: %r\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', %r, '-k', "
            "'not only_declared_symbols']))\n" % (HERE, ROOT, lib, os.path.join(HERE, "test_abi.py")))
    proc = run_child(code, runtime(clang_rt[0]))
    import re
    m = re.search(r"(\d+) passed", proc.stdout)
    assert m and int(m.group(1)) >= 12, proc.stdout[-2000:]
    assert "failed" not in proc.stdout and "error" not in proc.stdout.lower(), proc.stdout[-2000:]
