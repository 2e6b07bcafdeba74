"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle's C source is built with -fsanitize=address,undefined into a
temporary directory, and the pin and fuzz suites run against that build in
a subprocess (the ASan runtime preloaded into the interpreter, UBSan fatal).
A planted heap overflow in a separate scratch library shows that the set-up
does catch an error, so a clean run means something.  Nothing here touches
the GPU library.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_FLAGS = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]


def _asan_runtime():
    try:
        p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True, check=True)
    except (OSError, subprocess.CalledProcessError):
        return None
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _env(extra):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0",
                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", **extra)


def test_oracle_pins_and_fuzz_under_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    import oracle
    lib = oracle.compile_source(os.path.join(ROOT, "oracle", "hhr_oracle.c"), str(tmp_path / "liboracle_san.so"),
                                SAN_FLAGS)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_fuzz.py")],
                       cwd=ROOT, env=_env({"HHR_ORACLE_LIB": lib}), capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]


def test_sanitizer_set_up_catches_a_planted_overflow(tmp_path):
    src = tmp_path / "poke.c"
    src.write_text("#include <stdlib.h>\n"
                   "int poke(int n) { int* a = malloc(sizeof(int) * n); for (int i = 0; i < n; ++i) a[i] = i;\n"
                   "  int s = a[n]; free(a); return s; }\n")
    lib = tmp_path / "libpoke.so"
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", *SAN_FLAGS, "-o", str(lib), str(src)], check=True)
    r = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({str(lib)!r}).poke(4)"],
                       env=_env({}), capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr
