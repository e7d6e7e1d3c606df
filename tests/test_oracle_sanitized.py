"""The oracle's pins and property tests, run once more against a copy of
the C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

An out-of-bounds access, a use of freed memory, a signed overflow or an
invalid shift anywhere in bitnest_oracle.c that the pins reach aborts the
child process, so the test fails even where the wrong value would happen
to pass a pin. The child is a fresh interpreter with the sanitizer
runtime preloaded (an instrumented library cannot be loaded into a
process that started without it) and BITNEST_ORACLE_LIB pointing at the
instrumented copy.
"""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_pass_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c99",
                    "-D_GNU_SOURCE", "-Wall", "-Wextra", "-fPIC", "-shared", oracle._SRC, "-o", str(lib), "-lm"],
                   check=True)
    env = dict(os.environ)
    env["BITNEST_ORACLE_LIB"] = str(lib)
    env["LD_PRELOAD"] = asan
    # the interpreter's own allocations are not the oracle's: no leak report
    # at exit; any other finding ends the child with an error
    logs = tmp_path / "san"
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:log_path=%s" % logs
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:log_path=%s" % logs
    env["OMP_NUM_THREADS"] = "4"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-x",
                        os.path.join(HERE, "test_oracle.py"), os.path.join(HERE, "test_oracle_properties.py")],
                       env=env, capture_output=True, text=True, cwd=os.path.dirname(HERE), timeout=900)
    reports = "".join(open(f).read() for f in sorted(tmp_path.glob("san*")))
    tail = (r.stdout + r.stderr)[-2000:] + reports[:4000]
    assert r.returncode == 0 and not reports, tail
    assert " passed" in r.stdout and " failed" not in r.stdout, tail
