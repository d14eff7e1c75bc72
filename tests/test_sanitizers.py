"""The oracle (oracle/oracle.c) and the input generators (synth/gen.c) built
with AddressSanitizer and UndefinedBehaviorSanitizer, and the oracle's pins
and the generators' tests run against those builds in a child process (CPU
only). Any out-of-bounds access, use after free or undefined operation in
either C file aborts the child and fails the test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]


def _runtime():
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                         text=True).stdout.strip()
    return out if out and os.path.exists(out) else None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    if _runtime() is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    d = tmp_path_factory.mktemp("san")
    ora = str(d / "liboracle_san.so")
    syn = str(d / "libsynth_san.so")
    # the oracle keeps its strict IEEE flags; the generator its OpenMP
    subprocess.check_call(["gcc"] + SAN + ["-ffp-contract=off", "-fno-fast-math", "-fPIC",
                                           "-shared", os.path.join(ROOT, "oracle", "oracle.c"),
                                           "-o", ora, "-lm"])
    subprocess.check_call(["gcc"] + SAN + ["-fopenmp", "-fPIC", "-shared",
                                           os.path.join(ROOT, "synth", "gen.c"), "-o", syn,
                                           "-lm"])
    return ora, syn


def test_oracle_and_generators_under_sanitizers(sanitized):
    ora, syn = sanitized
    env = dict(os.environ, ORACLE_LIB=ora, SYNTH_LIB=syn, LD_PRELOAD=_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_oracle.py", "tests/test_synth.py", "-k",
                        "not thread_count"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
