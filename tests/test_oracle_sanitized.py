"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: its
pins (tableaux, closed forms, invariants, derivatives, dense output,
sensitivities, every method and system) run against a sanitized build of
oracle.cpp, in a child process that preloads the ASan runtime, with every
report fatal; and the set-up is shown to catch a planted out-of-bounds read
and a planted undefined shift in a copy of the source.  (The whole
`-m "not gpu"` suite passes against the sanitized build too; the command is
in the oracle's build notes.)"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime():
    path = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("no ASan runtime for g++")
    return path


def _env(lib):
    env = dict(os.environ)
    env.update(LD_PRELOAD=_runtime(), ORACLE_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


def _reports(text):
    return "AddressSanitizer" in text or "runtime error:" in text


def test_oracle_pins_pass_under_sanitizers():
    import oracle
    lib = oracle.build(force=True, sanitize=True)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-n", "4", "-p", "no:cacheprovider",
           "tests/test_oracle_pins.py", "tests/test_oracle_dense.py",
           "tests/test_oracle_user_rhs.py", "-k", "not scipy and not order and not global"]
    r = subprocess.run(cmd, cwd=ROOT, env=_env(lib), capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert not _reports(out), out[-3000:]
    assert " passed" in out


# (what to plant, the text it replaces, what replaces it, the report)
PLANTS = [
    ("an out-of-bounds read of the last trajectory's u0",
     "  for (int c = 0; c < d; ++c) y[c] = u0[c];\n  for (int s = 0; s < o.S; ++s) {",
     "  for (int c = 0; c <= d; ++c) y[c] = u0[c];\n  for (int s = 0; s < o.S; ++s) {",
     "AddressSanitizer"),
    ("a shift by more than the width of int",
     "  int nacc = 0, natt = 0, st = S_OK;\n  bool finite = true;",
     "  int nacc = 0, natt = 0, st = S_OK;\n  bool finite = (1 << (P->dim + 40)) != 0;",
     "runtime error:"),
]


@pytest.mark.parametrize("what,old,new,report", PLANTS, ids=["asan", "ubsan"])
def test_sanitizers_catch_a_planted_mistake(tmp_path, what, old, new, report):
    import oracle
    src = open(os.path.join(ROOT, "oracle", "oracle.cpp")).read()
    assert src.count(old) == 1, what
    path = tmp_path / "oracle_planted.cpp"
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / "liboracle_planted.so")
    subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fopenmp", "-fPIC",
                    "-shared", *oracle.SANITIZE_FLAGS, "-I", os.path.join(ROOT, "oracle"),
                    "-o", lib, str(path)], check=True)
    code = ("import numpy as np, oracle, workloads as W\n"
            "w = W.WORKLOADS[1]\n"
            "inp = W.make_inputs(1, 5)\n"
            "oracle.record(w.problem(), inp['u0'], inp['p'])\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=_env(lib),
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and report in r.stderr, (what, r.stderr[-2000:])
