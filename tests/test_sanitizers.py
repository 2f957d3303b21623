"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The oracle (plain C) built by gcc with -fsanitize=address,undefined runs its
  pins (tests/test_oracle_pins.py).
- libpkv with its host C++ instrumented (pkv_api.cpp: argument checks,
  schedule planning, workspace arithmetic, pkv_validate_host; device code
  unchanged) runs the C-ABI checks of tests/test_abi.py.
Each runs in a child process that preloads the sanitizer runtime; any report
aborts the child.  A copy of the oracle with a planted one-element
out-of-bounds read shows that the runtime is live.
"""
import os
import subprocess
import sys

import pytest

import oracle
from paged_kv_cache_92_amd import build as pkv_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer", "-g")


def _gcc_runtime():
    libs = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                           check=True).stdout.strip()
        if not os.path.isabs(p) or not os.path.exists(p):
            pytest.skip(f"gcc has no {name}")
        libs.append(p)
    return ":".join(libs)


def _child(kind, lib, test_file, preload, *extra):
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return subprocess.run([sys.executable, "-m", "tests.sanitizer_child", kind, lib, test_file, *extra],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = oracle.build(extra_flags=SAN, out_path=str(tmp_path / "liboracle_san.so"))
    r = _child("oracle", lib, os.path.join(ROOT, "tests", "test_oracle_pins.py"), _gcc_runtime())
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout


def test_planted_out_of_bounds_read_is_reported(tmp_path):
    # One element past the end of the query row: the oracle's dot product reads
    # q[d] as well (the mistake is planted in a copy, on the CPU).
    src = open(os.path.join(ROOT, "oracle", "pkv_oracle.c")).read()
    marker = "for (int e = 0; e < d; ++e) dot += q[e] * k[e];"
    assert src.count(marker) == 1
    bad = tmp_path / "pkv_oracle_oob.c"
    bad.write_text(src.replace(marker, "for (int e = 0; e <= d; ++e) dot += q[e] * k[e];"))
    lib = oracle.build(extra_flags=SAN, out_path=str(tmp_path / "liboracle_oob.so"), src=str(bad))
    r = _child("oracle", lib, os.path.join(ROOT, "tests", "test_oracle_pins.py"), _gcc_runtime(),
               "-k", "brute_force")
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr or "runtime error" in r.stderr, r.stderr[-3000:]


def test_library_host_checks_under_asan_ubsan(tmp_path):
    try:
        rt = pkv_build.host_asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = pkv_build.build_host_sanitized(str(tmp_path / "libpkv_hostsan.so"))
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "host code is not instrumented"
    r = _child("pkv", lib, os.path.join(ROOT, "tests", "test_abi.py"), rt)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout
