"""Child process of tests/test_sanitizers.py: point the oracle or the library
binding at a sanitizer-instrumented build, then run one test file in-process.

usage: python -m tests.sanitizer_child {oracle|pkv} LIBRARY TEST_FILE [pytest args...]
The parent preloads the matching sanitizer runtime (LD_PRELOAD)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def main():
    kind, lib, test_file, *rest = sys.argv[1:]
    if kind == "oracle":
        import oracle
        oracle.use_library(lib)
    elif kind == "pkv":
        import paged_kv_cache_92_amd._binding as binding
        binding.LIB_PATH = lib
    else:
        raise SystemExit(f"unknown kind {kind}")
    import pytest
    # -s: a sanitizer report goes to the real stderr, not to a capture that
    # the abort would discard.
    return pytest.main(["-q", "-x", "-s", "-p", "no:cacheprovider", "-m", "not gpu", test_file, *rest])


if __name__ == "__main__":
    sys.exit(main())
