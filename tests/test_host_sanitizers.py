"""The host-only C++ of the library (refcounted block pool, compression
planner, capacity rule, scheduler) built with AddressSanitizer and
UndefinedBehaviorSanitizer, and driven by the allocator / planner tests and
the scheduler's lockstep tests against the oracle, in a child Python with the
ASan runtime preloaded. Any sanitizer report aborts the child, which fails
this test. CPU only."""
import os
import subprocess
import sys

import pytest

from compressed_paged_kv_gqa_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

HOST_TESTS = [
    "tests/test_sched.py",
    "tests/test_abi.py::test_alloc_all_or_nothing_and_conservation",
    "tests/test_abi.py::test_planner_matches_oracle_and_commit_releases",
    "tests/test_abi.py::test_plan_without_free_blocks_changes_nothing_and_abort_frees",
    "tests/test_abi.py::test_plan_rejects_non_prefix_sharing_and_bad_tables",
    "tests/test_abi.py::test_random_allocator_sequences_conserve_blocks",
    "tests/test_abi.py::test_capacity_matches_oracle",
]


@pytest.mark.timeout(900)
def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    rt = _build.sanitizer_runtime()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("g++ has no AddressSanitizer runtime here")
    lib = _build.build_host_sanitized(str(tmp_path / "libzp_host_san.so"))
    env = dict(os.environ)
    env.update(ZP_LIBRARY=lib, LD_PRELOAD=rt,
               # Python's own allocations are never freed at exit: leak
               # checking would report the interpreter, not this library
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-p", "no:xdist", *HOST_TESTS], cwd=ROOT, env=env,
                       capture_output=True, text=True)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in tail and "runtime error" not in tail
