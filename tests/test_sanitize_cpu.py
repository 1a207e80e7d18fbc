"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): the planner (chunk and group sizes, workspace offsets), every
host-side validation path and the status strings.  build(sanitize=True)
compiles csrc/lce_api.hip with the sanitizers on its host side and links it
with tests/c_abi/lce_host_checks.c, a harness that walks valid and invalid
problem descriptions (sizes around every limit, seeded random ones) and the
error paths of each compute entry point with pointers that are never
dereferenced.  A sanitizer report or a failed invariant fails the test."""
import os
import subprocess

from linear_cross_entropy_chunk_amd import build


def test_host_code_under_asan_and_ubsan():
    exe = build.build_host_checks(verbose=False)     # seconds once liblce's objects exist
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
    word, created, tried = r.stdout.split()
    assert word == "ok" and int(created) > 1000 and int(tried) > 40000
