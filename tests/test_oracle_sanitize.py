"""The CPU oracle under AddressSanitizer, LeakSanitizer and UndefinedBehaviorSanitizer.

tests/oracle_sanitize.c includes the oracle's C source and walks every entry point
(decode steps in all threshold modes with eviction, contiguous and paged requests,
an empty batch row, append, gather, release, admission, prefill chunks, and the
degenerate sizes).  It is built here with gcc's sanitizers, host code only, and
must exit cleanly: any out-of-bounds access, use after free, leak or undefined
operation aborts it.
"""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_walk_is_clean_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    subprocess.run(["gcc", "-std=gnu99", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-ffp-contract=off", "-fopenmp", os.path.join(HERE, "oracle_sanitize.c"),
                    "-lm", "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
    m = re.search(r"ok \((\d+) steps, (\d+) evicted, (\d+) prefetched, (\d+) missed\)",
                  r.stdout)
    assert m, r.stdout
    # the walk reaches the eviction, prefetch and recall branches
    steps, evicted, prefetched, missed = map(int, m.groups())
    assert steps >= 20 and evicted > 0 and prefetched > 0 and missed > 0, r.stdout
