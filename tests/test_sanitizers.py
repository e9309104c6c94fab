"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

* The fp64 oracle's loop nests and partial-sum table walk, on small and
  degenerate shapes (N = 0, 1, ragged widths, T = 1 and 64).
* The C ABI's argument-check layer, sanitized on its host side, against the
  documented rejections and 20000 seeded fuzzed calls (descriptors,
  offsets tables, shard pointer arrays, NULL / misaligned / overlapping
  pointers): every call must end in an error status with a message, and
  none may reach a kernel launcher (there is no GPU here).
Builds take a few seconds (gcc, and hipcc with --cuda-host-only)."""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "sanitize"))

ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


@pytest.fixture(scope="module")
def san_dir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("sanitize"))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(san_dir):
    import build as sb
    exe = sb.build_oracle_driver(san_dir)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "OK", r.stdout + r.stderr


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not available")
def test_abi_checks_under_sanitizers(san_dir):
    import build as sb
    exe = sb.build_abi_driver(san_dir)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("OK"), r.stdout + r.stderr
