"""The library's host code under AddressSanitizer, no GPU needed:
tests/c_abi/usp_host_check (built by __graft_entry__.build() against a copy
of libusp whose host code is instrumented, its device code not) runs the
range splits, the head-chunk plan, the workspace size and the rejection of
invalid calls of every entry point, with pointer arrays allocated at exactly
their documented length, so any host read or write past them, use after
free or leak is reported and fails the run."""
import os
import subprocess

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "usp_host_check")


def test_host_code_under_address_sanitizer():
    assert os.path.exists(BIN), f"{BIN} is missing: run __graft_entry__.build() first"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "usp host check: ok" in r.stdout
    assert "AddressSanitizer" not in r.stderr, r.stderr
