"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): argument checks of every entry point, the host repack and its inverse,
the launch planners, workspace queries, KV-cache packing and the tree-MTP
planner, driven by tests/sanitize/host_checks.cpp."""

import importlib.util
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_host_code_under_sanitizers():
    spec = importlib.util.spec_from_file_location("sk_sanitize_build",
                                                  os.path.join(HERE, "sanitize", "build_checks.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    exe = mod.ensure_built()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks passed" in r.stdout
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
