"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
a host-sanitized build of liblps (device code unchanged) loaded with the clang
ASan runtime preloaded, running the host ABI tests (stage plans, the solver, the
RoPE table, every refusal that runs before an enqueue, the pending tokens)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_tests_pass_under_asan_and_ubsan():
    from layer_pipeline_stage_amd import build as b
    try:
        b.hipcc()
        rt = b.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    srcs = b.sources()
    stale = not os.path.exists(b.SAN_OUT) or any(
        os.path.getmtime(s) > os.path.getmtime(b.SAN_OUT) for s in srcs + [os.path.join(
            ROOT, "layer_pipeline_stage_amd", "csrc", h) for h in ("internal.h", "dev.h", "gemv_core.h")])
    if stale:
        b.build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", LPS_LIB_PATH=b.SAN_OUT)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
