"""The host side of libmoe under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Builds every source with the sanitizers on its host pass (build.build_sanitized) and runs
the host ABI tests against that library in a child process with the ASan runtime
preloaded: argument checks, workspace layouts, status strings and the no-allocation entry
point's checks all run instrumented, and any report is fatal.
"""
import os
import subprocess
import sys

import pytest

from mixture_experts_transformer_sigmoid_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(900)
def test_host_abi_under_asan_and_ubsan():
    lib = B.build_sanitized()
    with open(lib, "rb") as f:
        image = f.read()
    # instrumented: the host code calls the ASan and UBSan report hooks
    assert b"__asan_report_load" in image and b"__ubsan_handle_" in image
    env = B.sanitizer_env()
    probe = subprocess.run([sys.executable, "-c", "import mixture_experts_transformer_sigmoid_amd as M; "
                            "M.lib(); print(M.LIB_PATH)"], cwd=ROOT, env=env,
                           stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert probe.returncode == 0 and probe.stdout.strip().endswith("libmoe_san.so"), probe.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=600)
    print(r.stdout[-3000:])
    assert r.returncode == 0, r.stdout[-3000:]
    assert "ERROR: AddressSanitizer" not in r.stdout and "runtime error" not in r.stdout
    assert " passed" in r.stdout
