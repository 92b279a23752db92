"""The argument validation of the C ABI under AddressSanitizer (CPU only): tests/test_abi_cpu.py runs in a child
process against libheal built with its host code instrumented (error_compensated_gemm_amd.build.build_asan), with
the clang ASan runtime preloaded.  Every validation path there returns before any device call, so no GPU is
needed; an out-of-bounds read or write in the host code of the library fails the run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DRIVER = """
import sys
sys.path.insert(0, {root!r})
import error_compensated_gemm_amd as heal
heal.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(['-q', '-m', 'not gpu', '-p', 'no:cacheprovider', {test!r}]))
"""


@pytest.mark.slow
def test_abi_validation_under_asan():
    from error_compensated_gemm_amd import build as hb

    rt = hb.asan_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime in this ROCm install")
    lib = hb.build_asan()
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    code = DRIVER.format(root=ROOT, lib=lib, test=os.path.join(ROOT, "tests", "test_abi_cpu.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert "AddressSanitizer" not in out
    assert r.returncode == 0
    assert " passed" in out
