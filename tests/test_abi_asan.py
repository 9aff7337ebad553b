"""The C ABI's host code under AddressSanitizer (CPU only): the library is rebuilt with
-fsanitize=address on the host side (device code unchanged), and tests/test_abi.py runs against
it in a child process with the ASan runtime preloaded.  Any invalid host memory access in the
argument checks, the launch set-up or the status strings aborts that child with a report."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _sources_hash() -> str:
    from io_aware_softmax_mifa_amd import build as B

    h = hashlib.sha256()
    for p in B.SOURCES + [os.path.join(B.INCLUDE, "mifa.h"), os.path.join(B.PKG, "csrc", "mifa_common.h")]:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def test_abi_under_host_asan():
    from io_aware_softmax_mifa_amd import build as B

    try:
        B.hipcc()
        runtime = B.asan_runtime()
    except RuntimeError as e:
        pytest.skip(f"no ROCm toolchain / ASan runtime: {e}")
    out_dir = os.path.join(ROOT, "_build", "asan-" + _sources_hash())
    lib = os.path.join(out_dir, "libmifa.so")
    if not os.path.exists(lib):
        B.build_host_asan(out_dir)
    env = dict(os.environ, MIFA_LIBRARY=lib, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    print(r.stdout[-3000:], r.stderr[-3000:])
    assert r.returncode == 0, "test_abi.py failed under host ASan"
    assert "AddressSanitizer" not in r.stderr
