"""The host code of the library (the C ABI, the Eq. 1 solvers and the
KV-pressure scheduler's decision) under AddressSanitizer and
UndefinedBehaviorSanitizer: the library is rebuilt with those host sources
instrumented (kernels as usual) and the host tests of the boundary
(tests/test_capi_host.py: every exported entry point's argument and state
errors, the solvers against the oracle, the decision against its oracle)
run against it in a child interpreter with the sanitizer runtime preloaded.
Any report aborts the child. No GPU is used."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def san_lib():
    from mixed_precision_weight_page_amd import build
    try:
        rt = build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    return build.build_host_sanitized(), rt


def test_host_tests_pass_under_asan_and_ubsan(san_lib):
    lib, rt = san_lib
    env = dict(os.environ)
    env.update(PW_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_capi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out


def test_sanitized_library_is_the_one_loaded(san_lib):
    # the child really loads the instrumented build: its map holds the
    # sanitized library and the sanitizer runtime
    lib, rt = san_lib
    env = dict(os.environ)
    env.update(PW_LIBRARY=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0")
    code = ("from mixed_precision_weight_page_amd import pagedweight as p; p.lib(); "
            "print(open('/proc/self/maps').read())")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert os.path.basename(lib) in r.stdout and "asan" in r.stdout
