"""libpp's host code under AddressSanitizer: tests/asan/abi_driver (built by
personaplex_temporal_transformer_amd/build.py build_asan(), against libpp_asan.so whose host
code is instrumented) calls every entry point, error paths included. Without a GPU it runs
the host-only checks (NULL handles and arguments); on the GPU it also creates small models
and runs decode (graph, direct, allocation-free, batched), prefill and chunks, the readers,
the depth transformer, the generator with its snapshot, sampling and the error paths."""

import os
import subprocess

import pytest

from tests.helpers import have_gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "asan", "abi_driver")


def _run():
    if not os.path.exists(DRIVER):
        pytest.fail("tests/asan/abi_driver is not built: run the package build (build_asan)")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([DRIVER], capture_output=True, text=True, env=env, timeout=240)
    print(r.stdout[-2000:])
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, (r.returncode, r.stdout[-2000:], r.stderr[-2000:])
    return r.stdout


def test_asan_host_only_paths():
    if have_gpu():
        pytest.skip("the GPU variant below covers these paths too")
    assert "host-only checks ok" in _run()


@pytest.mark.gpu
def test_asan_every_entry_point_on_the_gpu():
    assert "abi_driver: ok" in _run()
