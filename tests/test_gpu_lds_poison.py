"""The prefill kernel's counted waits on the GPU: every prefill-kernel path (paged
prefill in both page modes, split and unsplit, the cascade's level 0, block-sparse, the
mixed batch) run with the debug build, whose LDS tile buffers start each item as NaN,
must still match the oracle; a tile read before its load landed would read NaN. The
cases run in a child process (tests/lds_poison_cases.py), which loads the debug build."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_prefill_paths_with_poisoned_lds():
    lib = os.path.join(os.path.dirname(HERE), "paged_kv_cache_173_amd", "libpkv_debug.so")
    assert os.path.exists(lib), "build the library first (it builds libpkv_debug.so too)"
    env = dict(os.environ, PKV_LIBRARY="libpkv_debug.so")
    res = subprocess.run([sys.executable, "-u", os.path.join(HERE, "lds_poison_cases.py")],
                         env=env, capture_output=True, text=True, timeout=240)
    print(res.stdout[-4000:])
    print(res.stderr[-4000:], file=sys.stderr)
    assert res.returncode == 0, res.stderr[-2000:]
    assert "lds poison:" in res.stdout and "cases ok" in res.stdout
