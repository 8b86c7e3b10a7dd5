"""Host-side checks of the benchmark: the one-GPU rule and the probe library
that supplies the achievable-peak denominators (loads and exports its entry
points; its argument checks run before any launch)."""
import ctypes
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.fixture(scope="module")
def P():
    from grouped_gemm_topk_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        B.build()
    L = ctypes.CDLL(B.PROBE_LIB)
    L.moe_probe_mfma_loop.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.moe_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                     ctypes.c_void_p]
    return L


def test_probe_exports(P):
    for n in ("moe_probe_mfma_loop", "moe_probe_hbm_read", "moe_probe_mfma_flops_per_wave_iter"):
        assert hasattr(P, n), n
    # 16 accumulators x one 32x32x16 MFMA (2 flops per multiply-add)
    assert P.moe_probe_mfma_flops_per_wave_iter() == 16 * 32 * 32 * 16 * 2


def test_probe_rejects_bad_arguments_before_launch(P):
    hip_invalid_value = 1
    assert P.moe_probe_mfma_loop(None, 1024, 10, None) == hip_invalid_value
    assert P.moe_probe_mfma_loop(ctypes.c_void_p(16), 0, 10, None) == hip_invalid_value
    assert P.moe_probe_hbm_read(None, 1 << 20, ctypes.c_void_p(16), 8, None) == hip_invalid_value
    assert P.moe_probe_hbm_read(ctypes.c_void_p(16), 24, ctypes.c_void_p(16), 8, None) == hip_invalid_value
