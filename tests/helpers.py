"""Shared test helpers: moving generator output to the GPU and comparing."""
import numpy as np

ATOL_MAX = 2e-2      # max |GPU - oracle| on the fp32 output
RTOL_L2 = 5e-3       # ||GPU - oracle||_2 / ||oracle||_2


def to_dev(a, dev="cuda"):
    """numpy -> torch on the GPU; uint16 arrays become bfloat16 (same bits)."""
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def out_errors(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    d = got - want
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    nrm = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(d) / nrm) if nrm > 0 else float(np.linalg.norm(d))
    return max_abs, rel


def assert_out_close(got, want, what=""):
    max_abs, rel = out_errors(got, want)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert max_abs <= ATOL_MAX and rel <= RTOL_L2, f"{what}: max|d|={max_abs:.3g} rel-L2={rel:.3g}"
    return max_abs, rel
