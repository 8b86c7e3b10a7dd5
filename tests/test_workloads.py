"""The seeded input generator: bit-level conversion, determinism and the
routing structure each workload recipe promises."""
import hashlib

import numpy as np
import pytest
import torch

from grouped_gemm_topk_amd import workloads as W
from oracle import moe_oracle as O


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1.0, -2.5, 1e-30, 3.0e38], np.float32)])
    # values halfway between two bf16 numbers (ties to even)
    halfway = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    a = np.concatenate([a, halfway, -halfway])
    ours = W.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(W.bf16_bits_to_f32(ours),
                          torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def _digest(inp):
    h = hashlib.sha256()
    for k in sorted(inp):
        h.update(k.encode())
        h.update(np.ascontiguousarray(inp[k]).tobytes())
    return h.hexdigest()


def test_determinism_and_independence():
    cfg = W.CONFIGS["tiny"]
    a = W.make_inputs(cfg)
    b = W.make_inputs(cfg, threads=1)
    assert _digest(a) == _digest(b)
    c = W.make_inputs(cfg, layer=1)
    assert _digest(a) != _digest(c)
    assert a["w13"].shape == (8, 1024, 256) and a["w2"].shape == (8, 256, 512)
    x = W.bf16_bits_to_f32(a["x"])
    assert abs(float(x.std()) - 1.0) < 0.05
    w = W.bf16_bits_to_f32(a["w13"])
    assert abs(float(w.std()) - 0.02) < 0.001


def test_dup3_logits_hit_duplicates():
    cfg = W.CONFIGS["decode_t3"]
    l = W.make_logits(cfg)
    ids = O.select_topk(l, cfg.top_k)
    distinct = np.unique(ids)
    assert distinct.size == 12            # 24 slots on 12 experts
    counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
    assert set(counts[counts > 0].tolist()) == {2}


def test_zipf_logits_are_uneven():
    cfg = W.CONFIGS["zipf128"]
    l = W.make_logits(cfg)
    ids = O.select_topk(l, cfg.top_k)
    counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
    assert counts.sum() == cfg.T * cfg.top_k
    assert counts.max() > 20 * max(1, counts.min())


@pytest.mark.parametrize("layer", range(4))
def test_dsv3_group_scores_have_no_near_ties(layer):
    """Grouped routing takes its group decision on fp64 sigmoid sums; the GPU and
    the CPU may differ in the last ulp of exp, so the generated logits must keep
    every pair of group scores of a token (and the top-k boundary) apart."""
    cfg = W.CONFIGS["dsv3"]
    l = W.make_logits(cfg, layer)
    gs = O.group_scores(l, cfg.n_group)
    s = np.sort(gs, axis=1)
    assert np.min(np.diff(s, axis=1)) > 1e-12
    assert np.all(np.isfinite(l))
