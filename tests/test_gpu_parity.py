"""GPU parity: libmoe's HIP path (through the C ABI) against the CPU oracle.

Routing outputs are compared bit for bit; the fp32 layer output within
max|d| <= 2e-2 and rel-L2 <= 5e-3; intermediate grouped-GEMM outputs within a
bound derived from bf16 rounding of the result (2^-8 relative) plus fp32
accumulation-order differences.
"""
import dataclasses

import numpy as np
import pytest

from grouped_gemm_topk_amd import workloads as W
from oracle import moe_oracle as O
from tests.helpers import assert_out_close, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def moe():
    from grouped_gemm_topk_amd import moe as M
    M.lib()
    return M


def _check_routing(res_gpu, ref, T, k, bm):
    if "status" in res_gpu:   # every bounded cross-workgroup wait ended normally
        assert int(res_gpu["status"].item()) == 0, "status word set"
    ids = res_gpu["topk_ids"].cpu().numpy()
    assert np.array_equal(ids, ref["topk_ids"]), "topk_ids"
    np.testing.assert_allclose(res_gpu["topk_weights"].cpu().numpy(), ref["topk_weights"],
                               rtol=2e-6, atol=1e-7)
    ntpp = int(res_gpu["num_tokens_post_padded"].cpu().item())
    assert ntpp == ref["num_tokens_post_padded"]
    st = res_gpu["sorted_token_ids"].cpu().numpy()[:ntpp]
    assert np.array_equal(st, ref["sorted_token_ids"]), "sorted_token_ids"
    ex = res_gpu["expert_ids"].cpu().numpy()[:ntpp // bm]
    assert np.array_equal(ex, ref["expert_ids"]), "expert_ids"


def _run_fused(moe, cfg, inp, block_m=None):
    p = moe.LayerParams.from_config(cfg, block_m=block_m)
    args = [to_dev(inp["x"]), to_dev(inp["logits"]), to_dev(inp["w13"]), to_dev(inp["w2"])]
    sh = [to_dev(inp["shared_w13"]), to_dev(inp["shared_w2"])] if cfg.n_shared else [None, None]
    out, routing = moe.moe_fused_forward(p, *args, *sh, return_routing=True)
    torch.cuda.synchronize()
    return out.cpu().numpy(), routing


# ---------------------------------------------------------------- align
@pytest.mark.parametrize("bm", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("T,k,E,mode", [
    (1, 8, 128, "rand"), (3, 8, 128, "rand"), (37, 2, 8, "rand"), (64, 2, 8, "rand"),
    (100, 4, 18, "rand"), (513, 6, 128, "rand"), (700, 8, 256, "rand"),
    (4096, 4, 18, "rand"), (8192, 8, 128, "zipf"), (5000, 1, 1, "rand"), (1023, 5, 64, "one"),
    (0, 4, 8, "rand"), (2049, 2, 8, "rand"),
    # the one-workgroup / two-kernel boundary (1024 slots), all slots on one
    # expert past it, and more than 64 x 1024 slots (chunks of several passes)
    (1024, 1, 4, "rand"), (1025, 1, 4, "rand"), (129, 8, 16, "one"),
    (20000, 8, 256, "rand"), (9000, 8, 64, "zipf"),
])
def test_align_bit_exact(moe, T, k, E, mode, bm):
    print(f"align T={T} k={k} E={E} mode={mode} bm={bm}", flush=True)
    rng = np.random.default_rng(T * 7 + E + bm)
    if mode == "rand":
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) if T else \
            np.zeros((0, k), np.int32)
    elif mode == "one":      # every slot on expert 3
        ids = np.full((T, k), 3, np.int32)
    else:                     # skewed
        pr = 1.0 / np.arange(1, E + 1) ** 1.1
        ids = np.stack([rng.choice(E, size=k, replace=False, p=pr / pr.sum())
                        for _ in range(T)]).astype(np.int32)
    ref = O.align(ids, E, bm)
    dev_ids = torch.from_numpy(ids).cuda() if T else torch.zeros((0, k), dtype=torch.int32,
                                                                 device="cuda")
    st, ex, ntpp = moe.moe_align(dev_ids, E, bm)
    torch.cuda.synchronize()
    n = int(ntpp.cpu().item())
    assert n == ref["num_tokens_post_padded"]
    assert np.array_equal(st.cpu().numpy()[:n], ref["sorted_token_ids"])
    assert np.array_equal(ex.cpu().numpy()[:n // bm], ref["expert_ids"])


# ---------------------------------------------------------------- grouped GEMM
@pytest.mark.parametrize("bm", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("epi,c32", [(O.EPI_STORE, 1), (O.EPI_STORE, 0), (O.EPI_SWIGLU, 0),
                                     (O.EPI_RELU2, 0), (O.EPI_WEIGHTED_SCATTER, 1),
                                     (O.EPI_SWIGLU, 1)])
@pytest.mark.parametrize("shape", [(45, 3, 6, 200, 80), (300, 2, 5, 136, 272)])
def test_grouped_gemm_vs_oracle(moe, shape, epi, c32, bm):
    T, k, E, K, N = shape
    print(f"grouped_gemm shape={shape} epi={epi} fp32={c32} bm={bm}", flush=True)
    rng = np.random.default_rng(T + 31 * epi + bm)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    wts = rng.random((T, k)).astype(np.float32)
    x_bits = W.f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    w_bits = W.f32_to_bf16_bits((0.1 * rng.standard_normal((E, N, K))).astype(np.float32))
    dev_ids = torch.from_numpy(ids).cuda()
    st, ex, ntpp = moe.moe_align(dev_ids, E, bm)
    al = O.align(ids, E, bm)
    ref = O.grouped_gemm(O.bf16_to_f64(x_bits), k, O.bf16_to_f64(w_bits), al["sorted_token_ids"],
                         al["expert_ids"], al["num_tokens_post_padded"], bm, T * k, epi, wts)
    cap = st.numel()
    ncols = N // 2 if epi == O.EPI_SWIGLU else N
    rows = T * k if epi == O.EPI_WEIGHTED_SCATTER else cap
    dt = torch.float32 if c32 else torch.bfloat16
    c = torch.full((rows, ncols), float("nan"), dtype=dt, device="cuda")
    moe.moe_grouped_gemm(to_dev(x_bits), k, to_dev(w_bits), st, ex, ntpp, bm, T * k, epi, c,
                         torch.from_numpy(wts.reshape(-1)).cuda())
    torch.cuda.synchronize()
    got = c.float().cpu().numpy()
    nt = al["num_tokens_post_padded"]
    if epi != O.EPI_WEIGHTED_SCATTER:
        got, ref = got[:nt], ref[:nt]
    assert np.all(np.isfinite(got)), "rows left unwritten"
    tol = (2.0 ** -8 if not c32 else 1e-5) * np.abs(ref) + 1e-4 * np.abs(ref).max()
    bad = np.abs(got - ref) > tol
    assert not bad.any(), f"{bad.sum()} mismatches, worst {np.abs(got - ref).max()}"


def test_grouped_gemm_contiguous_a(moe):
    """a_row_div = 0: A is read in padded order (the second GEMM's form)."""
    T, k, E, K, N, bm = 50, 2, 4, 96, 64, 32
    rng = np.random.default_rng(77)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    wts = rng.random((T, k)).astype(np.float32)
    st, ex, ntpp = moe.moe_align(torch.from_numpy(ids).cuda(), E, bm)
    al = O.align(ids, E, bm)
    cap = st.numel()
    a_bits = W.f32_to_bf16_bits(rng.standard_normal((cap, K)).astype(np.float32))
    w_bits = W.f32_to_bf16_bits((0.1 * rng.standard_normal((E, N, K))).astype(np.float32))
    ref = O.grouped_gemm(O.bf16_to_f64(a_bits), 0, O.bf16_to_f64(w_bits), al["sorted_token_ids"],
                         al["expert_ids"], al["num_tokens_post_padded"], bm, T * k,
                         O.EPI_WEIGHTED_SCATTER, wts)
    c = torch.full((T * k, N), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_grouped_gemm(to_dev(a_bits), 0, to_dev(w_bits), st, ex, ntpp, bm, T * k,
                         O.EPI_WEIGHTED_SCATTER, c, torch.from_numpy(wts.reshape(-1)).cuda())
    torch.cuda.synchronize()
    np.testing.assert_allclose(c.cpu().numpy(), ref, rtol=1e-5, atol=1e-4)


# ---------------------------------------------------------------- fused forward, small
SMALL = [
    W.CONFIGS["tiny"],
    W.small_config("small_swiglu", T=37, H=64, I=96, E=8, top_k=2),
    W.small_config("small_relu2", T=50, H=136, I=72, E=16, top_k=3, activation=W.ACT_RELU2),
    W.small_config("small_dsv3", T=70, H=128, I=64, E=18, top_k=4, scoring=W.SCORE_SIGMOID,
                   n_group=6, topk_group=4, n_shared=1, block_m=32),
    W.small_config("small_dsv3_s2.5", T=70, H=128, I=64, E=18, top_k=4, scoring=W.SCORE_SIGMOID,
                   n_group=6, topk_group=4, n_shared=1, scale=2.5, block_m=64),
    W.small_config("small_e128", T=9, H=256, I=128, E=128, top_k=8),
    W.small_config("small_norenorm", T=40, H=64, I=64, E=32, top_k=4, renormalize=0),
    W.small_config("small_sigmoid_flat", T=33, H=64, I=32, E=12, top_k=3,
                   scoring=W.SCORE_SIGMOID, renormalize=0),
    W.small_config("small_one_token", T=1, H=96, I=40, E=8, top_k=8),
    W.small_config("small_many_tokens", T=300, H=64, I=48, E=8, top_k=2, block_m=128),
    W.small_config("small_k1", T=65, H=64, I=64, E=4, top_k=1, block_m=64),
    # decode shapes (T <= 16 takes the GEMV path)
    W.small_config("small_dsv3_decode", T=5, H=136, I=72, E=18, top_k=4, scoring=W.SCORE_SIGMOID,
                   n_group=6, topk_group=4, n_shared=1, block_m=128),
    W.small_config("small_relu2_t16", T=16, H=264, I=40, E=32, top_k=6, activation=W.ACT_RELU2),
    W.small_config("small_t17_gemm", T=17, H=64, I=48, E=8, top_k=2),
    W.small_config("small_decode_ragged_k", T=3, H=600, I=328, E=64, top_k=8),
    # the decode path's two forms: from 48 slots (T * top_k) one fused launch,
    # below it GEMV1 + GEMV2; the boundary on both sides, and the fused form
    # with grouped routing and the shared expert (its own block and counter)
    W.small_config("small_decode_fused_edge", T=6, H=128, I=64, E=64, top_k=8),
    W.small_config("small_decode_below_fused", T=15, H=128, I=64, E=32, top_k=3),
    W.small_config("small_dsv3_decode_fused", T=14, H=136, I=72, E=18, top_k=4,
                   scoring=W.SCORE_SIGMOID, n_group=6, topk_group=4, n_shared=1, block_m=16),
    # the largest expert count and top-k the ABI accepts, on both paths
    W.small_config("small_max_e_k", T=20, H=64, I=32, E=256, top_k=16),
    W.small_config("small_max_e_k_decode", T=4, H=64, I=32, E=256, top_k=16),
    # one expert: the layer is a dense MLP with weight 1
    W.small_config("small_e1", T=24, H=64, I=40, E=1, top_k=1),
    W.small_config("small_e1_decode", T=2, H=64, I=40, E=1, top_k=1),
    # grouping that keeps every group (no restriction), with a shared expert
    W.small_config("small_groups_all", T=30, H=64, I=48, E=16, top_k=3,
                   scoring=W.SCORE_SIGMOID, n_group=4, topk_group=4, n_shared=1),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
@pytest.mark.parametrize("bm", [None, 16, 128, 256])
def test_fused_forward_small(moe, cfg, bm):
    print(f"fused {cfg.name} bm={bm}", flush=True)
    inp = W.make_inputs(cfg)
    ref = O.moe_forward_cfg(cfg if bm is None else dataclasses.replace(cfg, block_m=bm), inp)
    out, routing = _run_fused(moe, cfg, inp, bm)
    _check_routing(routing, ref, cfg.T, cfg.top_k, bm or cfg.block_m)
    assert_out_close(out, ref["out"], cfg.name)


@pytest.mark.parametrize("T", [6, 150])
def test_fused_forward_one_hot_expert(moe, T):
    """Every token's first choice is the same expert: one long run of blocks
    for that expert, the second choices spread over the rest."""
    cfg = W.small_config(f"one_hot_{T}", T=T, H=64, I=48, E=16, top_k=2, block_m=16)
    print(f"fused {cfg.name}", flush=True)
    inp = W.make_inputs(cfg)
    inp["logits"] = inp["logits"].copy()
    inp["logits"][:, 5] += 50.0
    ref = O.moe_forward_cfg(cfg, inp)
    assert np.all(ref["topk_ids"][:, 0] == 5)
    out, routing = _run_fused(moe, cfg, inp)
    _check_routing(routing, ref, cfg.T, cfg.top_k, cfg.block_m)
    assert_out_close(out, ref["out"], cfg.name)


def test_fused_forward_zero_tokens(moe):
    cfg = W.small_config("t0", T=0, H=64, I=32, E=8, top_k=2)
    p = moe.LayerParams.from_config(cfg)
    z = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    out = moe.moe_fused_forward(p, z, torch.empty((0, 8), device="cuda"),
                                torch.zeros((8, 64, 64), dtype=torch.bfloat16, device="cuda"),
                                torch.zeros((8, 64, 32), dtype=torch.bfloat16, device="cuda"))
    assert out.shape == (0, 64)


# ---------------------------------------------------------------- full-size configs
def _full_case(moe, name, bm=None):
    """Every config at its full size in the launch configuration the benchmark
    times: routing bit-exact and the whole [T, H] output against the oracle's
    layer (a per-expert loop over all tokens)."""
    cfg = W.CONFIGS[name]
    if bm is not None:
        cfg = dataclasses.replace(cfg, block_m=bm)
    print(f"full-size {name} bm={cfg.block_m}", flush=True)
    inp = W.make_inputs(cfg)
    out, routing = _run_fused(moe, cfg, inp, bm)
    ref = O.moe_forward_cfg(cfg, inp)
    _check_routing(routing, ref, cfg.T, cfg.top_k, cfg.block_m)
    max_abs, rel = assert_out_close(out, ref["out"], name)
    print(f"full-size {name}: max|d|={max_abs:.3g} rel-L2={rel:.3g}", flush=True)


@pytest.mark.parametrize("name", ["decode_t1", "decode_t3", "decode_t8", "relu2_t1", "relu2_t16"])
def test_full_decode_configs(moe, name):
    _full_case(moe, name)


@pytest.mark.parametrize("name", ["dsv3", "dsv3_s2.5", "zipf128", "relu2_t2048"])
def test_full_prefill_configs(moe, name):
    _full_case(moe, name)


@pytest.mark.parametrize("name,bm", [("dsv3", 128), ("dsv3", 256), ("zipf128", 128),
                                     ("zipf128", 256), ("relu2_t2048", 256)])
def test_full_prefill_block_m(moe, name, bm):
    """The full-size prefill layers laid out at the other large BLOCK_M."""
    _full_case(moe, name, bm)
