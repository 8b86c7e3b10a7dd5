"""Top-k ties on every gating path of the HIP library.

Experts are ranked by logit, ties going to the lower expert index (the rule
applied to the skill card's *Token-Expert Routing* step 1); +0.0 and -0.0 are
equal keys.  The logits here are built with exact ties (whole rows equal,
values on a 0.5 grid, signed zeros, three experts competing for the k-th
place, groups with equal scores), and every gating kernel is reached through
the C ABI by the shape that selects it:

* decode routing prologue of the first expert GEMV: T <= 16 and T*k < 48;
* the decode route kernel: T <= 16 and T*k >= 48;
* gating fused into the one-workgroup align: 16 < T <= 64 and T*k <= 1024;
* the gating kernel: T > 64;
* the router-logit GEMM with gating (moe_fused_forward_router), for which
  zero token rows give all-zero logits and duplicated router rows equal ones.

topk_ids, sorted_token_ids, expert_ids and num_tokens_post_padded must be bit
for bit the oracle's; weights and the layer output are held to the usual bars.
"""

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


def _check_routing(r, ids, wts, E, bm):
    assert int(r["status"].item()) == 0, "status word set"
    got_ids = r["topk_ids"].cpu().numpy()
    assert np.array_equal(got_ids, ids), f"topk_ids\n{got_ids}\n{ids}"
    np.testing.assert_allclose(r["topk_weights"].cpu().numpy(), wts, rtol=2e-6, atol=1e-7)
    al = O.align(ids, E, bm)
    nt = int(r["num_tokens_post_padded"].cpu().item())
    assert nt == al["num_tokens_post_padded"]
    assert np.array_equal(r["sorted_token_ids"].cpu().numpy()[:nt], al["sorted_token_ids"])
    assert np.array_equal(r["expert_ids"].cpu().numpy()[:nt // bm], al["expert_ids"])


def _no_near_group_ties(logits, n_group):
    """Group scores of one token are either exactly equal or far apart, so the
    CPU's and the GPU's float64 exp cannot order them differently."""
    gs = O.group_scores(logits, n_group)
    d = np.abs(gs[:, :, None] - gs[:, None, :])
    assert not np.any((d > 0) & (d < 1e-9)), "near-tie of group scores in the test input"


def _run_case(moe, cfg, logits):
    inp = W.make_inputs(cfg)
    inp["logits"] = logits
    if cfg.n_group > 1:
        _no_near_group_ties(logits, cfg.n_group)
    ref = O.moe_forward_cfg(cfg, inp)
    p = moe.LayerParams.from_config(cfg)
    sh = [to_dev(inp["shared_w13"]), to_dev(inp["shared_w2"])] if cfg.n_shared else [None, None]
    out, r = moe.moe_fused_forward(p, to_dev(inp["x"]), to_dev(logits), to_dev(inp["w13"]),
                                   to_dev(inp["w2"]), *sh, return_routing=True)
    torch.cuda.synchronize()
    _check_routing(r, ref["topk_ids"], ref["topk_weights"], cfg.E, cfg.block_m)
    assert_out_close(out.cpu().numpy(), ref["out"], cfg.name)
    return ref


# (label, T, E, k, block_m): the shape picks the gating kernel
PATHS = [
    ("prologue_t1", 1, 128, 8, 16),
    ("prologue_t3", 3, 128, 8, 16),
    ("prologue_t16_k2", 16, 32, 2, 16),
    ("prologue_e256_k16", 2, 256, 16, 16),
    ("route_kernel_t6", 6, 128, 8, 16),
    ("route_kernel_e256_k16", 16, 256, 16, 16),
    ("align_fused_t17", 17, 64, 4, 16),
    ("align_fused_t64_e256_k16", 64, 256, 16, 32),
    ("gate_kernel_t65", 65, 128, 8, 64),
    ("gate_kernel_t300_e256_k16", 300, 256, 16, 128),
]


@pytest.mark.parametrize("mode", ["equal", "coarse", "signed_zero", "kth"])
@pytest.mark.parametrize("label,T,E,k,bm", PATHS, ids=[p[0] for p in PATHS])
def test_ties_softmax(moe, label, T, E, k, bm, mode):
    print(f"ties softmax {label} mode={mode}", flush=True)
    cfg = W.small_config(f"ties_{label}_{mode}", T=T, H=64, I=32, E=E, top_k=k, block_m=bm)
    ref = _run_case(moe, cfg, W.make_tie_logits(T, E, k, mode))
    if mode == "equal":   # a full tie keeps experts 0 .. k-1
        assert np.array_equal(ref["topk_ids"], np.tile(np.arange(k, dtype=np.int32), (T, 1)))


@pytest.mark.parametrize("mode", ["equal", "kth"])
@pytest.mark.parametrize("T", [2, 8, 40, 100])
def test_ties_softmax_no_renorm(moe, T, mode):
    """Without renormalisation the weights use the full softmax denominator."""
    print(f"ties no-renorm T={T} mode={mode}", flush=True)
    cfg = W.small_config(f"ties_norenorm_{T}_{mode}", T=T, H=64, I=32, E=32, top_k=6,
                         renormalize=0)
    _run_case(moe, cfg, W.make_tie_logits(T, 32, 6, mode))


# grouped sigmoid routing (DeepSeek-V3 shaped: 18 experts, 6 groups keep 4,
# top-4, shared expert) and a wider grouping; T picks the gating kernel as above
@pytest.mark.parametrize("mode", ["equal", "groups_equal", "groups_two", "kth"])
@pytest.mark.parametrize("T", [1, 5, 14, 40, 100])
@pytest.mark.parametrize("E,n_group,topk_group,k", [(18, 6, 4, 4), (64, 8, 3, 6)])
def test_ties_grouped_sigmoid(moe, E, n_group, topk_group, k, T, mode):
    print(f"ties grouped E={E} T={T} mode={mode}", flush=True)
    cfg = W.small_config(f"ties_grouped_{E}_{T}_{mode}", T=T, H=64, I=32, E=E, top_k=k,
                         scoring=W.SCORE_SIGMOID, n_group=n_group, topk_group=topk_group,
                         n_shared=1, block_m=32, scale=2.5)
    ref = _run_case(moe, cfg, W.make_tie_logits(T, E, k, mode, n_group=n_group))
    if mode in ("equal", "groups_equal"):
        # every group score ties: the lowest topk_group groups are kept
        gs = E // n_group
        assert ref["topk_ids"].max() < topk_group * gs


@pytest.mark.parametrize("T", [1, 3, 8, 40, 100])
def test_ties_block_m_sweep(moe, T):
    """The same tied routing laid out at every BLOCK_M."""
    logits = W.make_tie_logits(T, 16, 3, "coarse", seed=7)
    for bm in (16, 32, 64, 128, 256):
        print(f"ties bm sweep T={T} bm={bm}", flush=True)
        cfg = W.small_config(f"ties_bm_{T}_{bm}", T=T, H=64, I=32, E=16, top_k=3, block_m=bm)
        _run_case(moe, cfg, logits)


# ---------------------------------------------------------------- router path
ROUTER = [
    W.small_config("rt_ties_decode_t3", T=3, H=128, I=64, E=128, top_k=8),
    W.small_config("rt_ties_decode_fused_t8", T=8, H=128, I=64, E=64, top_k=8),
    W.small_config("rt_ties_dsv3_t40", T=40, H=128, I=64, E=18, top_k=4, scoring=W.SCORE_SIGMOID,
                   n_group=6, topk_group=4, n_shared=1, block_m=32),
    W.small_config("rt_ties_e256_t100", T=100, H=64, I=32, E=256, top_k=16, block_m=64),
]


@pytest.mark.parametrize("cfg", ROUTER, ids=[c.name for c in ROUTER])
def test_ties_router(moe, cfg):
    """Logits formed by the library: every third token row is zero (all
    logits +0: a full tie) and router rows come in equal pairs (expert 2j+1
    copies expert 2j, so their logits are equal whatever the accumulation
    order).  Routing is checked bit-exact against the oracle's gating of the
    kernel's own logits."""
    print(f"ties router {cfg.name}", flush=True)
    inp = W.make_inputs(cfg)
    x = inp["x"].copy()
    x[::3] = 0
    inp["x"] = x
    wr = W.make_router_weight(cfg).copy()
    wr[1::2] = wr[0::2][:wr[1::2].shape[0]]
    p = moe.LayerParams.from_config(cfg)
    sh = [to_dev(inp["shared_w13"]), to_dev(inp["shared_w2"])] if cfg.n_shared else [None, None]
    out, r = moe.moe_fused_forward_router(p, to_dev(x), to_dev(wr), to_dev(inp["w13"]),
                                          to_dev(inp["w2"]), *sh, return_routing=True)
    torch.cuda.synchronize()
    lg = r["router_logits"].cpu().numpy()
    assert np.all(lg[::3] == 0.0), "zero rows must give zero logits"
    assert np.array_equal(lg[:, 1::2], lg[:, 0::2][:, :lg[:, 1::2].shape[1]]), "paired rows"
    if cfg.n_group > 1:
        _no_near_group_ties(lg, cfg.n_group)
    ids, wts = O.gate(lg, cfg.top_k, cfg.scoring, cfg.n_group, cfg.topk_group, cfg.renormalize,
                      cfg.scale)
    zero_rows = ids[::3]
    if cfg.n_group == 1:
        assert np.array_equal(zero_rows, np.tile(np.arange(cfg.top_k), (zero_rows.shape[0], 1)))
    _check_routing(r, ids, wts, cfg.E, cfg.block_m)
    x64 = O.bf16_to_f64(inp["x"])
    shw = [O.bf16_to_f64(inp["shared_w13"]), O.bf16_to_f64(inp["shared_w2"])] if cfg.n_shared \
        else [None, None]
    want = O.expert_loop(x64, O.bf16_to_f64(inp["w13"]), O.bf16_to_f64(inp["w2"]), ids, wts,
                         cfg.activation, *shw)
    assert_out_close(out.cpu().numpy(), want, cfg.name)


def test_ties_mxfp8_decode(moe):
    """The MXFP8 decode form shares the routing prologue: tied logits there too."""
    cfg = W.small_config("mx_ties", T=3, H=128, I=64, E=64, top_k=8)
    print("ties mxfp8 decode", flush=True)
    inp = W.make_inputs(cfg)
    inp["logits"] = W.make_tie_logits(3, 64, 8, "kth")
    mx = W.make_mxfp8_weights(inp)
    ref = O.moe_forward_mxfp8_cfg(cfg, inp, mx)
    p = moe.LayerParams.from_config(cfg)
    out, r = moe.moe_fused_forward_mxfp8(p, to_dev(inp["x"]), to_dev(inp["logits"]),
                                         to_dev(mx["w13_q"]), to_dev(mx["w13_s"]),
                                         to_dev(mx["w2_q"]), to_dev(mx["w2_s"]),
                                         return_routing=True)
    torch.cuda.synchronize()
    _check_routing(r, ref["topk_ids"], ref["topk_weights"], cfg.E, cfg.block_m)
    assert_out_close(out.cpu().numpy(), ref["out"], cfg.name)
