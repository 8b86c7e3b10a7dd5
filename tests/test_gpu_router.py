"""Parity of the layer with the router's linear layer fused into gating
(moe_fused_forward_router).

The kernel forms the router logits in fp32 and decides the routing on them,
so: the logits match the oracle's float64 product within the fp32 dot-product
error bound (H * 2^-24 times the sum of |x_h w_eh|); the routing outputs are
bit-exact against the oracle's gating and align of those same fp32 logits
(the decision taken in the kernel's precision); and the output meets the
usual bar against the oracle's layer with that routing.
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


def _run(moe, cfg, inp, wr):
    p = moe.LayerParams.from_config(cfg)
    sh = [to_dev(inp["shared_w13"]), to_dev(inp["shared_w2"])] if cfg.n_shared else [None, None]
    out, r = moe.moe_fused_forward_router(p, to_dev(inp["x"]), to_dev(wr), to_dev(inp["w13"]),
                                          to_dev(inp["w2"]), *sh, return_routing=True)
    torch.cuda.synchronize()
    return out.cpu().numpy(), {k: v.cpu().numpy() for k, v in r.items()}


def _check_logits(inp, wr, got):
    x64, w64 = O.bf16_to_f64(inp["x"]), O.bf16_to_f64(wr)
    ref = O.router_logits(x64, w64)
    bound = x64.shape[1] * 2.0 ** -24 * (np.abs(x64) @ np.abs(w64).T) * 1.01 + 1e-30
    assert not (np.abs(got - ref) > bound).any(), f"logits worst {np.abs(got - ref).max()}"


def _check_routing(cfg, r):
    assert int(r["status"][0]) == 0, "status word set"
    ids, wts = O.gate(r["router_logits"], cfg.top_k, cfg.scoring, cfg.n_group, cfg.topk_group,
                      cfg.renormalize, cfg.scale)
    assert np.array_equal(r["topk_ids"], ids)
    np.testing.assert_allclose(r["topk_weights"], wts, rtol=1e-5, atol=1e-7)
    al = O.align(ids, cfg.E, cfg.block_m)
    nt = int(r["num_tokens_post_padded"][0])
    assert nt == al["num_tokens_post_padded"]
    assert np.array_equal(r["sorted_token_ids"][:nt], al["sorted_token_ids"])
    assert np.array_equal(r["expert_ids"][:nt // cfg.block_m], al["expert_ids"])
    return ids, wts


SMALL = [
    W.small_config("rt_softmax", T=37, H=64, I=96, E=8, top_k=2),
    W.small_config("rt_ragged_h", T=90, H=136, I=72, E=16, top_k=3, activation=W.ACT_RELU2),
    W.small_config("rt_dsv3", T=70, H=128, I=64, E=18, top_k=4, scoring=W.SCORE_SIGMOID,
                   n_group=6, topk_group=4, n_shared=1, block_m=32),
    W.small_config("rt_max_e_k", T=20, H=64, I=32, E=256, top_k=16),
    W.small_config("rt_decode_t3", T=3, H=256, I=128, E=128, top_k=8),
    W.small_config("rt_decode_fused", T=8, H=256, I=128, E=64, top_k=8),
    W.small_config("rt_t0", T=0, H=64, I=32, E=8, top_k=2),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_router_layer_small(moe, cfg):
    print(f"router layer {cfg.name}", flush=True)
    inp = W.make_inputs(cfg)
    wr = W.make_router_weight(cfg)
    got, r = _run(moe, cfg, inp, wr)
    if cfg.T == 0:
        return
    _check_logits(inp, wr, r["router_logits"])
    ids, wts = _check_routing(cfg, r)
    x64 = O.bf16_to_f64(inp["x"])
    sh = [O.bf16_to_f64(inp["shared_w13"]), O.bf16_to_f64(inp["shared_w2"])] if cfg.n_shared else [None, None]
    want = O.expert_loop(x64, O.bf16_to_f64(inp["w13"]), O.bf16_to_f64(inp["w2"]), ids, wts,
                         cfg.activation, *sh).astype(np.float64)
    err = np.abs(got - want)
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert err.max() <= 2e-2 and rel <= 5e-3, f"max|d|={err.max():.3g} rel-L2={rel:.3g}"


@pytest.mark.parametrize("name", ["dsv3", "decode_t1"])
def test_router_layer_full_size(moe, name):
    print(f"router layer full size {name}", flush=True)
    cfg = W.CONFIGS[name]
    inp = W.make_inputs(cfg)
    wr = W.make_router_weight(cfg)
    got, r = _run(moe, cfg, inp, wr)
    _check_logits(inp, wr, r["router_logits"])
    ids, wts = _check_routing(cfg, r)
    # the whole [T, H] output against the oracle's layer on that routing
    x64 = O.bf16_to_f64(inp["x"])
    sh = [O.bf16_to_f64(inp["shared_w13"]), O.bf16_to_f64(inp["shared_w2"])] if cfg.n_shared \
        else [None, None]
    want = O.expert_loop(x64, O.bf16_to_f64(inp["w13"]), O.bf16_to_f64(inp["w2"]), ids, wts,
                         cfg.activation, *sh)
    max_abs, rel = assert_out_close(got, want, name)
    print(f"router layer full size {name}: max|d|={max_abs:.3g} rel-L2={rel:.3g}", flush=True)


@pytest.mark.parametrize("cfg", [
    W.small_config("rt_graph_prefill", T=70, H=128, I=64, E=18, top_k=4, scoring=W.SCORE_SIGMOID,
                   n_group=6, topk_group=4, n_shared=1, block_m=32),
    W.small_config("rt_graph_decode", T=3, H=256, I=128, E=64, top_k=8),
], ids=["prefill", "decode"])
def test_router_layer_graph_replays(moe, cfg):
    """The router-fused layer captured once and replayed with eager work in
    between: every replay within fp32 reassociation of the eager result."""
    inp = W.make_inputs(cfg)
    p = moe.LayerParams.from_config(cfg)
    sh = [to_dev(inp["shared_w13"]), to_dev(inp["shared_w2"])] if cfg.n_shared else [None, None]
    layer = moe.FusedLayer(p, to_dev(inp["x"]), None, to_dev(inp["w13"]), to_dev(inp["w2"]), *sh,
                           router_w=to_dev(W.make_router_weight(cfg)))
    eager = layer.run().clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = layer.run()
    torch.cuda.synchronize()
    want = eager.cpu().numpy()
    for rep in range(3):
        layer.tensors["out"].fill_(float("nan"))
        if rep == 1:
            layer.run()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_allclose(out.cpu().numpy(), want, rtol=1e-5,
                                   atol=1e-6 * np.abs(want).max(), err_msg=f"replay {rep}")
