"""moe_fused_forward_noalloc (no workspace argument; the library's device
scratch instead) against moe_fused_forward on the same inputs, through the C
ABI: two calls in a row on one GPU, the second with fewer tokens, so the
second call runs on scratch the first left written.  Routing must be bit-exact
and the output within the layer's bar (max|d| <= 2e-2, rel-L2 <= 5e-3); the
prefill path is deterministic, so there the output must also be identical.
A layer whose workspace exceeds the scratch is rejected before any launch."""
import numpy as np
import pytest

from grouped_gemm_topk_amd import workloads as W
from tests.helpers import assert_out_close, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def moe():
    from grouped_gemm_topk_amd import moe as M
    M.lib()
    return M


def _routing_bufs(moe, p, dev="cuda"):
    cap = moe.align_capacity(p.T, p.top_k, p.E, p.block_m)
    return dict(topk_ids=torch.full((p.T, p.top_k), -7, dtype=torch.int32, device=dev),
                topk_weights=torch.full((p.T, p.top_k), float("nan"), device=dev),
                sorted_token_ids=torch.full((cap,), -7, dtype=torch.int32, device=dev),
                expert_ids=torch.full((max(cap // p.block_m, 1),), -7, dtype=torch.int32,
                                      device=dev),
                num_tokens_post_padded=torch.full((1,), -7, dtype=torch.int32, device=dev))


def _both(moe, cfg):
    inp = W.make_inputs(cfg)
    p = moe.LayerParams.from_config(cfg)
    args = [to_dev(inp["x"]), to_dev(inp["logits"]), to_dev(inp["w13"]), to_dev(inp["w2"])]
    sh = [to_dev(inp["shared_w13"]), to_dev(inp["shared_w2"])] if cfg.n_shared else [None, None]
    ref, rr = moe.moe_fused_forward(p, *args, *sh, return_routing=True)
    out = torch.full((cfg.T, cfg.H), float("nan"), device="cuda")
    r = _routing_bufs(moe, p)
    moe.moe_fused_forward_noalloc(p, *args, *sh, out=out, routing=r)
    torch.cuda.synchronize()
    nt = int(rr["num_tokens_post_padded"].item())
    assert int(r["num_tokens_post_padded"].item()) == nt
    assert torch.equal(r["topk_ids"], rr["topk_ids"])
    assert torch.equal(r["topk_weights"], rr["topk_weights"])
    assert torch.equal(r["sorted_token_ids"][:nt], rr["sorted_token_ids"][:nt])
    assert torch.equal(r["expert_ids"][:nt // cfg.block_m], rr["expert_ids"][:nt // cfg.block_m])
    got, want = out.cpu().numpy(), ref.cpu().numpy()
    assert_out_close(got, want, cfg.name)
    if cfg.T > 16:   # the prefill kernels are deterministic
        assert np.array_equal(got, want), f"{cfg.name}: prefill output differs"


PAIRS = [
    # prefill (grouped sigmoid, shared expert), then a smaller prefill
    (W.small_config("na_dsv3_256", T=256, H=512, I=256, E=18, top_k=4, scoring=W.SCORE_SIGMOID,
                    n_group=6, topk_group=4, n_shared=1, block_m=64),
     W.small_config("na_dsv3_40", T=40, H=512, I=256, E=18, top_k=4, scoring=W.SCORE_SIGMOID,
                    n_group=6, topk_group=4, n_shared=1, block_m=64)),
    # decode: the fused form (from 48 slots), then the two-GEMV form
    (W.CONFIGS["decode_t8"], W.CONFIGS["decode_t1"]),
    # prefill, then decode on the scratch it left
    (W.CONFIGS["tiny"], W.small_config("na_decode_t3", T=3, H=256, I=512, E=8, top_k=2)),
    # 256-row tiles: a W13 launch of 8 x 40 = 320 tiles on the persistent grid
    # whose last round of 64 runs in 64-column slices, then half the tokens
    (W.small_config("na_split_256", T=2048, H=256, I=5120, E=1, top_k=1, block_m=256),
     W.small_config("na_half_256", T=1024, H=256, I=5120, E=1, top_k=1, block_m=256)),
]


@pytest.mark.parametrize("first,second", PAIRS, ids=[f"{a.name}-then-{b.name}" for a, b in PAIRS])
def test_noalloc_matches_fused_forward(moe, first, second):
    for cfg in (first, second):
        print(f"noalloc {cfg.name} T={cfg.T}", flush=True)
        _both(moe, cfg)


def test_noalloc_rejects_oversized_layer(moe):
    """dsv3 at 4096 tokens needs far more than the scratch: MOE_ERR_CAPACITY,
    nothing written."""
    cfg = W.CONFIGS["dsv3"]
    p = moe.LayerParams.from_config(cfg)
    assert moe.fused_workspace_bytes(p) > moe.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros((cfg.T, cfg.E), device="cuda")
    w13 = torch.zeros((cfg.E, cfg.M1, cfg.H), dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros((cfg.E, cfg.H, cfg.I), dtype=torch.bfloat16, device="cuda")
    sw13 = torch.zeros((cfg.M1, cfg.H), dtype=torch.bfloat16, device="cuda")
    sw2 = torch.zeros((cfg.H, cfg.I), dtype=torch.bfloat16, device="cuda")
    out = torch.full((cfg.T, cfg.H), float("nan"), device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_fused_forward_noalloc(p, x, lg, w13, w2, sw13, sw2, out=out)
    assert ei.value.status == -3
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
