"""Parity of the layer on the less common paths of the persistent 128- and
256-row grouped GEMM (one workgroup per CU running a sequence of tiles).

- more than 2048 routed m-blocks: the expert ids no longer fit the LDS copy
  and the tile mapping reads them from global memory;
- several tiles per workgroup with a one-step K loop (K <= 64): the next
  tile's first K steps are requested between the tiles, not ahead;
- a ragged last K step with several tiles per workgroup and the shared
  expert's dense tiles after the routed ones;
- a tile count that is an exact multiple of the CU count;
- two K steps per tile (with the loader waves of the 128-row tile, a tile's
  sorted ids are read three tiles after they are written).
- with 256-row tiles, a last round that fills at most a quarter of the
  grid: each workgroup runs its full rounds and then one of that round's
  tiles' 64-column slices (both GEMMs, ragged K,
  the shared expert's dense tiles in the sliced round, and a layer whose
  W13 launch keeps a last round of half the grid while its W2 launch
  splits).

Routing outputs bit for bit, the output at the layer's bar (max|d| <= 2e-2,
relative-L2 <= 5e-3), against the oracle on the whole output.
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


CASES = [
    # 264000 slots over 8 experts: about 2070 m-blocks of 128 rows (> 2048)
    W.small_config("p_many_blocks", T=33000, H=64, I=32, E=8, top_k=8, block_m=128),
    # K = 200 (three full steps and an 8-element tail), 4 act n-tiles, the
    # shared expert: about 200 m-blocks x 4 = 800 W13 tiles
    W.small_config("p_ragged_k_shared", T=8192, H=200, I=512, E=4, top_k=2, block_m=128,
                   scoring=W.SCORE_SIGMOID, n_group=2, topk_group=2, n_shared=1),
    # one expert, top-1: 128 m-blocks x 4 n-tiles = 512 tiles, two per CU
    W.small_config("p_exact_rounds", T=16384, H=64, I=512, E=1, top_k=1, block_m=128),
    # two K steps per tile (ragged K = 104, then K = 120), several tiles per
    # workgroup: the W13 launch (5 n-tiles x 259 m-blocks), then the W2
    # launch (3 n-tiles x 514 m-blocks); with the loader waves a tile's sorted
    # ids are read three tiles after they are written
    W.small_config("p_two_steps_w13", T=16384, H=104, I=520, E=4, top_k=2, block_m=128),
    W.small_config("p_two_steps_w2", T=32768, H=520, I=120, E=4, top_k=2, block_m=128),
    W.small_config("p_two_steps_w13_256", T=16384, H=104, I=520, E=4, top_k=2, block_m=256),
    # the same paths with 256-row tiles: 528000 slots, about 2070 m-blocks of 256
    W.small_config("p_many_blocks_256", T=66000, H=64, I=32, E=8, top_k=8, block_m=256),
    W.small_config("p_ragged_k_shared_256", T=8192, H=200, I=512, E=4, top_k=2, block_m=256,
                   scoring=W.SCORE_SIGMOID, n_group=2, topk_group=2, n_shared=1),
    # 64 m-blocks x 4 n-tiles = 256 tiles, one per CU
    W.small_config("p_exact_rounds_256", T=16384, H=64, I=512, E=1, top_k=1, block_m=256),
    # on 256 CUs: W13 384 tiles (last round 128: not split), W2 288 tiles
    # (last round 32: split), K = 600 and 400 (ragged)
    W.small_config("p_split_round_256", T=12000, H=600, I=400, E=4, top_k=2, block_m=256),
    # W13 and W2 280 tiles each (last rounds of 24 split), K = 1000 and 504
    W.small_config("p_split_both_256", T=8600, H=1000, I=504, E=4, top_k=2, block_m=256),
    # W13 and W2 312 tiles each (last rounds of 56, the shared expert's among them)
    W.small_config("p_split_round_shared_256", T=8600, H=520, I=384, E=4, top_k=2, block_m=256,
                   scoring=W.SCORE_SIGMOID, n_group=2, topk_group=2, n_shared=1),
]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_persistent_gemm_paths(moe, cfg):
    print(f"persistent gemm {cfg.name}", flush=True)
    inp = W.make_inputs(cfg)
    ref = O.moe_forward_cfg(cfg, inp)
    p = moe.LayerParams.from_config(cfg)
    sh = [to_dev(inp["shared_w13"]), to_dev(inp["shared_w2"])] if cfg.n_shared else [None, None]
    out, r = moe.moe_fused_forward(p, to_dev(inp["x"]), to_dev(inp["logits"]), to_dev(inp["w13"]),
                                   to_dev(inp["w2"]), *sh, return_routing=True)
    torch.cuda.synchronize()
    assert np.array_equal(r["topk_ids"].cpu().numpy(), ref["topk_ids"])
    ntpp = int(r["num_tokens_post_padded"].cpu().item())
    assert ntpp == ref["num_tokens_post_padded"]
    if cfg.name.startswith("p_many_blocks"):
        assert ntpp // cfg.block_m > 2048
    assert np.array_equal(r["sorted_token_ids"].cpu().numpy()[:ntpp], ref["sorted_token_ids"])
    assert np.array_equal(r["expert_ids"].cpu().numpy()[:ntpp // cfg.block_m], ref["expert_ids"])
    assert_out_close(out.cpu().numpy(), ref["out"], cfg.name)
