"""Graph replays of the fused forward.

The layer is captured once into a graph and replayed several times, with the
program's own eager work (other kernels, an eager run of the same layer) in
between.  Every replay must reproduce the eager result: bit for bit on the
prefill path, whose reduction order is fixed; within fp32 reassociation on the
decode path, whose routed contributions meet in fp32 atomics.  The kernels
clear what they accumulate into with ordinary stores, so a replay does not
depend on state left by the previous one.
"""
import numpy as np
import pytest

from grouped_gemm_topk_amd import workloads as W
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def moe():
    from grouped_gemm_topk_amd import moe as M
    M.lib()
    return M


CASES = [
    ("decode_t1", W.CONFIGS["decode_t1"], False),
    ("decode_t8", W.CONFIGS["decode_t8"], False),
    ("prefill_dsv3_small", W.small_config("prefill_dsv3_small", T=200, H=256, I=192, E=18,
                                          top_k=4, scoring=W.SCORE_SIGMOID, n_group=6,
                                          topk_group=4, n_shared=1, block_m=128), True),
    ("prefill_softmax_small", W.small_config("prefill_softmax_small", T=333, H=128, I=96,
                                             E=8, top_k=2, block_m=64), True),
    # the persistent 128-row grid (loader / compute split), several tiles per
    # workgroup in both GEMMs
    ("prefill_persistent_128", W.small_config("prefill_persistent_128", T=16384, H=104, I=520,
                                              E=4, top_k=2, block_m=128), True),
    # 256-row tiles whose last rounds (24 of 280 tiles in each GEMM on 256
    # CUs) run in 64-column slices
    ("prefill_split_256", W.small_config("prefill_split_256", T=8600, H=1000, I=504, E=4,
                                         top_k=2, block_m=256), True),
]


@pytest.mark.parametrize("name,cfg,exact", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(moe, name, cfg, exact):
    print(f"graph replay {name}", flush=True)
    inp = W.make_inputs(cfg)
    p = moe.LayerParams.from_config(cfg)
    sh = [to_dev(inp["shared_w13"]), to_dev(inp["shared_w2"])] if cfg.n_shared else [None, None]
    layer = moe.FusedLayer(p, to_dev(inp["x"]), to_dev(inp["logits"]), to_dev(inp["w13"]),
                           to_dev(inp["w2"]), *sh, routing_outputs=True)
    eager = layer.run().clone()
    eager_ids = layer.routing["sorted_token_ids"].clone()
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on the capture stream, as torch requires
        layer.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = layer.run()
    torch.cuda.synchronize()

    junk = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    for rep in range(3):
        # eager work between the replays: unrelated kernels that overwrite
        # the output and workspace-sized buffers, and an eager run
        junk.fill_(float(rep + 1))
        layer.tensors["out"].fill_(float("nan"))
        if rep == 1:
            layer.run()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        want = eager.cpu().numpy()
        assert np.all(np.isfinite(got)), f"replay {rep}: unwritten output"
        if exact:
            assert np.array_equal(got, want), f"replay {rep} differs from the eager run"
        else:
            np.testing.assert_allclose(got, want, rtol=1e-5, atol=1e-6 * np.abs(want).max(),
                                       err_msg=f"replay {rep}")
        ntpp = int(layer.routing["num_tokens_post_padded"].item())
        assert np.array_equal(layer.routing["sorted_token_ids"].cpu().numpy()[:ntpp],
                              eager_ids.cpu().numpy()[:ntpp]), f"replay {rep}: routing"
