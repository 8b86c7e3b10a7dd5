"""Parity of the indexed (contiguous) grouped GEMM against the oracle.

out[i] = x[i] @ w[expert_indices[i]].T through moe_align (top-1) and
moe_grouped_gemm (scatter by slot, weight 1).  Small cases are compared
element by element; the four full-size scenarios of the axolotl page's
benchmark table are run in the launch configuration the benchmark times and
checked on sampled rows (first and last row of every group plus random ones),
with every output row required to be written.
"""
import numpy as np
import pytest

from grouped_gemm_topk_amd import workloads as W
from oracle import moe_oracle as O
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def moe():
    from grouped_gemm_topk_amd import moe as M
    M.lib()
    return M


def _tol(ref, fp32):
    # bf16 output: one bf16 step of the value (round-to-nearest of an fp32
    # result that may sit on the other side of a rounding boundary); fp32:
    # accumulation-order differences over K
    rel = 1e-5 if fp32 else 2.0 ** -8
    return rel * np.abs(ref) + 1e-4 * np.abs(ref).max()


SMALL = [
    W.small_gemm_scenario("cg_uniform_pad"),                                   # 160-row groups, BM 128
    W.small_gemm_scenario("cg_uneven_empty", sizes=(0, 200, 280)),
    W.small_gemm_scenario("cg_shuffled", sizes=(100, 3, 377), shuffled=True),
    W.small_gemm_scenario("cg_g8_bm64", G=8, M=8 * 70, N=136, K=264, block_m=64),
    W.small_gemm_scenario("cg_g8_bm32", G=8, M=8 * 33, N=64, K=72, block_m=32),
    W.small_gemm_scenario("cg_g5_bm16", G=5, M=5 * 21, N=520, K=48, block_m=16),
    W.small_gemm_scenario("cg_g1", G=1, M=300, N=256, K=128),
    W.small_gemm_scenario("cg_one_row", G=4, M=1, N=64, K=64, sizes=(0, 0, 1, 0)),
]


@pytest.mark.parametrize("sc", SMALL, ids=[s.name for s in SMALL])
@pytest.mark.parametrize("fp32", [False, True], ids=["bf16", "fp32"])
def test_indexed_grouped_gemm_small(moe, sc, fp32):
    print(f"indexed grouped gemm {sc.name} fp32={fp32}", flush=True)
    inp = W.make_gemm_inputs(sc)
    ref = O.indexed_grouped_gemm(O.bf16_to_f64(inp["x"]), O.bf16_to_f64(inp["w"]),
                                 inp["expert_indices"])
    out = torch.full((sc.M, sc.N), float("nan"), device="cuda",
                     dtype=torch.float32 if fp32 else torch.bfloat16)
    moe.indexed_grouped_gemm(to_dev(inp["x"]), to_dev(inp["w"]), to_dev(inp["expert_indices"]),
                             sc.block_m, out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.all(np.isfinite(got)), "rows left unwritten"
    bad = np.abs(got - ref) > _tol(ref, fp32)
    assert not bad.any(), f"{bad.sum()} mismatches, worst {np.abs(got - ref).max()}"


def test_indexed_grouped_gemm_reuse_and_new_indices(moe):
    """The same object run twice, then with other indices written into its
    index tensor: every run reflects the indices it saw."""
    sc = W.small_gemm_scenario("cg_reuse", sizes=(50, 150, 280))
    inp = W.make_gemm_inputs(sc)
    xd, wd = to_dev(inp["x"]), to_dev(inp["w"])
    idx = to_dev(inp["expert_indices"])
    op = moe.IndexedGroupedGemm(xd, wd, idx, sc.block_m)
    x64, w64 = O.bf16_to_f64(inp["x"]), O.bf16_to_f64(inp["w"])
    for rep, new in enumerate([None, None, np.random.default_rng(3).integers(0, 3, sc.M)]):
        if new is not None:
            idx.copy_(torch.from_numpy(new.astype(np.int32)))
            ids_np = new
        else:
            ids_np = inp["expert_indices"]
        got = op.run().float().cpu().numpy()
        ref = O.indexed_grouped_gemm(x64, w64, ids_np)
        assert not (np.abs(got - ref) > _tol(ref, False)).any(), f"run {rep}"


FULL = list(W.GEMM_SCENARIOS.values())


SCHED = [
    # more tiles than CUs, so that the persistent grid runs tile sequences:
    # 190 m-blocks x 3 n-tiles at BLOCK_M 128, 120 x 4 at 256 (ragged K)
    W.small_gemm_scenario("sched_bm128", G=6, M=6 * 4000, N=520, K=264, block_m=128),
    W.small_gemm_scenario("sched_bm256", G=5, M=5 * 6000, N=1000, K=200, block_m=256),
    # 80 m-blocks x 4 n-tiles = 320 tiles: on 256 CUs the last round's 64
    # tiles run in 64-column slices
    W.small_gemm_scenario("sched_bm256_split", G=5, M=5 * 3900, N=1000, K=200, block_m=256),
    W.small_gemm_scenario("sched_bm64", G=8, M=8 * 70, N=136, K=264, block_m=64),
]


@pytest.mark.parametrize("sc", SCHED, ids=[s.name for s in SCHED])
def test_indexed_grouped_gemm_schedules(moe, sc):
    """One workgroup per tile (MOE_SCHED_PER_TILE) against the persistent
    default: the same output bit for bit, and both against the oracle."""
    print(f"indexed grouped gemm schedules {sc.name}", flush=True)
    inp = W.make_gemm_inputs(sc)
    ref = O.indexed_grouped_gemm(O.bf16_to_f64(inp["x"]), O.bf16_to_f64(inp["w"]),
                                 inp["expert_indices"])
    outs = []
    for sched in (moe.SCHED_PERSISTENT, moe.SCHED_PER_TILE):
        out = torch.full((sc.M, sc.N), float("nan"), device="cuda", dtype=torch.float32)
        op = moe.IndexedGroupedGemm(to_dev(inp["x"]), to_dev(inp["w"]),
                                    to_dev(inp["expert_indices"]), sc.block_m, out)
        op.align()
        op.gemm(schedule=sched)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    for got in outs:
        assert np.all(np.isfinite(got)), "rows left unwritten"
        bad = np.abs(got - ref) > _tol(ref, True)
        assert not bad.any(), f"{bad.sum()} mismatches, worst {np.abs(got - ref).max()}"
    assert np.array_equal(outs[0], outs[1]), "the schedules disagree"


@pytest.mark.parametrize("sc", FULL, ids=[s.name for s in FULL])
def test_indexed_grouped_gemm_full_size_sampled(moe, sc):
    print(f"indexed grouped gemm full size {sc.name}", flush=True)
    inp = W.make_gemm_inputs(sc)
    out = torch.full((sc.M, sc.N), float("nan"), device="cuda", dtype=torch.bfloat16)
    op = moe.IndexedGroupedGemm(to_dev(inp["x"]), to_dev(inp["w"]), to_dev(inp["expert_indices"]),
                                sc.block_m, out)
    op.run()
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "rows left unwritten"
    idx = inp["expert_indices"]
    starts = np.flatnonzero(np.r_[True, idx[1:] != idx[:-1]])
    ends = np.r_[starts[1:], sc.M] - 1
    rng = np.random.default_rng(11)
    rows = np.unique(np.r_[starts, ends, rng.integers(0, sc.M, 24)])
    ref = O.indexed_grouped_gemm(O.bf16_to_f64(inp["x"]), O.bf16_to_f64(inp["w"]), idx, rows=rows)
    got = out[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    bad = np.abs(got - ref) > _tol(ref, False)
    assert not bad.any(), f"{bad.sum()} mismatches, worst {np.abs(got - ref).max()}"


def test_indexed_grouped_gemm_graph_replays(moe):
    """Captured once (align + GEMM) and replayed with eager work in between:
    every replay equals the eager result bit for bit."""
    sc = W.small_gemm_scenario("cg_graph", G=6, M=6 * 300, N=384, K=256, sizes=(0, 700, 300, 1, 499, 300))
    inp = W.make_gemm_inputs(sc)
    op = moe.IndexedGroupedGemm(to_dev(inp["x"]), to_dev(inp["w"]), to_dev(inp["expert_indices"]),
                                sc.block_m)
    eager = op.run().clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        op.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = op.run()
    torch.cuda.synchronize()
    for rep in range(3):
        op.out.fill_(float("nan"))
        op.sorted.fill_(-7)
        if rep == 1:
            op.run()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"


# ---------------------------------------------------------------- backward
BWD_SMALL = SMALL + [
    W.small_gemm_scenario("cg_bwd_g6_uneven", G=6, M=900, N=264, K=136,
                          sizes=(0, 400, 1, 250, 0, 249), block_m=64),
    W.small_gemm_scenario("cg_bwd_empty_rows", G=3, M=0, N=64, K=64, sizes=(0, 0, 0)),
    # 512 weight-gradient tiles on the persistent grid, whose tile sequences
    # change K (the expert's padded rows: 0, 1024, 128, 1536) from tile to
    # tile: 256-row tiles (N >= 1024; 8 x 16 per expert) and 128-row tiles
    # (8 x 16 per expert)
    W.small_gemm_scenario("cg_bwd_persistent", G=4, M=2400, N=2048, K=4096,
                          sizes=(0, 900, 1, 1499)),
    W.small_gemm_scenario("cg_bwd_persistent_128", G=4, M=2400, N=1000, K=4096,
                          sizes=(0, 900, 1, 1499)),
]


@pytest.mark.parametrize("sc", BWD_SMALL, ids=[s.name for s in BWD_SMALL])
@pytest.mark.parametrize("fp32", [False, True], ids=["bf16", "fp32"])
def test_indexed_grouped_gemm_backward_small(moe, sc, fp32):
    print(f"indexed grouped gemm backward {sc.name} fp32={fp32}", flush=True)
    inp = W.make_gemm_inputs(sc, with_grad=True)
    x64, w64, dy64 = (O.bf16_to_f64(inp[k]) for k in ("x", "w", "dy"))
    rdx, rdw = O.indexed_grouped_gemm_backward(x64, w64, inp["expert_indices"], dy64)
    op = moe.IndexedGroupedGemm(to_dev(inp["x"]), to_dev(inp["w"]), to_dev(inp["expert_indices"]),
                                sc.block_m)
    op.align()
    dt = torch.float32 if fp32 else torch.bfloat16
    dx = torch.full((sc.M, sc.K), float("nan"), dtype=dt, device="cuda")
    dw = torch.full((sc.G, sc.N, sc.K), float("nan"), dtype=dt, device="cuda")
    op.backward(to_dev(inp["dy"]), dx, dw, out_fp32=fp32)
    torch.cuda.synchronize()
    gx, gw = dx.float().cpu().numpy(), dw.float().cpu().numpy()
    assert np.all(np.isfinite(gx)) and np.all(np.isfinite(gw)), "outputs left unwritten"
    if sc.M:
        assert not (np.abs(gx - rdx) > _tol(rdx, fp32)).any(), f"dx worst {np.abs(gx - rdx).max()}"
    tw = _tol(rdw, fp32) if np.abs(rdw).max() > 0 else 0.0
    assert not (np.abs(gw - rdw) > tw).any(), f"dw worst {np.abs(gw - rdw).max()}"


def test_indexed_grouped_gemm_backward_one_side(moe):
    """dx alone and dw alone (the other pointer NULL) give the same values."""
    sc = W.small_gemm_scenario("cg_bwd_sides", sizes=(100, 200, 180))
    inp = W.make_gemm_inputs(sc, with_grad=True)
    op = moe.IndexedGroupedGemm(to_dev(inp["x"]), to_dev(inp["w"]), to_dev(inp["expert_indices"]),
                                sc.block_m)
    op.align()
    dy = to_dev(inp["dy"])
    dx_both, dw_both = op.backward(dy)
    dx_only, none_w = op.backward(dy, want_dw=False)
    none_x, dw_only = op.backward(dy, want_dx=False)
    torch.cuda.synchronize()
    assert none_w is None and none_x is None
    assert torch.equal(dx_both, dx_only) and torch.equal(dw_both, dw_only)


@pytest.mark.parametrize("sc", FULL, ids=[s.name for s in FULL])
def test_indexed_grouped_gemm_backward_full_size_sampled(moe, sc):
    print(f"indexed grouped gemm backward full size {sc.name}", flush=True)
    inp = W.make_gemm_inputs(sc, with_grad=True)
    op = moe.IndexedGroupedGemm(to_dev(inp["x"]), to_dev(inp["w"]), to_dev(inp["expert_indices"]),
                                sc.block_m)
    op.align()
    dx = torch.full((sc.M, sc.K), float("nan"), dtype=torch.bfloat16, device="cuda")
    dw = torch.full((sc.G, sc.N, sc.K), float("nan"), dtype=torch.bfloat16, device="cuda")
    op.backward(to_dev(inp["dy"]), dx, dw)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(dx).all()) and bool(torch.isfinite(dw).all()), "outputs left unwritten"
    idx = inp["expert_indices"]
    rng = np.random.default_rng(12)
    starts = np.flatnonzero(np.r_[True, idx[1:] != idx[:-1]])
    xrows = np.unique(np.r_[starts, np.r_[starts[1:], sc.M] - 1, rng.integers(0, sc.M, 16)])
    wrows = [(e, int(n)) for e in range(sc.G) for n in np.r_[0, sc.N - 1, rng.integers(0, sc.N, 2)]]
    sx, sw = O.indexed_grouped_gemm_backward(O.bf16_to_f64(inp["x"]), O.bf16_to_f64(inp["w"]), idx,
                                             O.bf16_to_f64(inp["dy"]), dx_rows=xrows, dw_rows=wrows)
    gx = dx[torch.from_numpy(xrows).cuda()].float().cpu().numpy()
    gw = np.stack([dw[e, n].float().cpu().numpy() for e, n in wrows])
    assert not (np.abs(gx - sx) > _tol(sx, False)).any(), f"dx worst {np.abs(gx - sx).max()}"
    assert not (np.abs(gw - sw) > _tol(sw, False)).any(), f"dw worst {np.abs(gw - sw).max()}"


def test_indexed_grouped_gemm_backward_graph_replays(moe):
    """align + backward (dx, dw) captured once and replayed with eager work in
    between: every replay equals the eager result bit for bit (the layout
    kernels and the GEMMs are deterministic)."""
    sc = W.small_gemm_scenario("cg_bwd_graph", G=5, M=900, N=264, K=200, sizes=(0, 400, 1, 250, 249),
                               block_m=64)
    inp = W.make_gemm_inputs(sc, with_grad=True)
    op = moe.IndexedGroupedGemm(to_dev(inp["x"]), to_dev(inp["w"]), to_dev(inp["expert_indices"]),
                                sc.block_m)
    dy = to_dev(inp["dy"])
    dx = torch.empty((sc.M, sc.K), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((sc.G, sc.N, sc.K), dtype=torch.bfloat16, device="cuda")

    def step():
        op.align()
        op.backward(dy, dx, dw)

    step()
    torch.cuda.synchronize()
    ex, ew = dx.clone(), dw.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        dx.fill_(float("nan"))
        dw.fill_(float("nan"))
        if rep == 1:
            step()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dx, ex) and torch.equal(dw, ew), f"replay {rep}"
