"""Pins of the CPU oracle against things other than itself.

Every function of the oracle is checked here against hand-worked fixtures
(tests/golden), textbook/library routines (stable argsort, scipy softmax and
expit, torch's linear/silu), brute force on tiny inputs (all expert subsets,
all group subsets, the dense every-expert-on-every-token MLP), closed forms and
invariants.  None of these needs a GPU.
"""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import moe_oracle as O
from grouped_gemm_topk_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- top-k
def test_topk_golden_ties():
    for case in _golden("topk_ties.json")["cases"]:
        l = np.array([case["logits"]], dtype=np.float32)
        ids = O.select_topk(l, case["k"])
        assert ids[0].tolist() == case["ids"], case


@pytest.mark.parametrize("seed", range(5))
def test_topk_matches_stable_argsort(seed):
    rng = np.random.default_rng(seed)
    # coarse values force many exact ties
    l = np.round(rng.standard_normal((200, 16)), 1).astype(np.float32)
    for k in (1, 3, 8, 16):
        ref = np.argsort(-l, axis=1, kind="stable")[:, :k]
        assert np.array_equal(O.select_topk(l, k), ref)


@pytest.mark.parametrize("E,k", [(4, 1), (5, 2), (6, 3), (8, 4), (8, 8)])
def test_topk_bruteforce_subsets(E, k):
    rng = np.random.default_rng(E * 10 + k)
    l = rng.standard_normal((30, E)).astype(np.float32)   # distinct almost surely
    ids = O.select_topk(l, k)
    for t in range(l.shape[0]):
        best = max(itertools.combinations(range(E), k), key=lambda S: sum(float(l[t, e]) for e in S))
        assert set(ids[t].tolist()) == set(best)
        # selection order is by descending key
        keys = l[t, ids[t]]
        assert np.all(keys[:-1] >= keys[1:])


# ---------------------------------------------------------------- grouped routing
def _bruteforce_grouped(l, k, n_group, topk_group):
    T, E = l.shape
    gsize = E // n_group
    s = 1.0 / (1.0 + np.exp(-l.astype(np.float64)))
    gscore = np.sort(s.reshape(T, n_group, gsize), axis=2)[:, :, -2:].sum(axis=2)
    out = []
    for t in range(T):
        keep = max(itertools.combinations(range(n_group), topk_group),
                   key=lambda G: sum(gscore[t, g] for g in G))
        cand = [e for e in range(E) if e // gsize in keep]
        best = max(itertools.combinations(cand, k), key=lambda S: sum(float(l[t, e]) for e in S))
        out.append(set(best))
    return out


@pytest.mark.parametrize("E,n_group,topk_group,k", [(12, 4, 2, 3), (18, 6, 4, 4), (8, 4, 1, 2),
                                                    (9, 3, 2, 5)])
def test_grouped_topk_bruteforce(E, n_group, topk_group, k):
    rng = np.random.default_rng(E + n_group + k)
    l = rng.standard_normal((25, E)).astype(np.float32)
    ids = O.select_topk_grouped(l, k, n_group, topk_group)
    ref = _bruteforce_grouped(l, k, n_group, topk_group)
    for t in range(l.shape[0]):
        assert set(ids[t].tolist()) == ref[t]


def test_grouped_topk_all_groups_kept_is_plain_topk():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((50, 18)).astype(np.float32)
    assert np.array_equal(O.select_topk_grouped(l, 4, 6, 6), O.select_topk(l, 4))


def test_group_scores_top2():
    l = np.array([[0.0, 1.0, -1.0, 2.0, 2.0, -5.0]], dtype=np.float32)
    gs = O.group_scores(l, 2)
    ex = scipy.special.expit
    assert gs[0, 0] == pytest.approx(ex(1.0) + ex(0.0), abs=1e-15)
    assert gs[0, 1] == pytest.approx(2 * ex(2.0), abs=1e-15)


# ---------------------------------------------------------------- weights
def test_weights_softmax_renorm_closed_forms():
    rng = np.random.default_rng(7)
    l = rng.standard_normal((64, 8)).astype(np.float32)
    ids = O.select_topk(l, 3)
    w = O.routing_weights(l, ids, O.SCORE_SOFTMAX, 1)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= 1e-6)
    full = scipy.special.softmax(l.astype(np.float64), axis=1)
    sel = np.take_along_axis(full, ids, 1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-6)
    # k = E with renormalisation is the full softmax
    idsE = O.select_topk(l, 8)
    np.testing.assert_allclose(O.routing_weights(l, idsE, O.SCORE_SOFTMAX, 1),
                               np.take_along_axis(full, idsE, 1), rtol=1e-6)
    # k = 1 with renormalisation is exactly one
    assert np.all(O.routing_weights(l, O.select_topk(l, 1), O.SCORE_SOFTMAX, 1) == 1.0)


def test_weights_softmax_no_renorm_and_scale():
    rng = np.random.default_rng(8)
    l = rng.standard_normal((32, 16)).astype(np.float32)
    ids = O.select_topk(l, 4)
    full = scipy.special.softmax(l.astype(np.float64), axis=1)
    np.testing.assert_allclose(O.routing_weights(l, ids, O.SCORE_SOFTMAX, 0, 2.5),
                               2.5 * np.take_along_axis(full, ids, 1), rtol=1e-6)


def test_weights_sigmoid():
    rng = np.random.default_rng(9)
    l = rng.standard_normal((32, 18)).astype(np.float32)
    ids = O.select_topk_grouped(l, 4, 6, 4)
    s = np.take_along_axis(scipy.special.expit(l.astype(np.float64)), ids, 1)
    np.testing.assert_allclose(O.routing_weights(l, ids, O.SCORE_SIGMOID, 1, 2.5),
                               2.5 * s / s.sum(1, keepdims=True), rtol=1e-6)
    w1 = O.routing_weights(l, ids, O.SCORE_SIGMOID, 1, 1.0).astype(np.float64)
    assert np.all(np.abs(w1.sum(1) - 1.0) <= 1e-6)
    np.testing.assert_allclose(O.routing_weights(l, ids, O.SCORE_SIGMOID, 0), s, rtol=1e-6)


# ---------------------------------------------------------------- align
def test_align_golden():
    for case in _golden("align_small.json")["cases"]:
        ids = np.array(case["topk_ids"], dtype=np.int32)
        al = O.align(ids, case["E"], case["block_m"])
        assert al["sorted_token_ids"].tolist() == case["sorted_token_ids"]
        assert al["expert_ids"].tolist() == case["expert_ids"]
        assert al["num_tokens_post_padded"] == case["num_tokens_post_padded"]


def _check_align_invariants(ids, E, bm, al):
    T, k = ids.shape
    n = T * k
    flat = ids.reshape(-1)
    st, ex, ntpp = al["sorted_token_ids"], al["expert_ids"], al["num_tokens_post_padded"]
    counts = np.bincount(flat, minlength=E)
    # closed form of the padded total
    assert ntpp == int(sum(-(-c // bm) * bm for c in counts))
    assert ntpp <= O.align_capacity(T, k, E, bm)
    assert len(st) == ntpp and len(ex) * bm == ntpp
    valid = st[st < n]
    # valid ids are a permutation of the slots; pads are exactly n
    assert np.array_equal(np.sort(valid), np.arange(n))
    assert np.all(st[st >= n] == n)
    assert int((st == n).sum()) == ntpp - n
    # stable sort by expert (textbook routine) gives the valid ids in order
    assert np.array_equal(valid, np.argsort(flat, kind="stable"))
    # expert ids non-decreasing, every valid id in block b belongs to ex[b]
    assert np.all(np.diff(ex) >= 0)
    blk = np.arange(ntpp) // bm
    m = st < n
    assert np.array_equal(flat[st[m]], ex[blk[m]])
    # padded counts are multiples of BM and empty experts take no block
    pc = np.bincount(ex, minlength=E) * bm
    assert np.all(pc % bm == 0)
    assert np.array_equal(pc, -(-counts // bm) * bm)


@pytest.mark.parametrize("T,k,E,bm", [(1, 8, 128, 16), (3, 8, 128, 16), (37, 2, 8, 16),
                                      (64, 2, 8, 32), (100, 4, 18, 128), (513, 6, 128, 64),
                                      (2, 1, 1, 16), (0, 4, 8, 16)])
def test_align_invariants_random(T, k, E, bm):
    rng = np.random.default_rng(T * 1000 + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) if T else \
        np.zeros((0, k), np.int32)
    _check_align_invariants(ids, E, bm, O.align(ids, E, bm))


def test_align_offsets_match_cumulative_aligned_counts():
    """Cross-check against the count -> aligned size -> cumulative offset scheme of
    the axolotl branch's generate_permute_indices (without its clamp of empty
    experts to one block, which this library does not take)."""
    rng = np.random.default_rng(11)
    ids = rng.integers(0, 16, size=(300, 1)).astype(np.int32)
    ids[ids == 5] = 6     # one empty expert
    bm = 32
    al = O.align(ids, 16, bm)
    counts = np.bincount(ids.reshape(-1), minlength=16)
    m_sizes = (counts + bm - 1) // bm * bm
    m_offsets = np.cumsum(m_sizes)
    starts = m_offsets - m_sizes
    ex = al["expert_ids"]
    for e in range(16):
        blocks = np.nonzero(ex == e)[0]
        if m_sizes[e] == 0:
            assert blocks.size == 0
        else:
            assert blocks[0] * bm == starts[e] and (blocks[-1] + 1) * bm == m_offsets[e]


def test_align_capacity_is_tight():
    # every slot on its own expert: each needs a full block
    T, k, E, bm = 4, 2, 16, 16
    ids = np.arange(8, dtype=np.int32).reshape(T, k)
    assert O.align(ids, E, bm)["num_tokens_post_padded"] == O.align_capacity(T, k, E, bm)


# ---------------------------------------------------------------- expert MLP
def _torch_mlp(x, w13, w2, act):
    """Expert MLP with torch's linear (weight [out, in]) and silu, fp64 CPU."""
    xt = torch.from_numpy(np.asarray(x, np.float64))
    h = torch.nn.functional.linear(xt, torch.from_numpy(np.asarray(w13, np.float64)))
    if act == O.ACT_SWIGLU:
        I = w13.shape[0] // 2
        a = torch.nn.functional.silu(h[:, :I]) * h[:, I:]
    else:
        a = torch.relu(h) ** 2
    return torch.nn.functional.linear(a, torch.from_numpy(np.asarray(w2, np.float64))).numpy()


def _dense_bruteforce(x, w13, w2, ids, wts, act, sw13=None, sw2=None):
    """Every expert on every token, non-selected outputs masked by zero weights."""
    T, E = x.shape[0], w13.shape[0]
    M = np.zeros((T, E))
    for t in range(T):
        for j, e in enumerate(ids[t]):
            M[t, e] += float(wts[t, j])
    Y = np.stack([_torch_mlp(x, w13[e], w2[e], act) for e in range(E)], axis=1)   # [T,E,H]
    out = np.einsum("te,teh->th", M, Y)
    if sw13 is not None:
        out = out + _torch_mlp(x, sw13, sw2, act)
    return out


def test_golden_mlp():
    for case in _golden("mlp_small.json")["cases"]:
        out = O.expert_loop(np.array(case["x"]), np.array(case["w13"]), np.array(case["w2"]),
                            np.array(case["topk_ids"], dtype=np.int32),
                            np.array(case["topk_weights"], dtype=np.float32), case["activation"])
        np.testing.assert_allclose(out, np.array(case["out"]), rtol=1e-7, atol=0, err_msg=case["name"])


def _random_case(rng, T, E, k, H, I, act, grouped, shared):
    x = rng.standard_normal((T, H))
    M1 = 2 * I if act == O.ACT_SWIGLU else I
    w13 = rng.standard_normal((E, M1, H)) * 0.3
    w2 = rng.standard_normal((E, H, I)) * 0.3
    l = rng.standard_normal((T, E)).astype(np.float32)
    if grouped:
        ids = O.select_topk_grouped(l, k, 2, 1 if k <= E // 2 else 2)
        wts = O.routing_weights(l, ids, O.SCORE_SIGMOID, 1, 2.5)
    else:
        ids = O.select_topk(l, k)
        wts = O.routing_weights(l, ids, O.SCORE_SOFTMAX, 1)
    sw13 = rng.standard_normal((M1, H)) * 0.3 if shared else None
    sw2 = rng.standard_normal((H, I)) * 0.3 if shared else None
    return x, w13, w2, ids, wts, sw13, sw2


@pytest.mark.parametrize("seed", range(24))
def test_expert_loop_vs_dense_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(1, 10))
    E = int(rng.integers(1, 9))
    grouped = bool(seed % 3 == 1) and E % 2 == 0 and E >= 4
    k = int(rng.integers(1, E + 1))
    if grouped:
        k = min(k, E)
    H = int(rng.choice([8, 16, 32]))
    I = int(rng.choice([8, 16, 32]))
    act = seed % 2
    shared = seed % 4 >= 2
    x, w13, w2, ids, wts, sw13, sw2 = _random_case(rng, T, E, k, H, I, act, grouped, shared)
    out = O.expert_loop(x, w13, w2, ids, wts, act, sw13, sw2)
    ref = _dense_bruteforce(x, w13, w2, ids, wts, act, sw13, sw2)
    assert np.max(np.abs(out - ref)) <= 1e-5 * max(1.0, np.max(np.abs(ref)))


def test_single_expert_is_dense_mlp():
    rng = np.random.default_rng(5)
    for act in (O.ACT_SWIGLU, O.ACT_RELU2):
        x, w13, w2, _, _, _, _ = _random_case(rng, 7, 1, 1, 16, 8, act, False, False)
        ids = np.zeros((7, 1), np.int32)
        out = O.expert_loop(x, w13, w2, ids, np.ones((7, 1), np.float32), act)
        np.testing.assert_allclose(out, _torch_mlp(x, w13[0], w2[0], act), rtol=1e-6, atol=1e-6)


def test_k1_is_selected_expert_and_linear_in_weights():
    rng = np.random.default_rng(6)
    x, w13, w2, ids, wts, _, _ = _random_case(rng, 9, 5, 2, 16, 16, O.ACT_SWIGLU, False, False)
    a = O.expert_loop(x, w13, w2, ids, wts, 0).astype(np.float64)
    b = O.expert_loop(x, w13, w2, ids, 2 * wts, 0).astype(np.float64)
    np.testing.assert_allclose(b, 2 * a, rtol=1e-6, atol=1e-7)
    # k = 1: out = weight * selected expert's MLP
    ids1 = ids[:, :1].copy()
    o1 = O.expert_loop(x, w13, w2, ids1, np.full((9, 1), 0.5, np.float32), 0)
    for t in range(9):
        e = ids1[t, 0]
        np.testing.assert_allclose(o1[t], 0.5 * _torch_mlp(x[t:t + 1], w13[e], w2[e], 0)[0],
                                   rtol=1e-6, atol=1e-7)


def test_expert_relabelling_invariance():
    rng = np.random.default_rng(12)
    x, w13, w2, ids, wts, _, _ = _random_case(rng, 11, 6, 3, 16, 8, O.ACT_RELU2, False, False)
    p = rng.permutation(6)              # new label of old expert e is p[e]
    w13p = np.empty_like(w13)
    w2p = np.empty_like(w2)
    w13p[p] = w13
    w2p[p] = w2
    a = O.expert_loop(x, w13, w2, ids, wts, 1)
    b = O.expert_loop(x, w13p, w2p, p[ids].astype(np.int32), wts, 1)
    np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-7)


def test_token_output_matches_loop():
    cfg = W.small_config(T=13, H=32, I=16, E=6, top_k=3, n_shared=1, scoring=W.SCORE_SIGMOID,
                         n_group=3, topk_group=2)
    inp = W.make_inputs(cfg)
    res = O.moe_forward_cfg(cfg, inp)
    for t in (0, 5, 12):
        got = O.token_output(inp, t, res["topk_ids"][t], res["topk_weights"][t], cfg.activation, 1)
        np.testing.assert_allclose(got, res["out"][t], rtol=1e-6, atol=1e-7)


# ---------------------------------------------------------------- grouped GEMM oracle
@pytest.mark.parametrize("epi", [O.EPI_STORE, O.EPI_SWIGLU, O.EPI_RELU2, O.EPI_WEIGHTED_SCATTER])
def test_grouped_gemm_rows_direct(epi):
    rng = np.random.default_rng(20 + epi)
    T, k, E, K, N, bm = 11, 3, 5, 24, 16, 4
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    wts = rng.random((T, k)).astype(np.float32)
    al = O.align(ids, E, bm)
    x = rng.standard_normal((T, K))
    w = rng.standard_normal((E, N, K))
    c = O.grouped_gemm(x, k, w, al["sorted_token_ids"], al["expert_ids"],
                       al["num_tokens_post_padded"], bm, T * k, epi, wts)
    flat = ids.reshape(-1)
    st = al["sorted_token_ids"]
    for i, s in enumerate(st):
        if s >= T * k:
            if epi != O.EPI_WEIGHTED_SCATTER:
                assert np.all(c[i] == 0.0)
            continue
        t, e = s // k, flat[s]
        h = torch.nn.functional.linear(torch.from_numpy(x[t]), torch.from_numpy(w[e])).numpy()
        if epi == O.EPI_STORE:
            ref, row = h, i
        elif epi == O.EPI_SWIGLU:
            ref, row = torch.nn.functional.silu(torch.from_numpy(h[:N // 2])).numpy() * h[N // 2:], i
        elif epi == O.EPI_RELU2:
            ref, row = np.maximum(h, 0) ** 2, i
        else:
            ref, row = float(wts.reshape(-1)[s]) * h, s
        np.testing.assert_allclose(c[row], ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- whole layer
def test_tiny_config_vs_dense_bruteforce():
    cfg = W.CONFIGS["tiny"]
    inp = W.make_inputs(cfg)
    res = O.moe_forward_cfg(cfg, inp)
    x = O.bf16_to_f64(inp["x"])
    ref = _dense_bruteforce(x, O.bf16_to_f64(inp["w13"]), O.bf16_to_f64(inp["w2"]),
                            res["topk_ids"], res["topk_weights"], cfg.activation)
    assert np.max(np.abs(res["out"] - ref)) <= 1e-4 * np.max(np.abs(ref))
    _check_align_invariants(res["topk_ids"], cfg.E, cfg.block_m, res)


def test_dsv3_small_shape_with_shared_vs_dense():
    cfg = W.small_config(T=21, H=32, I=24, E=18, top_k=4, scoring=W.SCORE_SIGMOID, n_group=6,
                         topk_group=4, n_shared=1, scale=2.5, block_m=32)
    inp = W.make_inputs(cfg)
    res = O.moe_forward_cfg(cfg, inp)
    ref = _dense_bruteforce(O.bf16_to_f64(inp["x"]), O.bf16_to_f64(inp["w13"]),
                            O.bf16_to_f64(inp["w2"]), res["topk_ids"], res["topk_weights"],
                            cfg.activation, O.bf16_to_f64(inp["shared_w13"]),
                            O.bf16_to_f64(inp["shared_w2"]))
    assert np.max(np.abs(res["out"] - ref)) <= 1e-4 * np.max(np.abs(ref))
    assert np.all(np.abs(res["topk_weights"].astype(np.float64).sum(1) - 2.5) <= 1e-5)


# ---------------------------------------------------------------- indexed grouped GEMM
def test_indexed_grouped_gemm_bruteforce():
    """Every output element as a pure-Python sum over K (no matmul)."""
    rng = np.random.default_rng(5)
    M, K, N, E = 7, 5, 4, 3
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((E, N, K))
    idx = np.array([2, 0, 0, 1, 2, 2, 0])
    got = O.indexed_grouped_gemm(x, w, idx)
    for i in range(M):
        for n in range(N):
            s = 0.0
            for kk in range(K):
                s += float(x[i, kk]) * float(w[idx[i], n, kk])
            assert abs(got[i, n] - s) <= 1e-12 * max(1.0, abs(s))
    np.testing.assert_allclose(O.indexed_grouped_gemm(x, w, idx, rows=[6, 0]), got[[6, 0]],
                               rtol=1e-14, atol=1e-14)


def test_indexed_grouped_gemm_permutation_weights():
    """W[e] a permutation matrix P_e (not symmetric): row i must come out as
    P_e x[i] -- a transposed operand would give P_e^T x[i], a wrong expert
    another permutation."""
    rng = np.random.default_rng(6)
    K = 6
    perms = [rng.permutation(K) for _ in range(3)]
    w = np.zeros((3, K, K))
    for e, p in enumerate(perms):
        w[e, np.arange(K), p] = 1.0          # (P_e x)[n] = x[p[n]]
    x = rng.standard_normal((9, K))
    idx = np.array([0, 1, 2, 2, 1, 0, 1, 1, 2])
    got = O.indexed_grouped_gemm(x, w, idx)
    for i in range(9):
        assert np.array_equal(got[i], x[i, perms[idx[i]]])


def test_indexed_grouped_gemm_row_permutation_equivariance():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((20, 8))
    w = rng.standard_normal((4, 6, 8))
    idx = rng.integers(0, 4, 20)
    p = rng.permutation(20)
    np.testing.assert_allclose(O.indexed_grouped_gemm(x[p], w, idx[p]),
                               O.indexed_grouped_gemm(x, w, idx)[p], rtol=1e-13, atol=1e-13)


def test_indexed_grouped_gemm_equals_aligned_scatter():
    """The library's composition: align the per-row indices with top_k = 1,
    then the aligned grouped GEMM with a plain scatter by slot (weight 1)."""
    rng = np.random.default_rng(8)
    M, K, N, E, bm = 45, 16, 24, 5, 16
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((E, N, K))
    idx = np.repeat(np.arange(E), [0, 17, 3, 25, 0]).astype(np.int32)   # contiguous, uneven
    al = O.align(idx.reshape(M, 1), E, bm)
    via = O.grouped_gemm(x, 1, w, al["sorted_token_ids"], al["expert_ids"],
                         al["num_tokens_post_padded"], bm, M, O.EPI_WEIGHTED_SCATTER, None)
    np.testing.assert_allclose(via, O.indexed_grouped_gemm(x, w, idx), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- its backward
def test_indexed_backward_bruteforce():
    """dx and dw element by element as pure-Python sums."""
    rng = np.random.default_rng(15)
    M, K, N, E = 6, 4, 3, 4
    x, w, dy = rng.standard_normal((M, K)), rng.standard_normal((E, N, K)), rng.standard_normal((M, N))
    idx = np.array([1, 1, 3, 0, 3, 3])            # expert 2 has no rows
    dx, dw = O.indexed_grouped_gemm_backward(x, w, idx, dy)
    for i in range(M):
        for k in range(K):
            s = sum(float(dy[i, n]) * float(w[idx[i], n, k]) for n in range(N))
            assert abs(dx[i, k] - s) <= 1e-12 * max(1.0, abs(s))
    for e in range(E):
        for n in range(N):
            for k in range(K):
                s = sum(float(dy[i, n]) * float(x[i, k]) for i in range(M) if idx[i] == e)
                assert abs(dw[e, n, k] - s) <= 1e-12 * max(1.0, abs(s))
    assert np.all(dw[2] == 0.0)


def test_indexed_backward_adjoint_identities():
    """The gradients are the adjoints of the forward: for any directions hx,
    hw, <dy, F(hx, w)> = <dx, hx> and <dy, F(x, hw)> = <dw, hw> (F bilinear),
    with F the pinned forward."""
    rng = np.random.default_rng(16)
    M, K, N, E = 40, 12, 9, 5
    x, w, dy = rng.standard_normal((M, K)), rng.standard_normal((E, N, K)), rng.standard_normal((M, N))
    idx = rng.integers(0, E, M)
    dx, dw = O.indexed_grouped_gemm_backward(x, w, idx, dy)
    hx, hw = rng.standard_normal((M, K)), rng.standard_normal((E, N, K))
    lhs_x = float(np.sum(dy * O.indexed_grouped_gemm(hx, w, idx)))
    lhs_w = float(np.sum(dy * O.indexed_grouped_gemm(x, hw, idx)))
    assert abs(lhs_x - float(np.sum(dx * hx))) <= 1e-10 * abs(lhs_x)
    assert abs(lhs_w - float(np.sum(dw * hw))) <= 1e-10 * abs(lhs_w)


def test_indexed_backward_matches_autograd():
    """torch.autograd (CPU, float64) of the per-row forward."""
    rng = np.random.default_rng(17)
    M, K, N, E = 30, 8, 10, 4
    x, w, dy = rng.standard_normal((M, K)), rng.standard_normal((E, N, K)), rng.standard_normal((M, N))
    idx = rng.integers(0, E, M)
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    out = torch.einsum("mk,mnk->mn", xt, wt[torch.from_numpy(idx)])
    out.backward(torch.tensor(dy))
    dx, dw = O.indexed_grouped_gemm_backward(x, w, idx, dy)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_indexed_backward_sampled_rows_match_full():
    rng = np.random.default_rng(18)
    M, K, N, E = 25, 8, 6, 3
    x, w, dy = rng.standard_normal((M, K)), rng.standard_normal((E, N, K)), rng.standard_normal((M, N))
    idx = np.r_[np.zeros(10, int), np.full(15, 2)]       # expert 1 empty
    dx, dw = O.indexed_grouped_gemm_backward(x, w, idx, dy)
    sx, sw = O.indexed_grouped_gemm_backward(x, w, idx, dy, dx_rows=[3, 24], dw_rows=[(0, 5), (1, 0), (2, 2)])
    np.testing.assert_allclose(sx, dx[[3, 24]], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(sw, np.stack([dw[0, 5], dw[1, 0], dw[2, 2]]), rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- MXFP8 decoding
def test_e4m3_decoding_matches_torch_and_hand_values():
    bits = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(bits).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = O.e4m3_to_f64(bits)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    # hand values: 1.0, the largest, the smallest subnormal, -2, NaN
    assert O.e4m3_to_f64(np.uint8(0x38)) == 1.0
    assert O.e4m3_to_f64(np.uint8(0x7E)) == 448.0
    assert O.e4m3_to_f64(np.uint8(0x01)) == 2.0 ** -9
    assert O.e4m3_to_f64(np.uint8(0xC0)) == -2.0
    assert np.isnan(O.e4m3_to_f64(np.uint8(0x7F)))


def test_e8m0_and_block_scaling():
    assert O.e8m0_to_f64(np.uint8(127)) == 1.0
    assert O.e8m0_to_f64(np.uint8(0)) == 2.0 ** -127
    assert O.e8m0_to_f64(np.uint8(130)) == 8.0
    assert np.isnan(O.e8m0_to_f64(np.uint8(255)))
    q = np.full((2, 64), 0x38, np.uint8)         # every element 1.0
    s = np.array([[127, 130], [120, 0]], np.uint8)
    w = O.mxfp8_to_f64(q, s)
    assert np.array_equal(w[0, :32], np.ones(32)) and np.array_equal(w[0, 32:], np.full(32, 8.0))
    assert np.array_equal(w[1, :32], np.full(32, 2.0 ** -7))


def test_mxfp8_quantisation_error_is_bounded():
    """The workload's MXFP8 weights decode (oracle) to within half an E4M3 step
    of each element: |w - deq| <= 2^-4 |w| for normal elements, 2^-10 * scale
    below (subnormal E4M3), and no element saturates."""
    rng = np.random.default_rng(20)
    wb = W.f32_to_bf16_bits((0.02 * rng.standard_normal((8, 256))).astype(np.float32))
    q, s = W.quantize_mxfp8(wb)
    w = W.bf16_bits_to_f32(wb).astype(np.float64)
    deq = O.mxfp8_to_f64(q, s)
    scale = np.repeat(O.e8m0_to_f64(s), 32, axis=-1)
    assert np.all(np.abs(w - deq) <= np.maximum(2.0 ** -4 * np.abs(w), 2.0 ** -10 * scale) + 1e-30)
    assert np.all(np.abs(deq) <= 448.0 * scale)


def test_mxfp8_layer_equals_layer_on_decoded_weights():
    """The MXFP8 layer is the bf16-input layer run on the decoded weights
    (exactly representable in bf16: 3 mantissa bits times a power of two)."""
    cfg = W.small_config("mx_small", T=5, H=64, I=96, E=8, top_k=2, n_shared=1)
    inp = W.make_inputs(cfg)
    mx = W.make_mxfp8_weights(inp)
    got = O.moe_forward_mxfp8_cfg(cfg, inp, mx)["out"]
    dec = dict(inp)
    for name in ("w13", "w2", "shared_w13", "shared_w2"):
        wf = O.mxfp8_to_f64(mx[name + "_q"], mx[name + "_s"]).astype(np.float32)
        bits = W.f32_to_bf16_bits(wf)
        assert np.array_equal(W.bf16_bits_to_f32(bits), wf), "decoded MXFP8 is exact in bf16"
        dec[name] = bits
    want = O.moe_forward_cfg(cfg, dec)["out"]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- router logits
def test_router_logits_bruteforce():
    rng = np.random.default_rng(30)
    x, wr = rng.standard_normal((3, 5)), rng.standard_normal((4, 5))
    got = O.router_logits(x, wr)
    for t in range(3):
        for e in range(4):
            s = sum(float(x[t, h]) * float(wr[e, h]) for h in range(5))
            assert abs(got[t, e] - s) <= 1e-12 * max(1.0, abs(s))
