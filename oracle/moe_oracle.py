"""CPU oracle of the fused Mixture-of-Experts forward.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module; the library's product
path never does.  It shares no code with the HIP implementation.

The oracle is deliberately plain and slow: a per-expert loop, the structure the
pages use as their reference (the skill card's *Verification* checks against
one matmul per expert after top-k selection; the per-group matmul
loop ``pytorch_reference`` in the axolotl branch's ``cg_forward.py``; the
per-expert Python loop of the Gemma-4 training note).  Floating point is
carried in float64; bf16 inputs are widened exactly.

Steps, in the order the skill card's *Token-Expert Routing* lists them:

1. top-k gating (``select_topk``, ``select_topk_grouped``, ``routing_weights``)
2. sort by expert and pad to BLOCK_M (``align``)
3. per-expert MLP and routed-weight combine (``expert_loop``)

plus ``grouped_gemm`` (one grouped GEMM over the aligned layout),
``indexed_grouped_gemm`` (the standalone contiguous grouped GEMM of the
axolotl page, rows mapped to experts by an index per row),
``indexed_grouped_gemm_backward`` (its input and weight gradients) and
``moe_forward`` (the whole layer).

Readings where the pages are silent (each is pinned by a test unless marked):

* top-k order: experts by logit descending, ties to the lower expert index;
  sigmoid and softmax are strictly monotone, so selecting on the logit equals
  selecting on the exact score.
* grouped routing (DeepSeek-V3 config of the axolotl benchmark, ``n_group`` /
  ``topk_group``): contiguous groups of E/n_group experts, group score = sum
  of the two largest fp64 sigmoids, keep the ``topk_group`` best groups (ties
  to the lower group index), then top-k over the kept experts.  The group-score
  rule itself comes from the DeepSeek-V3 convention, not from the pages:
  parity unpinned against the pages (it is pinned against brute force).
* weights: softmax over the selected logits (renormalised) or over all logits;
  sigmoid divided by the selected sum (renormalised) or raw; then times the
  routed scaling factor.  fp64, stored as fp32.
* align: stable (ascending slot id) within an expert, pads are exactly T*k,
  an expert with no slots takes no block.
* pad rows of a row-ordered grouped GEMM output are zero.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

SCORE_SOFTMAX, SCORE_SIGMOID = 0, 1
ACT_SWIGLU, ACT_RELU2 = 0, 1
EPI_STORE, EPI_SWIGLU, EPI_RELU2, EPI_WEIGHTED_SCATTER = 0, 1, 2, 3


# ----------------------------------------------------------------------------
# bf16 helpers (the oracle's own; exact widening of raw bit patterns)
# ----------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)



# ----------------------------------------------------------------------------
# 1. gating
# ----------------------------------------------------------------------------
def router_logits(x: np.ndarray, router_w: np.ndarray) -> np.ndarray:
    """The gate's linear layer before the top-k (the HF gate the axolotl
    benchmark calls on the hidden states): logits[t, e] = x[t] . W[e], float64."""
    return np.asarray(x, np.float64) @ np.asarray(router_w, np.float64).T


def select_topk(logits: np.ndarray, k: int, allowed: Optional[np.ndarray] = None) -> np.ndarray:
    """Top-k expert ids per token, as k rounds of arg-max.

    Fused Moe Kernel skill card, *Token-Expert Routing* step 1 (each token
    keeps k experts).  Each round picks the largest remaining logit; among
    equal logits ``np.argmax`` returns the first, i.e. the lower expert index.
    ``allowed`` (bool [T,E]) restricts the candidates (grouped routing).
    Returns int32 [T,k] in selection order.
    """
    key = np.array(logits, dtype=np.float32, copy=True)
    T, E = key.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    taken = np.zeros((T, E), dtype=bool)
    if allowed is not None:
        taken |= ~allowed
    ids = np.empty((T, k), dtype=np.int32)
    rows = np.arange(T)
    for j in range(k):
        masked = np.where(taken, -np.inf, key)
        pick = np.argmax(masked, axis=1)
        if np.any(taken[rows, pick]):
            raise ValueError("fewer than k candidate experts")
        ids[:, j] = pick
        taken[rows, pick] = True
    return ids


def sigmoid64(logits: np.ndarray) -> np.ndarray:
    """Logistic function in float64."""
    l = np.asarray(logits, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-l))


def group_scores(logits: np.ndarray, n_group: int) -> np.ndarray:
    """Per-token group scores [T, n_group]: sum of the two largest fp64 sigmoids
    of each contiguous group of E/n_group experts (DeepSeek-V3 grouped routing,
    the ``n_group``/``topk_group`` fields of the axolotl DeepSeek-V3 config)."""
    T, E = logits.shape
    gsize = E // n_group
    s = sigmoid64(logits).reshape(T, n_group, gsize)
    out = np.empty((T, n_group), dtype=np.float64)
    for t in range(T):
        for g in range(n_group):
            vals = sorted(s[t, g].tolist(), reverse=True)
            out[t, g] = vals[0] + (vals[1] if gsize > 1 else 0.0)
    return out


def select_topk_grouped(logits: np.ndarray, k: int, n_group: int, topk_group: int) -> np.ndarray:
    """Grouped top-k: keep the ``topk_group`` best groups, then top-k inside them."""
    T, E = logits.shape
    if E % n_group != 0:
        raise ValueError("E must be a multiple of n_group")
    gsize = E // n_group
    if topk_group * gsize < k:
        raise ValueError("kept groups hold fewer than k experts")
    gs = group_scores(logits, n_group)
    allowed = np.zeros((T, E), dtype=bool)
    for t in range(T):
        # groups by score descending, ties to the lower group index
        order = sorted(range(n_group), key=lambda g: (-gs[t, g], g))
        for g in order[:topk_group]:
            allowed[t, g * gsize:(g + 1) * gsize] = True
    return select_topk(logits, k, allowed)


def routing_weights(logits: np.ndarray, ids: np.ndarray, scoring: int, renormalize: int,
                    scale: float = 1.0) -> np.ndarray:
    """Routed weights [T,k] float32 for the selected ids.

    softmax: exp(l_j - m) / sum_i exp(l_i - m) over the selected set when
    renormalising (the full-softmax denominator cancels), else over all experts.
    sigmoid: sigma_j / sum over the selected set, or sigma_j alone.
    Then times ``scale`` (``routed_scaling_factor`` of the DeepSeek-V3 config,
    ``norm_topk_prob`` = renormalise).  Computed in fp64.
    """
    l = np.asarray(logits, dtype=np.float64)
    T, k = ids.shape
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        sel = l[t, ids[t]]
        if scoring == SCORE_SOFTMAX:
            if renormalize:
                m = sel.max()
                e = np.exp(sel - m)
                w[t] = e / e.sum()
            else:
                m = l[t].max()
                w[t] = np.exp(sel - m) / np.exp(l[t] - m).sum()
        elif scoring == SCORE_SIGMOID:
            s = 1.0 / (1.0 + np.exp(-sel))
            w[t] = s / s.sum() if renormalize else s
        else:
            raise ValueError("unknown scoring")
    return (w * scale).astype(np.float32)


def gate(logits: np.ndarray, k: int, scoring: int = SCORE_SOFTMAX, n_group: int = 1,
         topk_group: int = 1, renormalize: int = 1, scale: float = 1.0):
    """Gating step: (topk_ids int32 [T,k], topk_weights float32 [T,k])."""
    if n_group > 1:
        ids = select_topk_grouped(logits, k, n_group, topk_group)
    else:
        ids = select_topk(logits, k)
    return ids, routing_weights(logits, ids, scoring, renormalize, scale)


# ----------------------------------------------------------------------------
# 2. align: sort slots by expert, pad each expert to a multiple of BLOCK_M
# ----------------------------------------------------------------------------
def align_capacity(T: int, k: int, E: int, block_m: int) -> int:
    """Upper bound of the padded length: round_up(T*k + min(E, T*k)*(BM-1), BM)."""
    n = T * k
    c = n + min(E, n) * (block_m - 1)
    return (c + block_m - 1) // block_m * block_m


def align(topk_ids: np.ndarray, E: int, block_m: int) -> Dict[str, np.ndarray]:
    """Skill card *Token-Expert Routing* steps 2-3 and *Grouped GEMM Structure*.

    Slot s = t*k + j.  For expert e with c_e slots: padded count
    p_e = ceil(c_e / BM) * BM (0 stays 0), offset o_e = sum_{e'<e} p_e'.
    sorted_token_ids[o_e + r] is the r-th smallest slot of expert e (r < c_e) and
    T*k for pads; expert_ids[b] = e for the blocks of expert e.
    Returns sorted_token_ids, expert_ids (both int32, length = padded total and
    padded total / BM) and num_tokens_post_padded (int).
    """
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    n = flat.size
    sorted_ids = []
    expert_ids = []
    for e in range(E):
        slots = np.nonzero(flat == e)[0].tolist()          # ascending slot order
        c = len(slots)
        p = -(-c // block_m) * block_m
        sorted_ids.extend(slots)
        sorted_ids.extend([n] * (p - c))
        expert_ids.extend([e] * (p // block_m))
    return {
        "sorted_token_ids": np.array(sorted_ids, dtype=np.int32),
        "expert_ids": np.array(expert_ids, dtype=np.int32),
        "num_tokens_post_padded": len(sorted_ids),
    }


# ----------------------------------------------------------------------------
# 3. expert MLP and combine
# ----------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z), the SiLU activation of the DeepSeek-V3 config."""
    return z / (1.0 + np.exp(-z))


def activation(h: np.ndarray, act: int, I: int) -> np.ndarray:
    """SwiGLU: silu of the gate half h[:, :I] times the up half h[:, I:] (the
    order of the axolotl MoE forward), or squared ReLU max(h, 0)^2 (mlxcel fc1 -> relu^2)."""
    if act == ACT_SWIGLU:
        return silu(h[:, :I]) * h[:, I:]
    if act == ACT_RELU2:
        return np.maximum(h, 0.0) ** 2
    raise ValueError("unknown activation")


def expert_mlp(xr: np.ndarray, w13: np.ndarray, w2: np.ndarray, act: int) -> np.ndarray:
    """One expert on rows xr (fp64): act(xr @ w13^T) @ w2^T."""
    I = w2.shape[1]
    h = xr @ w13.T
    return activation(h, act, I) @ w2.T


def expert_loop(x: np.ndarray, w13: np.ndarray, w2: np.ndarray, topk_ids: np.ndarray,
                topk_weights: np.ndarray, act: int,
                shared_w13: Optional[np.ndarray] = None,
                shared_w2: Optional[np.ndarray] = None) -> np.ndarray:
    """Routed-expert MLPs as a per-expert loop, then the weighted combine.

    x [T,H], w13 [E,M1,H], w2 [E,H,I], topk_weights [T,k] — float arrays
    (already widened).  For each expert e: its slots S_e in ascending order,
    tokens S_e // k (skill card *Common Pitfalls* 1), rows times the slot's
    routed weight (*Common Pitfalls* 4).  out[t] = sum_j ys[t*k + j] in j order,
    plus the always-on shared expert with weight 1 (``n_shared_experts=1``).
    Returns float32 [T,H].
    """
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    E = w13.shape[0]
    k = topk_ids.shape[1]
    flat = topk_ids.reshape(-1)
    wflat = np.asarray(topk_weights, dtype=np.float64).reshape(-1)
    ys = np.zeros((T * k, H), dtype=np.float64)
    for e in range(E):
        slots = np.nonzero(flat == e)[0]
        if slots.size == 0:
            continue
        y = expert_mlp(x[slots // k], np.asarray(w13[e], np.float64),
                       np.asarray(w2[e], np.float64), act)
        ys[slots] = wflat[slots, None] * y
    out = np.zeros((T, H), dtype=np.float64)
    for j in range(k):
        out += ys[j::k]
    if shared_w13 is not None:
        out += expert_mlp(x, np.asarray(shared_w13, np.float64),
                          np.asarray(shared_w2, np.float64), act)
    return out.astype(np.float32)


def grouped_gemm(a: np.ndarray, a_row_div: int, w: np.ndarray, sorted_token_ids: np.ndarray,
                 expert_ids: np.ndarray, num_tokens_post_padded: int, block_m: int,
                 num_valid: int, epilogue: int,
                 topk_weights: Optional[np.ndarray] = None) -> np.ndarray:
    """One grouped GEMM over the aligned layout (skill card *Grouped GEMM
    Structure*): padded row i uses expert expert_ids[i // BM] and A row
    sorted_token_ids[i] // a_row_div (a_row_div = 0: A row i).

    Epilogues: STORE h, SWIGLU silu(h[:N/2]) * h[N/2:], RELU2 max(h,0)^2 —
    written at row i, zero for pad rows; WEIGHTED_SCATTER writes
    topk_weights[s] * h at row s = sorted_token_ids[i] for valid rows only
    (weight 1 when topk_weights is None: a plain scatter by slot).
    Rows at or beyond num_tokens_post_padded are not produced (NaN here).
    Returns float64.
    """
    a = np.asarray(a, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    N = w.shape[1]
    ncols = N // 2 if epilogue == EPI_SWIGLU else N
    if epilogue == EPI_WEIGHTED_SCATTER:
        c = np.full((num_valid, ncols), np.nan)
        wf = (np.ones(num_valid) if topk_weights is None
              else np.asarray(topk_weights, dtype=np.float64).reshape(-1))
    else:
        c = np.full((len(sorted_token_ids), ncols), np.nan)
    for i in range(num_tokens_post_padded):
        e = int(expert_ids[i // block_m])
        sid = int(sorted_token_ids[i])
        valid = sid < num_valid
        if epilogue == EPI_WEIGHTED_SCATTER:
            if valid:
                row = a[i] if a_row_div == 0 else a[sid // a_row_div]
                c[sid] = wf[sid] * (w[e] @ row)
            continue
        if not valid:
            c[i] = 0.0
            continue
        row = a[i] if a_row_div == 0 else a[sid // a_row_div]
        h = w[e] @ row
        if epilogue == EPI_STORE:
            c[i] = h
        elif epilogue == EPI_SWIGLU:
            c[i] = silu(h[:ncols]) * h[ncols:]
        elif epilogue == EPI_RELU2:
            c[i] = np.maximum(h, 0.0) ** 2
        else:
            raise ValueError("unknown epilogue")
    return c


def indexed_grouped_gemm(x: np.ndarray, w: np.ndarray, expert_indices: np.ndarray,
                         rows: Optional[np.ndarray] = None) -> np.ndarray:
    """The contiguous grouped GEMM of the axolotl page (``cg_forward.py``,
    ``cg_grouped_gemm_forward`` and its per-block ``pytorch_reference``):
    output row i is input row i times the transposed weight of its expert,
    ``x[i] @ w[expert_indices[i]].T``.  The page takes one index per block of
    ``group_size_m`` rows and requires each block to share it; read per row,
    the definition needs no such condition and agrees where it holds.

    One matmul per expert over its rows, float64.  ``rows``: only these output
    rows, in the given order (each computed alone; for spot checks of large
    cases)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    idx = np.asarray(expert_indices).reshape(-1)
    if rows is not None:
        return np.stack([w[int(idx[r])] @ x[r] for r in rows]) if len(rows) else \
            np.zeros((0, w.shape[1]))
    out = np.full((x.shape[0], w.shape[1]), np.nan)
    for e in range(w.shape[0]):
        sel = np.nonzero(idx == e)[0]
        if sel.size:
            out[sel] = x[sel] @ w[e].T
    return out


def indexed_grouped_gemm_backward(x: np.ndarray, w: np.ndarray, expert_indices: np.ndarray,
                                  dy: np.ndarray, dx_rows=None, dw_rows=None):
    """Gradients of the indexed grouped GEMM ``out[i] = x[i] @ w[idx[i]].T``
    for an output gradient ``dy`` (the axolotl page's ``cg_backward.py``:
    ``cg_grouped_gemm_backward_inputs`` and ``..._weights``):

        dx[i] = dy[i] @ w[idx[i]]                       ([M, K])
        dw[e] = sum over rows i with idx[i] == e of outer(dy[i], x[i])
              = dy[rows_e].T @ x[rows_e]                ([E, N, K]; zero if no rows)

    Read per row, like the forward.  One matmul per expert, float64.

    Spot checks of large cases: ``dx_rows`` (row ids) and ``dw_rows`` ((e, n)
    pairs) return only those rows of dx and dw, each from the same
    definition: ``(dx[dx_rows], [dw[e, n] for e, n in dw_rows])``."""
    idx = np.asarray(expert_indices).reshape(-1)
    if dx_rows is not None or dw_rows is not None:
        sx = [np.asarray(dy[r], np.float64) @ np.asarray(w[int(idx[r])], np.float64)
              for r in (dx_rows if dx_rows is not None else [])]
        sw = []
        for e, n in (dw_rows if dw_rows is not None else []):
            sel = np.nonzero(idx == e)[0]
            sw.append(np.asarray(dy[sel, n], np.float64) @ np.asarray(x[sel], np.float64)
                      if sel.size else np.zeros(np.shape(x)[1]))
        return np.array(sx), np.array(sw)
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    E, N, K = w.shape
    dx = np.full((x.shape[0], K), np.nan)
    dw = np.zeros((E, N, K))
    for e in range(E):
        sel = np.nonzero(idx == e)[0]
        if sel.size:
            dx[sel] = dy[sel] @ w[e]
            dw[e] = dy[sel].T @ x[sel]
    return dx, dw


def e4m3_to_f64(bits: np.ndarray) -> np.ndarray:
    """FP8 E4M3 ("fn": no infinities) bits -> float64, from the format's
    definition (OCP 8-bit floating point): sign, 4 exponent bits with bias 7,
    3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    s = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def e8m0_to_f64(bits: np.ndarray) -> np.ndarray:
    """E8M0 scale bits -> 2^(bits - 127) (255 is NaN), OCP Microscaling."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.float64)
    return np.where(b == 255, np.nan, np.exp2(b - 127.0))


def mxfp8_to_f64(q: np.ndarray, s: np.ndarray, block: int = 32) -> np.ndarray:
    """MXFP8 weights [..., K] (E4M3 bits) with E8M0 scales [..., K / block]:
    every element times the scale of its block of ``block`` elements along K."""
    v = e4m3_to_f64(q)
    return v * np.repeat(e8m0_to_f64(s), block, axis=-1)


# ----------------------------------------------------------------------------
# the whole layer
# ----------------------------------------------------------------------------
def moe_forward(inp: Dict[str, np.ndarray], *, top_k: int, block_m: int,
                scoring: int = SCORE_SOFTMAX, n_group: int = 1, topk_group: int = 1,
                renormalize: int = 1, scale: float = 1.0, activation_kind: int = ACT_SWIGLU,
                n_shared: int = 0) -> Dict[str, np.ndarray]:
    """Gating -> align -> per-expert MLP loop -> combine, on the bf16-bit inputs
    produced by the workload generator (``x``, ``logits``, ``w13``, ``w2`` and
    optionally ``shared_w13``/``shared_w2``).  Returns the routing outputs and
    ``out`` float32 [T,H]."""
    logits = np.asarray(inp["logits"], dtype=np.float32)
    E = logits.shape[1]
    ids, wts = gate(logits, top_k, scoring, n_group, topk_group, renormalize, scale)
    al = align(ids, E, block_m)
    x = bf16_to_f64(inp["x"])
    w13 = bf16_to_f64(inp["w13"])
    w2 = bf16_to_f64(inp["w2"])
    sw13 = sw2 = None
    if n_shared:
        sw13 = bf16_to_f64(inp["shared_w13"])
        sw2 = bf16_to_f64(inp["shared_w2"])
    out = expert_loop(x, w13, w2, ids, wts, activation_kind, sw13, sw2)
    return {"topk_ids": ids, "topk_weights": wts, **al, "out": out}


def moe_forward_cfg(cfg, inp: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """``moe_forward`` with the fields of a workload config object."""
    return moe_forward(inp, top_k=cfg.top_k, block_m=cfg.block_m, scoring=cfg.scoring,
                       n_group=cfg.n_group, topk_group=cfg.topk_group,
                       renormalize=cfg.renormalize, scale=cfg.scale,
                       activation_kind=cfg.activation, n_shared=cfg.n_shared)


class _MxExperts:
    """Expert weights kept in MXFP8 and decoded (mxfp8_to_f64) one expert at a
    time when the loop asks for it."""

    def __init__(self, q: np.ndarray, s: np.ndarray):
        self.q, self.s, self.shape = q, s, q.shape

    def __getitem__(self, e):
        return mxfp8_to_f64(self.q[e], self.s[e])


def moe_forward_mxfp8_cfg(cfg, inp: Dict[str, np.ndarray], mx: Dict[str, np.ndarray]):
    """The layer with MXFP8 expert weights (``mx``: w13_q/_s, w2_q/_s and the
    shared expert's): the same gating, align and per-expert loop as
    ``moe_forward``, on the weights the MXFP8 encoding represents."""
    logits = np.asarray(inp["logits"], dtype=np.float32)
    ids, wts = gate(logits, cfg.top_k, cfg.scoring, cfg.n_group, cfg.topk_group, cfg.renormalize,
                    cfg.scale)
    al = align(ids, logits.shape[1], cfg.block_m)
    sw13 = sw2 = None
    if cfg.n_shared:
        sw13 = mxfp8_to_f64(mx["shared_w13_q"], mx["shared_w13_s"])
        sw2 = mxfp8_to_f64(mx["shared_w2_q"], mx["shared_w2_s"])
    out = expert_loop(bf16_to_f64(inp["x"]), _MxExperts(mx["w13_q"], mx["w13_s"]),
                      _MxExperts(mx["w2_q"], mx["w2_s"]), ids, wts, cfg.activation, sw13, sw2)
    return {"topk_ids": ids, "topk_weights": wts, **al, "out": out}


def token_output(inp: Dict[str, np.ndarray], t: int, ids_t: np.ndarray, wts_t: np.ndarray,
                 activation_kind: int, n_shared: int = 0) -> np.ndarray:
    """out[t] for one token alone (for sampled checks at full size): the routed
    experts of that token in j order, plus the shared expert."""
    x = bf16_to_f64(inp["x"][t:t + 1])
    acc = np.zeros(x.shape[1], dtype=np.float64)
    for j, e in enumerate(np.asarray(ids_t).tolist()):
        y = expert_mlp(x, bf16_to_f64(inp["w13"][e]), bf16_to_f64(inp["w2"][e]),
                       activation_kind)[0]
        acc += float(wts_t[j]) * y
    if n_shared:
        acc += expert_mlp(x, bf16_to_f64(inp["shared_w13"]), bf16_to_f64(inp["shared_w2"]),
                          activation_kind)[0]
    return acc.astype(np.float32)
