"""Seeded synthetic MoE-layer workloads.

This module only draws numbers: it holds none of the MoE arithmetic (no
gating, no sorting, no matrix products).  It is the single source of inputs for
both the CPU oracle and the HIP library, so that the two are compared on exactly
the same bits.

Shapes follow the workloads described on the pages:

* the fused-MoE skill card ("Fused Moe Kernel", *Key Parameters* and
  *Small-M heuristic*) for BLOCK_M choices and small token counts;
* the DeepSeek-V3 ~8.3B random-weight model built by the axolotl benchmark
  scripts (``build_deepseek_v3_8b.py``, ``build_config``): H 3072, MoE
  intermediate 2560, 18 routed experts, top-4, 6 groups / 4 kept, one shared
  expert, ``initializer_range`` 0.02;
* the squared-ReLU expert MLP of the mlxcel PR (fc1 -> relu^2 -> fc2);
* decode batches of 1-3 tokens with duplicate experts across tokens, as in the
  B70 grouped-Q8 experiment (*Intent*).

Every tensor is drawn from ``numpy.random.default_rng(SeedSequence(key))`` with
a key built from (family, tokens, layer, tensor id[, expert]), so any tensor can
be regenerated alone.  bf16 tensors are produced as raw ``uint16`` bit
patterns by round-to-nearest-even of a float32 draw.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np

# tensor ids used in the seed keys
_TID_X, _TID_LOGITS, _TID_W13, _TID_W2, _TID_SW13, _TID_SW2, _TID_PERM = 1, 2, 3, 4, 5, 6, 7
_TID_ROUTER = 8

SCORE_SOFTMAX, SCORE_SIGMOID = 0, 1
ACT_SWIGLU, ACT_RELU2 = 0, 1


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """One MoE layer shape plus the recipe of its synthetic inputs."""

    name: str
    family: int            # seed namespace (1 tiny, 2 decode, 3 DeepSeek-V3-shaped, 4 Zipf, 5 relu^2)
    T: int
    H: int
    I: int
    E: int
    top_k: int
    scoring: int = SCORE_SOFTMAX
    n_group: int = 1
    topk_group: int = 1
    renormalize: int = 1
    scale: float = 1.0
    activation: int = ACT_SWIGLU
    n_shared: int = 0
    block_m: int = 16
    logits_mode: str = "normal"   # "normal" | "dup3" | "zipf"
    w_std: float = 0.02

    @property
    def M1(self) -> int:
        """Rows of the first weight matrix per expert (2I for SwiGLU, I for relu^2)."""
        return 2 * self.I if self.activation == ACT_SWIGLU else self.I

    @property
    def mats(self) -> int:
        return 3 if self.activation == ACT_SWIGLU else 2

    def flops(self, routed_only: bool = False) -> float:
        """Useful flops of one layer: 2 * T * k_eff * mats * H * I (no padding)."""
        k_eff = self.top_k + (0 if routed_only else self.n_shared)
        return 2.0 * self.T * k_eff * self.mats * self.H * self.I


CONFIGS: Dict[str, MoEConfig] = {
    # tiny layer, softmax top-2 of 8, BLOCK_M 16
    "tiny": MoEConfig("tiny", 1, T=64, H=256, I=512, E=8, top_k=2, block_m=16),
    # decode-shaped, 128 experts top-8
    "decode_t1": MoEConfig("decode_t1", 2, T=1, H=2048, I=768, E=128, top_k=8, block_m=16),
    "decode_t3": MoEConfig("decode_t3", 2, T=3, H=2048, I=768, E=128, top_k=8, block_m=16,
                           logits_mode="dup3"),
    "decode_t8": MoEConfig("decode_t8", 2, T=8, H=2048, I=768, E=128, top_k=8, block_m=16),
    # DeepSeek-V3-8B-shaped: grouped sigmoid routing plus one shared expert
    # (BLOCK_M 256: 2-4 % faster per layer than 128 on MI355X; 18 experts with
    # about 900 slots each pad little)
    "dsv3": MoEConfig("dsv3", 3, T=4096, H=3072, I=2560, E=18, top_k=4,
                      scoring=SCORE_SIGMOID, n_group=6, topk_group=4, n_shared=1, block_m=256),
    "dsv3_s2.5": MoEConfig("dsv3_s2.5", 3, T=4096, H=3072, I=2560, E=18, top_k=4,
                           scoring=SCORE_SIGMOID, n_group=6, topk_group=4, n_shared=1,
                           scale=2.5, block_m=256),
    # 128 experts with a Zipf(1.1) popularity prior (BLOCK_M 128: measured faster
    # than 64 despite the extra padding, fewer weight-tile passes)
    "zipf128": MoEConfig("zipf128", 4, T=8192, H=2816, I=704, E=128, top_k=8, block_m=128,
                         logits_mode="zipf"),
    # squared-ReLU experts
    "relu2_t1": MoEConfig("relu2_t1", 5, T=1, H=2688, I=1856, E=128, top_k=6,
                          activation=ACT_RELU2, block_m=16),
    "relu2_t16": MoEConfig("relu2_t16", 5, T=16, H=2688, I=1856, E=128, top_k=6,
                           activation=ACT_RELU2, block_m=16),
    "relu2_t2048": MoEConfig("relu2_t2048", 5, T=2048, H=2688, I=1856, E=128, top_k=6,
                             activation=ACT_RELU2, block_m=128),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32)
    rounded = (b + (((b >> 16) & 1) + np.uint32(0x7FFF))) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(shape, std: float, *key: int) -> np.ndarray:
    z = _rng(*key).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        z *= np.float32(std)
    return f32_to_bf16_bits(z)


def _expert_stack(cfg: MoEConfig, layer: int, tid: int, rows: int, cols: int,
                  threads: Optional[int]) -> np.ndarray:
    """[E, rows, cols] bf16 bits, one independent stream per expert."""
    out = np.empty((cfg.E, rows, cols), dtype=np.uint16)

    def fill(e: int) -> None:
        out[e] = _normal_bf16((rows, cols), cfg.w_std, cfg.family, layer, tid, e)

    nthreads = threads or min(16, len(os.sched_getaffinity(0)))
    if nthreads <= 1 or cfg.E == 1:
        for e in range(cfg.E):
            fill(e)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(fill, range(cfg.E)))
    return out


def make_logits(cfg: MoEConfig, layer: int = 0) -> np.ndarray:
    """Router logits [T, E] float32 following the config's recipe.

    * ``normal``: i.i.d. N(0, 1).
    * ``dup3``  : three decode tokens whose preferred expert sets overlap so that
      half of the 24 slots repeat an expert of another token.  With a seeded
      permutation p of the experts, token 0 prefers p[0:8], token 1 prefers
      p[0:4] + p[8:12], token 2 prefers p[4:8] + p[8:12]; preferred logits are
      z + 6 and the others z, with z ~ N(0,1) clipped to [-2.5, 2.5] so every
      preferred logit (>= 3.5) exceeds every other one (<= 2.5).
    * ``zipf``  : z - 1.1 * ln(rank_e) with rank_e a seeded permutation of
      1..E, i.e. a softmax prior proportional to rank^-1.1.
    """
    rng = _rng(cfg.family, cfg.T, layer, _TID_LOGITS)
    z = rng.standard_normal(size=(cfg.T, cfg.E), dtype=np.float32)
    if cfg.logits_mode == "normal":
        return z
    perm = _rng(cfg.family, cfg.T, layer, _TID_PERM).permutation(cfg.E)
    if cfg.logits_mode == "dup3":
        if cfg.T != 3 or cfg.top_k != 8 or cfg.E < 12:
            raise ValueError("dup3 logits need T=3, top_k=8, E>=12")
        z = np.clip(z, -2.5, 2.5)
        sets = [perm[0:8], np.concatenate([perm[0:4], perm[8:12]]),
                np.concatenate([perm[4:8], perm[8:12]])]
        for t, s in enumerate(sets):
            z[t, s] += np.float32(6.0)
        return z.astype(np.float32)
    if cfg.logits_mode == "zipf":
        rank = (perm + 1).astype(np.float64)
        bias = (-1.1 * np.log(rank)).astype(np.float32)
        return (z + bias[None, :]).astype(np.float32)
    raise ValueError(f"unknown logits_mode {cfg.logits_mode!r}")


def make_inputs(cfg: MoEConfig, layer: int = 0, with_weights: bool = True,
                threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """All inputs of one layer as numpy arrays.

    Returns ``x`` (uint16 bf16 bits [T,H]), ``logits`` (float32 [T,E]) and, with
    ``with_weights``, ``w13`` (bf16 bits [E,M1,H]; SwiGLU rows [0,I) gate,
    [I,2I) up), ``w2`` (bf16 bits [E,H,I]) and, when ``n_shared`` is 1,
    ``shared_w13`` ([M1,H]) and ``shared_w2`` ([H,I]).
    """
    inp: Dict[str, np.ndarray] = {
        "x": _normal_bf16((cfg.T, cfg.H), 1.0, cfg.family, cfg.T, layer, _TID_X),
        "logits": make_logits(cfg, layer),
    }
    if with_weights:
        inp["w13"] = _expert_stack(cfg, layer, _TID_W13, cfg.M1, cfg.H, threads)
        inp["w2"] = _expert_stack(cfg, layer, _TID_W2, cfg.H, cfg.I, threads)
        if cfg.n_shared:
            inp["shared_w13"] = _normal_bf16((cfg.M1, cfg.H), cfg.w_std, cfg.family, layer,
                                             _TID_SW13)
            inp["shared_w2"] = _normal_bf16((cfg.H, cfg.I), cfg.w_std, cfg.family, layer,
                                            _TID_SW2)
    return inp


def small_config(name: str = "small", **kw) -> MoEConfig:
    """A config for oracle-sized parity cases; keyword arguments override fields."""
    base = dict(name=name, family=100, T=37, H=64, I=96, E=8, top_k=2, block_m=16)
    base.update(kw)
    return MoEConfig(**base)


# ---------------------------------------------------------------------------
# standalone grouped GEMM (rows mapped to experts by an index per row)
# ---------------------------------------------------------------------------
_TID_GX, _TID_GW, _TID_GPERM, _TID_GDY = 11, 12, 13, 14


@dataclasses.dataclass(frozen=True)
class GemmScenario:
    """One contiguous grouped GEMM: M rows of K, G expert matrices [N, K].

    The four full-size scenarios are the table of the axolotl page's
    ``benchmark_cg_gemm`` script (uniform groups of M / G rows, inputs and
    weights drawn from N(0, 1) as that script's ``randn`` does).  ``sizes``
    gives uneven (contiguous) groups instead; ``shuffled`` permutes the rows'
    indices so that groups are not contiguous."""

    name: str
    family: int
    G: int
    M: int
    N: int
    K: int
    sizes: Optional[tuple] = None
    shuffled: bool = False
    block_m: int = 128

    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


GEMM_SCENARIOS: Dict[str, GemmScenario] = {
    s.name: s for s in (
        GemmScenario("cg_g4_m8192_n4096_k7168", 6, G=4, M=8192, N=4096, K=7168),
        GemmScenario("cg_g4_m8192_n7168_k2048", 6, G=4, M=8192, N=7168, K=2048),
        GemmScenario("cg_g8_m4096_n4096_k7168", 6, G=8, M=4096, N=4096, K=7168),
        GemmScenario("cg_g8_m4096_n7168_k2048", 6, G=8, M=4096, N=7168, K=2048),
    )
}


def small_gemm_scenario(name: str = "cg_small", **kw) -> GemmScenario:
    """A grouped-GEMM scenario for oracle-sized parity cases."""
    base = dict(name=name, family=106, G=3, M=480, N=320, K=200)
    base.update(kw)
    return GemmScenario(**base)


def make_gemm_inputs(sc: GemmScenario, threads: Optional[int] = None,
                     with_grad: bool = False) -> Dict[str, np.ndarray]:
    """``x`` (bf16 bits [M, K]), ``w`` (bf16 bits [G, N, K], one stream per
    expert) and ``expert_indices`` (int32 [M]); with ``with_grad`` also an
    output gradient ``dy`` (bf16 bits [M, N], N(0, 1))."""
    if sc.sizes is not None:
        sizes = np.asarray(sc.sizes, dtype=np.int64)
        if sizes.size != sc.G or int(sizes.sum()) != sc.M:
            raise ValueError("group sizes must be G entries summing to M")
    else:
        if sc.M % sc.G:
            raise ValueError("uniform groups need M divisible by G")
        sizes = np.full(sc.G, sc.M // sc.G, dtype=np.int64)
    idx = np.repeat(np.arange(sc.G, dtype=np.int32), sizes)
    if sc.shuffled:
        idx = idx[_rng(sc.family, sc.M, _TID_GPERM).permutation(sc.M)]
    w = np.empty((sc.G, sc.N, sc.K), dtype=np.uint16)

    def fill(e: int) -> None:
        w[e] = _normal_bf16((sc.N, sc.K), 1.0, sc.family, sc.M, _TID_GW, e)

    nthreads = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(max(1, nthreads)) as ex:
        list(ex.map(fill, range(sc.G)))
    out = {"x": _normal_bf16((sc.M, sc.K), 1.0, sc.family, sc.M, _TID_GX),
           "w": w, "expert_indices": np.ascontiguousarray(idx)}
    if with_grad:
        out["dy"] = _normal_bf16((sc.M, sc.N), 1.0, sc.family, sc.M, _TID_GDY)
    return out


# ---------------------------------------------------------------------------
# MXFP8 expert weights (decode): an input format, produced from the bf16 weights
# ---------------------------------------------------------------------------
MX_BLOCK = 32          # elements per shared scale (OCP Microscaling)
E4M3_MAX = 448.0       # largest finite FP8 E4M3 value


def quantize_mxfp8(bits: np.ndarray):
    """bf16 weights [..., K] (K a multiple of 32) -> (FP8 E4M3 bits [..., K]
    uint8, E8M0 scale bits [..., K / 32] uint8), the way a bf16 checkpoint is
    converted to MXFP8 (OCP Microscaling): per block of 32 consecutive
    elements along K, the smallest power-of-two scale 2^x with max |w| / 2^x
    <= 448 (so no element saturates), elements w / 2^x rounded to
    nearest-even E4M3; an all-zero block gets scale bits 0.  Quantisation
    happens before the library (like any checkpoint conversion); the library
    and the oracle only decode."""
    import torch
    shp = bits.shape
    if shp[-1] % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    w = bf16_bits_to_f32(bits).reshape(*shp[:-1], shp[-1] // MX_BLOCK, MX_BLOCK)
    amax = np.abs(w).max(axis=-1)
    with np.errstate(divide="ignore"):
        shared = np.where(amax > 0, np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / E4M3_MAX)),
                          -127.0)
    sbits = np.clip(shared + 127, 0, 254).astype(np.uint8)
    scale = np.ldexp(np.float32(1.0), sbits.astype(np.int32) - 127).astype(np.float32)
    scaled = np.clip(w / scale[..., None], -E4M3_MAX, E4M3_MAX)
    q = torch.from_numpy(np.ascontiguousarray(scaled, dtype=np.float32)).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy().reshape(shp), sbits


def make_mxfp8_weights(inp: Dict[str, np.ndarray], experts=None) -> Dict[str, np.ndarray]:
    """MXFP8 forms of the layer's weights, expert by expert: w13_q / w13_s,
    w2_q / w2_s and, with a shared expert, shared_w13_q / _s, shared_w2_q / _s.
    ``experts``: convert only these (the others stay zero bytes), for timing
    runs whose routing is known to read no other expert."""
    out: Dict[str, np.ndarray] = {}
    for name in ("w13", "w2"):
        w = inp[name]
        q = np.zeros(w.shape, dtype=np.uint8)
        s = np.zeros(w.shape[:-1] + (w.shape[-1] // MX_BLOCK,), dtype=np.uint8)
        for e in (range(w.shape[0]) if experts is None else experts):
            q[e], s[e] = quantize_mxfp8(w[e])
        out[name + "_q"], out[name + "_s"] = q, s
    for name in ("shared_w13", "shared_w2"):
        if name in inp:
            out[name + "_q"], out[name + "_s"] = quantize_mxfp8(inp[name])
    return out


# ---------------------------------------------------------------------------
# router weight (the gate's linear layer): for the path that computes the
# router logits itself
# ---------------------------------------------------------------------------
def make_router_weight(cfg: MoEConfig, layer: int = 0) -> np.ndarray:
    """bf16 bits [E, H] ~ N(0, w_std): the gate's weight, logits = x . W^T
    (the HF DeepSeek-V3 gate's linear layer, ``initializer_range``)."""
    return _normal_bf16((cfg.E, cfg.H), cfg.w_std, cfg.family, layer, _TID_ROUTER)


# ---------------------------------------------------------------------------
# router logits with exact ties (for the lower-index tie rule of top-k)
# ---------------------------------------------------------------------------
_TID_TIES = 9
TIE_MODES = ("equal", "coarse", "signed_zero", "kth", "groups_equal", "groups_two")


def make_tie_logits(T: int, E: int, k: int, mode: str, seed: int = 0,
                    n_group: int = 1) -> np.ndarray:
    """Router logits [T, E] float32 built so that many keys are exactly equal.

    * ``equal``: every row constant (values from {-1.5, -0.0, +0.0, 0.5, 2});
      all experts tie.
    * ``coarse``: N(0, 1) rounded to multiples of 0.5; ties everywhere,
      often across the k-th place.
    * ``signed_zero``: a mix of +0.0 and -0.0 with a few +-1 entries; +0 and
      -0 are equal keys.
    * ``kth``: k-1 distinct leaders (4, 4.25, ...), then three experts at 3.0
      competing for the k-th place, the rest N(0, 1) clipped to 2.5.
    * ``groups_equal`` (n_group contiguous groups): every group holds a
      permutation of one multiset of non-negative multiples of 0.5, so all
      group scores are equal and equal values repeat across groups.
    * ``groups_two``: two multisets, a clearly stronger one (values + 2) on a
      random half of the groups; the groups of each multiset tie.
    """
    rng = _rng(200, T, E, k, seed, TIE_MODES.index(mode), _TID_TIES)
    if mode == "equal":
        vals = np.array([-1.5, -0.0, 0.0, 0.5, 2.0], np.float32)
        return np.repeat(vals[rng.integers(0, vals.size, T)][:, None], E, axis=1)
    if mode == "coarse":
        return (np.round(rng.standard_normal((T, E)) * 2.0) / 2.0).astype(np.float32)
    if mode == "signed_zero":
        z = np.where(rng.random((T, E)) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
        few = rng.random((T, E)) < 0.05
        z[few] = np.where(rng.random(few.sum()) < 0.5, -1.0, 1.0).astype(np.float32)
        return z
    if mode == "kth":
        z = np.clip(rng.standard_normal((T, E)), -2.5, 2.5).astype(np.float32)
        for t in range(T):
            p = rng.permutation(E)
            z[t, p[:k - 1]] = 4.0 + 0.25 * np.arange(k - 1, dtype=np.float32)
            z[t, p[k - 1:k + 2]] = 3.0
        return z
    if mode in ("groups_equal", "groups_two"):
        if n_group < 2 or E % n_group:
            raise ValueError("group modes need E a multiple of n_group >= 2")
        gs = E // n_group
        z = np.empty((T, E), np.float32)
        for t in range(T):
            base = (rng.integers(0, 7, gs) * 0.5).astype(np.float32)
            strong = rng.random(n_group) < 0.5 if mode == "groups_two" else np.zeros(n_group, bool)
            for g in range(n_group):
                z[t, g * gs:(g + 1) * gs] = rng.permutation(base) + (2.0 if strong[g] else 0.0)
        return z
    raise ValueError(f"unknown tie mode {mode!r}")
