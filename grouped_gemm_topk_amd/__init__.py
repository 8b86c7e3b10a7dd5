"""libmoe: fused Mixture-of-Experts forward for MI355X (gfx950).

The compute lives in ``libmoe.so`` (hand-written HIP kernels behind a C ABI,
``include/moe.h``); :mod:`grouped_gemm_topk_amd.moe` is its Python binding.
"""
from .moe import (  # noqa: F401
    ACT_RELU2, ACT_SWIGLU, EPI_RELU2, EPI_STORE, EPI_SWIGLU, EPI_WEIGHTED_SCATTER,
    SCORE_SIGMOID, SCORE_SOFTMAX, FusedLayer, LayerParams, MoeError, align_capacity, lib,
    moe_align, moe_fused_forward, moe_grouped_gemm,
)
