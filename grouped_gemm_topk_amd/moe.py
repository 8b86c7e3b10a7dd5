"""Python binding of libmoe: the three C-ABI calls with the same names.

Argument marshalling only: tensors are checked for device, dtype and
contiguity, their device pointers and the current HIP stream are handed to the
library, and a negative status becomes an exception.  Every step of the MoE
forward runs in libmoe's HIP kernels; there is no other implementation here,
and a missing or unbuildable library is an error.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
SCORE_SOFTMAX, SCORE_SIGMOID = 0, 1
ACT_SWIGLU, ACT_RELU2 = 0, 1
EPI_STORE, EPI_SWIGLU, EPI_RELU2, EPI_WEIGHTED_SCATTER = 0, 1, 2, 3
SCHED_PERSISTENT, SCHED_PER_TILE = 0, 1

EXPORTED = ("moe_align", "moe_grouped_gemm", "moe_grouped_gemm_backward", "moe_fused_forward",
            "moe_fused_forward_mxfp8", "moe_fused_forward_router", "moe_fused_forward_noalloc",
            "moe_fused_forward_status_offset", "moe_align_capacity", "moe_status_string")

NOALLOC_SCRATCH_BYTES = 32 << 20


class MoeError(RuntimeError):
    def __init__(self, call: str, status: int, text: str):
        super().__init__(f"{call} failed with status {status}: {text}")
        self.status = status


class MoeLayerParams(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("top_k", ctypes.c_int32), ("block_m", ctypes.c_int32),
                ("scoring", ctypes.c_int32), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("routed_scaling_factor", ctypes.c_float), ("activation", ctypes.c_int32),
                ("n_shared", ctypes.c_int32)]


class MoeGemmArgs(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("a_row_div", ctypes.c_int32), ("w", ctypes.c_void_p),
                ("E", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("sorted_token_ids", ctypes.c_void_p), ("expert_ids", ctypes.c_void_p),
                ("num_tokens_post_padded", ctypes.c_void_p), ("block_m", ctypes.c_int32),
                ("num_valid", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("epilogue", ctypes.c_int32), ("topk_weights", ctypes.c_void_p),
                ("c", ctypes.c_void_p), ("c_is_fp32", ctypes.c_int32), ("schedule", ctypes.c_int32)]


class MoeGemmBackwardArgs(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("w", ctypes.c_void_p), ("dy", ctypes.c_void_p),
                ("M", ctypes.c_int32), ("E", ctypes.c_int32), ("N", ctypes.c_int32),
                ("K", ctypes.c_int32), ("sorted_token_ids", ctypes.c_void_p),
                ("expert_ids", ctypes.c_void_p), ("num_tokens_post_padded", ctypes.c_void_p),
                ("block_m", ctypes.c_int32), ("capacity", ctypes.c_int32), ("dx", ctypes.c_void_p),
                ("dw", ctypes.c_void_p), ("out_fp32", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmoe.so is not built ({LIB_PATH}); run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)
        L.moe_align.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, i64, vp, sz, vp]
        L.moe_align.restype = ctypes.c_int
        L.moe_grouped_gemm.argtypes = [ctypes.POINTER(MoeGemmArgs), vp, sz, vp]
        L.moe_grouped_gemm.restype = ctypes.c_int
        L.moe_grouped_gemm_backward.argtypes = [ctypes.POINTER(MoeGemmBackwardArgs), vp, sz, vp]
        L.moe_grouped_gemm_backward.restype = ctypes.c_int
        L.moe_fused_forward.argtypes = [ctypes.POINTER(MoeLayerParams), vp, vp, vp, vp, vp, vp,
                                        vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_fused_forward.restype = ctypes.c_int
        L.moe_fused_forward_mxfp8.argtypes = [ctypes.POINTER(MoeLayerParams), vp, vp, vp, vp, vp,
                                              vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                              vp]
        L.moe_fused_forward_mxfp8.restype = ctypes.c_int
        L.moe_fused_forward_router.argtypes = [ctypes.POINTER(MoeLayerParams), vp, vp, vp, vp, vp,
                                               vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_fused_forward_router.restype = ctypes.c_int
        L.moe_fused_forward_noalloc.argtypes = [ctypes.POINTER(MoeLayerParams), vp, vp, vp, vp, vp,
                                                vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_fused_forward_noalloc.restype = ctypes.c_int
        L.moe_fused_forward_status_offset.argtypes = [ctypes.POINTER(MoeLayerParams)]
        L.moe_fused_forward_status_offset.restype = ctypes.c_int64
        L.moe_align_capacity.argtypes = [i32, i32, i32, i32]
        L.moe_align_capacity.restype = ctypes.c_int64
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(call: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(call, status, lib().moe_status_string(status).decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtype, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def align_capacity(T: int, k: int, E: int, block_m: int) -> int:
    return int(lib().moe_align_capacity(T, k, E, block_m))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- moe_align
def moe_align(topk_ids: torch.Tensor, E: int, block_m: int, sorted_token_ids=None,
              expert_ids=None, num_tokens_post_padded=None, workspace=None, stream=None):
    """Sort slots by expert and pad to block_m.  Returns (sorted_token_ids,
    expert_ids, num_tokens_post_padded) as int32 GPU tensors of capacity length
    (entries beyond the padded count are unspecified)."""
    _dev(topk_ids, "topk_ids", torch.int32)
    T, k = topk_ids.shape
    cap = align_capacity(T, k, E, block_m)
    dev = topk_ids.device
    if sorted_token_ids is None:
        sorted_token_ids = torch.empty(cap, dtype=torch.int32, device=dev)
    if expert_ids is None:
        expert_ids = torch.empty(max(cap // block_m, 1), dtype=torch.int32, device=dev)
    if num_tokens_post_padded is None:
        num_tokens_post_padded = torch.empty(1, dtype=torch.int32, device=dev)
    n = ctypes.c_size_t(0)
    L = lib()
    if workspace is None:
        _check("moe_align", L.moe_align(_ptr(topk_ids), T, k, E, block_m, None, None, None, cap,
                                        None, ctypes.byref(n), None))
        workspace = _workspace(n.value, dev)
    n = ctypes.c_size_t(workspace.numel())
    _check("moe_align", L.moe_align(_ptr(topk_ids), T, k, E, block_m, _ptr(sorted_token_ids),
                                    _ptr(expert_ids), _ptr(num_tokens_post_padded),
                                    sorted_token_ids.numel(), _ptr(workspace), ctypes.byref(n),
                                    _stream(stream)))
    return sorted_token_ids, expert_ids, num_tokens_post_padded


# ---------------------------------------------------------------- moe_grouped_gemm
def moe_grouped_gemm(a: torch.Tensor, a_row_div: int, w: torch.Tensor,
                     sorted_token_ids: torch.Tensor, expert_ids: torch.Tensor,
                     num_tokens_post_padded: torch.Tensor, block_m: int, num_valid: int,
                     epilogue: int, c: torch.Tensor, topk_weights: Optional[torch.Tensor] = None,
                     stream=None, schedule: int = 0) -> torch.Tensor:
    """One grouped GEMM over the aligned layout; writes and returns ``c``.
    ``schedule``: SCHED_PERSISTENT (default) or SCHED_PER_TILE."""
    _dev(a, "a", torch.bfloat16)
    _dev(w, "w", torch.bfloat16)
    E, N, K = w.shape
    if a.shape[-1] != K:
        raise ValueError("a and w disagree on K")
    for name, t in (("sorted_token_ids", sorted_token_ids), ("expert_ids", expert_ids),
                    ("num_tokens_post_padded", num_tokens_post_padded)):
        _dev(t, name, torch.int32)
    if topk_weights is not None:
        _dev(topk_weights, "topk_weights", torch.float32)
    if c.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("c must be float32 or bfloat16")
    _dev(c, "c", c.dtype)
    args = MoeGemmArgs(a=_ptr(a), a_row_div=a_row_div, w=_ptr(w), E=E, N=N, K=K,
                       sorted_token_ids=_ptr(sorted_token_ids), expert_ids=_ptr(expert_ids),
                       num_tokens_post_padded=_ptr(num_tokens_post_padded), block_m=block_m,
                       num_valid=num_valid, capacity=sorted_token_ids.numel(), epilogue=epilogue,
                       topk_weights=_ptr(topk_weights), c=_ptr(c),
                       c_is_fp32=1 if c.dtype == torch.float32 else 0, schedule=schedule)
    n = ctypes.c_size_t(0)
    _check("moe_grouped_gemm", lib().moe_grouped_gemm(ctypes.byref(args), None, ctypes.byref(n),
                                                      _stream(stream)))
    return c


class IndexedGroupedGemm:
    """The contiguous grouped GEMM of the axolotl page (``cg_grouped_gemm_forward``):
    ``out[i] = x[i] @ w[expert_indices[i]].T`` for x bf16 [M, K], w bf16
    [G, N, K] and int32 indices [M] (any grouping).  Two library calls:
    ``moe_align`` over the indices as top-1 routing, then ``moe_grouped_gemm``
    with the scatter epilogue and no weights.  The align outputs and the
    workspace are allocated once here, so ``run()`` only launches."""

    def __init__(self, x: torch.Tensor, w: torch.Tensor, expert_indices: torch.Tensor,
                 block_m: int = 128, out: Optional[torch.Tensor] = None):
        _dev(x, "x", torch.bfloat16)
        _dev(w, "w", torch.bfloat16)
        G, N, K = w.shape
        M = x.shape[0]
        if x.dim() != 2 or x.shape[1] != K:
            raise ValueError("x must be [M, K] with the K of w")
        _dev(expert_indices, "expert_indices", torch.int32, (M,))
        if out is None:
            out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
        _dev(out, "out", out.dtype, (M, N))
        self.x, self.w, self.out, self.block_m = x, w, out, block_m
        self.ids = expert_indices.view(M, 1)
        self.G, self.M = G, M
        cap = align_capacity(M, 1, G, block_m)
        dev = x.device
        self.sorted = torch.empty(cap, dtype=torch.int32, device=dev)
        self.expert_ids = torch.empty(max(cap // block_m, 1), dtype=torch.int32, device=dev)
        self.ntpp = torch.empty(1, dtype=torch.int32, device=dev)
        n = ctypes.c_size_t(0)
        _check("moe_align", lib().moe_align(_ptr(self.ids), M, 1, G, block_m, None, None, None,
                                            cap, None, ctypes.byref(n), None))
        self.workspace = _workspace(n.value, dev)

    def align(self, stream=None):
        moe_align(self.ids, self.G, self.block_m, self.sorted, self.expert_ids, self.ntpp,
                  self.workspace, stream)

    def gemm(self, stream=None, schedule: int = 0) -> torch.Tensor:
        return moe_grouped_gemm(self.x, 1, self.w, self.sorted, self.expert_ids, self.ntpp,
                                self.block_m, self.M, EPI_WEIGHTED_SCATTER, self.out, None, stream,
                                schedule)

    def run(self, stream=None) -> torch.Tensor:
        self.align(stream)
        return self.gemm(stream)

    def backward(self, dy: torch.Tensor, dx: Optional[torch.Tensor] = None,
                 dw: Optional[torch.Tensor] = None, want_dx: bool = True, want_dw: bool = True,
                 out_fp32: bool = False, stream=None):
        """Gradients for the output gradient ``dy`` (bf16 [M, N]) through
        ``moe_grouped_gemm_backward``: returns ``(dx, dw)`` (bf16, or float32
        with ``out_fp32``; None where not wanted).  Uses the aligned layout of
        the last ``align()``/``run()``; the workspace is kept between calls."""
        G, N, K = self.w.shape
        _dev(dy, "dy", torch.bfloat16, (self.M, N))
        dt = torch.float32 if out_fp32 else torch.bfloat16
        dev = dy.device
        if want_dx and dx is None:
            dx = torch.empty((self.M, K), dtype=dt, device=dev)
        if want_dw and dw is None:
            dw = torch.empty((G, N, K), dtype=dt, device=dev)
        if dx is not None:
            _dev(dx, "dx", dt, (self.M, K))
        if dw is not None:
            _dev(dw, "dw", dt, (G, N, K))
        args = MoeGemmBackwardArgs(x=_ptr(self.x), w=_ptr(self.w), dy=_ptr(dy), M=self.M, E=G, N=N,
                                   K=K, sorted_token_ids=_ptr(self.sorted),
                                   expert_ids=_ptr(self.expert_ids),
                                   num_tokens_post_padded=_ptr(self.ntpp), block_m=self.block_m,
                                   capacity=self.sorted.numel(), dx=_ptr(dx) if want_dx else None,
                                   dw=_ptr(dw) if want_dw else None, out_fp32=int(out_fp32))
        n = ctypes.c_size_t(0)
        L = lib()
        _check("moe_grouped_gemm_backward",
               L.moe_grouped_gemm_backward(ctypes.byref(args), None, ctypes.byref(n), None))
        key = (want_dx, want_dw)
        ws = getattr(self, "_bwd_ws", {}).get(key)
        if ws is None or ws.numel() < n.value:
            ws = _workspace(n.value, dev)
            self._bwd_ws = {**getattr(self, "_bwd_ws", {}), key: ws}
        n = ctypes.c_size_t(ws.numel())
        _check("moe_grouped_gemm_backward",
               L.moe_grouped_gemm_backward(ctypes.byref(args), _ptr(ws), ctypes.byref(n),
                                           _stream(stream)))
        return (dx if want_dx else None), (dw if want_dw else None)


def indexed_grouped_gemm(x: torch.Tensor, w: torch.Tensor, expert_indices: torch.Tensor,
                         block_m: int = 128, out: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """One-shot form of :class:`IndexedGroupedGemm`; returns ``out`` (bf16
    [M, N] unless a float32 ``out`` is passed)."""
    return IndexedGroupedGemm(x, w, expert_indices, block_m, out).run(stream)


# ---------------------------------------------------------------- moe_fused_forward
@dataclass
class LayerParams:
    T: int
    H: int
    I: int
    E: int
    top_k: int
    block_m: int = 16
    scoring: int = SCORE_SOFTMAX
    n_group: int = 1
    topk_group: int = 1
    renormalize: int = 1
    routed_scaling_factor: float = 1.0
    activation: int = ACT_SWIGLU
    n_shared: int = 0

    def c_struct(self) -> MoeLayerParams:
        return MoeLayerParams(self.T, self.H, self.I, self.E, self.top_k, self.block_m,
                              self.scoring, self.n_group, self.topk_group, self.renormalize,
                              float(self.routed_scaling_factor), self.activation, self.n_shared)

    @property
    def M1(self) -> int:
        return 2 * self.I if self.activation == ACT_SWIGLU else self.I

    @classmethod
    def from_config(cls, cfg, T: Optional[int] = None, block_m: Optional[int] = None):
        return cls(T=cfg.T if T is None else T, H=cfg.H, I=cfg.I, E=cfg.E, top_k=cfg.top_k,
                   block_m=cfg.block_m if block_m is None else block_m, scoring=cfg.scoring,
                   n_group=cfg.n_group, topk_group=cfg.topk_group, renormalize=cfg.renormalize,
                   routed_scaling_factor=cfg.scale, activation=cfg.activation,
                   n_shared=cfg.n_shared)


def fused_workspace_bytes(p: LayerParams) -> int:
    n = ctypes.c_size_t(0)
    cp = p.c_struct()
    _check("moe_fused_forward", lib().moe_fused_forward(
        ctypes.byref(cp), None, None, None, None, None, None, None, None, None, None, None, None,
        None, ctypes.byref(n), None))
    return n.value


class FusedLayer:
    """A ready-to-run moe_fused_forward call: checked tensors, outputs and the
    workspace are bound once, ``run()`` only enqueues the library call (the
    form used for timing and graph capture).

    With ``router_w`` (bf16 [E, H]) the router logits are computed by the
    library (moe_fused_forward_router) into ``logits`` (allocated when None).

    With ``scales`` (a dict of uint8 tensors ``w13``, ``w2`` and, with a
    shared expert, ``shared_w13``, ``shared_w2``: E8M0 bytes, one per 32
    elements along each row) the weight tensors are MXFP8 (uint8 FP8 E4M3
    bytes of the same shapes) and the call is moe_fused_forward_mxfp8."""

    def __init__(self, p: LayerParams, x, logits, w13, w2, shared_w13=None, shared_w2=None,
                 out=None, routing_outputs: bool = False, workspace=None, scales=None,
                 router_w=None):
        self.p = p
        dev = x.device
        wt = torch.uint8 if scales is not None else torch.bfloat16
        _dev(x, "x", torch.bfloat16, (p.T, p.H))
        if router_w is not None:
            if scales is not None:
                raise ValueError("the router path takes bf16 expert weights")
            _dev(router_w, "router_w", torch.bfloat16, (p.E, p.H))
            if logits is None:
                logits = torch.empty((p.T, p.E), dtype=torch.float32, device=dev)
        _dev(logits, "router_logits", torch.float32, (p.T, p.E))
        _dev(w13, "w13", wt, (p.E, p.M1, p.H))
        _dev(w2, "w2", wt, (p.E, p.H, p.I))
        if p.n_shared:
            _dev(shared_w13, "shared_w13", wt, (p.M1, p.H))
            _dev(shared_w2, "shared_w2", wt, (p.H, p.I))
        self.scales = scales
        if scales is not None:
            if p.H % 32 or p.I % 32:
                raise ValueError("MXFP8 weights need H and I multiples of 32")
            _dev(scales["w13"], "w13 scales", torch.uint8, (p.E, p.M1, p.H // 32))
            _dev(scales["w2"], "w2 scales", torch.uint8, (p.E, p.H, p.I // 32))
            if p.n_shared:
                _dev(scales["shared_w13"], "shared_w13 scales", torch.uint8, (p.M1, p.H // 32))
                _dev(scales["shared_w2"], "shared_w2 scales", torch.uint8, (p.H, p.I // 32))
        if out is None:
            out = torch.empty((p.T, p.H), dtype=torch.float32, device=dev)
        _dev(out, "out", torch.float32, (p.T, p.H))
        self.tensors = dict(x=x, logits=logits, w13=w13, w2=w2, shared_w13=shared_w13,
                            shared_w2=shared_w2, out=out)
        self.routing = {}
        if routing_outputs:
            cap = align_capacity(p.T, p.top_k, p.E, p.block_m)
            self.routing = dict(
                topk_ids=torch.empty((p.T, p.top_k), dtype=torch.int32, device=dev),
                topk_weights=torch.empty((p.T, p.top_k), dtype=torch.float32, device=dev),
                sorted_token_ids=torch.empty(cap, dtype=torch.int32, device=dev),
                expert_ids=torch.empty(max(cap // p.block_m, 1), dtype=torch.int32, device=dev),
                num_tokens_post_padded=torch.empty(1, dtype=torch.int32, device=dev))
        need = fused_workspace_bytes(p)
        if workspace is None:
            workspace = _workspace(need, dev)
        elif workspace.numel() < need:
            raise ValueError(f"workspace needs {need} bytes")
        self.workspace = workspace
        self._cp = p.c_struct()
        r = self.routing
        t = self.tensors
        tail = [_ptr(t["out"]), _ptr(r.get("topk_ids")), _ptr(r.get("topk_weights")),
                _ptr(r.get("sorted_token_ids")), _ptr(r.get("expert_ids")),
                _ptr(r.get("num_tokens_post_padded")), _ptr(workspace)]
        if router_w is not None:
            self._call = "moe_fused_forward_router"
            self.tensors["router_w"] = router_w
            self._args = [ctypes.byref(self._cp), _ptr(t["x"]), _ptr(router_w), _ptr(t["logits"]),
                          _ptr(t["w13"]), _ptr(t["w2"]), _ptr(t["shared_w13"]),
                          _ptr(t["shared_w2"])] + tail
        elif scales is None:
            self._call = "moe_fused_forward"
            self._args = [ctypes.byref(self._cp), _ptr(t["x"]), _ptr(t["logits"]), _ptr(t["w13"]),
                          _ptr(t["w2"]), _ptr(t["shared_w13"]), _ptr(t["shared_w2"])] + tail
        else:
            self._call = "moe_fused_forward_mxfp8"
            self._args = [ctypes.byref(self._cp), _ptr(t["x"]), _ptr(t["logits"]), _ptr(t["w13"]),
                          _ptr(scales["w13"]), _ptr(t["w2"]), _ptr(scales["w2"]),
                          _ptr(t["shared_w13"]), _ptr(scales.get("shared_w13")),
                          _ptr(t["shared_w2"]), _ptr(scales.get("shared_w2"))] + tail
        self._fn = getattr(lib(), self._call)
        self._n = ctypes.c_size_t(workspace.numel())

    @property
    def out(self) -> torch.Tensor:
        return self.tensors["out"]

    def status(self) -> torch.Tensor:
        """The layer's status word in the workspace (int32 [1] view, on the
        device): 0 after a call whose cross-workgroup waits all ended normally,
        1 when a bounded wait expired (that call's output is invalid)."""
        off = int(lib().moe_fused_forward_status_offset(ctypes.byref(self._cp)))
        if off < 0:
            _check("moe_fused_forward_status_offset", off)
        return self.workspace[off:off + 4].view(torch.int32)

    def run(self, stream=None) -> torch.Tensor:
        self._n.value = self.workspace.numel()
        _check(self._call, self._fn(*self._args, ctypes.byref(self._n), _stream(stream)))
        return self.tensors["out"]


def _with_status(layer: "FusedLayer") -> dict:
    r = dict(layer.routing)
    if layer.p.T > 0:
        r["status"] = layer.status()
    return r


def moe_fused_forward_mxfp8(p: LayerParams, x, router_logits, w13_q, w13_scale, w2_q, w2_scale,
                            shared_w13_q=None, shared_w13_scale=None, shared_w2_q=None,
                            shared_w2_scale=None, out=None, return_routing: bool = False,
                            stream=None):
    """The layer with MXFP8 expert weights (decode shapes, T <= 16): uint8 FP8
    E4M3 weight bytes and uint8 E8M0 scales, one per 32 elements along a row.
    With ``return_routing`` the dict also holds ``status`` (see FusedLayer.status)."""
    sc = {"w13": w13_scale, "w2": w2_scale}
    if p.n_shared:
        sc["shared_w13"], sc["shared_w2"] = shared_w13_scale, shared_w2_scale
    layer = FusedLayer(p, x, router_logits, w13_q, w2_q, shared_w13_q, shared_w2_q, out,
                       routing_outputs=return_routing, scales=sc)
    if p.T > 0:
        layer.run(stream)
    return (layer.out, _with_status(layer)) if return_routing else layer.out


def moe_fused_forward_router(p: LayerParams, x, router_w, w13, w2, shared_w13=None,
                             shared_w2=None, out=None, return_routing: bool = False, stream=None):
    """The layer from the hidden states and the router weight: returns ``out``
    (or ``(out, routing_dict)`` with the computed ``router_logits`` in it)."""
    layer = FusedLayer(p, x, None, w13, w2, shared_w13, shared_w2, out,
                       routing_outputs=return_routing, router_w=router_w)
    if p.T > 0:
        layer.run(stream)
    if return_routing:
        return layer.out, {**_with_status(layer), "router_logits": layer.tensors["logits"]}
    return layer.out


def moe_fused_forward(p: LayerParams, x, router_logits, w13, w2, shared_w13=None, shared_w2=None,
                      out=None, return_routing: bool = False, stream=None):
    """The whole MoE layer.  Returns ``out`` (fp32 [T,H]) or, with
    ``return_routing``, ``(out, routing_dict)``; the dict also holds the
    call's ``status`` word (see FusedLayer.status)."""
    layer = FusedLayer(p, x, router_logits, w13, w2, shared_w13, shared_w2, out,
                       routing_outputs=return_routing)
    if p.T > 0:
        layer.run(stream)
    return (layer.out, _with_status(layer)) if return_routing else layer.out


def moe_fused_forward_noalloc(p: LayerParams, x, router_logits, w13, w2, shared_w13=None,
                              shared_w2=None, out=None, routing=None, stream=None):
    """The layer through moe_fused_forward_noalloc: no workspace, the library's
    device-resident scratch instead (layers whose workspace exceeds it are
    rejected).  ``out`` (fp32 [T, H]) and ``routing`` (a dict holding any of
    topk_ids, topk_weights, sorted_token_ids, expert_ids,
    num_tokens_post_padded) are caller tensors and are only checked here, so
    that the call allocates nothing when they are given.  Returns ``out``."""
    dev = x.device
    _dev(x, "x", torch.bfloat16, (p.T, p.H))
    _dev(router_logits, "router_logits", torch.float32, (p.T, p.E))
    _dev(w13, "w13", torch.bfloat16, (p.E, p.M1, p.H))
    _dev(w2, "w2", torch.bfloat16, (p.E, p.H, p.I))
    if p.n_shared:
        _dev(shared_w13, "shared_w13", torch.bfloat16, (p.M1, p.H))
        _dev(shared_w2, "shared_w2", torch.bfloat16, (p.H, p.I))
    if out is None:
        out = torch.empty((p.T, p.H), dtype=torch.float32, device=dev)
    _dev(out, "out", torch.float32, (p.T, p.H))
    r = routing or {}
    cap = align_capacity(p.T, p.top_k, p.E, p.block_m)
    shapes = dict(topk_ids=(torch.int32, (p.T, p.top_k)),
                  topk_weights=(torch.float32, (p.T, p.top_k)),
                  sorted_token_ids=(torch.int32, None), expert_ids=(torch.int32, None),
                  num_tokens_post_padded=(torch.int32, (1,)))
    for name, t in r.items():
        dt, shp = shapes[name]
        _dev(t, name, dt, shp)
    if "sorted_token_ids" in r and r["sorted_token_ids"].numel() < cap:
        raise ValueError(f"sorted_token_ids needs {cap} entries")
    if "expert_ids" in r and r["expert_ids"].numel() < max(cap // p.block_m, 1):
        raise ValueError(f"expert_ids needs {max(cap // p.block_m, 1)} entries")
    cp = p.c_struct()
    _check("moe_fused_forward_noalloc", lib().moe_fused_forward_noalloc(
        ctypes.byref(cp), _ptr(x), _ptr(router_logits), _ptr(w13), _ptr(w2), _ptr(shared_w13),
        _ptr(shared_w2), _ptr(out), _ptr(r.get("topk_ids")), _ptr(r.get("topk_weights")),
        _ptr(r.get("sorted_token_ids")), _ptr(r.get("expert_ids")),
        _ptr(r.get("num_tokens_post_padded")), _stream(stream)))
    return out
