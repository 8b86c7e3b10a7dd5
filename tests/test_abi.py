"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects invalid arguments on the host before touching a device."""
import ctypes
import os
import re

import pytest

from grouped_gemm_topk_amd import moe as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|const char\s*\*)\s+(moe_\w+)\s*\(", src,
                                 flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(M.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return M.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert set(names) >= {"moe_align", "moe_grouped_gemm", "moe_fused_forward"}
    for n in names:
        assert hasattr(L, n), n
    assert set(M.EXPORTED) <= set(names)


def test_capacity_matches_macro(L):
    for T, k, E, bm in [(1, 8, 128, 16), (4096, 4, 18, 128), (8192, 8, 128, 64), (0, 2, 8, 16),
                        (3, 2, 64, 32)]:
        n = T * k
        want = (n + min(E, n) * (bm - 1) + bm - 1) // bm * bm
        assert L.moe_align_capacity(T, k, E, bm) == want
    assert L.moe_align_capacity(1, 1, 1, 24) == -1


def _layer(**kw):
    base = dict(T=4, H=64, I=32, E=8, top_k=2, block_m=16)
    base.update(kw)
    return M.LayerParams(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), -2), (dict(H=60), -2), (dict(I=12), -2), (dict(E=0), -2), (dict(E=257), -2),
    (dict(top_k=0), -2), (dict(top_k=9), -2), (dict(top_k=17, E=32), -2), (dict(block_m=24), -2),
    (dict(scoring=2), -2), (dict(n_group=3), -2), (dict(n_group=4, topk_group=5), -2),
    (dict(n_group=4, topk_group=1, top_k=3, scoring=1), -2),
    (dict(n_group=2, topk_group=1), -4), (dict(activation=3), -2), (dict(n_shared=2), -2),
    (dict(renormalize=2), -2), (dict(routed_scaling_factor=float("inf")), -2),
])
def test_fused_forward_rejects_bad_params(L, kw, status):
    p = _layer(**kw).c_struct()
    n = ctypes.c_size_t(0)
    st = L.moe_fused_forward(ctypes.byref(p), None, None, None, None, None, None, None, None, None,
                             None, None, None, None, ctypes.byref(n), None)
    assert st == status
    assert n.value == 0


def test_fused_forward_size_query_and_null_checks(L):
    p = _layer().c_struct()
    n = ctypes.c_size_t(0)
    assert L.moe_fused_forward(ctypes.byref(p), *([None] * 13), ctypes.byref(n), None) == 0
    assert n.value > 0
    need = n.value
    fake = 1 << 20     # never dereferenced: validation fails first
    small = ctypes.c_size_t(need - 1)
    assert L.moe_fused_forward(ctypes.byref(p), *([fake] * 12), fake, ctypes.byref(small),
                               None) == -3
    ok = ctypes.c_size_t(need)
    args = [fake] * 13
    args[0] = None   # x missing
    assert L.moe_fused_forward(ctypes.byref(p), *args, ctypes.byref(ok), None) == -1
    args = [fake] * 13
    args[0] = fake + 2   # misaligned x
    assert L.moe_fused_forward(ctypes.byref(p), *args, ctypes.byref(ok), None) == -5
    p2 = _layer(n_shared=1).c_struct()
    n2 = ctypes.c_size_t(0)
    L.moe_fused_forward(ctypes.byref(p2), *([None] * 13), ctypes.byref(n2), None)
    assert n2.value > need
    args = [fake] * 13
    args[4] = None   # shared_w13 missing
    assert L.moe_fused_forward(ctypes.byref(p2), *args, ctypes.byref(n2), None) == -1
    assert L.moe_fused_forward(ctypes.byref(p), *([fake] * 13), None, None) == -1


def test_fused_forward_t0_is_noop(L):
    p = _layer(T=0).c_struct()
    n = ctypes.c_size_t(0)
    assert L.moe_fused_forward(ctypes.byref(p), *([None] * 13), ctypes.byref(n), None) == 0
    ws = ctypes.c_size_t(n.value)
    assert L.moe_fused_forward(ctypes.byref(p), *([None] * 12), 1 << 20, ctypes.byref(ws),
                               None) == 0


def test_align_validation(L):
    fake = 1 << 20           # never dereferenced: validation fails first
    A = L.moe_align

    def call(ids=fake, T=4, k=2, E=8, bm=16, st=fake, ex=fake, nt=fake, cap=None, ws=fake,
             wsb=1 << 30):
        if cap is None:
            cap = max(L.moe_align_capacity(T, k, E, bm), 0)
        n = ctypes.c_size_t(wsb or 0)
        return A(ids, T, k, E, bm, st, ex, nt, cap, ws, None if wsb is None else ctypes.byref(n),
                 None)

    assert call(bm=24) == -2
    assert call(k=9) == -2
    assert call(T=-1) == -2
    assert call(k=17, E=32) == -2
    assert call(E=300, k=2) == -2
    assert call(cap=L.moe_align_capacity(4, 2, 8, 16) - 1) == -3
    assert call(st=None) == -1
    assert call(ids=None) == -1
    assert call(st=fake + 1) == -5
    assert call(ws=fake + 4) == -5
    assert call(wsb=None) == -1
    # a NULL workspace is a size query: nothing else is checked or launched
    n = ctypes.c_size_t(5)
    assert A(None, 4, 2, 8, 16, None, None, None, 0, None, ctypes.byref(n), None) == 0
    assert n.value == 0
    n = ctypes.c_size_t(0)
    assert A(fake, 8192, 8, 128, 64, fake, fake, fake, 1 << 20, None, ctypes.byref(n), None) == 0
    assert n.value > 0
    assert call(T=8192, k=8, E=128, bm=64, wsb=n.value - 1) == -3


def test_grouped_gemm_validation(L):
    fake = 1 << 20
    base = dict(a=fake, a_row_div=2, w=fake, E=8, N=64, K=64, sorted_token_ids=fake,
                expert_ids=fake, num_tokens_post_padded=fake, block_m=16, num_valid=8,
                capacity=128, epilogue=0, topk_weights=None, c=fake, c_is_fp32=1)

    def call(**kw):
        d = dict(base)
        d.update(kw)
        args = M.MoeGemmArgs(**d)
        n = ctypes.c_size_t(7)
        return L.moe_grouped_gemm(ctypes.byref(args), None, ctypes.byref(n), None)

    assert call(K=60) == -2
    assert call(N=60) == -2
    assert call(epilogue=1, N=56) == -2
    assert call(epilogue=4) == -2
    assert call(schedule=2) == -2          # MOE_SCHED_* only
    assert call(schedule=-1) == -2
    assert call(block_m=48) == -2
    assert call(capacity=100) == -2
    assert call(E=0) == -2
    assert call(num_valid=7) == -2         # not a multiple of a_row_div
    assert call(a=None) == -1
    assert call(epilogue=3, capacity=0) == 0   # scatter without weights is valid (weight 1)
    assert call(w=fake + 8) == -5
    assert call(capacity=0) == 0           # nothing to do
    # operand buffers must stay below the kernel's masked-load offset
    # (0x7fff0000 bytes): one expert's weights of 8 x K bf16 just past it, and
    # an A operand of 2 x K bf16 rows just past it, are rejected
    k_band = (0x7fff0000 // 16 + 8) // 8 * 8
    assert 0x7fff0000 <= 16 * k_band < 1 << 31
    assert call(N=8, K=k_band) == -4
    k_a = (0x7fff0000 // 32 + 8) // 8 * 8            # 16 A rows of k_a bf16 in the band
    assert 0x7fff0000 <= 32 * k_a < 1 << 31
    assert call(a_row_div=1, num_valid=16, N=8, K=k_a) == -4


def test_grouped_gemm_backward_validation_and_sizes(L):
    fake = 1 << 20
    M_, E, N, K, bm = 100, 4, 64, 96, 32
    cap = L.moe_align_capacity(M_, 1, E, bm)
    base = dict(x=fake, w=fake, dy=fake, M=M_, E=E, N=N, K=K, sorted_token_ids=fake,
                expert_ids=fake, num_tokens_post_padded=fake, block_m=bm, capacity=cap,
                dx=fake, dw=fake, out_fp32=0)

    def call(ws=None, n=0, **kw):
        d = dict(base)
        d.update(kw)
        args = M.MoeGemmBackwardArgs(**d)
        sz = ctypes.c_size_t(n)
        st = L.moe_grouped_gemm_backward(ctypes.byref(args), ws, ctypes.byref(sz), None)
        return st, sz.value

    r = lambda b: (b + 255) // 256 * 256
    assert call(dw=None) == (0, r(E * N * K * 2))
    assert call(dx=None) == (0, r(N * cap * 2) + r(K * cap * 2) + r(2 * E * 4))
    assert call() == (0, r(E * N * K * 2) + r(N * cap * 2) + r(K * cap * 2) + r(2 * E * 4))
    assert call(K=60)[0] == -2
    assert call(N=12)[0] == -2
    assert call(E=0)[0] == -2
    assert call(block_m=48)[0] == -2
    assert call(capacity=cap - bm)[0] == -3          # below MOE_ALIGN_CAPACITY
    assert call(ws=fake, n=10)[0] == -3              # workspace too small
    assert call(ws=fake, n=1 << 30, dx=None, dw=None)[0] == 0   # nothing requested: no launch
    assert call(ws=fake, n=1 << 30, dy=None)[0] == -1
    assert call(ws=fake, n=1 << 30, dw=None, w=None)[0] == -1
    assert call(ws=fake, n=1 << 30, dx=None, x=None)[0] == -1
    assert call(ws=fake, n=1 << 30, expert_ids=None)[0] == -1
    assert call(ws=fake + 8, n=1 << 30)[0] == -5
    assert L.moe_grouped_gemm_backward(None, None, None, None) == -1


def test_fused_forward_mxfp8_validation(L):
    """MXFP8 entry point: decode shapes only, rows in blocks of 32, scales
    required; the workspace is the bf16 layer's."""
    p = _layer(H=64, I=64).c_struct()
    n = ctypes.c_size_t(0)
    assert L.moe_fused_forward_mxfp8(ctypes.byref(p), *([None] * 17), ctypes.byref(n), None) == 0
    nb = ctypes.c_size_t(0)
    assert L.moe_fused_forward(ctypes.byref(p), *([None] * 13), ctypes.byref(nb), None) == 0
    assert n.value == nb.value > 0
    for kw, status in [(dict(T=17, H=64, I=64), -4), (dict(H=72, I=64), -2),
                       (dict(H=64, I=40), -2)]:
        q = _layer(**kw).c_struct()
        m = ctypes.c_size_t(0)
        assert L.moe_fused_forward_mxfp8(ctypes.byref(q), *([None] * 17), ctypes.byref(m),
                                         None) == status
    fake = 1 << 20
    ok = ctypes.c_size_t(n.value)
    args = [fake] * 17
    args[3] = None   # w13 scales missing
    assert L.moe_fused_forward_mxfp8(ctypes.byref(p), *args, ctypes.byref(ok), None) == -1
    ps = _layer(H=64, I=64, n_shared=1).c_struct()
    ns = ctypes.c_size_t(0)
    L.moe_fused_forward_mxfp8(ctypes.byref(ps), *([None] * 17), ctypes.byref(ns), None)
    for i in (7, 9):   # shared_w13 scales, shared_w2 scales missing
        args = [fake] * 17
        args[i] = None
        assert L.moe_fused_forward_mxfp8(ctypes.byref(ps), *args, ctypes.byref(ns), None) == -1


def test_fused_forward_router_validation(L):
    """Router entry point: the workspace is the layer's; router_w is required
    and 16-byte aligned; router_logits_out may be NULL."""
    p = _layer(H=64, I=64).c_struct()
    n = ctypes.c_size_t(0)
    assert L.moe_fused_forward_router(ctypes.byref(p), *([None] * 14), ctypes.byref(n), None) == 0
    nb = ctypes.c_size_t(0)
    assert L.moe_fused_forward(ctypes.byref(p), *([None] * 13), ctypes.byref(nb), None) == 0
    assert n.value == nb.value > 0
    fake = 1 << 20
    ok = ctypes.c_size_t(n.value)
    args = [fake] * 14
    args[1] = None   # router_w missing
    assert L.moe_fused_forward_router(ctypes.byref(p), *args, ctypes.byref(ok), None) == -1
    args = [fake] * 14
    args[1] = fake + 4   # router_w misaligned
    assert L.moe_fused_forward_router(ctypes.byref(p), *args, ctypes.byref(ok), None) == -5


def test_status_offset(L):
    """The status word lies inside the layer's workspace, 4-byte aligned, for
    prefill and decode shapes; invalid parameters give their status."""
    for kw in (dict(), dict(T=1, E=128, top_k=8), dict(T=4096, H=3072, I=2560, E=18, top_k=4,
                                                       block_m=128, n_shared=1)):
        p = _layer(**kw).c_struct()
        n = ctypes.c_size_t(0)
        assert L.moe_fused_forward(ctypes.byref(p), *([None] * 13), ctypes.byref(n), None) == 0
        off = L.moe_fused_forward_status_offset(ctypes.byref(p))
        assert 0 <= off and off + 4 <= n.value and off % 4 == 0
    assert L.moe_fused_forward_status_offset(ctypes.byref(_layer(block_m=24).c_struct())) == -2
