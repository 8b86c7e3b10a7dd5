"""Benchmark of the fused MoE forward (libmoe) on one MI355X.

One step = one moe_fused_forward call over one batch (gating, align, GEMM1 +
activation, GEMM2 + routed weight, combine) on the DeepSeek-V3-8B-shaped layer
(T=4096, H=3072, I=2560, 18 routed experts top-4 with grouped sigmoid routing,
one shared expert, SwiGLU, bf16 weights).  Inputs are seeded synthetic tensors
resident in HBM before timing starts.

Prints ONE JSON line: TFLOPS of the layer (2*T*k_eff*3*H*I / latency), the
roofline entry of the dominant kernel (the SwiGLU grouped GEMM, timed alone
with HIP events on its stream), decode microseconds per layer at T = 1, 3, 8
(128 experts top-8) and of the squared-ReLU layer at T = 1, 16, each cycling
through enough distinct layers that the 256 MB Infinity Cache cannot hold the
touched weights and cross-checked with an explicit cache flush before every
call, the standalone grouped GEMM at the four shapes of the axolotl page's
benchmark table, the layer with the router logits fused into gating against a
separate router GEMM, the achievable peaks of this GPU from the probe library's own MFMA-loop
and streaming-read kernels, and the CPU oracle's rate on a bounded sample of
the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MALL_BYTES = 256 << 20           # Infinity Cache
# decode-shaped layers (GEMV path): 128 experts top-8 SwiGLU at T = 1, 3, 8 and
# the squared-ReLU layer (128 experts top-6) at T = 1, 16
DECODE_CASES = ("decode_t1", "decode_t3", "decode_t8", "relu2_t1", "relu2_t16")
# the other MFMA-path layers, timed like the headline one: 128 experts top-8
# with a Zipf(1.1) load (T = 8192) and the squared-ReLU layer at T = 2048
PREFILL_CASES = ("zipf128", "relu2_t2048")

# HBM-side bytes per launch of the dominant kernel (routed SwiGLU grouped GEMM
# of the dsv3 layer) from two rocprofv3 counter passes: FETCH_SIZE x 2.0 and
# WRITE_SIZE x 1.0, the factors that turn the same counters into the known
# bytes of a 1 GiB device copy.  Valid only for the kernel source with this
# digest; any other source reports traffic null until it is measured again.
# the SwiGLU grouped GEMM instantiation a layer of each BLOCK_M launches
DOMINANT_KERNEL = {
    256: "grouped_gemm_kernel<256, 256, 4, 2, true, 64, 2, 1, false, false>",
    128: "grouped_gemm_kernel<128, 256, 2, 4, true, 64, 3, 1, false, true>",
}

DOMINANT_TRAFFIC = {
    "src": "grouped_gemm_topk_amd/csrc/gemm.hip",
    "sha256": "b5d922985dcb8baad466192d8ad6824bea27542d557be1d540dbdfd58450dc9f",
    "config": "dsv3",
    # one call, one persistent launch
    "fetch_bytes": 898884203,
    "write_bytes": 95288517,
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="dsv3")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode measurements")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode measurements (one JSON line with them), for profiler passes")
    ap.add_argument("--no-peaks", action="store_true", help="skip the achievable-peak probes")
    ap.add_argument("--no-gemm-scenarios", action="store_true",
                    help="skip the standalone grouped-GEMM scenarios")
    ap.add_argument("--no-router", action="store_true", help="skip the router-fusion comparison")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the other prefill layers (zipf128, relu2_t2048)")
    ap.add_argument("--router-only", action="store_true",
                    help="only the router-fusion comparison (one JSON line)")
    ap.add_argument("--gemm-scenarios-only", action="store_true",
                    help="only the standalone grouped-GEMM scenarios (one JSON line), for profiler passes")
    ap.add_argument("--cpu-tokens", type=int, default=4096,
                    help="tokens of the workload the CPU oracle runs on")
    ap.add_argument("--extra", default="", help="comma list of more configs to time (report only)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a device-to-device copy of known size (scales the HBM "
                         "byte counters of a profiler pass) and exit")
    return ap.parse_args()


def _to_dev(a, torch):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _layer(cfg, inp, torch, moe, routing=False, weights=None):
    p = moe.LayerParams.from_config(cfg)
    w = weights or {k: _to_dev(inp[k], torch) for k in ("w13", "w2", "shared_w13", "shared_w2")
                    if k in inp}
    return moe.FusedLayer(p, _to_dev(inp["x"], torch), _to_dev(inp["logits"], torch), w["w13"],
                          w["w2"], w.get("shared_w13"), w.get("shared_w2"),
                          routing_outputs=routing), w


def time_layer(layer, steps, warmup, torch, spread=False):
    """Mean ms per step over `steps` back-to-back calls (events around the
    whole run), the wall time, and with `spread` the p10/p50/p90 of per-step
    event pairs (a second timed run, so the first stays free of them)."""
    for _ in range(warmup):
        layer.run()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(s)
    for _ in range(steps):
        layer.run()
    e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean = e0.elapsed_time(e1) / steps
    if not spread:
        return mean, wall, None
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(s)
    for i in range(steps):
        layer.run()
        ev[i + 1].record(s)
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    return mean, wall, {q: round(float(np.percentile(per, int(q[1:]))), 4) for q in ("p10", "p50", "p90")}


def time_dominant_gemm(cfg, layer, steps, warmup, torch, moe):
    """The SwiGLU grouped GEMM (GEMM1 of the routed experts) alone, same inputs
    and launch configuration as inside the layer, timed with events on the
    stream it is launched on."""
    r = layer.routing
    t = layer.tensors
    cap = r["sorted_token_ids"].numel()
    act = torch.empty((cap, cfg.I), dtype=torch.bfloat16, device="cuda")

    def go():
        moe.moe_grouped_gemm(t["x"], cfg.top_k, t["w13"], r["sorted_token_ids"], r["expert_ids"],
                             r["num_tokens_post_padded"], cfg.block_m, cfg.T * cfg.top_k,
                             moe.EPI_SWIGLU, act)
    for _ in range(warmup):
        go()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        go()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def gpu_topk_ids(cfg, inp, torch, moe):
    """The layer's routing as the library decides it (topk_ids, numpy): one
    call with the routing outputs requested.  Used to count the experts whose
    weights a layer reads."""
    layer, w = _layer(cfg, inp, torch, moe, routing=True)
    layer.run()
    ids = layer.routing["topk_ids"].cpu().numpy()
    del layer, w
    torch.cuda.empty_cache()
    return ids


def decode_case(name, torch, moe, W, reps=20, flush_reps=20, mxfp8=False):
    """µs per layer at decode shape, cycling L distinct copies of the weights
    from a captured graph; cross-checked by timing one layer eagerly with a
    1 GiB copy (4 x the Infinity Cache) between calls, events around the layer
    alone, so that every call starts with cold caches.  ``mxfp8``: the layer
    with MXFP8 expert weights (the touched experts converted)."""
    cfg = W.CONFIGS[name]
    inp = W.make_inputs(cfg)
    ids = gpu_topk_ids(cfg, inp, torch, moe)
    touched = int(np.unique(ids).size)
    # bytes per weight: bf16 2; MXFP8 1 plus one scale byte per 32
    per_expert = cfg.mats * cfg.H * cfg.I * (1 + 1 / 32 if mxfp8 else 2)
    wbytes = touched * per_expert
    nlayers = max(2, int(np.ceil(4 * MALL_BYTES / wbytes)))
    mx = W.make_mxfp8_weights(inp, experts=np.unique(ids).tolist()) if mxfp8 else None
    if mxfp8:
        base = {k + s: torch.from_numpy(mx[k + s]).cuda() for k in ("w13", "w2") for s in ("_q", "_s")}
    else:
        base = {k: _to_dev(inp[k], torch) for k in ("w13", "w2")}
    layers = []
    for li in range(nlayers):
        w = base if li == 0 else {k: v.clone() for k, v in base.items()}
        if mxfp8:
            p = moe.LayerParams.from_config(cfg)
            layers.append(moe.FusedLayer(p, _to_dev(inp["x"], torch), _to_dev(inp["logits"], torch),
                                         w["w13_q"], w["w2_q"],
                                         scales={"w13": w["w13_s"], "w2": w["w2_s"]}))
        else:
            layers.append(_layer(cfg, inp, torch, moe, weights=w)[0])
    for l in layers:
        l.run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for l in layers:
            l.run()
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * nlayers)
    del g
    # cross-check: cold-cache calls of one layer, the flush queued ahead of them
    fa = torch.empty(MALL_BYTES * 2 // 4, dtype=torch.float32, device="cuda")
    fb = torch.empty_like(fa)
    lay = layers[0]
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(flush_reps)]
    for a, b in evs:
        fb.copy_(fa)
        a.record()
        lay.run()
        b.record()
    torch.cuda.synchronize()
    flushed = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    us_flushed = flushed[len(flushed) // 2]
    del fa, fb
    alg_bytes = wbytes + cfg.T * cfg.H * 2 + cfg.T * cfg.H * 4 + cfg.T * cfg.E * 4
    gbs = alg_bytes / (us * 1e-6) / 1e9
    del layers, base
    torch.cuda.empty_cache()
    return {"config": name, "weights": "mxfp8" if mxfp8 else "bf16", "T": cfg.T,
            "us_per_layer": round(us, 2),
            "us_flushed_median": round(us_flushed, 2), "touched_experts": touched,
            "alg_bytes": int(alg_bytes), "GBps": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "layers_cycled": nlayers}


_ONE_THREAD = r"""
import json, sys, time
sys.path.insert(0, sys.argv[1])
from grouped_gemm_topk_amd import workloads as W
from oracle import moe_oracle as O
cfg = W.CONFIGS[sys.argv[2]]
ntok = int(sys.argv[3])
inp = W.make_inputs(cfg)
inp["x"] = inp["x"][:ntok]
inp["logits"] = inp["logits"][:ntok]
reps, t0 = 0, time.perf_counter()
while True:
    O.moe_forward_cfg(cfg, inp)
    reps += 1
    dt = time.perf_counter() - t0
    if dt >= float(sys.argv[4]) or reps >= 50:
        break
print(json.dumps({"reps": reps, "seconds": dt}))
"""


def cpu_baseline_one_thread(cfg, ntok, min_seconds=10.0):
    """The same oracle in a child process whose BLAS runs one thread (the
    thread counts are fixed before numpy loads)."""
    import subprocess
    env = dict(os.environ)
    for v in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS", "MKL_NUM_THREADS"):
        env[v] = "1"
    env["HIP_VISIBLE_DEVICES"] = ""   # the child never needs the GPU
    r = subprocess.run([sys.executable, "-c", _ONE_THREAD, ROOT, cfg.name, str(ntok),
                        str(min_seconds)], env=env, capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        return {"error": r.stderr.strip().splitlines()[-1:] if r.stderr else "failed"}
    d = json.loads(r.stdout.strip().splitlines()[-1])
    flops = cfg.flops() * ntok / cfg.T * d["reps"]
    return {"value": round(flops / d["seconds"] / 1e12, 6), "unit": "TFLOPS", "cores": 1,
            "sample": f"{d['reps']} x the first {ntok} of {cfg.T} tokens ({d['seconds']:.2f} s)"}


def cpu_baseline(cfg, inp, ntok, W, O, min_seconds=10.0):
    """The CPU oracle as it stands on the first ``ntok`` tokens of the workload,
    repeated until at least ``min_seconds`` of CPU work have been timed."""
    sub = {k: v for k, v in inp.items()}
    sub["x"] = inp["x"][:ntok]
    sub["logits"] = inp["logits"][:ntok]
    threads = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = threads
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.moe_forward_cfg(cfg, sub)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= 50:
            break
    flops = cfg.flops() * ntok / cfg.T * reps
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOPS", "cores": int(min(threads, blas)),
            "kind": "oracle",
            "sample": f"{reps} x the first {ntok} of {cfg.T} tokens of the {cfg.name} layer "
                      f"({dt:.2f} s, fp64 numpy per-expert loop incl. weight widening)"}


def layer_roofline(cfg, ms, ids):
    """The layer against its roofline: flops at the bf16 MFMA peak and the
    algorithmic bytes (every touched expert's weights once, x, logits, the fp32
    output) at the HBM peak; the larger time is the bound.  ``ids``: the
    layer's topk_ids as the library routed them."""
    touched = int(np.unique(ids).size) + cfg.n_shared
    wbytes = touched * cfg.mats * cfg.H * cfg.I * 2
    alg_bytes = wbytes + cfg.T * cfg.H * 2 + cfg.T * cfg.E * 4 + cfg.T * cfg.H * 4
    t_mfma = cfg.flops() / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    t_hbm = alg_bytes / (HBM_PEAK_GBS * 1e9)
    bound = "mfma" if t_mfma >= t_hbm else "hbm"
    t = ms * 1e-3
    return {"bound": bound, "roof_us": round(max(t_mfma, t_hbm) * 1e6, 1),
            "frac": round(max(t_mfma, t_hbm) / t, 4),
            "mfma_frac": round(t_mfma / t, 4), "hbm_frac": round(t_hbm / t, 4),
            "alg_bytes": int(alg_bytes), "touched_experts": touched}


def prefill_case(name, steps, warmup, torch, moe, W):
    """One more MFMA-path layer, timed like the headline one (events around
    back-to-back calls, inputs resident)."""
    cfg = W.CONFIGS[name]
    inp = W.make_inputs(cfg)
    layer, w = _layer(cfg, inp, torch, moe, routing=True)
    ms, _, spread = time_layer(layer, steps, warmup, torch, spread=True)
    ids = layer.routing["topk_ids"].cpu().numpy()
    res = {"config": name, "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "top_k": cfg.top_k,
           "block_m": cfg.block_m, "activation": "relu2" if cfg.activation else "swiglu",
           "ms": round(ms, 4), "TFLOPS": round(cfg.flops() / (ms * 1e-3) / 1e12, 2),
           "step_ms_spread": spread, "roofline": layer_roofline(cfg, ms, ids)}
    del layer, w
    torch.cuda.empty_cache()
    return res


CPU_CASES = ("decode_t1", "decode_t3", "decode_t8", "relu2_t1", "relu2_t16", "zipf128",
             "relu2_t2048")


def cpu_per_config(W, O, prefill_tokens=1 << 30):
    """The CPU oracle as it stands, one call per config on the whole layer
    (``prefill_tokens`` can cut the prefill layers to their first tokens; the
    weights are widened whole either way, and ms per layer is then scaled to
    the config's T)."""
    res = []
    for name in CPU_CASES:
        cfg = W.CONFIGS[name]
        inp = W.make_inputs(cfg)
        ntok = min(cfg.T, prefill_tokens)
        inp["x"] = inp["x"][:ntok]
        inp["logits"] = inp["logits"][:ntok]
        t0 = time.perf_counter()
        O.moe_forward_cfg(cfg, inp)
        dt = time.perf_counter() - t0
        ms_layer = dt * 1e3 * cfg.T / ntok
        res.append({"config": name, "ms_per_layer": round(ms_layer, 2),
                    "GFLOPS": round(cfg.flops() / (ms_layer * 1e-3) / 1e9, 3),
                    "sample": f"one call on {ntok} of {cfg.T} tokens ({dt:.2f} s)"})
        del inp
    return res


def _event_ms(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _interleaved_ms(fns, steps, warmup, torch, rounds=5):
    """Median ms per call of each function, timed in alternation over several
    rounds (the order within a run otherwise favours whichever comes later)."""
    for f in fns:
        for _ in range(warmup):
            f()
    times = [[] for _ in fns]
    for _ in range(rounds):
        for i, f in enumerate(fns):
            times[i].append(_event_ms(f, steps, 1, torch))
    return [float(np.median(t)) for t in times]


def gemm_scenarios(steps, warmup, torch, moe, W):
    """The contiguous grouped GEMM at the four shapes of the axolotl page's
    benchmark table (uniform groups): the whole call (align of the per-row
    indices + grouped GEMM), the GEMM launch alone with the persistent grid
    and with one workgroup per tile (the page's table times its persistent and
    its non-persistent kernel side by side), plus hipBLASLt (one torch.matmul
    per group on a contiguous transposed weight) as context; then
    the backward (input and weight gradients, each with its layout kernels)
    beside hipBLASLt per group.  Timed in alternation over five rounds; medians."""
    res = []
    for sc in W.GEMM_SCENARIOS.values():
        inp = W.make_gemm_inputs(sc)
        x, w = _to_dev(inp["x"], torch), _to_dev(inp["w"], torch)
        op = moe.IndexedGroupedGemm(x, w, _to_dev(inp["expert_indices"], torch), sc.block_m)
        op.run()
        gsz = sc.M // sc.G
        wt = [w[g].t().contiguous() for g in range(sc.G)]
        xs = [x[g * gsz:(g + 1) * gsz] for g in range(sc.G)]
        ref_out = torch.empty((sc.M, sc.N), dtype=torch.bfloat16, device="cuda")
        outs = [ref_out[g * gsz:(g + 1) * gsz] for g in range(sc.G)]

        def blas():
            for g in range(sc.G):
                torch.matmul(xs[g], wt[g], out=outs[g])
        per_tile = lambda: op.gemm(schedule=moe.SCHED_PER_TILE)
        ms_call, ms_gemm, ms_tile, ms_blas = _interleaved_ms([op.run, op.gemm, per_tile, blas],
                                                             steps, warmup, torch)
        # backward: dx (weight transpose + grouped GEMM) and dw (segment table,
        # gathered transposes of dy and x + segmented GEMM), each 2 M N K flops
        dy = _to_dev(W.make_gemm_inputs(sc, with_grad=True)["dy"], torch)
        dxb = torch.empty((sc.M, sc.K), dtype=torch.bfloat16, device="cuda")
        dwb = torch.empty((sc.G, sc.N, sc.K), dtype=torch.bfloat16, device="cuda")
        op.backward(dy, dxb, dwb)
        bdx = lambda: op.backward(dy, dxb, None, want_dw=False)
        bdw = lambda: op.backward(dy, None, dwb, want_dx=False)
        dys = [dy[g * gsz:(g + 1) * gsz] for g in range(sc.G)]
        dyt = [d.t().contiguous() for d in dys]
        ref_dx = torch.empty((sc.M, sc.K), dtype=torch.bfloat16, device="cuda")
        ref_dw = torch.empty((sc.G, sc.N, sc.K), dtype=torch.bfloat16, device="cuda")

        def blas_dx():
            for g in range(sc.G):
                torch.matmul(dys[g], w[g], out=ref_dx[g * gsz:(g + 1) * gsz])

        def blas_dw():
            for g in range(sc.G):
                torch.matmul(dyt[g], xs[g], out=ref_dw[g])
        ms_bdx, ms_bdw, ms_rdx, ms_rdw = _interleaved_ms([bdx, bdw, blas_dx, blas_dw], steps, warmup,
                                                         torch)
        f = sc.flops()
        res.append({"scenario": sc.name, "G": sc.G, "M": sc.M, "N": sc.N, "K": sc.K,
                    "block_m": sc.block_m, "ms": round(ms_call, 4),
                    "TFLOPS": round(f / (ms_call * 1e-3) / 1e12, 1),
                    "gemm_ms": round(ms_gemm, 4),
                    "gemm_TFLOPS": round(f / (ms_gemm * 1e-3) / 1e12, 1),
                    "mfma_frac": round(f / (ms_gemm * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                    "gemm_per_tile_ms": round(ms_tile, 4),
                    "gemm_per_tile_TFLOPS": round(f / (ms_tile * 1e-3) / 1e12, 1),
                    "hipblaslt_per_group_ms": round(ms_blas, 4),
                    "hipblaslt_per_group_TFLOPS": round(f / (ms_blas * 1e-3) / 1e12, 1),
                    "backward": {
                        "dx_ms": round(ms_bdx, 4), "dx_TFLOPS": round(f / (ms_bdx * 1e-3) / 1e12, 1),
                        "dw_ms": round(ms_bdw, 4), "dw_TFLOPS": round(f / (ms_bdw * 1e-3) / 1e12, 1),
                        "hipblaslt_per_group_dx_ms": round(ms_rdx, 4),
                        "hipblaslt_per_group_dw_ms": round(ms_rdw, 4)}})
        del op, x, w, wt, xs, outs, ref_out, dy, dxb, dwb, dys, dyt, ref_dx, ref_dw
        torch.cuda.empty_cache()
    return res


def router_cases(steps, warmup, torch, moe, W):
    """The layer from the hidden states and the router weight: the router's
    linear layer fused into gating (moe_fused_forward_router) against the
    separate pipeline (an fp32 torch.matmul for the logits, as the HF gate
    computes them, then moe_fused_forward).  Prefill: eager calls in
    alternation; decode: graph replays of one call each (weights stay in the
    caches, the same for both)."""
    res = []
    for name in ("dsv3", "decode_t1"):
        cfg = W.CONFIGS[name]
        inp = W.make_inputs(cfg)
        p = moe.LayerParams.from_config(cfg)
        x = _to_dev(inp["x"], torch)
        wr = _to_dev(W.make_router_weight(cfg), torch)
        w = {k: _to_dev(inp[k], torch) for k in ("w13", "w2", "shared_w13", "shared_w2") if k in inp}
        sh = (w.get("shared_w13"), w.get("shared_w2"))
        fused = moe.FusedLayer(p, x, None, w["w13"], w["w2"], *sh, router_w=wr)
        logits = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device="cuda")
        layer = moe.FusedLayer(p, x, logits, w["w13"], w["w2"], *sh)
        xf, wrt = x.float(), wr.float().t().contiguous()

        def separate():
            torch.matmul(xf, wrt, out=logits)
            layer.run()
        if cfg.T > 16:
            ms_f, ms_s = _interleaved_ms([fused.run, separate], steps, warmup, torch)
        else:
            ms_f, ms_s = [_graph_replay_ms(f, steps, warmup, torch) for f in (fused.run, separate)]
        res.append({"config": name, "fused_router_ms": round(ms_f, 4),
                    "separate_router_ms": round(ms_s, 4),
                    "timing": "eager, alternating" if cfg.T > 16 else "graph replays, warm caches"})
        del fused, layer, w, x, wr, xf, wrt, logits
        torch.cuda.empty_cache()
    return res


def _graph_replay_ms(fn, steps, warmup, torch):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(10):
            fn()
    ms = _event_ms(g.replay, max(1, steps // 10), max(1, warmup // 10), torch) / 10
    del g
    return ms


def achievable_peaks(torch, reps=5):
    """This GPU's achievable rates from the probe library (libmoe_probe.so,
    built beside libmoe.so): dense bf16 MFMA TFLOP/s of a loop of independent
    32x32x16 MFMAs with no memory traffic, and GB/s of a non-temporal
    streaming read of 4 GiB.  Best of ``reps`` launches each."""
    import ctypes
    from grouped_gemm_topk_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        return {"error": "libmoe_probe.so is not built"}
    L = ctypes.CDLL(B.PROBE_LIB)
    L.moe_probe_mfma_loop.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.moe_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                     ctypes.c_void_p]
    s = torch.cuda.current_stream()
    sp = ctypes.c_void_p(s.cuda_stream)

    def best(launch):
        launch()
        times = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            launch()
            e1.record(s)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3)
        return min(times)

    grid, iters = 1024, 2000   # 4 workgroups of 4 waves per CU
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")

    def mf():
        rc = L.moe_probe_mfma_loop(ctypes.c_void_p(out.data_ptr()), grid, iters, sp)
        if rc:
            raise RuntimeError(f"moe_probe_mfma_loop: hip error {rc}")
    t = best(mf)
    flops = grid * 4 * iters * L.moe_probe_mfma_flops_per_wave_iter()
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    rgrid = 1024
    rout = torch.empty(rgrid * 256, dtype=torch.int32, device="cuda")

    def rd():
        rc = L.moe_probe_hbm_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                  ctypes.c_void_p(rout.data_ptr()), rgrid, sp)
        if rc:
            raise RuntimeError(f"moe_probe_hbm_read: hip error {rc}")
    tr = best(rd)
    del buf
    torch.cuda.empty_cache()
    return {"mfma_bf16_TFLOPS": round(flops / t / 1e12, 1), "hbm_read_GBps": round(nbytes / tr / 1e9, 1),
            "how": f"best of {reps}: {grid} x 4 waves x {iters} rounds of 16 independent 32x32x16 bf16 "
                   f"MFMAs; non-temporal 16 B/lane streaming read of {nbytes >> 30} GiB"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def dominant_traffic(cfg_name):
    """Counter-derived bytes per launch, or None when the kernel source has
    changed since the counters were taken (or for another workload)."""
    import hashlib
    t = DOMINANT_TRAFFIC
    try:
        with open(os.path.join(ROOT, t["src"]), "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    if digest != t["sha256"] or cfg_name != t["config"]:
        return None
    return t["fetch_bytes"] + t["write_bytes"]


def copy_calibration(torch, nbytes=1 << 30, reps=4):
    """Copies of ``nbytes`` (read nbytes, write nbytes per launch), for turning
    the FETCH_SIZE / WRITE_SIZE counters of the same profiler into bytes: a
    device-to-device ``copy_`` and an elementwise negation (a streaming kernel
    of the same traffic that is certain to be a shader dispatch)."""
    a = torch.full((nbytes // 4,), 1.0, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    for _ in range(reps):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": nbytes, "bytes_written": nbytes,
                                           "launches": reps}}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the MoE layer runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    import torch

    from grouped_gemm_topk_amd import moe
    from grouped_gemm_topk_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    moe.lib()
    if args.router_only:
        print(json.dumps({"router_fused": router_cases(args.steps, args.warmup, torch, moe, W)}),
              flush=True)
        return
    if args.gemm_scenarios_only:
        print(json.dumps({"grouped_gemm_scenarios": gemm_scenarios(args.steps, args.warmup, torch,
                                                                   moe, W)}), flush=True)
        return
    if args.decode_only:
        print(json.dumps({"decode": [decode_case(n, torch, moe, W) for n in DECODE_CASES],
                          "decode_mxfp8": [decode_case(n, torch, moe, W, mxfp8=True)
                                           for n in DECODE_CASES]}), flush=True)
        return
    cfg = W.CONFIGS[args.config]
    inp = W.make_inputs(cfg)
    layer, _ = _layer(cfg, inp, torch, moe, routing=True)
    layer.run()
    torch.cuda.synchronize()
    print(f"# {cfg.name}: inputs resident, timing {args.steps} steps", file=sys.stderr, flush=True)
    ms, wall, spread = time_layer(layer, args.steps, args.warmup, torch, spread=True)
    flops = cfg.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    # dominant kernel: routed SwiGLU grouped GEMM
    gemm_ms = time_dominant_gemm(cfg, layer, args.steps, args.warmup, torch, moe)
    gemm_flops = 2.0 * cfg.T * cfg.top_k * cfg.H * 2 * cfg.I
    gemm_tf = gemm_flops / (gemm_ms * 1e-3) / 1e12
    # algorithmic bytes: every routed expert's W13 once, each token row once,
    # the activation rows of every (token, slot) pair written once
    gemm_alg_bytes = (cfg.E * 2 * cfg.I * cfg.H + cfg.T * cfg.H + cfg.T * cfg.top_k * cfg.I) * 2
    line = {
        "metric": "fused-MoE layer TFLOPS at T=4096 + decode us/layer (T=1..8) vs roofline",
        "value": round(tflops, 2), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} "
                               f"top_k={cfg.top_k} groups={cfg.n_group}/{cfg.topk_group} "
                               f"shared={cfg.n_shared} block_m={cfg.block_m} SwiGLU bf16",
                   "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "top_k": cfg.top_k,
                   "block_m": cfg.block_m, "flops_per_step": flops,
                   "routed_only_TFLOPS": round(cfg.flops(routed_only=True) / (ms * 1e-3) / 1e12, 2),
                   "mfma_frac_of_layer": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                   "wall_s_timed": round(wall, 3),
                   "step_ms_spread": spread},
        "roofline": {"bound": "mfma", "kernel": f"{DOMINANT_KERNEL.get(cfg.block_m, 'grouped_gemm_kernel')} (routed W13 + SwiGLU)",
                     "achieved": round(gemm_tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": dominant_traffic(cfg.name),
                     "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled)",
                     "alg_bytes_per_launch": gemm_alg_bytes,
                     "avg_launch_us": round(gemm_ms * 1e3, 2),
                     "alg_flops_per_launch": gemm_flops},
    }
    peaks = None if args.no_peaks else achievable_peaks(torch)
    if peaks and "mfma_bf16_TFLOPS" in peaks:
        line["roofline"]["achievable_peak"] = peaks["mfma_bf16_TFLOPS"]
        line["roofline"]["frac_of_achievable"] = round(gemm_tf / peaks["mfma_bf16_TFLOPS"], 4)
        line["config"]["mfma_frac_of_achievable"] = round(tflops / peaks["mfma_bf16_TFLOPS"], 4)
    if peaks:
        line["achievable_peaks"] = peaks
    if not args.no_decode:
        line["decode"] = [decode_case(n, torch, moe, W) for n in DECODE_CASES]
        line["decode_mxfp8"] = [decode_case(n, torch, moe, W, mxfp8=True) for n in DECODE_CASES]
        if peaks and "hbm_read_GBps" in peaks:
            for d in line["decode"] + line["decode_mxfp8"]:
                d["frac_of_achievable_hbm"] = round(d["GBps"] / peaks["hbm_read_GBps"], 4)
    if not args.no_gemm_scenarios:
        line["grouped_gemm_scenarios"] = gemm_scenarios(args.steps, args.warmup, torch, moe, W)
    if not args.no_router:
        line["router_fused"] = router_cases(args.steps, args.warmup, torch, moe, W)
    line["prefill"] = [dict(config=cfg.name, T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, top_k=cfg.top_k,
                            block_m=cfg.block_m, activation="swiglu", ms=round(ms, 4),
                            TFLOPS=round(tflops, 2), step_ms_spread=spread,
                            roofline=layer_roofline(cfg, ms,
                                                    layer.routing["topk_ids"].cpu().numpy()))]
    if not args.no_prefill:
        for name in PREFILL_CASES:
            print(f"# {name}: timing", file=sys.stderr, flush=True)
            line["prefill"].append(prefill_case(name, args.steps, args.warmup, torch, moe, W))
    extra = [e for e in args.extra.split(",") if e]
    if extra:
        line["extra"] = {}
        for name in extra:
            c2 = W.CONFIGS[name]
            i2 = W.make_inputs(c2)
            l2, _ = _layer(c2, i2, torch, moe)
            ms2, _, _ = time_layer(l2, args.steps, args.warmup, torch)
            line["extra"][name] = {"ms": round(ms2, 4),
                                   "TFLOPS": round(c2.flops() / (ms2 * 1e-3) / 1e12, 2)}
            del l2
            torch.cuda.empty_cache()
    if not args.no_cpu:
        # the CPU leg: the oracle, timed as a reported baseline
        from oracle import moe_oracle as O
        line["cpu_baseline"] = cpu_baseline(cfg, inp, min(args.cpu_tokens, cfg.T), W, O)
        line["cpu_baseline"]["single_thread"] = cpu_baseline_one_thread(cfg, min(512, cfg.T))
        line["cpu_baseline"]["cpu_model"] = cpu_model()
        print("# CPU oracle per config", file=sys.stderr, flush=True)
        line["cpu_baseline"]["per_config"] = cpu_per_config(W, O)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
