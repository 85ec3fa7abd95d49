#!/usr/bin/env python3
"""Benchmark of the fused mixed-precision MoE expert layer on one MI355X.

One step = one pw_moe_forward call (route, gate_up + SwiGLU, down, combine) on
seeded synthetic inputs resident in HBM.  The reported line is the
Mixtral-8x7B-shaped decode layer at T = 64 tokens (H=4096, I=14336, E=8,
top-2, per-block committed bitwidths uniform in 3..8: the largest layer with
mixed 3-8-bit experts); every other layer shape of the study -- tiny, the
Qwen1.5-MoE-A2.7B-shaped decode (T=4) and batched (T=256, Zipf) layers,
Mixtral decode at T = 1 and 8, Mixtral prefill (T=4096) -- gets its own timed
region under `per_config`.  The routed experts' storage is kept in R copies at
different addresses (R x the bytes a call reads >= 1 GB) and the steps rotate
through them, so weights come from HBM and not from the 256 MB last-level cache.

Roofline of each call's dominant kernel: its algorithmic bytes (or flops) per
launch over its average duration, taken from start / stop events that the
library hands to the kernel launch itself (the kernel's own execution).

Prints one JSON line.  --only NAME runs one configuration (for profiling).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + achieved HBM GB/s (% peak) at mixed 3–8-bit experts"

# (name, workload, T) of every configuration; the first field names the
# profile summaries under profiles/ as well.
CONFIGS = [
    ("tiny", "tiny", None),
    ("qwen_decode", "qwen_decode", None),
    ("qwen_batched", "qwen_batched", None),
    ("mixtral_decode_T1", "mixtral_decode", 1),
    ("mixtral_decode_T8", "mixtral_decode", 8),
    ("mixtral_decode_T64", "mixtral_decode", 64),
    ("mixtral_prefill", "mixtral_prefill", None),
]
HEADLINE = "mixtral_decode_T64"

KERNEL_NAMES = {("gemv", 0): "gemv_kernel<true>", ("gemv", 1): "gemv_kernel<false>",
                ("mgemv", 0): "mgemv_kernel<true>", ("mgemv", 1): "mgemv_kernel<false>",
                ("mfma", 0): "mfma_kernel<true>", ("mfma", 1): "mfma_kernel<false>"}


class HipEvents:
    """Raw hipEvent_t handles (the library records them on its own stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
        return ev.value

    def destroy(self, ev) -> None:
        self.hip.hipEventDestroy(ctypes.c_void_p(ev))

    def record(self, ev, stream) -> None:
        assert self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) == 0

    def elapsed_ms(self, a, b) -> float:
        out = ctypes.c_float()
        assert self.hip.hipEventSynchronize(ctypes.c_void_p(b)) == 0
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return float(out.value)


def source_hash() -> str:
    """sha256[:16] over the library's kernel and host sources (a profile summary
    taken on other sources no longer describes these kernels)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "any_precision_bitplane_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def profile_fields(name: str, kind: str, kernel: str):
    """Fields of `kernel` in profiles/<kind>_<name>.txt if that summary was taken
    on the current sources, else None.  kind: "kernels" (rocprofv3 kernel-trace
    stats: avg_ns) or "traffic" (FETCH_SIZE / WRITE_SIZE: traffic_bytes_per_launch)."""
    path = os.path.join(ROOT, "profiles", f"{kind}_{name}.txt")
    if not os.path.exists(path):
        return None
    fields, sha = {}, None
    for line in open(path):
        if line.startswith("source_sha256_16:"):
            sha = line.split(":", 1)[1].strip()
        elif line.startswith(kernel + ":"):
            for tok in line.split()[1:]:
                k, v = tok.split("=")
                fields[k] = float(v)
    if sha != source_hash() or not fields:
        return None
    return fields


def cpu_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    return model, int(threads), os.cpu_count()


def cpu_baseline(layer, budget_s: float):
    """The oracle as it stands, on the host cores, over a bounded sample of the
    same workload: whole experts (every slot routed to the expert, its two
    blocks dequantized and its FFN run), in ascending expert id until the
    budget is spent; the layer's time is the mean per-expert time times the
    number of routed experts."""
    import oracle.pagedweight_oracle as orc
    model, threads, ncpu = cpu_info()
    routed = [int(e) for e in layer.active_experts()]
    done, spent = [], 0.0
    for e in routed:
        ids_e = np.where(layer.ids == e, layer.ids, -1).astype(np.int32)
        t0 = time.perf_counter()
        orc.moe_forward_layer(layer, ids=ids_e)
        spent += time.perf_counter() - t0
        done.append(e)
        if spent >= budget_s:
            break
    layer_s = spent / len(done) * len(routed)
    T = layer.wl.T
    return {"value": T / layer_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"experts {done} of the {len(routed)} routed (all their slots), {spent:.1f} s of fp64 numpy; "
                      f"layer time = mean per expert x {len(routed)}",
            "os_cpu_count": ncpu, "blas_threads": threads, "cpu_model": model}


def timed_ms(evs, stream, fn, n: int) -> float:
    """Average ms per call of fn() over n calls, from HIP events on `stream`."""
    a, b = evs.create(), evs.create()
    evs.record(a, stream.cuda_stream)
    for i in range(n):
        fn(i)
    evs.record(b, stream.cuda_stream)
    return evs.elapsed_ms(a, b) / n


def next_rows(layer, dev, copies, opts, stream, evs, steps: int):
    """Secondary measurements of the parts around the fused layer, on the same
    layer: the router (and the routed layer call), a captured HIP graph of
    consecutive layer calls, and the pager's asynchronous plane reload."""
    import torch
    from any_precision_bitplane_amd import binding as B
    from any_precision_bitplane_amd import synth
    from any_precision_bitplane_amd.device import PagedLayer
    wl = layer.wl
    out = {}
    # router: logits + top-k + statistics, and router + layer in one call
    wr = torch.from_numpy(synth.draw_router_weights(wl.seed, wl.E, wl.H)).to(dev.device)
    ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device=dev.device)
    w = torch.empty((wl.T, wl.k), dtype=torch.float32, device=dev.device)
    cnt = torch.zeros(wl.E, dtype=torch.int32, device=dev.device)
    mass = torch.zeros(wl.E, dtype=torch.float32, device=dev.device)
    y2 = torch.empty_like(dev.y)
    route = lambda i: B.pw_router_topk(dev.shape, wl.T, dev.x, wr, ids, w, cnt, mass, dev.ws, stream=stream)
    routed = lambda i: B.pw_moe_forward_routed(dev.shape, wl.T, dev.x, wr, dev.blocks[i % copies], dev.q, y2, cnt,
                                               mass, dev.ws, opts=opts, stream=stream)
    for i in range(10):
        routed(i)
    torch.cuda.synchronize()
    out["router_us"] = 1e3 * timed_ms(evs, stream, route, steps)
    out["routed_layer_us"] = 1e3 * timed_ms(evs, stream, routed, steps)
    # the layer alone on the router's own routing (which routes other experts
    # than the synthetic ids the plain layer call uses), for a like-for-like
    # cost of the router inside the routed call
    route(0)
    same = lambda i: B.pw_moe_forward(dev.shape, wl.T, dev.x, ids, w, dev.blocks[i % copies], dev.q, y2, dev.ws,
                                      opts=opts, stream=stream)
    out["layer_on_router_ids_us"] = 1e3 * timed_ms(evs, stream, same, steps)
    torch.cuda.synchronize()
    # HIP graph of G consecutive layer calls (rotating storage copies), replayed
    G = 16
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for i in range(G):
            dev.forward(opts, copy=i % copies)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(G):
            dev.forward(opts, copy=i % copies)
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // G)
    out["graph_layer_us"] = 1e3 * timed_ms(evs, stream, lambda i: g.replay(), reps) / G
    out["eager_layer_us"] = 1e3 * timed_ms(evs, stream, lambda i: dev.forward(opts, copy=i % copies, stream=stream),
                                           steps)
    del g
    torch.cuda.synchronize()
    # pager: all blocks lowered to 3 bits, then the layer's bitwidths reloaded
    # from pinned host memory on a copy stream while layer calls run
    full = sum(8 * (2 * wl.I * wl.H if b % 2 == 0 else wl.H * wl.I) // 8 for b in range(2 * wl.E))
    paged = PagedLayer(layer, 2 * full + (1 << 20), device=dev.device)
    copy = torch.cuda.Stream()
    paged.request(layer.q)
    paged.execute(copy)
    paged.commit(stream, wait=True)
    paged.request(np.full(layer.q.shape, 3, np.uint8))
    paged.execute(copy)
    paged.commit(stream, wait=True)
    torch.cuda.synchronize()
    pfwd = lambda i: paged.forward(opts, stream=stream)
    for i in range(5):
        pfwd(i)
    torch.cuda.synchronize()
    alone_us = 1e3 * timed_ms(evs, stream, pfwd, steps)
    torch.cuda.synchronize()
    paged.request(layer.q)
    a, b = evs.create(), evs.create()
    evs.record(a, copy.cuda_stream)
    paged.execute(copy)
    evs.record(b, copy.cuda_stream)
    c, d = evs.create(), evs.create()
    evs.record(c, stream.cuda_stream)
    n_during = 0
    while True:   # layer calls enqueued while the copies are in flight
        pfwd(n_during)
        n_during += 1
        if n_during >= 20 and (B.pw_pager_info(paged.pager, 0).state != B.PW_PAGE_IN_TRANSFER or n_during >= 400):
            break
    evs.record(d, stream.cuda_stream)
    reload_ms = evs.elapsed_ms(a, b)
    during_us = 1e3 * evs.elapsed_ms(c, d) / n_during
    paged.commit(stream, wait=True)
    torch.cuda.synchronize()
    pb = [(2 * wl.I * wl.H if b % 2 == 0 else wl.H * wl.I) // 8 for b in range(2 * wl.E)]
    moved = sum((int(layer.q.reshape(-1)[b]) - 3) * pb[b] for b in range(2 * wl.E))
    out["pager"] = {"reload_bytes": moved, "reload_ms": reload_ms, "reload_h2d_gbs": moved / (reload_ms * 1e-3) / 1e9,
                    "layer_us_alone_q3": alone_us, "layer_us_during_reload": during_us,
                    "layer_calls_during_reload": n_during}
    paged.close()
    out["layers"] = multi_layer_rows(layer, opts, stream, evs, steps)
    # planner: host time for 24 layers of this shape
    nb = 24 * 2 * wl.E
    sens = synth.draw_sensitivity(wl.seed, nb)
    pbs = np.array(pb * 24, np.int64)
    t0 = time.perf_counter()
    _, plan, used, fits = B.pw_plan_bitwidths(np.full(nb, 8), pbs, np.arange(nb) // 2, sens,
                                              routing_mass=np.tile(mass.cpu().numpy(), 24), hot_fraction=0.2,
                                              floor_hot=6, hot_multiplier=2.0,
                                              budget_bytes=int(0.5 * (8 * pbs).sum()))
    out["planner_ms_24_layers"] = 1e3 * (time.perf_counter() - t0)
    return out


def build_layers(name, workload, T, cache):
    """The synthetic layer of one configuration.  The Mixtral decode layers at
    T = 1, 8 and 64 share one storage draw (same seed; their tokens and routing
    are prefixes of the same streams)."""
    from any_precision_bitplane_amd import synth
    wl = synth.WORKLOADS[workload]
    if T is not None:
        wl = wl.with_T(T)
    if workload == "mixtral_decode":
        if "mixtral_decode_full" not in cache:
            cache["mixtral_decode_full"] = synth.make_layer(synth.WORKLOADS[workload].with_T(64))
        full = cache["mixtral_decode_full"]
        ids, w = synth.draw_router(wl)
        return synth.Layer(wl, full.planes, full.luts, synth.draw_q(wl, ids, w), synth.draw_x(wl.seed, wl.T, wl.H),
                           ids, w)
    return synth.make_routed_layer(wl)


def measure(name, layer, dev, copies, args, evs, stream, opts_kw):
    """Timed region, repeats, and kernel-event pass of one configuration."""
    import torch
    from any_precision_bitplane_amd import binding as B
    from any_precision_bitplane_amd import roofline as RL
    wl = layer.wl
    H, I, E, k, T = wl.H, wl.I, wl.E, wl.k, wl.T
    routed = [int(e) for e in layer.active_experts()]
    opts = B.make_options(**opts_kw)
    info = B.pw_moe_path_info(dev.shape, T, opts)
    family = [f for f in ("gemv", "mgemv", "mfma") if getattr(info, f)]
    lbytes = RL.layer_bytes(layer.q, layer.ids, H, I, E, T, k)
    flops = RL.layer_flops(T, k, H, I)

    for i in range(args.warmup):
        dev.forward(opts, copy=i % copies, stream=stream)
    torch.cuda.synchronize()

    # Timed region: exactly K layer calls, bracketed by synchronizations, with a
    # pair of HIP events on the stream around the loop.
    ev_a, ev_b = evs.create(), evs.create()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs.record(ev_a, stream.cuda_stream)
    for i in range(args.steps):
        dev.forward(opts, copy=i % copies, stream=stream)
    evs.record(ev_b, stream.cuda_stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_step_ms = evs.elapsed_ms(ev_a, ev_b) / args.steps
    ms_per_step = wall * 1e3 / args.steps

    reps = []
    for _ in range(5):
        ra, rb = evs.create(), evs.create()
        torch.cuda.synchronize()
        evs.record(ra, stream.cuda_stream)
        for i in range(args.steps):
            dev.forward(opts, copy=i % copies, stream=stream)
        evs.record(rb, stream.cuda_stream)
        torch.cuda.synchronize()
        reps.append(evs.elapsed_ms(ra, rb) / args.steps)
        evs.destroy(ra)
        evs.destroy(rb)

    # Kernel pass: the same K calls with the product kernels' own start / stop
    # events (gate_up: events 0/1, down: 2/3).
    kev = [[evs.create() for _ in range(4)] for _ in range(args.steps)]
    kopts = [B.make_options(events=kev[i], event_mode=B.PW_EVENTS_KERNELS, **opts_kw) for i in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        dev.forward(kopts[i], copy=i % copies, stream=stream)
    torch.cuda.synchronize()
    kern = np.array([[evs.elapsed_ms(kev[i][0], kev[i][1]), evs.elapsed_ms(kev[i][2], kev[i][3])]
                     for i in range(args.steps)])
    for row in kev:
        for e in row:
            evs.destroy(e)
    # Stage pass: events between the kernels on the stream (kernel plus launch gap).
    sev = [[evs.create() for _ in range(B.PW_NUM_STAGES + 1)] for _ in range(args.steps)]
    sopts = [B.make_options(events=sev[i], **opts_kw) for i in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        dev.forward(sopts[i], copy=i % copies, stream=stream)
    torch.cuda.synchronize()
    stage = np.array([[evs.elapsed_ms(sev[i][s], sev[i][s + 1]) for s in range(B.PW_NUM_STAGES)]
                      for i in range(args.steps)]).mean(axis=0)
    for row in sev:
        for e in row:
            evs.destroy(e)
    evs.destroy(ev_a)
    evs.destroy(ev_b)

    kms = kern.mean(axis=0)
    m = 0 if kms[0] >= kms[1] else 1
    # the product's kernels, one per family that runs (the start / stop events
    # bracket all of them: e.g. prefill's MFMA tiles and its tails on the
    # matrix-core GEMV)
    knames = [KERNEL_NAMES[(f, m)] for f in (family or ["gemv"])]
    kname = " + ".join(knames)
    dom_bytes = RL.module_bytes(layer.q, layer.ids, H, I, E, T, k, m)
    dom_flops = RL.module_flops(T, k, H, I, m)
    bound = RL.bound(dom_flops, dom_bytes)

    def rate(ms):
        if bound == "mfma":
            return dom_flops / (ms * 1e-3) / 1e12
        return dom_bytes / (ms * 1e-3) / 1e9
    peak = RL.MFMA_FP16_PEAK_TFLOPS if bound == "mfma" else RL.HBM_PEAK_GBS
    achieved = rate(float(kms[m]))
    span_ms = float(stage[1 + m])
    roof = {
        "kernel": f"{kname} ({['gate_up', 'down'][m]})",
        "bound": bound,
        "achieved": achieved,
        "peak": peak,
        "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
        "frac": achieved / peak,
        "traffic": None,
        "algorithmic_bytes_per_launch": dom_bytes,
        "algorithmic_flops_per_launch": dom_flops,
        "avg_kernel_ms": float(kms[m]),
        "timing": "kernel start/stop events handed to the launch (hipExtLaunchKernelGGL), mean of K launches",
        "event_span": {"avg_ms": span_ms, "frac": rate(span_ms) / peak,
                       "what": "events on the stream before and after the product (includes the launch gap)"},
    }
    tr = [profile_fields(name, "traffic", kn) for kn in knames]
    if all(t is not None for t in tr):
        roof["traffic"] = sum(t["traffic_bytes_per_launch"] for t in tr)
    kt = [profile_fields(name, "kernels", kn) for kn in knames]
    if all(t is not None for t in kt):
        kt_ms = sum(t["avg_ns"] for t in kt) * 1e-6
        roof["kernel_trace"] = {"avg_ms": kt_ms, "frac": rate(kt_ms) / peak,
                                "profile": f"profiles/kernels_{name}.txt"}

    status = dev.status()
    y = dev.y.float().cpu().numpy()
    ok = bool(np.all(np.isfinite(y))) and status == 0
    return {
        "workload": name,
        "description": wl.description or wl.name,
        "H": H, "I": I, "E": E, "top_k": k, "T": T,
        "routed_experts": len(routed),
        "mean_q_routed": float(np.mean([layer.q[e] for e in routed])),
        "kernel_family": family,
        "storage_copies_rotated": copies,
        "ms_per_step": ms_per_step,
        "tokens_per_s": T / (ms_per_step * 1e-3),
        "gpu_ms_per_step": gpu_step_ms,
        "repeats_gpu_ms_per_step": reps,
        "median_gpu_ms_per_step": float(np.median(reps)),
        "algorithmic_bytes": lbytes,
        "algorithmic_flops": flops,
        "hbm_gbs": lbytes / (ms_per_step * 1e-3) / 1e9,
        "hbm_frac": lbytes / (ms_per_step * 1e-3) / 1e9 / RL.HBM_PEAK_GBS,
        "tflops": flops / (ms_per_step * 1e-3) / 1e12,
        "mfma_frac": flops / (ms_per_step * 1e-3) / 1e12 / RL.MFMA_FP16_PEAK_TFLOPS,
        "kernel_ms": {"gate_up": float(kms[0]), "down": float(kms[1])},
        "stage_ms": {"route": float(stage[0]), "gate_up": float(stage[1]), "down": float(stage[2]),
                     "combine": float(stage[3])},
        "roofline": roof,
        "output_finite_and_status_clear": ok,
    }


def multi_layer_rows(layer, opts, stream, evs, steps: int, nlayers: int = 8):
    """Decode step through `nlayers` layers of this shape, each with its own
    device storage (copies of one full draw) and its own router, chained in
    one pw_moe_forward_layers call: per-layer time eager and as a replayed HIP
    graph, against one routed layer call and one unrouted layer call."""
    import torch
    from any_precision_bitplane_amd import binding as B
    from any_precision_bitplane_amd import synth
    from any_precision_bitplane_amd.device import DeviceLayer
    wl = layer.wl
    full = synth.make_layer(wl)
    devs = [DeviceLayer(full) for _ in range(nlayers)]
    wrs = [torch.from_numpy(synth.draw_router_weights(wl.seed + 17 * l, wl.E, wl.H)).cuda() for l in range(nlayers)]
    shp = devs[0].shape
    ws = torch.empty(B.pw_workspace_bytes(shp, wl.T), dtype=torch.uint8, device="cuda")
    B.pw_workspace_init(ws)
    x0 = devs[0].x
    y = torch.empty((wl.T, wl.H), dtype=torch.float16, device="cuda")
    blocks = [d.blocks[0] for d in devs]
    qs = [d.q for d in devs]
    # A chain of SwiGLU layers without a residual path is quadratic in the
    # activation scale; each layer's down tables are scaled so that its output
    # on its actual input has unit RMS, so every layer routes O(1) inputs (with
    # vanishing inputs every token would pick the same experts).
    x = x0
    for l in range(nlayers):
        B.pw_moe_forward_routed(shp, wl.T, x, wrs[l], blocks[l], qs[l], y, None, None, ws)
        torch.cuda.synchronize()
        rms = float(y.float().pow(2).mean().sqrt())
        for e in range(wl.E):
            devs[l].luts[0][e][1].view(torch.float16).mul_(1.0 / max(rms, 1e-6))
        x_next = torch.empty_like(y)
        B.pw_moe_forward_routed(shp, wl.T, x, wrs[l], blocks[l], qs[l], x_next, None, None, ws)
        x = x_next
    torch.cuda.synchronize()
    call = lambda i: B.pw_moe_forward_layers(shp, wl.T, x0, wrs, blocks, qs, y, None, None, ws, opts=opts,
                                             stream=stream)
    routed = lambda i: B.pw_moe_forward_routed(shp, wl.T, x0, wrs[i % nlayers], blocks[i % nlayers], qs[i % nlayers],
                                               y, None, None, ws, opts=opts, stream=stream)
    plain = lambda i: devs[i % nlayers].forward(opts, stream=stream)
    for i in range(5):
        call(i)
        routed(i)
        plain(i)
    torch.cuda.synchronize()
    n = max(4, steps // 4)
    res = {"layers": nlayers,
           "eager_us_per_layer": 1e3 * timed_ms(evs, stream, call, n) / nlayers,
           "routed_single_layer_us": 1e3 * timed_ms(evs, stream, routed, steps),
           "unrouted_single_layer_us": 1e3 * timed_ms(evs, stream, plain, steps)}
    # each layer alone on the ids its router gives for its input in the chain
    xin, ids, w = x0, [], []
    for l in range(nlayers):
        i_l = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
        w_l = torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda")
        B.pw_router_topk(shp, wl.T, xin, wrs[l], i_l, w_l, None, None, ws)
        x_next = torch.empty_like(y)
        B.pw_moe_forward(shp, wl.T, xin, i_l, w_l, blocks[l], qs[l], x_next, ws)
        ids.append(i_l)
        w.append(w_l)
        xin = x_next
    torch.cuda.synchronize()
    same = lambda i: B.pw_moe_forward(shp, wl.T, x0, ids[i % nlayers], w[i % nlayers], blocks[i % nlayers],
                                      qs[i % nlayers], y, ws, opts=opts, stream=stream)
    res["layers_alone_on_their_routing_us"] = 1e3 * timed_ms(evs, stream, same, steps)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        B.pw_moe_forward_layers(shp, wl.T, x0, wrs, blocks, qs, y, None, None, ws, opts=opts)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        B.pw_moe_forward_layers(shp, wl.T, x0, wrs, blocks, qs, y, None, None, ws, opts=opts)
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    res["graph_us_per_layer"] = 1e3 * timed_ms(evs, stream, lambda i: g.replay(), n) / nlayers
    del g
    torch.cuda.synchronize()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--only", default=None, choices=[c[0] for c in CONFIGS],
                    help="run one configuration and report it as the line")
    ap.add_argument("--copies", type=int, default=0, help="storage copies to rotate (0: auto, >= 1 GB)")
    ap.add_argument("--path", type=int, default=0, help="0 auto, 1 GEMV, 2 MFMA, 3 matrix-core GEMV")
    ap.add_argument("--mfma-min", type=int, default=0, help="AUTO: MFMA from this many tokens (0: library default)")
    ap.add_argument("--mgemv-min", type=int, default=0,
                    help="AUTO: matrix-core GEMV from this many tokens (0: library default)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes (counter calibration)")
    ap.add_argument("--no-extras", action="store_true", help="skip the router / graph / pager measurements")
    ap.add_argument("--uniform-q", type=int, default=0,
                    help="commit one bitwidth for every block (mixed-vs-uniform comparison)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the layer's multi-GPU sharding is "
              f"designed (expert parallelism over RCCL) but not built.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_bytes:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(max(args.steps, 1)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "copies": max(args.steps, 1)}))
        return
    from any_precision_bitplane_amd import binding as B
    from any_precision_bitplane_amd import roofline as RL
    from any_precision_bitplane_amd.device import DeviceLayer

    B.load()
    evs = HipEvents()
    stream = torch.cuda.current_stream()
    opts_kw = dict(path=args.path, mfma_min_tokens=args.mfma_min, mgemv_min_tokens=args.mgemv_min)
    headline = args.only or HEADLINE
    run = [c for c in CONFIGS if args.only is None or c[0] == args.only]

    results, extras, base_layer = {}, None, None
    cache = {}
    dev = None
    for name, workload, T in run:
        print(f"[bench] {name}: building", file=sys.stderr, flush=True)
        layer = build_layers(name, workload, T, cache)
        if args.uniform_q:
            layer.q[:] = args.uniform_q
        lbytes = RL.layer_bytes(layer.q, layer.ids, layer.wl.H, layer.wl.I, layer.wl.E, layer.wl.T, layer.wl.k)
        copies = args.copies or max(2, int(np.ceil(1.0e9 / max(lbytes, 1))))
        copies = min(copies, 64)
        if workload == "mixtral_decode" and dev is not None and getattr(dev, "_shared", None) == "mixtral_decode":
            dev.set_tokens(layer)
            dev.set_q(layer.q)
            copies = dev.copies
        else:
            dev = None
            torch.cuda.empty_cache()
            routed = [int(e) for e in layer.active_experts()]
            if workload == "mixtral_decode":
                routed = list(range(layer.wl.E))   # one device copy serves T = 1, 8, 64
            dev = DeviceLayer(layer, copies=copies, experts=routed)
            dev._shared = workload
            dev.copies = copies
        print(f"[bench] {name}: timing ({copies} storage copies)", file=sys.stderr, flush=True)
        results[name] = measure(name, layer, dev, copies, args, evs, stream, opts_kw)
        if name == headline:
            base_layer = layer
        if name == "qwen_decode" and not args.no_extras and not args.uniform_q:
            print("[bench] qwen_decode: around the layer", file=sys.stderr, flush=True)
            extras = next_rows(layer, dev, copies, B.make_options(**opts_kw), stream, evs, args.steps)
        if workload != "mixtral_decode":
            dev = None
    dev = None
    torch.cuda.empty_cache()

    head = results[headline]
    rec = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": head["description"],
            "H": head["H"], "I": head["I"], "E": head["E"], "top_k": head["top_k"], "T": head["T"],
            "routed_experts": head["routed_experts"],
            "mean_q_routed": head["mean_q_routed"],
            "storage_copies_rotated": head["storage_copies_rotated"],
            "path": ["auto", "gemv", "mfma", "mgemv"][args.path],
            "kernel_family": head["kernel_family"],
            "bitwidths": f"uniform {args.uniform_q}" if args.uniform_q else "per block, uniform in 3..8",
        },
        "hbm_gbs": head["hbm_gbs"],
        "hbm_frac_of_peak": head["hbm_frac"],
        "roofline": head["roofline"],
        "layer": {k: v for k, v in head.items() if k != "roofline"},
        "per_config": [results[c[0]] for c in run if c[0] != headline],
    }
    if extras is not None:
        rec["around_the_layer"] = extras
    if not args.no_cpu and base_layer is not None:
        print("[bench] oracle on the host cores", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(base_layer, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
