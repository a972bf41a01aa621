"""Benchmark of the latent MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1..4]

A step is one moe_latent_forward over one batch of synthetic tokens (router,
top-K, permutation, pooler, expert gate/up + SwiGLU, expert down, post-expert
norm + weighted sum, unpooler). Main workload: the real-shape layer
(H 8192, L 4096, 256 experts top-8, SwiGLU I 4096, MXFP4 experts) at decode
T = 1; without --config the verify (T = 32), skewed (T = 512) and prefill
(T = 4096) workloads follow, each with its own tokens/s and roofline under
"workloads". Inputs are resident in HBM before the timed region. To keep
the 256 MB last-level cache from serving the weight stream, steps rotate
over token sets (different experts) and 4 copies of the dense weights.

Prints one JSON line with layer tokens/s (K steps timed by the host clock,
no events in the stream), the roofline of the dominant kernel (timed over K
further steps with HIP events that its own launch records, on the library's
stream), the measured copy/read/MFMA ceilings of this GPU, and the CPU
oracle baseline (all host threads up to 16, and one thread).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps of the main workload (default 400 at T=1, 100 at T=32, "
                         "40 at T=512, 20 at T=4096)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=None,
                    help="workload id 1..4 (see synth.CONFIGS); default: decode T=1 as the main "
                         "line plus the other three workloads under 'workloads'")
    ap.add_argument("--only-main", action="store_true", help="time only the main workload")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured copy/MFMA ceilings")
    ap.add_argument("--token-sets", type=int, default=None)
    ap.add_argument("--weight-copies", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--format", choices=("mxfp4", "nvfp4"), default="mxfp4",
                    help="expert weight format (nvfp4: E4M3 scales per 16 and per-tensor scales)")
    ap.add_argument("--expert-split-rows", type=int, default=0,
                    help="moe_dims.expert_split_rows: the expert projections' two loops in the "
                         "row-tile regime (-1: one loop; 1..16: experts with at most that many "
                         "routes on the streaming kernels; 0: the library's choice)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the routing-replay and block timings (profiling runs: one kernel mix)")
    ap.add_argument("--cpu-tokens", type=int, default=320, help="tokens in the oracle sample (about 10 s of host work)")
    ap.add_argument("--cpu-tokens-1t", type=int, default=16,
                    help="tokens in the one-thread oracle sample (about 10 s of host work)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain copy of this size, 3 times (the HBM counter calibration: "
                         "the peaks library's copy_kernel reads and writes this many bytes)")
    return ap.parse_args()


def stage_bytes(dims: dict, T: int, U: int, sblock: int = 32) -> dict:
    """Algorithmic HBM bytes of each step for T tokens touching U experts
    (sblock: elements per scale byte, 32 for MXFP4, 16 for NVFP4)."""
    H, L, I, E, K = (dims[k] for k in ("hidden", "latent", "inter", "n_experts", "top_k"))
    R = T * K
    w13 = 2 * I * (L // 2) + 2 * I * (L // sblock)
    w2 = L * (I // 2) + L * (I // sblock)
    return dict(
        router=E * H * 4 + T * H * 2 + T * E * 4,
        topk=T * E * 4 + R * 8,
        permute=R * 4 * 2 + (E + 1) * 4,
        pool=L * H * 2 + T * H * 2 + T * L * 2,
        gateup=U * w13 + T * L * 2 + R * I * 2,
        down=U * w2 + R * I * 2 + R * L * 4,
        combine=R * L * 4 + R * 8 + T * L * 2 + L * 2,
        unpool=H * L * 2 + T * L * 2 + T * H * 2,
    )


def layer_bytes(dims: dict, T: int, U: int, sblock: int = 32) -> int:
    H, L, I, E = (dims[k] for k in ("hidden", "latent", "inter", "n_experts"))
    expert = 2 * I * (L // 2) + 2 * I * (L // sblock) + L * (I // 2) + L * (I // sblock)
    return E * H * 4 + L * H * 2 + H * L * 2 + U * expert + T * H * 2 * 2


def stage_flops(dims: dict, T: int) -> dict:
    H, L, I, E, K = (dims[k] for k in ("hidden", "latent", "inter", "n_experts", "top_k"))
    R = T * K
    return dict(router=2 * T * H * E, pool=2 * T * H * L, gateup=2 * R * L * 2 * I,
                down=2 * R * I * L, unpool=2 * T * L * H)


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()  # over the comma-separated source files, in order
    for name in rec["source"].split(","):
        h.update(open(os.path.join(ROOT, "latent_mixture_experts_amd", "csrc", name), "rb").read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    return rec["hbm_bytes_per_launch"]


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(lay, dev, n_tokens: int, n_tokens_1t: int, cfg_id: int):
    """The oracle as it stands, on the host cores, over a bounded sample of
    the same workload: single-token layer passes (tokens drawn like the
    benchmark's, from a token set of their own), one per thread, on all the
    host threads the box grants (at most 16), and again on one thread. Expert
    bytes are copied to the host first and the copy is not timed."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    from latent_mixture_experts_amd import synth

    xs = synth.token_batch(cfg_id, n_tokens, token_set=1000)
    logits = oracle.router_logits(xs, lay.router)
    ids, _ = oracle.topk(logits, lay.dims["top_k"])
    cache = {int(e): tuple(dev[k][int(e)].cpu().numpy() for k in synth.EXPERT_TENSORS)
             for e in np.unique(ids)}
    nproc = os.cpu_count() or 1
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = nproc
    cores = min(len(xs), avail, 16)
    fn = lambda t: oracle.token_forward(lay.dims, xs[t], lay.router, lay.pooler, lay.gain,
                                        lay.unpooler, lay.eps, lay.gain_per_expert, cache.__getitem__)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(cores) as ex:
        list(ex.map(fn, range(len(xs))))
    dt = time.perf_counter() - t0
    n1 = min(n_tokens_1t, len(xs))
    t1 = time.perf_counter()
    for t in range(n1):
        fn(t)
    dt1 = time.perf_counter() - t1
    return {"value": round(len(xs) / dt, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "one_thread": {"value": round(n1 / dt1, 3), "unit": "tokens/s", "cores": 1,
                           "sample": f"{n1} single-token layer passes, {dt1:.1f} s"},
            "host": {"nproc": nproc, "threads_available": avail, "cpu_model": _cpu_model()},
            "sample": f"{len(xs)} single-token layer passes (real shape, one thread each), "
                      f"{dt:.1f} s wall on {cores} host threads; input generation and "
                      "expert-byte copies excluded"}


def _peaks_lib():
    import ctypes

    lib = ctypes.CDLL(os.path.join(ROOT, "latent_mixture_experts_amd", "libmoe_peaks.so"))
    lib.moe_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                  ctypes.c_void_p]
    lib.moe_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_void_p]
    lib.moe_peak_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.moe_peak_mfma_bf16_flops.restype = ctypes.c_double
    lib.moe_peak_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    return lib


def copy_probe(dev_name: str, mib: int):
    """A plain copy of `mib` MiB, three launches (the kernel that the HBM
    counter runs calibrate against: it reads and writes that many bytes)."""
    import ctypes

    import torch

    lib = _peaks_lib()
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev_name).fill_(1)
    dst = torch.empty_like(src)
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(3):
        if lib.moe_peak_copy(src.data_ptr(), dst.data_ptr(), n, 4096, sp) != 0:
            raise RuntimeError("copy probe launch failed")
    torch.cuda.synchronize()


def measured_peaks(dev_name: str):
    """The ceilings one kernel reaches on this GPU (libmoe_peaks.so): a copy
    and a read of 2 GiB buffers (HBM bytes / time), and bf16 MFMA 16x16x32
    issued from registers by 2048 workgroups of 4 wavefronts. Best of 5."""
    import ctypes

    import torch

    lib = _peaks_lib()
    st = torch.cuda.current_stream()
    sp = ctypes.c_void_p(st.cuda_stream)
    n = 2 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev_name).fill_(3)
    b = torch.empty_like(a)
    sink = torch.empty(1 << 16, dtype=torch.int32, device=dev_name)
    wg = 4096

    def best(launch, nbytes_or_flops):
        vals = []
        for _ in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            rc = launch()
            e1.record(st)
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"peak kernel launch failed ({rc})")
            vals.append(nbytes_or_flops / (e0.elapsed_time(e1) * 1e-3))
        return max(vals[1:])

    copy = best(lambda: lib.moe_peak_copy(a.data_ptr(), b.data_ptr(), n, wg, sp), 2 * n) / 1e9
    read = best(lambda: lib.moe_peak_read(a.data_ptr(), n, sink.data_ptr(), wg, sp), n) / 1e9
    out = torch.empty(2048 * 256, dtype=torch.float32, device=dev_name)
    mfma_by_wg = {}
    for mwg in (256, 512, 1024, 2048):  # 1, 2, 4, 8 wavefronts per SIMD
        iters = 8 * 1024 * 256 // mwg
        mfma_by_wg[mwg] = best(lambda: lib.moe_peak_mfma_bf16(out.data_ptr(), mwg, iters, sp),
                               lib.moe_peak_mfma_bf16_flops(mwg, iters)) / 1e12
    mfma = max(mfma_by_wg.values())
    del a, b
    return {"hbm_copy_GBps": round(copy, 1), "hbm_read_GBps": round(read, 1),
            "bf16_mfma_TFLOPs": round(mfma, 1),
            "bf16_mfma_by_waves_per_simd": {str(w // 256): round(v, 1) for w, v in mfma_by_wg.items()},
            "how": "best of 5 event-timed launches: copy and read of 2 GiB (HBM bytes moved / time); "
                   "bf16 MFMA 16x16x32 from registers, 4-wavefront workgroups with 8 independent "
                   "chains each, 1 to 8 wavefronts per SIMD (the best)"}


# default steps per workload id (the step counts keep each timed region short)
DEFAULT_STEPS = {1: 400, 2: 100, 3: 20, 4: 40}
DEFAULT_TOKEN_SETS = {1: 8, 2: 8, 3: 2, 4: 4}


def run_workload(args, cfg_id: int, experts, dev_name: str, steps: int, warmup: int,
                 token_sets: int, variants: bool, peaks: dict | None):
    """One workload: inputs resident in HBM, a pass with events on every
    step, K timed steps, K more steps for the dominant kernel's duration
    (events recorded by that kernel's own launch), and optionally the
    routing-replay and block entry points. Returns (result dict, layer)."""
    import numpy as np
    import torch

    from latent_mixture_experts_amd import binding as B
    from latent_mixture_experts_amd import synth

    cfg = synth.CONFIGS[cfg_id]
    dims, T = cfg["dims"], cfg["T"]
    print(f"bench: workload {cfg['name']} (T={T}), {steps} steps", file=sys.stderr, flush=True)
    lay = synth.config_layer(cfg_id)
    nv = args.format == "nvfp4"
    sblock = 16 if nv else 32
    workload = cfg["name"] + ("_nvfp4" if nv else "")
    to_dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).view(dt).to(dev_name)
    copies = []
    for c in range(args.weight_copies):
        w = dict(router=to_dev(lay.router, torch.float32), pooler=to_dev(lay.pooler, torch.int16),
                 unpooler=to_dev(lay.unpooler, torch.int16), norm_gain=to_dev(lay.gain, torch.int16),
                 **experts)
        copies.append((w, B.make_weights(w)))
    token_sets_dev = [to_dev(synth.token_batch(cfg_id, T, token_set=s), torch.int16)
                      for s in range(token_sets)]
    d = B.make_dims(dims, lay.eps, lay.gain_per_expert, B.FMT_NVFP4 if nv else B.FMT_MXFP4,
                    expert_split_rows=args.expert_split_rows)
    ws = B.alloc_workspace(d, T, device=dev_name)
    out = torch.empty((T, dims["hidden"]), dtype=torch.int16, device=dev_name)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    # touched experts per token set (from the library's own routing), and
    # that routing kept for the routing-replay timing
    touched, routings = [], []
    K = dims["top_k"]
    for x in token_sets_dev:
        B.latent_forward(d, x, copies[0][1], out, ws)
        torch.cuda.synchronize()
        offs = B.workspace_view(d, T, ws, "offsets", torch.int32, (dims["n_experts"] + 1,)).cpu().numpy()
        touched.append(int((np.diff(offs) > 0).sum()))
        routings.append((B.workspace_view(d, T, ws, "ids", torch.int32, (T, K)).clone(),
                         B.workspace_view(d, T, ws, "weights", torch.float32, (T, K)).clone()))
    step = lambda i, **kw: B.latent_forward(d, token_sets_dev[i % len(token_sets_dev)],
                                            copies[i % len(copies)][1], out, ws, stream=stream, **kw)

    # ---- warmup; a pass with events on every step for the breakdown ----
    nst = 2 * B.N_STAGES
    for i in range(warmup):
        step(i)
    n_pre = max(10, min(steps, 100))
    events = B.create_events(n_pre * nst)
    for i in range(n_pre):
        step(i, events=events[i * nst:(i + 1) * nst])
    torch.cuda.synchronize()
    stage_ms = np.zeros(B.N_STAGES)
    for i in range(n_pre):
        ev = events[i * nst:(i + 1) * nst]
        stage_ms += [B.elapsed_ms(ev[2 * s], ev[2 * s + 1]) for s in range(B.N_STAGES)]
    stage_ms /= n_pre
    B.destroy_events(events)
    dom = max(range(B.N_STAGES), key=lambda s: stage_ms[s])

    # ---- K timed steps (no events: recording them stalls the stream) ----
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # ---- K more steps in which the dominant kernel's launch records its own
    # start/stop events (the roofline's kernel duration) ----
    kev = B.create_events(2 * steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        evs = [None] * nst
        evs[2 * dom], evs[2 * dom + 1] = kev[2 * i], kev[2 * i + 1]
        step(i, events=evs)
    torch.cuda.synchronize()
    elapsed_ev = time.perf_counter() - t1
    dom_ms = float(np.mean([B.elapsed_ms(kev[2 * i], kev[2 * i + 1]) for i in range(steps)]))
    B.destroy_events(kev)

    elapsed_routed = elapsed_block = elapsed_persist = None
    if variants and T <= 2 and dims == synth.REAL:
        print("bench: persistent decode layer", file=sys.stderr, flush=True)
        B.workspace_view(d, T, ws, "sync", torch.int32, (64,)).zero_()
        # ---- the persistent decode layer: K steps of moe_latent_forward_persistent ----
        pers = lambda i: B.latent_forward_persistent(d, token_sets_dev[i % len(token_sets_dev)],
                                                     copies[i % len(copies)][1], out, ws, stream=stream)
        for i in range(min(warmup, 5)):
            pers(i)
        torch.cuda.synchronize()
        tp = time.perf_counter()
        for i in range(steps):
            pers(i)
        torch.cuda.synchronize()
        elapsed_persist = time.perf_counter() - tp
        st = B.workspace_view(d, T, ws, "sync", torch.int32, (64,)).cpu().numpy()
        if st[1] & 2:
            raise RuntimeError("persistent decode layer: a bounded wait gave up")
        # the last call's stamps (the 100 MHz clock; from workgroup 0's start):
        # routing done and barriers 1-4 released, workgroup 0's phase ends
        since = lambda v: round(((int(v) - int(st[16])) & 0xFFFFFFFF) / 100.0, 2)
        # (with the route sum the combine is part of the unpooler's phase: no barrier 4)
        rsum = B.workspace_view_range(d, T, "rows_bf16")[1] > 0
        persist_stamps = {"released_us": [since(v) for v in st[8:12 if rsum else 13]],
                          "workgroup0_us": [since(v) for v in st[17:22]],
                          "workgroups": int(st[3])}
        persist_note = ("released: routing done, barriers 1-3 released; workgroup 0: end of phases "
                        "1-3 (router+pooler, gate/up, down), then the start and end of the unpooler's "
                        "phase with the post-norm and weighted sum" if rsum else
                        "released: routing done, barriers 1-4 released; workgroup 0: end of phases 1-5 "
                        "(router+pooler, gate/up, down, combine, unpool)")
    if variants:
        # ---- routing replay: K steps of moe_latent_forward_routed with each
        # token set's recorded routing (no router, no top-k) ----
        def routed(i):
            r_ids, r_w = routings[i % len(routings)]
            B.latent_forward_routed(d, token_sets_dev[i % len(token_sets_dev)], r_ids, r_w,
                                    copies[i % len(copies)][1], out, ws, stream=stream)
        for i in range(min(warmup, 5)):
            routed(i)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for i in range(steps):
            routed(i)
        torch.cuda.synchronize()
        elapsed_routed = time.perf_counter() - t2

        # ---- the block around the layer (pre-norm, layer, post-norm + residual):
        # K steps of moe_block_forward with the token sets as the residual stream ----
        pre_np, post_np = synth.block_gains(dims)
        pre_g, post_g = to_dev(pre_np, torch.int16), to_dev(post_np, torch.int16)
        ws_blk = B.alloc_block_workspace(d, T, device=dev_name)
        out_blk = torch.empty_like(out)
        blk = lambda i: B.block_forward(d, token_sets_dev[i % len(token_sets_dev)], pre_g, post_g,
                                        1e-6, copies[i % len(copies)][1], out_blk, ws_blk, stream=stream)
        for i in range(min(warmup, 5)):
            blk(i)
        torch.cuda.synchronize()
        t3 = time.perf_counter()
        for i in range(steps):
            blk(i)
        torch.cuda.synchronize()
        elapsed_block = time.perf_counter() - t3
        del ws_blk

    ms_per_step = elapsed * 1e3 / steps
    U = float(np.mean([touched[i % len(touched)] for i in range(steps)]))
    sb = stage_bytes(dims, T, U, sblock)
    sf = stage_flops(dims, T)
    if T <= 16:  # the router and the pooler share one launch (timed as "router")
        sb["router"] += sb.pop("pool")
        sb["pool"] = 0
        sf["router"] += sf.pop("pool")
    # few route rows: the post-norm and the weighted sum inside the unpooler's
    # launch (timed as "unpool"; the workspace then holds the gain-scaled rows)
    route_sum = B.workspace_view_range(d, T, "rows_bf16")[1] > 0
    if route_sum:
        sb["unpool"] += sb.pop("combine")
        sb["combine"] = 0
    stages = {}
    for s, name in enumerate(B.STAGES):
        us = stage_ms[s] * 1e3
        entry = {"us": round(us, 2), "GBps": round(sb[name] / max(us * 1e-6, 1e-12) / 1e9, 1)}
        # (a step without a kernel of its own records its two events back to
        # back: its figure is that pair's overhead, not work)
        no_kernel = " (no kernel of its own: two events recorded back to back)"
        fused_route = T <= 8 and T * dims["top_k"] <= 64
        if T <= 16 and name in ("router", "pool", "permute"):
            entry["note"] = {"router": "router + pooler (one launch)", "pool": "in the router launch" + no_kernel,
                             "permute": "in the top-k launch" + no_kernel}[name]
        if fused_route and name in ("router", "topk", "permute"):
            entry["note"] = {"router": "router + pooler + top-K + grouping (one launch)",
                             "topk": "in the router launch" + no_kernel,
                             "permute": "in the router launch" + no_kernel}[name]
        if route_sum and name in ("combine", "unpool"):
            entry["note"] = {"combine": "in the unpooler launch" + no_kernel,
                             "unpool": "post-norm + weighted sum + unpooler (one launch)"}[name]
        if name in sf:
            entry["TFLOPs"] = round(sf[name] / max(us * 1e-6, 1e-12) / 1e12, 2)
        stages[name] = entry
    dom_name = B.STAGES[dom]
    dom_s = dom_ms * 1e-3
    mfma_bound = T >= 1024
    if mfma_bound and dom_name in sf:
        achieved = sf[dom_name] / dom_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4)}
        if peaks:
            roof["frac_of_measured"] = round(achieved / peaks["bf16_mfma_TFLOPs"], 4)
    else:
        achieved = sb[dom_name] / dom_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
        if peaks:
            roof["frac_of_measured"] = round(achieved / peaks["hbm_read_GBps"], 4)
    roof["traffic"] = traffic_for(dom_name, workload)
    roof["kernel"] = dom_name
    roof["kernel_us"] = round(dom_ms * 1e3, 2)
    roof["ms_per_step_with_events"] = round(elapsed_ev * 1e3 / steps, 4)

    layer_gbs = layer_bytes(dims, T, U, sblock) / (ms_per_step * 1e-3) / 1e9
    mfma_flops = 4 * T * dims["hidden"] * dims["latent"] + 2 * T * K * 3 * dims["latent"] * dims["inter"]
    res = {
        "value": round(T * steps / elapsed, 2),
        "ms_per_step": round(ms_per_step, 4),
        "steps": steps,
        "config": {"workload": workload, "T": T, "hidden": dims["hidden"],
                   "latent": dims["latent"], "inter": dims["inter"],
                   "n_experts": dims["n_experts"], "top_k": dims["top_k"],
                   "experts": ("NVFP4 (E2M1 + E4M3/16 + fp32 per tensor), W4A16" if nv
                               else "MXFP4 (E2M1 + E8M0/32), W4A16"), "touched_experts": U,
                   "token_sets": token_sets, "weight_copies": args.weight_copies,
                   "expert_split_rows": args.expert_split_rows},
        "roofline": roof,
        "layer_hbm": {"GBps": round(layer_gbs, 1), "frac": round(layer_gbs / HBM_PEAK_GBS, 4),
                      "algorithmic_bytes": int(layer_bytes(dims, T, U, sblock))},
        "layer_mfma": {"TFLOPs": round(mfma_flops / (ms_per_step * 1e-3) / 1e12, 1),
                       "frac": round(mfma_flops / (ms_per_step * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                       "flops": int(mfma_flops)},
        "stages": stages,
    }
    if peaks:
        res["layer_hbm"]["frac_of_measured"] = round(layer_gbs / peaks["hbm_read_GBps"], 4)
    if elapsed_routed is not None:
        res["routed"] = {
            "entry": "moe_latent_forward_routed (routing replay: the recorded routing of each "
                     "token set; no router, no top-k)",
            "value": round(T * steps / elapsed_routed, 2),
            "unit": "tokens/s",
            "ms_per_step": round(elapsed_routed * 1e3 / steps, 4),
            "layer_hbm_frac": round((layer_bytes(dims, T, U, sblock) - 4 * dims["n_experts"] * dims["hidden"])
                                    / (elapsed_routed / steps) / 1e9 / HBM_PEAK_GBS, 4),
        }
    if elapsed_persist is not None:
        res["persistent"] = {
            "entry": "moe_latent_forward_persistent (the whole layer in one launch: phases separated "
                     "by barriers between its workgroups)",
            "value": round(T * steps / elapsed_persist, 2),
            "unit": "tokens/s",
            "ms_per_step": round(elapsed_persist * 1e3 / steps, 4),
            "layer_hbm_frac": round(layer_bytes(dims, T, U, sblock) / (elapsed_persist / steps) / 1e9
                                    / HBM_PEAK_GBS, 4),
            "stamps": dict(persist_stamps, note=persist_note),
        }
    if elapsed_block is not None:
        res["block"] = {
            "entry": "moe_block_forward (resid + post_norm(layer(pre_norm(resid))); the token "
                     "sets as the residual stream)",
            "value": round(T * steps / elapsed_block, 2),
            "unit": "tokens/s",
            "ms_per_step": round(elapsed_block * 1e3 / steps, 4),
            "extra_ms_per_step": round((elapsed_block - elapsed) * 1e3 / steps, 4),
        }
    del copies, token_sets_dev, ws, out
    torch.cuda.empty_cache()
    return res, lay


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the layer runs on one GPU only; --gpus must be 1 "
                          "(its expert-parallel sharding is described, not implemented)"}))
        sys.exit(2)

    import torch

    from latent_mixture_experts_amd import synth

    dev_name = "cuda:0"
    torch.cuda.set_device(0)
    nv = args.format == "nvfp4"
    main_cfg = args.config if args.config is not None else 1
    peaks = None if args.no_peaks else measured_peaks(dev_name)
    experts = (synth.all_nvfp4_expert_bytes(synth.REAL, 0, device=dev_name) if nv
               else synth.all_expert_bytes(synth.REAL, 0, device=dev_name))
    torch.cuda.synchronize()
    if args.copy_probe_mib:
        copy_probe(dev_name, args.copy_probe_mib)

    steps = args.steps if args.steps is not None else DEFAULT_STEPS[main_cfg]
    token_sets = args.token_sets if args.token_sets is not None else DEFAULT_TOKEN_SETS[main_cfg]
    res, lay = run_workload(args, main_cfg, experts, dev_name, steps, args.warmup, token_sets,
                            not args.no_variants, peaks)
    result = {
        "metric": "latent-MoE layer tokens/s",
        "value": res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
    }
    result.update({k: v for k, v in res.items() if k not in ("value", "ms_per_step", "steps")})
    if peaks:
        result["measured_peaks"] = peaks
    # the other workloads of the metric (one line per workload, under "workloads")
    if args.config is None and not args.only_main:
        others = {}
        for c in (2, 4, 3):
            r, _ = run_workload(args, c, experts, dev_name, DEFAULT_STEPS[c], min(args.warmup, 5),
                                DEFAULT_TOKEN_SETS[c], False, peaks)
            others[synth.CONFIGS[c]["name"]] = {k: r[k] for k in ("value", "ms_per_step", "steps",
                                                                  "roofline", "layer_hbm",
                                                                  "layer_mfma", "config")}
        result["workloads"] = others
    if not args.no_cpu_baseline and not nv:  # (the oracle baseline is taken on the MXFP4 layer)
        print("bench: CPU baseline (the oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(lay, experts, args.cpu_tokens, args.cpu_tokens_1t,
                                              main_cfg)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
