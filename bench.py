"""Benchmark of the latent MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1]

A step is one moe_latent_forward over one batch of synthetic tokens (router,
top-K, permutation, pooler, expert gate/up + SwiGLU, expert down, post-expert
norm + weighted sum, unpooler). Default workload: the real-shape layer
(H 8192, L 4096, 256 experts top-8, SwiGLU I 4096, MXFP4 experts) at decode
T = 1. Inputs are resident in HBM before the timed region. To keep the
256 MB last-level cache from serving the weight stream, steps rotate over 8
token sets (different experts) and 4 copies of the dense weights.

Prints one JSON line with layer tokens/s (K steps timed by the host clock,
no events in the stream), the roofline of the dominant kernel (timed over K
further steps with HIP events that its own launch records, on the library's
stream) and the CPU oracle baseline.
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
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1, help="workload id 1..4 (see synth.CONFIGS)")
    ap.add_argument("--token-sets", type=int, default=8)
    ap.add_argument("--weight-copies", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--format", choices=("mxfp4", "nvfp4"), default="mxfp4",
                    help="expert weight format (nvfp4: E4M3 scales per 16 and per-tensor scales)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the routing-replay and block timings (profiling runs: one kernel mix)")
    ap.add_argument("--cpu-tokens", type=int, default=320, help="tokens in the oracle sample (about 10 s of host work)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run an elementwise copy of this size (HBM counter calibration)")
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


def cpu_baseline(lay, dev, n_tokens: int, cfg_id: int):
    """The oracle as it stands, on the host cores, over a bounded sample of
    the same workload: n_tokens single-token layer passes (tokens drawn like
    the benchmark's, from a token set of their own), one per thread. Expert bytes are copied to the host first and the
    copy is not timed."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    from latent_mixture_experts_amd import synth

    xs = synth.token_batch(cfg_id, n_tokens, token_set=1000)
    logits = oracle.router_logits(xs, lay.router)
    ids, _ = oracle.topk(logits, lay.dims["top_k"])
    cache = {int(e): tuple(dev[k][int(e)].cpu().numpy() for k in synth.EXPERT_TENSORS)
             for e in np.unique(ids)}
    cores = min(len(xs), os.cpu_count() or 1, 16)
    fn = lambda t: oracle.token_forward(lay.dims, xs[t], lay.router, lay.pooler, lay.gain,
                                        lay.unpooler, lay.eps, lay.gain_per_expert, cache.__getitem__)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(cores) as ex:
        list(ex.map(fn, range(len(xs))))
    dt = time.perf_counter() - t0
    return {"value": len(xs) / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(xs)} single-token layer passes (real shape, one thread each), "
                      f"{dt:.1f} s wall on {cores} host threads; input generation and "
                      "expert-byte copies excluded"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the layer runs on one GPU only; --gpus must be 1 "
                          "(its expert-parallel sharding is described, not implemented)"}))
        sys.exit(2)

    import numpy as np
    import torch

    from latent_mixture_experts_amd import binding as B
    from latent_mixture_experts_amd import synth

    cfg = synth.CONFIGS[args.config]
    dims, T = cfg["dims"], cfg["T"]
    dev_name = "cuda:0"
    torch.cuda.set_device(0)

    # ---- inputs, resident in HBM -------------------------------------------
    t_gen = time.time()
    lay = synth.config_layer(args.config)
    nv = args.format == "nvfp4"
    experts = (synth.all_nvfp4_expert_bytes(dims, 0, device=dev_name) if nv
               else synth.all_expert_bytes(dims, 0, device=dev_name))
    sblock = 16 if nv else 32
    workload = cfg["name"] + ("_nvfp4" if nv else "")
    to_dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).view(dt).to(dev_name)
    copies = []
    for c in range(args.weight_copies):
        w = dict(router=to_dev(lay.router, torch.float32), pooler=to_dev(lay.pooler, torch.int16),
                 unpooler=to_dev(lay.unpooler, torch.int16), norm_gain=to_dev(lay.gain, torch.int16),
                 **experts)
        copies.append((w, B.make_weights(w)))
    token_sets_np = [synth.token_batch(args.config, T, token_set=s) for s in range(args.token_sets)]
    token_sets = [to_dev(x, torch.int16) for x in token_sets_np]
    d = B.make_dims(dims, lay.eps, lay.gain_per_expert, B.FMT_NVFP4 if nv else B.FMT_MXFP4)
    ws = B.alloc_workspace(d, T, device=dev_name)
    out = torch.empty((T, dims["hidden"]), dtype=torch.int16, device=dev_name)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen

    # touched experts per token set (from the library's own routing), and
    # that routing kept for the routing-replay timing
    touched, routings = [], []
    K = dims["top_k"]
    for x in token_sets:
        B.latent_forward(d, x, copies[0][1], out, ws)
        torch.cuda.synchronize()
        offs = B.workspace_view(d, T, ws, "offsets", torch.int32, (dims["n_experts"] + 1,)).cpu().numpy()
        touched.append(int((np.diff(offs) > 0).sum()))
        routings.append((B.workspace_view(d, T, ws, "ids", torch.int32, (T, K)).clone(),
                         B.workspace_view(d, T, ws, "weights", torch.float32, (T, K)).clone()))

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev_name).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):  # an elementwise kernel that reads n and writes n bytes
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()

    # ---- warmup; a pass with events on every step for the breakdown ----
    nst = 2 * B.N_STAGES
    for i in range(args.warmup):
        B.latent_forward(d, token_sets[i % len(token_sets)], copies[i % len(copies)][1], out, ws)
    n_pre = max(20, min(args.steps, 100))
    events = B.create_events(n_pre * nst)
    for i in range(n_pre):
        B.latent_forward(d, token_sets[i % len(token_sets)], copies[i % len(copies)][1], out, ws,
                         stream=stream, events=events[i * nst:(i + 1) * nst])
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
    for i in range(args.steps):
        B.latent_forward(d, token_sets[i % len(token_sets)], copies[i % len(copies)][1], out, ws,
                         stream=stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # ---- K more steps in which the dominant kernel's launch records its own
    # start/stop events (the roofline's kernel duration) ----
    kev = B.create_events(2 * args.steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(args.steps):
        evs = [None] * nst
        evs[2 * dom], evs[2 * dom + 1] = kev[2 * i], kev[2 * i + 1]
        B.latent_forward(d, token_sets[i % len(token_sets)], copies[i % len(copies)][1], out, ws,
                         stream=stream, events=evs)
    torch.cuda.synchronize()
    elapsed_ev = time.perf_counter() - t1
    dom_ms = float(np.mean([B.elapsed_ms(kev[2 * i], kev[2 * i + 1]) for i in range(args.steps)]))
    B.destroy_events(kev)

    # ---- routing replay: K steps of moe_latent_forward_routed with each
    # token set's recorded routing (no router, no top-k) ----
    elapsed_routed = elapsed_block = None
    for i in range(0 if args.no_variants else min(args.warmup, 5)):
        r_ids, r_w = routings[i % len(routings)]
        B.latent_forward_routed(d, token_sets[i % len(token_sets)], r_ids, r_w,
                                copies[i % len(copies)][1], out, ws, stream=stream)
    if not args.no_variants:
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for i in range(args.steps):
            r_ids, r_w = routings[i % len(routings)]
            B.latent_forward_routed(d, token_sets[i % len(token_sets)], r_ids, r_w,
                                    copies[i % len(copies)][1], out, ws, stream=stream)
        torch.cuda.synchronize()
        elapsed_routed = time.perf_counter() - t2

        # ---- the block around the layer (pre-norm, layer, post-norm + residual):
        # K steps of moe_block_forward with the token sets as the residual stream ----
        pre_np, post_np = synth.block_gains(dims)
        pre_g, post_g = to_dev(pre_np, torch.int16), to_dev(post_np, torch.int16)
        ws_blk = B.alloc_block_workspace(d, T, device=dev_name)
        out_blk = torch.empty_like(out)
        for i in range(min(args.warmup, 5)):
            B.block_forward(d, token_sets[i % len(token_sets)], pre_g, post_g, 1e-6,
                            copies[i % len(copies)][1], out_blk, ws_blk, stream=stream)
        torch.cuda.synchronize()
        t3 = time.perf_counter()
        for i in range(args.steps):
            B.block_forward(d, token_sets[i % len(token_sets)], pre_g, post_g, 1e-6,
                            copies[i % len(copies)][1], out_blk, ws_blk, stream=stream)
        torch.cuda.synchronize()
        elapsed_block = time.perf_counter() - t3
        del ws_blk

    ms_per_step = elapsed * 1e3 / args.steps
    U = float(np.mean([touched[i % len(touched)] for i in range(args.steps)]))
    sb = stage_bytes(dims, T, U, sblock)
    sf = stage_flops(dims, T)
    if T <= 16:  # the router and the pooler share one launch (timed as "router")
        sb["router"] += sb.pop("pool")
        sb["pool"] = 0
        sf["router"] += sf.pop("pool")
    stages = {}
    for s, name in enumerate(B.STAGES):
        us = stage_ms[s] * 1e3
        entry = {"us": round(us, 2), "GBps": round(sb[name] / (us * 1e-6) / 1e9, 1)}
        if T <= 16 and name in ("router", "pool", "permute"):
            entry["note"] = {"router": "router + pooler (one launch)", "pool": "in the router launch",
                             "permute": "in the top-k launch"}[name]
        if name in sf:
            entry["TFLOPs"] = round(sf[name] / (us * 1e-6) / 1e12, 2)
        stages[name] = entry
    dom_name = B.STAGES[dom]
    dom_s = dom_ms * 1e-3
    mfma_bound = T >= 1024
    if mfma_bound and dom_name in sf:
        achieved = sf[dom_name] / dom_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4)}
    else:
        achieved = sb[dom_name] / dom_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["kernel"] = dom_name
    roof["kernel_us"] = round(dom_ms * 1e3, 2)
    roof["ms_per_step_with_events"] = round(elapsed_ev * 1e3 / args.steps, 4)
    roof["traffic"] = traffic_for(dom_name, workload)

    layer_gbs = layer_bytes(dims, T, U, sblock) / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": "latent-MoE layer tokens/s",
        "value": round(T * args.steps / elapsed, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "T": T, "hidden": dims["hidden"],
                   "latent": dims["latent"], "inter": dims["inter"],
                   "n_experts": dims["n_experts"], "top_k": dims["top_k"],
                   "experts": ("NVFP4 (E2M1 + E4M3/16 + fp32 per tensor), W4A16" if nv
                               else "MXFP4 (E2M1 + E8M0/32), W4A16"), "touched_experts": U,
                   "token_sets": args.token_sets, "weight_copies": args.weight_copies},
        "roofline": roof,
        "layer_hbm": {"GBps": round(layer_gbs, 1), "frac": round(layer_gbs / HBM_PEAK_GBS, 4),
                      "algorithmic_bytes": int(layer_bytes(dims, T, U, sblock))},
        "stages": stages,
    }
    if elapsed_routed is not None:
        result["routed"] = {
            "entry": "moe_latent_forward_routed (routing replay: the recorded routing of each "
                     "token set; no router, no top-k)",
            "value": round(T * args.steps / elapsed_routed, 2),
            "unit": "tokens/s",
            "ms_per_step": round(elapsed_routed * 1e3 / args.steps, 4),
            "layer_hbm_frac": round((layer_bytes(dims, T, U, sblock) - 4 * dims["n_experts"] * dims["hidden"])
                                    / (elapsed_routed / args.steps) / 1e9 / HBM_PEAK_GBS, 4),
        }
    if elapsed_block is not None:
        result["block"] = {
            "entry": "moe_block_forward (resid + post_norm(layer(pre_norm(resid))); the token "
                     "sets as the residual stream)",
            "value": round(T * args.steps / elapsed_block, 2),
            "unit": "tokens/s",
            "ms_per_step": round(elapsed_block * 1e3 / args.steps, 4),
            "extra_ms_per_step": round((elapsed_block - elapsed) * 1e3 / args.steps, 4),
        }
    if not args.no_cpu_baseline and not nv:  # (the oracle baseline is taken on the MXFP4 layer)
        result["cpu_baseline"] = cpu_baseline(lay, copies[0][0], args.cpu_tokens, args.config)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
