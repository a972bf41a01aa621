"""Helpers shared by the GPU tests: seeded inputs on the device, the HIP path
through the C ABI, the oracle on the host, and the comparison bars."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
from latent_mixture_experts_amd import binding as B
from latent_mixture_experts_amd import synth
from tests import exact

HOST_WORKERS = min(16, os.cpu_count() or 1)

# Output bar: max |delta| <= 2e-2 and relative RMS <= 1e-2 in bf16.
OUT_ATOL = 2e-2
OUT_REL_RMS = 1e-2


def log(msg: str) -> None:
    print(msg, flush=True)


def device_layer(lay: synth.Layer, experts: dict | None = None, device="cuda") -> dict:
    """Dense tensors of the layer on the device, plus expert bytes (generated
    on the device from the counter-based generator unless given)."""
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).view(dt).to(device)
    dev = dict(
        x=t(lay.x, torch.int16), router=t(lay.router, torch.float32),
        pooler=t(lay.pooler, torch.int16), unpooler=t(lay.unpooler, torch.int16),
        norm_gain=t(lay.gain, torch.int16))
    if experts is None:
        experts = synth.all_expert_bytes(lay.dims, lay.seed, device=device)
    for k, v in experts.items():
        dev[k] = v.to(device).contiguous()
    return dev


def run_gpu(lay: synth.Layer, dev: dict, T: int | None = None, x: torch.Tensor | None = None):
    """moe_latent_forward; returns (out tensor, dims, workspace)."""
    x = dev["x"] if x is None else x
    T = x.shape[0] if T is None else T
    d = B.make_dims(lay.dims, lay.eps, lay.gain_per_expert)
    ws = B.alloc_workspace(d, T)
    out = torch.empty((T, lay.dims["hidden"]), dtype=torch.int16, device=x.device)
    B.latent_forward(d, x, B.make_weights(dev), out, ws)
    torch.cuda.synchronize()
    return out, d, ws


def rows16_written(d, T: int) -> bool:
    """Whether moe_latent_forward takes the post-norm, the weighted sum and
    the unpooler in one launch for T tokens (then the workspace holds the
    gain-scaled bf16 route rows and no y)."""
    off, nb = B.workspace_view_range(d, T, "rows_bf16")
    return nb > 0


def views(lay: synth.Layer, d, ws, T: int) -> dict:
    """The intermediates of the last call (moe_latent_forward and its
    variants); y is None and rows16 ([T*K][L] bf16 bits, route-major)
    present when the weighted sum was taken after the unpooler's products."""
    L, I, E, K = (lay.dims[k] for k in ("latent", "inter", "n_experts", "top_k"))
    v = lambda name, dt, shape: B.workspace_view(d, T, ws, name, dt, shape).cpu().numpy()
    r16 = rows16_written(d, T)
    return dict(
        logits=v("logits", torch.float32, (T, E)), ids=v("ids", torch.int32, (T, K)),
        w=v("weights", torch.float32, (T, K)), offsets=v("offsets", torch.int32, (E + 1,)),
        sorted=v("sorted", torch.int32, (T * K,)),
        lat=v("latent", torch.int16, (T, L)).view(np.uint16),
        h=v("h", torch.int16, (T * K, I)).view(np.uint16),
        rows=v("rows", torch.float32, (T * K, L)),
        y=None if r16 else v("y", torch.int16, (T, L)).view(np.uint16),
        rows16=v("rows_bf16", torch.int16, (T * K, L)).view(np.uint16) if r16 else None)


def assert_y_or_rows16(got: dict, lay: synth.Layer, y_ref_bits, what: str = "y", t=None, out_bits=None):
    """y against the oracle's when the layer wrote it, else the gain-scaled
    route rows it took instead against the route rows (all of them) and, with
    out_bits, the output of the route sum from them (token t, or all)."""
    if got["y"] is not None:
        assert_out_close(got["y"] if t is None else got["y"][t], y_ref_bits, what)
    else:
        assert_rows16_from_rows(got, lay.gain, lay.gain_per_expert)
        if out_bits is not None:
            assert_route_sum_output(got, lay, out_bits, None if t is None else [t])


def assert_route_sum_output(got: dict, lay: synth.Layer, out_bits, tokens=None):
    """The output of the route sum from the GPU's own intermediates, in
    fp64: each route row's scale c = w / sqrt(mean(row^2) + eps) from its
    fp32 row, the unpooler applied to the gain-scaled bf16 rows, and each
    token's products added with their scales; the GPU's bf16 output is that
    value rounded, within one bf16 ulp (its fp32 accumulations can move a
    value across a rounding boundary) or, where the terms cancel, 2^-16 of
    the sum of the terms' magnitudes (fp32 accumulation of 4096 products).
    This checks the fused epilogue itself, apart from the choice of rounding
    point that the oracle's bar covers."""
    K = lay.dims["top_k"]
    L = lay.dims["latent"]
    T = np.asarray(out_bits).shape[0]
    tokens = range(T) if tokens is None else tokens
    rows = got["rows"].astype(np.float64)
    c = got["w"].reshape(-1).astype(np.float64) / np.sqrt((rows * rows).sum(axis=1) / L + float(lay.eps))
    u = bf16(lay.unpooler)
    r16 = bf16(got["rows16"])
    ua = np.abs(u)
    for t in tokens:
        z = r16[t * K:(t + 1) * K] @ u.T                      # [K][H]
        ref = (c[t * K:(t + 1) * K, None] * z).sum(axis=0)
        mag = (np.abs(c[t * K:(t + 1) * K, None]) * (np.abs(r16[t * K:(t + 1) * K]) @ ua.T)).sum(axis=0)
        g = bf16(np.asarray(out_bits)[t])
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
        bad = np.abs(g - ref) > np.maximum(ulp, 2.0 ** -16 * mag)
        assert not bad.any(), f"route sum t={t}: {int(bad.sum())} outputs beyond one bf16 ulp"


def assert_rows16_from_rows(got: dict, gain_bits, gain_per_expert: bool):
    """The gain-scaled bf16 route rows are the GPU's own fp32 route rows
    times the bf16 gain (of the route's expert when the gain is per expert),
    one fp32 product rounded to nearest-even bf16 (torch's conversion), bit
    for bit."""
    rows = got["rows"].astype(np.float32)
    g = exact.bf16_to_f64(np.asarray(gain_bits).view(np.uint16)).astype(np.float32)
    gr = g[got["ids"].reshape(-1)] if gain_per_expert else np.broadcast_to(g, rows.shape)
    want = torch.from_numpy(np.ascontiguousarray(rows * gr)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(got["rows16"], want.view(np.uint16)), "gain-scaled route rows"



def host_experts(dev: dict) -> dict:
    return {k: dev[k].cpu().numpy() for k in synth.EXPERT_TENSORS}


def oracle_full(lay: synth.Layer, ex_host: dict) -> dict:
    return oracle.latent_forward(lay.dims, lay.x, lay.router, lay.pooler, ex_host["w13_codes"],
                                 ex_host["w13_scales"], ex_host["w2_codes"], ex_host["w2_scales"],
                                 lay.gain, lay.unpooler, lay.eps, lay.gain_per_expert)


def oracle_router_all(lay: synth.Layer):
    """Oracle logits and top-K for every token (tokens split over threads)."""
    T = lay.T
    chunks = [(a, min(T, a + 64)) for a in range(0, T, 64)]
    with ThreadPoolExecutor(HOST_WORKERS) as ex:
        parts = list(ex.map(lambda c: oracle.router_logits(lay.x[c[0]:c[1]], lay.router), chunks))
    logits = np.concatenate(parts)
    ids, w = oracle.topk(logits, lay.dims["top_k"])
    return logits, ids, w


def oracle_tokens(lay: synth.Layer, dev: dict, tokens, fmt: int = oracle.MXFP4) -> list[dict]:
    """oracle.token_forward for selected tokens; expert bytes copied from the
    device on demand (they come from the shared input generator). NVFP4:
    dev also holds the per-tensor scales w13_global / w2_global [E]."""
    cache = {}

    def get(e):
        if e not in cache:
            t = tuple(dev[k][e].cpu().numpy() for k in synth.EXPERT_TENSORS)
            if fmt == oracle.NVFP4:
                t = t + (float(dev["w13_global"][e]), float(dev["w2_global"][e]))
            cache[e] = t
        return cache[e]

    # fetch the experts first (device copies), then run the host math in threads
    logits = oracle.router_logits(lay.x[list(tokens)], lay.router)
    ids, _ = oracle.topk(logits, lay.dims["top_k"])
    for e in np.unique(ids):
        get(int(e))
    fn = lambda t: oracle.token_forward(lay.dims, lay.x[t], lay.router, lay.pooler, lay.gain,
                                        lay.unpooler, lay.eps, lay.gain_per_expert, get, fmt)
    with ThreadPoolExecutor(HOST_WORKERS) as ex:
        return list(ex.map(fn, tokens))


def oracle_expert_rows(lay: synth.Layer, ex_host: dict, lat_bits, ids, fmt: int = oracle.MXFP4,
                       routes=None):
    """Steps A5 and A6 alone: oracle.expert_row for each route r = t*K + k
    (all, or those listed), fed with the given latent rows (the GPU's, so that
    A4's roundings do not enter) and expert ids[t][k]. ex_host maps the expert
    tensor names to [E][...] arrays (NVFP4: plus w13_global, w2_global).
    Returns (h [n][I], rows [n][L]) in route order."""
    K = lay.dims["top_k"]
    ids = np.asarray(ids).reshape(-1)
    routes = range(ids.size) if routes is None else routes

    def one(r):
        e, lat = int(ids[r]), lat_bits[r // K]
        if fmt == oracle.NVFP4:
            return oracle.expert_row_fmt(oracle.NVFP4, lat, ex_host["w13_codes"][e],
                                         ex_host["w13_scales"][e], float(ex_host["w13_global"][e]),
                                         ex_host["w2_codes"][e], ex_host["w2_scales"][e],
                                         float(ex_host["w2_global"][e]))
        return oracle.expert_row(lat, ex_host["w13_codes"][e], ex_host["w13_scales"][e],
                                 ex_host["w2_codes"][e], ex_host["w2_scales"][e])

    with ThreadPoolExecutor(HOST_WORKERS) as ex:
        res = list(ex.map(one, routes))
    return np.stack([r[0] for r in res]), np.stack([r[1] for r in res])


def bf16(a) -> np.ndarray:
    return exact.bf16_to_f64(np.asarray(a).view(np.uint16))


def out_errors(got_bits, ref_bits) -> tuple[float, float]:
    g, r = bf16(got_bits), bf16(ref_bits)
    d = g - r
    return float(np.abs(d).max()), float(np.sqrt((d * d).mean() / max((r * r).mean(), 1e-30)))


def assert_out_close(got_bits, ref_bits, what="out"):
    mx, rel = out_errors(got_bits, ref_bits)
    assert mx <= OUT_ATOL and rel <= OUT_REL_RMS, f"{what}: max|d|={mx:.3g} relRMS={rel:.3g}"


def assert_rel_close(got, ref, rel_rms, what):
    g, r = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    d = g - r
    rel = float(np.sqrt((d * d).mean() / max((r * r).mean(), 1e-30)))
    assert rel <= rel_rms, f"{what}: relRMS={rel:.3g}"


def assert_rows_elementwise(got, ref, rel_elem: float, what: str):
    """Per element of fp32 route rows: |got - ref| <= rel_elem * RMS of the
    reference row (the GPU's fp32 sums against the oracle's exact ones, and
    the rare one-ulp flips of a bf16 h element they feed)."""
    g = np.asarray(got, np.float64).reshape(-1, np.shape(ref)[-1])
    r = np.asarray(ref, np.float64).reshape(g.shape)
    rms = np.sqrt((r * r).mean(axis=1, keepdims=True))
    bad = np.abs(g - r) > rel_elem * np.maximum(rms, 1e-30)
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond {rel_elem} x row RMS " \
                          f"(worst {float((np.abs(g - r) / np.maximum(rms, 1e-30)).max()):.3g})"


def assert_h_elementwise(got_bits, ref_bits, what: str = "h"):
    """Per element of bf16 h rows: within one bf16 ulp of the reference, or
    1e-3 of the row's RMS where h is near zero (h = bf16(silu(g) * u) with
    g, u fp32 sums on the GPU and exact sums in the oracle, both from the same
    latent rows), and at least 95% identical."""
    g = bf16(np.asarray(got_bits)).reshape(-1, np.shape(ref_bits)[-1])
    r = bf16(np.asarray(ref_bits)).reshape(g.shape)
    ulp = np.ldexp(1.0, np.frexp(np.abs(r))[1] - 8)
    rms = np.sqrt((r * r).mean(axis=1, keepdims=True))
    d = np.abs(g - r)
    ok = d <= np.maximum(ulp, 1e-3 * rms)
    assert ok.all(), f"{what}: {int((~ok).sum())} elements beyond one ulp"
    assert (d == 0).mean() > 0.95, f"{what}: only {(d == 0).mean():.3f} identical"


def ulp_diff_f32(a, b) -> np.ndarray:
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


def assert_latent_close(got_bits, ref_bits):
    """Latent rows: the GPU rounds an fp32-accumulated sum to bf16, the oracle
    its exact sum. They agree bit for bit almost everywhere and differ by at
    most one bf16 ulp where the result is not small against the row's scale;
    near zero the fp32 accumulation error (a few 2^-24 of the row's RMS) may
    exceed one ulp of the result itself."""
    g = bf16(np.asarray(got_bits)).astype(np.float64)
    r = bf16(np.asarray(ref_bits)).astype(np.float64)
    ulp = np.ldexp(1.0, np.frexp(np.abs(r))[1] - 8)  # bf16 ulp at |r|
    rms = np.sqrt(np.mean(r * r))
    d = np.abs(g - r)
    assert (d <= np.maximum(ulp, 1e-5 * rms)).all(), (d.max(), rms)
    assert (d == 0).mean() > 0.95
