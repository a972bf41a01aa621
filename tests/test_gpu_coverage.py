"""GPU parity on paths the layer tests reach only in part.

* moe_route at decode sizes (T = 1, 4, 8, 16: the one-pass router and the
  one-workgroup top-K + grouping), with tied router rows;
* the generation word of the routing done inside the router launch
  (T <= 8) advances by exactly one per call, and no workgroup gives up;
* the post-norm and weighted sum in the unpooler's launch at widths off the
  real shape (rows staged through registers, no K split, per-expert gains,
  NVFP4, a full 16-row fragment);
* every route row is written: the h and route-row buffers are filled with
  NaN before the call (real prefill shape; a routed case whose experts hold
  1, 2, 3 and 4 row tiles, on both sides of the threshold where the row
  tiles are listed in pairs), and that case's rows match the oracle;
* every route row of the three most-loaded experts at the real prefill and
  skewed shapes, element by element against the oracle's expert_row fed
  with the GPU's latent rows (so A5/A6 are checked apart from A4);
* NVFP4 experts at the real shape: decode (all rows), verify and prefill
  (sampled tokens).

Sources: "Muse Spark Open on Gaudi 2", section "The latent MoE: A' with a
per-expert norm" (one row per route, grouped by expert); "Soporte de día 0
para Muse Spark Open en vLLM", section "Aspectos destacados" (NVFP4
checkpoint).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from latent_mixture_experts_amd import binding as B
from latent_mixture_experts_amd import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


# ---- moe_route at decode sizes -----------------------------------------------------
@pytest.mark.parametrize("T", [1, 4, 8, 16])
def test_route_entry_point_at_decode_sizes(T):
    """moe_route for T <= 16 (one-pass router per expert, then top-K and the
    grouping in one workgroup) at the real expert count and top-K, with
    duplicated router rows (exact ties that go to the lower id) and one
    all-zero token (ids 0..K-1)."""
    dims = dict(hidden=2048, latent=128, inter=128, n_experts=256, top_k=8)
    lay = synth.make_layer(dims, T, seed=70 + T)
    r = lay.router.copy()
    r[128:256] = r[0:128]          # expert e and e + 128 tie for every token
    x = lay.x.copy()
    if T > 1:
        x[T - 1] = 0               # every logit 0: ids 0..7
    G.log(f"moe_route T={T}")
    d = B.make_dims(dims)
    ws = B.alloc_workspace(d, T)
    got = B.route(d, torch.from_numpy(x).view(torch.int16).cuda(), torch.from_numpy(r).cuda(), ws)
    torch.cuda.synchronize()
    logits = oracle.router_logits(x, r)
    ids, w = oracle.topk(logits, dims["top_k"])
    off, sr = oracle.permute(ids, dims["n_experts"])
    assert np.array_equal(got["ids"].cpu().numpy(), ids)
    assert np.array_equal(got["offsets"].cpu().numpy(), off)
    assert np.array_equal(got["sorted"].cpu().numpy(), sr)
    assert np.allclose(got["w"].cpu().numpy(), w, rtol=1e-6, atol=0)
    ud = G.ulp_diff_f32(got["logits"].cpu().numpy(), logits)
    assert ud.max() <= 1 and (ud == 0).mean() >= 0.99
    # the ties really are exercised: some chosen experts have their twin chosen too
    assert any(len(set(row) & {e + 128 for e in row}) > 0 for row in ids.tolist())
    if T > 1:
        assert (ids[T - 1] == np.arange(8)).all()


# ---- the generation word of the in-launch routing -----------------------------------
@pytest.mark.parametrize("T", [1, 5])
def test_generation_word_advances_by_one_per_call(T):
    dims = dict(hidden=1024, latent=512, inter=512, n_experts=64, top_k=8)
    lay = synth.make_layer(dims, T, seed=80)
    dev = G.device_layer(lay)
    d = B.make_dims(lay.dims, lay.eps, lay.gain_per_expert)
    w = B.make_weights(dev)
    ws = B.alloc_workspace(d, T)
    ws.zero_()
    sync = B.workspace_view(d, T, ws, "sync", torch.int32, (64,))
    ref = G.oracle_full(lay, G.host_experts(dev))
    out = torch.empty((T, dims["hidden"]), dtype=torch.int16, device="cuda")
    gens = []
    for rep in range(4):
        B.latent_forward(d, dev["x"], w, out, ws)
        torch.cuda.synchronize()
        s = sync.cpu().numpy()
        gens.append(int(s[0]))
        assert s[1] == 0, "a router workgroup gave up waiting for the routing"
        assert np.array_equal(G.views(lay, d, ws, T)["ids"], ref["ids"])
    assert gens == [1, 2, 3, 4], gens
    G.assert_out_close(out.cpu().numpy(), ref["out"])


# ---- the route sum at widths off the real shape -----------------------------------------
@pytest.mark.parametrize("dims,T,nv,gpe", [
    (dict(hidden=512, latent=384, inter=256, n_experts=24, top_k=6), 2, False, True),   # 3 chunks: no K split
    (dict(hidden=512, latent=384, inter=256, n_experts=24, top_k=6), 1, True, False),   # NVFP4 one-row form
    (dict(hidden=640, latent=640, inter=384, n_experts=16, top_k=8), 2, False, False),   # a full 16-row fragment
    (dict(hidden=256, latent=256, inter=256, n_experts=32, top_k=1), 16, False, True),   # one route per token
    (dict(hidden=256, latent=256, inter=256, n_experts=32, top_k=3), 5, False, False)],  # tokens across lane groups
    ids=["l384_t2_gpe", "l384_t1_nvfp4", "l640_t2_16rows", "k1_t16", "k3_t5"])
def test_route_sum_odd_widths(dims, T, nv, gpe):
    """The post-norm and weighted sum in the unpooler's launch where the
    latent width is not a multiple of 512 (rows staged through registers,
    not copied straight to LDS), with an odd chunk count (no K split), per-
    expert gains, NVFP4 experts and 16 route rows: every stage against the
    oracle, the gain-scaled rows bit for bit against the route rows."""
    lay = synth.make_layer(dims, T, seed=87, gain_per_expert=gpe)
    dev = G.device_layer(lay, experts=synth.all_nvfp4_expert_bytes(lay.dims, 87, device="cuda") if nv else None)
    d = B.make_dims(lay.dims, lay.eps, lay.gain_per_expert, B.FMT_NVFP4 if nv else B.FMT_MXFP4)
    assert G.rows16_written(d, T)
    G.log(f"route sum dims={dims} T={T} nvfp4={nv} gpe={gpe}")
    ws = B.alloc_workspace(d, T)
    out = torch.empty((T, dims["hidden"]), dtype=torch.int16, device="cuda")
    B.latent_forward(d, dev["x"], B.make_weights(dev), out, ws)
    torch.cuda.synchronize()
    got = G.views(lay, d, ws, T)
    assert got["y"] is None
    names = synth.EXPERT_TENSORS + (("w13_global", "w2_global") if nv else ())
    ex = {k: dev[k].cpu().numpy() for k in names}
    kw = dict(fmt=oracle.NVFP4, w13_global=ex["w13_global"], w2_global=ex["w2_global"]) if nv else {}
    ref = oracle.latent_forward(lay.dims, lay.x, lay.router, lay.pooler, ex["w13_codes"], ex["w13_scales"],
                                ex["w2_codes"], ex["w2_scales"], lay.gain, lay.unpooler, lay.eps,
                                lay.gain_per_expert, **kw)
    assert np.array_equal(got["ids"], ref["ids"])
    h_ref, rows_ref = G.oracle_expert_rows(lay, ex, got["lat"], got["ids"], oracle.NVFP4 if nv else oracle.MXFP4)
    G.assert_h_elementwise(got["h"], h_ref[got["sorted"]])
    G.assert_rows_elementwise(got["rows"], rows_ref, 5e-3, "rows")
    G.assert_rows16_from_rows(got, lay.gain, lay.gain_per_expert)
    G.assert_route_sum_output(got, lay, out.cpu().numpy())
    G.assert_out_close(out.cpu().numpy(), ref["out"])


# ---- every route row written ----------------------------------------------------------
def _nan_fill(d, T, ws, I, L, K):
    B.workspace_view(d, T, ws, "h", torch.int16, (T * K, I)).fill_(0x7FC0)   # bf16 NaN
    B.workspace_view(d, T, ws, "rows", torch.float32, (T * K, L)).fill_(float("nan"))


def _routed_ids(counts, K, seed):
    """Expert ids with the given per-expert route counts, shuffled into [T][K]."""
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    np.random.default_rng(seed).shuffle(ids)
    return ids.reshape(-1, K)


@pytest.mark.parametrize("extra", [-2, 0, 2], ids=["below_pair_threshold", "at_pair_threshold",
                                                   "above_pair_threshold"])
def test_routed_tiles_of_one_to_four_every_row(extra):
    """Experts holding 1, 2, 3 and 4 row tiles of 128 (LDS-staged kernel) and
    12 experts with about 2 routes each: 2R just below E * 128, exactly
    there (from where the row tiles are listed with even-tile experts first)
    and just above.
    The h and route-row buffers start as NaN; every route row must be
    written, and every row equals the oracle's routed layer."""
    dims = dict(hidden=512, latent=512, inter=512, n_experts=16, top_k=2)
    counts = [400, 300, 200, 100] + [2] * 12
    counts[4] += extra
    ids = _routed_ids(counts, 2, seed=90 + extra)
    T = ids.shape[0]
    lay = synth.make_layer(dims, T, seed=91)
    dev = G.device_layer(lay)
    rng = np.random.default_rng(92)
    # (weights in [0.05, 0.3]: |y| stays below 4, where one bf16 ulp is within the 2e-2 bar)
    wts = rng.uniform(0.05, 0.3, ids.shape).astype(np.float32)
    d = B.make_dims(lay.dims, lay.eps, lay.gain_per_expert)
    ws = B.alloc_workspace(d, T)
    L, I, K = dims["latent"], dims["inter"], dims["top_k"]
    _nan_fill(d, T, ws, I, L, K)
    out = torch.empty((T, dims["hidden"]), dtype=torch.int16, device="cuda")
    G.log(f"routed T={T} R={T * K} counts={counts[:5]}")
    B.latent_forward_routed(d, dev["x"], torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda(),
                            B.make_weights(dev), out, ws)
    torch.cuda.synchronize()
    got = G.views(lay, d, ws, T)
    assert np.isfinite(got["rows"]).all()
    assert np.isfinite(G.bf16(got["h"])).all()
    ex = G.host_experts(dev)
    ref = oracle.latent_forward_routed(dims, lay.x, ids, wts, lay.pooler, ex["w13_codes"],
                                       ex["w13_scales"], ex["w2_codes"], ex["w2_scales"], lay.gain,
                                       lay.unpooler, lay.eps, lay.gain_per_expert)
    off, sr = oracle.permute(ids, dims["n_experts"])
    assert np.array_equal(got["offsets"], off) and np.array_equal(got["sorted"], sr)
    G.assert_latent_close(got["lat"], ref["lat"])
    G.assert_rel_close(got["rows"], ref["rows"], 1e-2, "rows")
    h_ref, rows_ref = G.oracle_expert_rows(lay, ex, got["lat"], ids)
    G.assert_h_elementwise(got["h"], h_ref[sr])
    G.assert_rows_elementwise(got["rows"], rows_ref, 5e-3, "rows")
    G.assert_y_or_rows16(got, lay, ref["ybf"])
    G.assert_out_close(out.cpu().numpy(), ref["out"])


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_routed_light_tiles_every_row(fmt):
    """Row tiles of at most 16 rows take the LDS-staged kernel's light ring
    (four slots of 16 activation rows, copies three stages ahead): experts
    with 1, 15, 16 and 17 routes, with 31, 32 and 33 (one or three
    fragments of 16 rows), and with 144 and 145 (a full tile and a 16- or
    17-row tail), beside a heavy one. h and the route rows start as NaN;
    every row is written and equals the oracle's routed layer."""
    dims = dict(hidden=512, latent=512, inter=512, n_experts=10, top_k=2)
    counts = [144, 145, 16, 17, 1, 15, 32, 33, 31, 250]
    ids = _routed_ids(counts, 2, seed=95)
    T = ids.shape[0]
    lay = synth.make_layer(dims, T, seed=96)
    nv = fmt == "nvfp4"
    dev = G.device_layer(lay, experts=synth.all_nvfp4_expert_bytes(lay.dims, 96, device="cuda") if nv else None)
    rng = np.random.default_rng(97)
    wts = rng.uniform(0.05, 0.3, ids.shape).astype(np.float32)
    d = B.make_dims(lay.dims, lay.eps, lay.gain_per_expert, B.FMT_NVFP4 if nv else B.FMT_MXFP4)
    ws = B.alloc_workspace(d, T)
    L, I, K = dims["latent"], dims["inter"], dims["top_k"]
    _nan_fill(d, T, ws, I, L, K)
    out = torch.empty((T, dims["hidden"]), dtype=torch.int16, device="cuda")
    G.log(f"routed light tiles {fmt} T={T} counts={counts}")
    B.latent_forward_routed(d, dev["x"], torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda(),
                            B.make_weights(dev), out, ws)
    torch.cuda.synchronize()
    got = G.views(lay, d, ws, T)
    assert np.isfinite(got["rows"]).all()
    assert np.isfinite(G.bf16(got["h"])).all()
    names = synth.EXPERT_TENSORS + (("w13_global", "w2_global") if nv else ())
    ex = {k: dev[k].cpu().numpy() for k in names}
    kw = dict(fmt=oracle.NVFP4, w13_global=ex["w13_global"], w2_global=ex["w2_global"]) if nv else {}
    ref = oracle.latent_forward_routed(dims, lay.x, ids, wts, lay.pooler, ex["w13_codes"],
                                       ex["w13_scales"], ex["w2_codes"], ex["w2_scales"], lay.gain,
                                       lay.unpooler, lay.eps, lay.gain_per_expert, **kw)
    off, sr = oracle.permute(ids, dims["n_experts"])
    assert np.array_equal(got["offsets"], off) and np.array_equal(got["sorted"], sr)
    G.assert_latent_close(got["lat"], ref["lat"])
    h_ref, rows_ref = G.oracle_expert_rows(lay, ex, got["lat"], ids, oracle.NVFP4 if nv else oracle.MXFP4)
    G.assert_h_elementwise(got["h"], h_ref[sr])
    G.assert_rows_elementwise(got["rows"], rows_ref, 5e-3, "rows")
    G.assert_y_or_rows16(got, lay, ref["ybf"])
    G.assert_out_close(out.cpu().numpy(), ref["out"])


def _expert_rows_check(lay, dev, got, experts):
    """Every route row of the given experts against oracle.expert_row fed
    with the GPU's latent rows: h (grouped order) and the fp32 rows."""
    K = lay.dims["top_k"]
    sr, off = got["sorted"], got["offsets"]
    jobs = []
    for e in experts:
        wt = tuple(dev[k][e].cpu().numpy() for k in synth.EXPERT_TENSORS)
        for i in range(off[e], off[e + 1]):
            jobs.append((e, i, int(sr[i]), wt))
    G.log(f"  {len(jobs)} route rows of experts {list(experts)}")
    fn = lambda j: oracle.expert_row(got["lat"][j[2] // K], *j[3])
    with ThreadPoolExecutor(G.HOST_WORKERS) as ex:
        res = list(ex.map(fn, jobs))
    h_ref = np.stack([r[0] for r in res])
    rows_ref = np.stack([r[1] for r in res])
    G.assert_h_elementwise(got["h"][[j[1] for j in jobs]], h_ref, "h")
    G.assert_rows_elementwise(got["rows"][[j[2] for j in jobs]], rows_ref, 5e-3, "rows")
    G.assert_rel_close(got["rows"][[j[2] for j in jobs]], rows_ref, 1e-3, "rows")


@pytest.mark.parametrize("cfg", [3, 4], ids=["prefill_t4096", "skewed_t512"])
def test_most_loaded_experts_every_row_real_shape(cfg, real_experts):
    """The three most-loaded experts' route rows (full, partial and, skewed,
    several-tile row tiles), with h and rows pre-filled with NaN: every route
    row of the call is written, and those experts' rows match the oracle
    element by element."""
    lay = synth.config_layer(cfg)
    dev = G.device_layer(lay, real_experts)
    d = B.make_dims(lay.dims, lay.eps, lay.gain_per_expert)
    T, L, I, K = lay.T, lay.dims["latent"], lay.dims["inter"], lay.dims["top_k"]
    ws = B.alloc_workspace(d, T)
    _nan_fill(d, T, ws, I, L, K)
    out = torch.empty((T, lay.dims["hidden"]), dtype=torch.int16, device="cuda")
    G.log(f"config {cfg} T={T}")
    B.latent_forward(d, dev["x"], B.make_weights(dev), out, ws)
    torch.cuda.synchronize()
    rows_dev = B.workspace_view(d, T, ws, "rows", torch.float32, (T * K, L))
    assert bool(torch.isfinite(rows_dev).all())
    got = G.views(lay, d, ws, T)
    counts = np.diff(got["offsets"])
    top = np.argsort(-counts, kind="stable")[:3]
    G.log(f"  most-loaded experts {top.tolist()} with {counts[top].tolist()} routes")
    _expert_rows_check(lay, dev, got, top)


# ---- NVFP4 at the real shape --------------------------------------------------------
@pytest.fixture(scope="module")
def real_nvfp4_experts():
    G.log("generating real-shape NVFP4 expert bytes on the device")
    ex = synth.all_nvfp4_expert_bytes(synth.REAL, 0, device="cuda")
    torch.cuda.synchronize()
    return ex


@pytest.mark.parametrize("cfg,tokens", [(1, [0]), (2, [0, 13, 31]), (3, [0, 2048, 4095])],
                         ids=["decode_t1", "verify_t32", "prefill_t4096"])
def test_nvfp4_real_shape(cfg, tokens, real_nvfp4_experts):
    lay = synth.config_layer(cfg)
    dev = G.device_layer(lay, real_nvfp4_experts)
    d = B.make_dims(lay.dims, lay.eps, lay.gain_per_expert, B.FMT_NVFP4)
    T, K = lay.T, lay.dims["top_k"]
    ws = B.alloc_workspace(d, T)
    out = torch.empty((T, lay.dims["hidden"]), dtype=torch.int16, device="cuda")
    G.log(f"NVFP4 config {cfg} T={T}")
    B.latent_forward(d, dev["x"], B.make_weights(dev), out, ws)
    torch.cuda.synchronize()
    got = G.views(lay, d, ws, T)
    refs = G.oracle_tokens(lay, dev, tokens, fmt=oracle.NVFP4)
    out_np = out.cpu().numpy()
    touched = np.unique(got["ids"][tokens])
    ex = {k: {int(e): dev[k][int(e)].cpu().numpy() for e in touched}
          for k in synth.EXPERT_TENSORS + ("w13_global", "w2_global")}
    for t, ref in zip(tokens, refs):
        assert np.array_equal(got["ids"][t], ref["ids"])
        G.assert_latent_close(got["lat"][t], ref["lat"])
        G.assert_rel_close(got["rows"][t * K:(t + 1) * K], ref["rows"], 1e-2, f"rows t={t}")
        routes = [t * K + k for k in range(K)]
        h_ref, rows_ref = G.oracle_expert_rows(lay, ex, got["lat"], got["ids"], oracle.NVFP4, routes)
        mine = [int(np.nonzero(got["sorted"] == r)[0][0]) for r in routes]
        G.assert_h_elementwise(got["h"][mine], h_ref, f"h t={t}")
        G.assert_rows_elementwise(got["rows"][routes], rows_ref, 5e-3, f"rows t={t}")
        G.assert_y_or_rows16(got, lay, ref["ybf"], f"y t={t}", t, out_np)
        G.assert_out_close(out_np[t], ref["out"], f"out t={t}")
