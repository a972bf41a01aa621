"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Routing ids, expert offsets and the route permutation must match bit for bit;
router logits within one fp32 ulp; weights within 1e-6 relative; the layer
output within max |delta| <= 2e-2 and relative RMS <= 1e-2 (bf16).
Intermediates are read from the workspace (moe_workspace_view)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from latent_mixture_experts_amd import binding as B
from latent_mixture_experts_amd import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _check_all_stages(lay, got, ref, dev=None, ex_host=None, fmt=oracle.MXFP4, rows_elem=5e-3, out_bits=None):
    T, K = lay.T, lay.dims["top_k"]
    # A1: logits, fp32 rounding of an fp64 sum on both sides
    ud = G.ulp_diff_f32(got["logits"], ref["logits"])
    assert ud.max() <= 1 and (ud == 0).mean() >= 0.999
    # A2: ids bit-exact, weights to 1e-6 relative
    assert np.array_equal(got["ids"], ref["ids"])
    assert np.allclose(got["w"], ref["w"], rtol=1e-6, atol=0)
    # A3: permutation bit-exact (against the oracle's own grouping)
    off, sr = oracle.permute(ref["ids"], lay.dims["n_experts"])
    assert np.array_equal(got["offsets"], off) and np.array_equal(got["sorted"], sr)
    # A4: latent rows, bf16 rounding of fp32 vs fp64 sums
    G.assert_latent_close(got["lat"], ref["lat"])
    # A5: h in sorted order vs the oracle's route-major h
    G.assert_rel_close(G.bf16(got["h"]), G.bf16(ref["h"][got["sorted"]]), 1e-2, "h")
    # A6: fp32 route rows, route-major
    G.assert_rel_close(got["rows"], ref["rows"], 1e-2, "rows")
    # A5 and A6 element by element, from the GPU's own latent rows
    if ex_host is not None:
        h_ref, rows_ref = G.oracle_expert_rows(lay, ex_host, got["lat"], got["ids"], fmt)
        G.assert_h_elementwise(got["h"], h_ref[got["sorted"]])
        G.assert_rows_elementwise(got["rows"], rows_ref, rows_elem, "rows")
    # A7: normed weighted sum; for few route rows it is taken after the
    # unpooler's products, from the gain-scaled bf16 route rows (then checked
    # against the route rows bit for bit, and through the output)
    if got["y"] is not None:
        G.assert_out_close(got["y"], ref["ybf"], "y")
    else:
        G.assert_rows16_from_rows(got, lay.gain, lay.gain_per_expert)
        if out_bits is not None:
            G.assert_route_sum_output(got, lay, out_bits)


def _run_and_compare(lay):
    G.log(f"dims={lay.dims} T={lay.T} gain_per_expert={lay.gain_per_expert}")
    dev = G.device_layer(lay)
    out, d, ws = G.run_gpu(lay, dev)
    got = G.views(lay, d, ws, lay.T)
    ex = G.host_experts(dev)
    ref = G.oracle_full(lay, ex)
    _check_all_stages(lay, got, ref, ex_host=ex, out_bits=out.cpu().numpy())
    G.assert_out_close(out.cpu().numpy(), ref["out"])
    return out, ref


@pytest.mark.parametrize("gain_per_expert", [False, True])
def test_tiny_config_all_stages(gain_per_expert):
    _run_and_compare(synth.config_layer(0, gain_per_expert=gain_per_expert))


SHAPES = [
    # several tiles in every dimension, ragged token count
    (dict(hidden=512, latent=384, inter=256, n_experts=24, top_k=6), 45, 0.02),
    # many rows per expert (several 16-row passes), ragged
    (dict(hidden=256, latent=256, inter=384, n_experts=8, top_k=2), 100, 0.02),
    # all 256 experts, K = 8, one token past a 32-row block
    (dict(hidden=384, latent=128, inter=128, n_experts=256, top_k=8), 33, 0.02),
    # K = E: every expert is used by every token
    (dict(hidden=256, latent=128, inter=256, n_experts=5, top_k=5), 3, 0.02),
    # a single token
    (dict(hidden=1024, latent=512, inter=512, n_experts=64, top_k=8), 1, 0.02),
    # prefill regime (tiled kernels): ragged 128-row tiles, tails of 1..127 rows
    (dict(hidden=512, latent=512, inter=256, n_experts=8, top_k=2), 300, 0.02),
    # prefill regime, experts with more than one 128-row tile
    (dict(hidden=256, latent=256, inter=256, n_experts=4, top_k=2), 400, 0.02),
    # prefill regime with few tokens (tiny expert count)
    (dict(hidden=256, latent=256, inter=256, n_experts=4, top_k=4), 16, 0.02),
    # LDS-staged expert tiles (128 rows): a full tile and a 22-row tile per
    # expert (its second wavefront row has no rows), K = 512 and 1024
    (dict(hidden=512, latent=512, inter=1024, n_experts=8, top_k=2), 600, 0.02),
    # one partial 128-row tile per expert, K = 512
    (dict(hidden=1024, latent=512, inter=512, n_experts=4, top_k=4), 100, 0.02),
    # 24 tokens: the pooler on the LDS-staged dense kernel with a 16-way K
    # split (16 column tiles of one row tile), the unpooler on the
    # register-staged tiles
    (dict(hidden=1024, latent=4096, inter=256, n_experts=8, top_k=2), 24, 0.02),
]


@pytest.mark.parametrize("dims,T,rstd", SHAPES, ids=[f"T{s[1]}_E{s[0]['n_experts']}" for s in SHAPES])
def test_reduced_shapes(dims, T, rstd):
    _run_and_compare(synth.make_layer(dims, T, seed=3, router_std=rstd, gain_per_expert=T % 2 == 1))


def test_route_entry_point_with_ties():
    """moe_route alone: duplicated router rows give exactly tied logits, which
    must go to the lower expert id; all-zero router rows tie every expert."""
    dims = dict(hidden=512, latent=128, inter=128, n_experts=40, top_k=8)
    lay = synth.make_layer(dims, 50, seed=5)
    r = lay.router.copy()
    r[20:40] = r[0:20]            # experts e and e+20 tie for every token
    r[10:20] = 0.0                # ten experts at logit exactly 0
    x = lay.x.copy()
    x[:5] = 0                     # five tokens with every logit 0
    d = B.make_dims(dims)
    ws = B.alloc_workspace(d, lay.T)
    got = B.route(d, torch.from_numpy(x).view(torch.int16).cuda(), torch.from_numpy(r).cuda(), ws)
    torch.cuda.synchronize()
    logits = oracle.router_logits(x, r)
    ids, w = oracle.topk(logits, dims["top_k"])
    off, sr = oracle.permute(ids, dims["n_experts"])
    assert np.array_equal(got["ids"].cpu().numpy(), ids)
    assert np.array_equal(got["offsets"].cpu().numpy(), off)
    assert np.array_equal(got["sorted"].cpu().numpy(), sr)
    assert np.allclose(got["w"].cpu().numpy(), w, rtol=1e-6, atol=0)
    assert G.ulp_diff_f32(got["logits"].cpu().numpy(), logits).max() <= 1
    assert (ids[:5] == np.arange(8)).all()


def test_deterministic_across_runs():
    lay = synth.make_layer(SHAPES[0][0], 45, seed=9)
    dev = G.device_layer(lay)
    o1, d, ws1 = G.run_gpu(lay, dev)
    v1 = G.views(lay, d, ws1, lay.T)
    o2, _, ws2 = G.run_gpu(lay, dev)
    v2 = G.views(lay, d, ws2, lay.T)
    for k in ("ids", "offsets", "sorted", "logits", "w"):
        assert np.array_equal(v1[k], v2[k]), k
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("fill", ["zeros", "ones", "random", "stale"])
def test_routing_in_router_launch_independent_of_workspace(fill):
    """For T <= 8 the router workgroups also take the top K and group the
    routes (their logits carry a tag derived from a generation word in the
    workspace; every workgroup that finds all tags routes, writing the
    same values).
    Whatever the workspace held before (zero bytes, 0xFF bytes, random
    bytes, or a previous call's words for other tokens), a call routes
    exactly as the oracle, and calls in a row on one workspace each route
    their own tokens."""
    for dims, T in ((SHAPES[0][0], 1), (SHAPES[3][0], 3), (SHAPES[2][0], 8), (SHAPES[4][0], 1)):
        G.log(f"fill={fill} dims={dims} T={T}")
        lay = synth.make_layer(dims, T, seed=31)
        dev = G.device_layer(lay)
        d = B.make_dims(lay.dims, lay.eps, lay.gain_per_expert)
        w = B.make_weights(dev)
        ws = B.alloc_workspace(d, T)
        if fill == "zeros":
            ws.zero_()
        elif fill == "ones":
            ws.fill_(255)
        elif fill == "random":
            g = torch.Generator(device="cpu").manual_seed(T)
            ws.copy_(torch.randint(0, 256, ws.shape, generator=g, dtype=torch.uint8))
        else:  # a call with other tokens first
            other = synth.make_layer(dims, T, seed=31, token_set=1)
            x_other = torch.from_numpy(other.x).view(torch.int16).cuda()
            B.latent_forward(d, x_other, w, torch.empty((T, dims["hidden"]), dtype=torch.int16,
                                                        device="cuda"), ws)
        ref = G.oracle_full(lay, G.host_experts(dev))
        for rep in range(3):  # calls in a row on the same workspace
            out = torch.empty((T, dims["hidden"]), dtype=torch.int16, device="cuda")
            B.latent_forward(d, dev["x"], w, out, ws)
            torch.cuda.synchronize()
            got = G.views(lay, d, ws, T)
            assert np.array_equal(got["ids"], ref["ids"]), (fill, T, rep)
            off, sr = oracle.permute(ref["ids"], dims["n_experts"])
            assert np.array_equal(got["offsets"], off) and np.array_equal(got["sorted"], sr)
            G.assert_out_close(out.cpu().numpy(), ref["out"])


def test_routing_on_one_workspace_across_token_counts():
    """One workspace (sized for 16 tokens) used by calls with T = 8, 1, 16,
    3, 1 in a row: calls with T <= 8 route inside the router launch (tagged
    logits placed after the generation word, where a call with another T
    keeps other data), T = 16 routes in its own launch. Each call routes its
    own tokens exactly as the oracle."""
    dims = SHAPES[2][0]  # E = 256, K = 8
    lay16 = synth.make_layer(dims, 16, seed=41)
    dev = G.device_layer(lay16)
    d = B.make_dims(lay16.dims, lay16.eps, lay16.gain_per_expert)
    w = B.make_weights(dev)
    ws = B.alloc_workspace(d, 16)
    ex = G.host_experts(dev)
    for T, token_set in ((8, 1), (1, 2), (16, 3), (3, 4), (1, 5)):
        lay = synth.make_layer(dims, T, seed=41, token_set=token_set)
        G.log(f"T={T} token_set={token_set}")
        x = torch.from_numpy(lay.x).view(torch.int16).cuda()
        out = torch.empty((T, dims["hidden"]), dtype=torch.int16, device="cuda")
        B.latent_forward(d, x, w, out, ws)
        torch.cuda.synchronize()
        got = G.views(lay, d, ws, T)
        ref = G.oracle_full(lay, ex)
        assert np.array_equal(got["ids"], ref["ids"]), T
        off, sr = oracle.permute(ref["ids"], dims["n_experts"])
        assert np.array_equal(got["offsets"], off) and np.array_equal(got["sorted"], sr), T
        G.assert_out_close(out.cpu().numpy(), ref["out"])


def test_dense_projection_split_over_k():
    """A prefill pooler with too few 128 x 256 tiles to fill the GPU (2 x 16
    here) runs with K split eight ways, fp32 partial sums in the workspace
    and an in-order sum: every stage against the oracle. (Top-8 routing as
    in the real shape keeps |y| below 4, where one bf16 ulp is 0.03.)"""
    dims = dict(hidden=1024, latent=4096, inter=128, n_experts=16, top_k=8)
    lay = synth.make_layer(dims, 160, seed=61)
    _run_and_compare(lay)


def test_zero_tokens_is_a_no_op():
    lay = synth.config_layer(0)
    dev = G.device_layer(lay)
    d = B.make_dims(lay.dims)
    out = torch.full((1, lay.dims["hidden"]), 7, dtype=torch.int16, device="cuda")
    ws = B.alloc_workspace(d, 1)
    B.latent_forward(d, dev["x"][:0], B.make_weights(dev), out, ws)
    torch.cuda.synchronize()
    assert (out == 7).all()


def test_output_invariant_to_expert_output_scale():
    """The post-expert norm removes a power-of-two scale on W2: doubling every
    W2 scale leaves the output unchanged (up to eps), on the GPU alone."""
    lay = synth.make_layer(SHAPES[0][0], 45, seed=4)
    dev = G.device_layer(lay)
    o1, _, _ = G.run_gpu(lay, dev)
    dev2 = dict(dev)
    dev2["w2_scales"] = dev["w2_scales"] + 1
    o2, _, _ = G.run_gpu(lay, dev2)
    d = np.abs(G.bf16(o1.cpu().numpy()) - G.bf16(o2.cpu().numpy()))
    assert d.max() <= 1e-2 and (d == 0).mean() > 0.99


def test_generator_same_bytes_on_cpu_and_gpu():
    dims = synth.REAL
    for name in synth.EXPERT_TENSORS:
        a = synth.expert_bytes(dims, 0, name, [0, 77, 255], device="cpu")
        b = synth.expert_bytes(dims, 0, name, [0, 77, 255], device="cuda").cpu()
        assert torch.equal(a, b), name


# ---- full-size workloads ----------------------------------------------------------
FULL = {1: [0], 2: [0, 13, 31], 3: [0, 1337, 4095], 4: [0, 200, 511]}


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_full_size_config(cfg, real_experts):
    lay = synth.config_layer(cfg)
    G.log(f"config {cfg}: T={lay.T}")
    dev = G.device_layer(lay, real_experts)
    out, d, ws = G.run_gpu(lay, dev)
    got = G.views(lay, d, ws, lay.T)
    G.log("  oracle router on all tokens")
    logits, ids, w = G.oracle_router_all(lay)
    ud = G.ulp_diff_f32(got["logits"], logits)
    assert ud.max() <= 1 and (ud == 0).mean() >= 0.999
    assert np.array_equal(got["ids"], ids)
    assert np.allclose(got["w"], w, rtol=1e-6, atol=0)
    off, sr = oracle.permute(ids, lay.dims["n_experts"])
    assert np.array_equal(got["offsets"], off) and np.array_equal(got["sorted"], sr)
    G.log(f"  oracle layer on tokens {FULL[cfg]}")
    refs = G.oracle_tokens(lay, dev, FULL[cfg])
    out_np = out.cpu().numpy()
    K = lay.dims["top_k"]
    touched = np.unique(ids[FULL[cfg]])
    ex = {k: {int(e): dev[k][int(e)].cpu().numpy() for e in touched} for k in synth.EXPERT_TENSORS}
    routes = [t * K + k for t in FULL[cfg] for k in range(K)]
    h_ref, rows_ref = G.oracle_expert_rows(lay, ex, got["lat"], ids, routes=routes)
    pos = np.argsort(got["sorted"])  # sorted position of each route
    G.assert_h_elementwise(got["h"][pos[routes]], h_ref)
    G.assert_rows_elementwise(got["rows"][routes], rows_ref, 5e-3, "rows")
    for t, ref in zip(FULL[cfg], refs):
        assert np.array_equal(ref["ids"], ids[t])
        G.assert_latent_close(got["lat"][t], ref["lat"])
        G.assert_rel_close(got["rows"][t * K:(t + 1) * K], ref["rows"], 1e-2, f"rows t={t}")
        G.assert_y_or_rows16(got, lay, ref["ybf"], f"y t={t}", t, out_np)
        G.assert_out_close(out_np[t], ref["out"], f"out t={t}")


def test_maximum_token_count(real_experts):
    """The largest T the boundary accepts at the real shape (h takes just
    under 2^31 bytes): routing of sampled tokens (the last ones included)
    against the oracle, the grouping of all routes, and the layer on tokens
    at the start, middle and end, whose rows sit at the highest offsets."""
    T = 32767
    lay = synth.make_layer(synth.REAL, T, seed=0, router_std=synth.CONFIGS[3]["router_std"])
    G.log(f"T={T}")
    dev = G.device_layer(lay, real_experts)
    out, d, ws = G.run_gpu(lay, dev)
    K, E, L = lay.dims["top_k"], lay.dims["n_experts"], lay.dims["latent"]
    view = lambda name, dt, shape: B.workspace_view(d, T, ws, name, dt, shape)
    ids = view("ids", torch.int32, (T, K)).cpu().numpy()
    sample = np.unique(np.r_[np.arange(0, T, 257), T - 3, T - 2, T - 1])
    logits = oracle.router_logits(lay.x[sample], lay.router)
    want, _ = oracle.topk(logits, K)
    assert np.array_equal(ids[sample], want)
    off, sr = oracle.permute(ids, E)
    assert np.array_equal(view("offsets", torch.int32, (E + 1,)).cpu().numpy(), off)
    assert np.array_equal(view("sorted", torch.int32, (T * K,)).cpu().numpy(), sr)
    toks = [0, T // 2, T - 1]
    refs = G.oracle_tokens(lay, dev, toks)
    rows = view("rows", torch.float32, (T * K, L))
    lat = view("latent", torch.int16, (T, L))
    y = view("y", torch.int16, (T, L))
    for t, ref in zip(toks, refs):
        G.assert_latent_close(lat[t].cpu().numpy().view(np.uint16), ref["lat"])
        G.assert_rel_close(rows[t * K:(t + 1) * K].cpu().numpy(), ref["rows"], 1e-2, f"rows t={t}")
        G.assert_out_close(y[t].cpu().numpy().view(np.uint16), ref["ybf"], f"y t={t}")
        G.assert_out_close(out[t].cpu().numpy(), ref["out"], f"out t={t}")


@pytest.mark.parametrize("T", [3, 40])
def test_timed_entry_point_matches_and_records_every_step(T):
    """moe_latent_forward_timed: same output as moe_latent_forward, and every
    step's start/stop events are recorded (small-T and large-T routing)."""
    dims = SHAPES[0][0]
    lay = synth.make_layer(dims, T, seed=6)
    dev = G.device_layer(lay)
    o1, d, ws = G.run_gpu(lay, dev)
    evs = B.create_events(2 * B.N_STAGES)
    o2 = torch.empty_like(o1)
    B.latent_forward(d, dev["x"], B.make_weights(dev), o2, ws, events=evs)
    torch.cuda.synchronize()
    times = [B.elapsed_ms(evs[2 * s], evs[2 * s + 1]) for s in range(B.N_STAGES)]
    B.destroy_events(evs)
    assert torch.equal(o1, o2)
    assert all(t >= 0.0 for t in times), times


@pytest.mark.parametrize("dims,T", [(SHAPES[4][0], 1), (SHAPES[0][0], 3), (SHAPES[6][0], 400), (SHAPES[8][0], 600)],
                         ids=["one_token_route_sum", "few_tokens", "tiled", "lds_tiles"])
def test_graph_capture_replays_match_eager(dims, T):
    """moe_latent_forward captured into a HIP graph: every replay, with eager
    work and synchronizations in between and new token values copied into the
    captured input, gives the eager result bit for bit (the library
    enqueues kernels only: no allocation, memset or host synchronization)."""
    lay = synth.make_layer(dims, T, seed=8)
    dev = G.device_layer(lay)
    d = B.make_dims(lay.dims, lay.eps, lay.gain_per_expert)
    w = B.make_weights(dev)
    ws = B.alloc_workspace(d, T)
    xs = [dev["x"]] + [torch.from_numpy(synth.make_layer(dims, T, seed=8, token_set=s).x)
                       .view(torch.int16).cuda() for s in (1, 2)]
    x_static = xs[0].clone()
    out_static = torch.empty((T, dims["hidden"]), dtype=torch.int16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        B.latent_forward(d, x_static, w, out_static, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.latent_forward(d, x_static, w, out_static, ws)
    torch.cuda.synchronize()
    for rep in range(6):
        x = xs[rep % len(xs)]
        x_static.copy_(x)
        graph.replay()
        torch.cuda.synchronize()
        got = out_static.clone()
        eager = torch.empty_like(out_static)
        ws2 = B.alloc_workspace(d, T)
        B.latent_forward(d, x, w, eager, ws2)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(got, eager), f"replay {rep}"
