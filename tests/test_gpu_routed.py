"""moe_latent_forward_routed (routing replay) through the C ABI.

Replaying the router's own choice reproduces moe_latent_forward bit for bit;
any other routing (repeated experts within a token, unsorted ids, weights
that do not sum to one) is compared with the oracle's routed layer: the
grouping bit for bit, the output within max |delta| <= 2e-2 and relative
RMS <= 1e-2 (bf16)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from latent_mixture_experts_amd import binding as B
from latent_mixture_experts_amd import synth
from tests import gpu_util as G
from tests.test_gpu_parity import SHAPES

pytestmark = pytest.mark.gpu

# few tokens (streaming kernels), one token, tiled, LDS-tiled; more than
# 6144 routes, grouped by several workgroups in chunks of 2048 (6400 routes
# over 256 experts, the last chunk ragged; 6400 routes over 4 experts, many
# row tiles per expert, and an unpooler whose 52 tiles do not fill whole
# groups of the tile order)
CASES = [(SHAPES[0][0], 3), (SHAPES[4][0], 1), (SHAPES[6][0], 400), (SHAPES[8][0], 600),
         (SHAPES[2][0], 800), (SHAPES[9][0], 1600)]
CASE_IDS = ["few_tokens", "one_token", "tiled", "lds_tiles", "chunks_256_experts",
            "chunks_4_experts"]


def _routed_gpu(lay, dev, ids, w):
    d = B.make_dims(lay.dims, lay.eps, lay.gain_per_expert)
    ws = B.alloc_workspace(d, lay.T)
    out = torch.empty((lay.T, lay.dims["hidden"]), dtype=torch.int16, device="cuda")
    B.latent_forward_routed(d, dev["x"], torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda(),
                            torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda(),
                            B.make_weights(dev), out, ws)
    torch.cuda.synchronize()
    return out, d, ws


@pytest.mark.parametrize("dims,T", CASES, ids=CASE_IDS)
def test_replay_of_the_router_choice_is_bit_identical(dims, T):
    lay = synth.make_layer(dims, T, seed=11, gain_per_expert=True)
    G.log(f"dims={dims} T={T}")
    dev = G.device_layer(lay)
    out, d, ws = G.run_gpu(lay, dev)
    v = G.views(lay, d, ws, T)
    out2, _, ws2 = _routed_gpu(lay, dev, v["ids"], v["w"])
    v2 = G.views(lay, d, ws2, T)
    assert torch.equal(out, out2)
    for k in ("ids", "offsets", "sorted"):
        assert np.array_equal(v[k], v2[k]), k


def _arbitrary_routing(lay, seed):
    """Random ids with some tokens repeating an expert and a third of all
    routes on expert 0 (uneven groups). Weights are random, scaled to sum to
    0.9 per token: not one, and at the scale of router weights, which the
    absolute output bar assumes (outputs of order one)."""
    T, K, E = lay.T, lay.dims["top_k"], lay.dims["n_experts"]
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, (T, K)).astype(np.int32)
    ids[rng.random((T, K)) < 0.33] = 0
    if K > 1:
        ids[::3, 1] = ids[::3, 0]
    w = rng.uniform(0.05, 1.0, (T, K))
    w = (0.9 * w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


@pytest.mark.parametrize("dims,T", [(synth.CONFIGS[0]["dims"], 4)] + CASES,
                         ids=["tiny"] + CASE_IDS)
def test_arbitrary_routing_matches_oracle(dims, T):
    lay = synth.make_layer(dims, T, seed=12, gain_per_expert=T % 2 == 0)
    G.log(f"dims={dims} T={T}")
    dev = G.device_layer(lay)
    ids, w = _arbitrary_routing(lay, 13)
    out, d, ws = _routed_gpu(lay, dev, ids, w)
    got = G.views(lay, d, ws, T)
    ex = G.host_experts(dev)
    ref = oracle.latent_forward_routed(lay.dims, lay.x, ids, w, lay.pooler, ex["w13_codes"],
                                       ex["w13_scales"], ex["w2_codes"], ex["w2_scales"], lay.gain,
                                       lay.unpooler, lay.eps, lay.gain_per_expert)
    off, sr = oracle.permute(ids, lay.dims["n_experts"])
    assert np.array_equal(got["ids"], ids)
    assert np.array_equal(got["offsets"], off) and np.array_equal(got["sorted"], sr)
    G.assert_latent_close(got["lat"], ref["lat"])
    G.assert_rel_close(G.bf16(got["h"]), G.bf16(ref["h"][got["sorted"]]), 1e-2, "h")
    G.assert_rel_close(got["rows"], ref["rows"], 1e-2, "rows")
    G.assert_y_or_rows16(got, lay, ref["ybf"])
    G.assert_out_close(out.cpu().numpy(), ref["out"])


@pytest.mark.parametrize("dims,T", [(SHAPES[0][0], 9), (SHAPES[2][0], 800)],
                         ids=["one_workgroup", "chunks"])
def test_out_of_range_ids_are_clamped(dims, T):
    """Ids outside [0, E) are clamped into range (documented as unspecified
    results, but with no access outside the weights): the call equals the
    same call with the clamped ids."""
    G.log(f"dims={dims} T={T}")
    lay = synth.make_layer(dims, T, seed=14)
    dev = G.device_layer(lay)
    E, K = dims["n_experts"], dims["top_k"]
    ids, w = _arbitrary_routing(lay, 15)
    bad = ids.copy()
    bad[0, 0], bad[2, 1], bad[5, 3] = -3, E + 7, np.iinfo(np.int32).max
    o1, d, ws1 = _routed_gpu(lay, dev, bad, w)
    o2, _, ws2 = _routed_gpu(lay, dev, np.clip(bad, 0, E - 1), w)
    assert torch.equal(o1, o2)
    assert np.array_equal(G.views(lay, d, ws1, T)["ids"], np.clip(bad, 0, E - 1))


@pytest.mark.parametrize("which", ["first", "last"])
def test_every_route_on_one_expert(which):
    """6400 routes (the grouping over several workgroups) all on expert 0 or
    all on expert E-1: one touched expert holds every row (400 passes of 16
    rows in the streaming expert kernels), every other work-list entry is
    unused. Grouping bit for bit, output against the oracle."""
    dims, T = SHAPES[2][0], 800
    G.log(f"dims={dims} T={T} expert={which}")
    lay = synth.make_layer(dims, T, seed=16)
    dev = G.device_layer(lay)
    E, K = dims["n_experts"], dims["top_k"]
    ids = np.full((T, K), 0 if which == "first" else E - 1, np.int32)
    w = np.full((T, K), 0.9 / K, np.float32)
    out, d, ws = _routed_gpu(lay, dev, ids, w)
    got = G.views(lay, d, ws, T)
    off, sr = oracle.permute(ids, E)
    assert np.array_equal(got["offsets"], off) and np.array_equal(got["sorted"], sr)
    ex = G.host_experts(dev)
    ref = oracle.latent_forward_routed(lay.dims, lay.x, ids, w, lay.pooler, ex["w13_codes"],
                                       ex["w13_scales"], ex["w2_codes"], ex["w2_scales"], lay.gain,
                                       lay.unpooler, lay.eps, lay.gain_per_expert)
    G.assert_rel_close(got["rows"], ref["rows"], 1e-2, "rows")
    G.assert_out_close(out.cpu().numpy(), ref["out"])
