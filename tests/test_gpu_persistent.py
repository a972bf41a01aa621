"""The persistent decode layer (moe_latent_forward_persistent: the whole
layer for one or two tokens in one launch, its phases separated by barriers
between its workgroups) through the C ABI.

At T = 1 every phase runs the per-step kernels' bodies with the same K
splits and weight stages (with few route rows both take the post-norm and
the weighted sum in the unpooler's phase), so the output and every
intermediate equal moe_latent_forward's bit for bit; at T = 2 the split of
one projection differs, and the output is held to the oracle's bar.
Routing is bit-exact against the oracle in both. The status word shows no wait that gave up,
the generation word advances by one per call, calls in a row on one
workspace each route their own tokens, and graph replays equal the eager
result."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from latent_mixture_experts_amd import binding as B
from latent_mixture_experts_amd import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

# the smallest shape the phases are compiled for (hidden and latent multiples
# of 4096 or 2048 as the real shape's, inter a multiple of 2048)
DIMS = dict(hidden=2048, latent=4096, inter=2048, n_experts=64, top_k=8)


def _sync(d, T, ws):
    return B.workspace_view(d, T, ws, "sync", torch.int32, (64,))


def _persistent(d, x, w, ws, H):
    out = torch.full((x.shape[0], H), 7, dtype=torch.int16, device="cuda")
    B.latent_forward_persistent(d, x, w, out, ws)
    torch.cuda.synchronize()
    s = _sync(d, x.shape[0], ws).cpu().numpy()
    # status bits: 2 a wait gave up, 4 routing flag, 8 release, 16 logits; word 3 the
    # workgroup count
    us = lambda v: [round(((int(t) - int(s[16])) & 0xFFFFFFFF) / 100.0, 1) for t in v]  # 100 MHz
    assert s[1] & 2 == 0, (f"status {s[1]:#x} workgroups {s[3]}; us from workgroup "
                           f"0's start: routing, barriers 1-4 released {us(s[8:13])}; workgroup 0's "
                           f"phases 1-5 ended {us(s[17:22])}")
    return out


def _status(d, T, ws):
    return _sync(d, T, ws).cpu().numpy()


@pytest.mark.parametrize("T", [1, 2])
def test_persistent_matches_oracle_reduced_shape(T):
    lay = synth.make_layer(DIMS, T, seed=111, gain_per_expert=T == 2)
    G.log(f"persistent dims={DIMS} T={T}")
    dev = G.device_layer(lay)
    d = B.make_dims(lay.dims, lay.eps, lay.gain_per_expert)
    ws = B.alloc_workspace(d, T)
    _sync(d, T, ws).zero_()
    out = _persistent(d, dev["x"], B.make_weights(dev), ws, DIMS["hidden"])
    assert _status(d, T, ws)[1] == 0
    got = G.views(lay, d, ws, T)
    ex = G.host_experts(dev)
    ref = G.oracle_full(lay, ex)
    assert np.array_equal(got["ids"], ref["ids"])
    off, sr = oracle.permute(ref["ids"], DIMS["n_experts"])
    assert np.array_equal(got["offsets"], off) and np.array_equal(got["sorted"], sr)
    G.assert_latent_close(got["lat"], ref["lat"])
    h_ref, rows_ref = G.oracle_expert_rows(lay, ex, got["lat"], got["ids"])
    G.assert_h_elementwise(got["h"], h_ref[sr])
    G.assert_rows_elementwise(got["rows"], rows_ref, 5e-3, "rows")
    G.assert_y_or_rows16(got, lay, ref["ybf"])
    G.assert_out_close(out.cpu().numpy(), ref["out"])
    # the step-by-step path on the same inputs
    ws2 = B.alloc_workspace(d, T)
    out2 = torch.empty_like(out)
    B.latent_forward(d, dev["x"], B.make_weights(dev), out2, ws2)
    torch.cuda.synchronize()
    if T == 1:
        assert torch.equal(out, out2)
        step = G.views(lay, d, ws2, T)
        for k in ("lat", "h", "rows", "y", "rows16"):
            assert (got[k] is None and step[k] is None) or np.array_equal(got[k], step[k]), k
    else:
        G.assert_out_close(out.cpu().numpy(), out2.cpu().numpy(), "against moe_latent_forward")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_persistent_real_shape_one_token_bit_identical(fmt, real_experts):
    lay = synth.config_layer(1)
    nv = fmt == "nvfp4"
    experts = synth.all_nvfp4_expert_bytes(synth.REAL, 0, device="cuda") if nv else real_experts
    dev = G.device_layer(lay, experts)
    d = B.make_dims(lay.dims, lay.eps, lay.gain_per_expert, B.FMT_NVFP4 if nv else B.FMT_MXFP4)
    w = B.make_weights(dev)
    H = lay.dims["hidden"]
    ws = B.alloc_workspace(d, 1)
    ws2 = B.alloc_workspace(d, 1)
    _sync(d, 1, ws).zero_()
    for token_set in range(4):  # calls in a row on one workspace, other tokens each time
        x = torch.from_numpy(synth.token_batch(1, 1, token_set)).view(torch.int16).cuda()
        G.log(f"real shape {fmt} token set {token_set}")
        gen0 = int(_status(d, 1, ws)[0])
        out = _persistent(d, x, w, ws, H)
        s = _status(d, 1, ws)
        assert s[1] == 0 and int(s[0]) == gen0 + 1
        out2 = torch.empty_like(out)
        B.latent_forward(d, x, w, out2, ws2)
        torch.cuda.synchronize()
        assert torch.equal(out, out2), token_set
        mine, step = G.views(lay, d, ws, 1), G.views(lay, d, ws2, 1)
        for k in ("ids", "rows16"):
            assert (mine[k] is None and step[k] is None) or np.array_equal(mine[k], step[k]), (k, token_set)
    if not nv:  # and the oracle, for the last token set
        ref = oracle.token_forward(lay.dims, x.cpu().numpy().view(np.uint16)[0], lay.router, lay.pooler,
                                   lay.gain, lay.unpooler, lay.eps, 0,
                                   lambda e: tuple(dev[k][e].cpu().numpy() for k in synth.EXPERT_TENSORS))
        G.assert_out_close(out.cpu().numpy()[0], ref["out"])


def test_persistent_graph_replays_match_eager():
    T = 1
    lay = synth.make_layer(DIMS, T, seed=112)
    dev = G.device_layer(lay)
    d = B.make_dims(lay.dims, lay.eps, lay.gain_per_expert)
    w = B.make_weights(dev)
    ws = B.alloc_workspace(d, T)
    _sync(d, T, ws).zero_()
    xs = [torch.from_numpy(synth.make_layer(DIMS, T, seed=112, token_set=s).x).view(torch.int16).cuda()
          for s in range(3)]
    x_static = xs[0].clone()
    out_static = torch.empty((T, DIMS["hidden"]), dtype=torch.int16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.latent_forward_persistent(d, x_static, w, out_static, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.latent_forward_persistent(d, x_static, w, out_static, ws)
    torch.cuda.synchronize()
    for rep in range(6):
        x = xs[rep % len(xs)]
        x_static.copy_(x)
        graph.replay()
        torch.cuda.synchronize()
        got = out_static.clone()
        assert _status(d, T, ws)[1] == 0
        eager = torch.empty_like(got)
        ws2 = B.alloc_workspace(d, T)
        _sync(d, T, ws2).zero_()
        B.latent_forward_persistent(d, x, w, eager, ws2)
        torch.cuda.synchronize()
        assert torch.equal(got, eager), f"replay {rep}"
        step = torch.empty_like(got)  # and the per-step path
        B.latent_forward(d, x, w, step, B.alloc_workspace(d, T))
        torch.cuda.synchronize()
        assert torch.equal(got, step), f"replay {rep} against moe_latent_forward"


def test_persistent_rejects_what_it_is_not_built_for():
    lay = synth.make_layer(DIMS, 3, seed=113)
    dev = G.device_layer(lay)
    d = B.make_dims(lay.dims)
    ws = B.alloc_workspace(d, 3)
    out = torch.full((3, DIMS["hidden"]), 7, dtype=torch.int16, device="cuda")
    with pytest.raises(B.MoeError) as e:
        B.latent_forward_persistent(d, dev["x"], B.make_weights(dev), out, ws)
    assert e.value.status == B.MOE_EUNSUPPORTED
    small = dict(hidden=512, latent=384, inter=256, n_experts=24, top_k=6)
    lay = synth.make_layer(small, 1, seed=114)
    dev = G.device_layer(lay)
    d = B.make_dims(small)
    with pytest.raises(B.MoeError) as e:
        B.latent_forward_persistent(d, dev["x"], B.make_weights(dev),
                                    torch.empty((1, 512), dtype=torch.int16, device="cuda"),
                                    B.alloc_workspace(d, 1))
    assert e.value.status == B.MOE_EUNSUPPORTED
    torch.cuda.synchronize()
    assert (out == 7).all()
