"""moe_block_forward (the layer inside its sandwich norms, plus the residual)
through the C ABI, against the oracle's block.

The pre-norm's fp32 output (the router input) within one fp32 ulp and
almost always identical, so that the routing stays bit-exact; the layer's
output at the layer's bar (max |delta| <= 2e-2, relative RMS <= 1e-2); the
block's output within max(2e-2, one bf16 ulp of the result) and relative
RMS <= 1e-2: the residual add rounds a value whose size is the residual
stream's, so one rounding step there is the sum's rounding, not an error of
the layer."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from latent_mixture_experts_amd import binding as B
from latent_mixture_experts_amd import synth
from tests import exact
from tests import gpu_util as G
from tests.test_gpu_parity import SHAPES

pytestmark = pytest.mark.gpu

# tiny; few tokens and one token (one-pass router); T = 40 (MFMA router);
# tiled and LDS-tiled experts
CASES = [(synth.CONFIGS[0]["dims"], 4), (SHAPES[0][0], 3), (SHAPES[4][0], 1), (SHAPES[0][0], 40),
         (SHAPES[6][0], 400), (SHAPES[8][0], 600)]
CASE_IDS = ["tiny", "few_tokens", "one_token", "mfma_router", "tiled", "lds_tiles"]
BLOCK_EPS = 1e-6


def _gains(H, seed):
    rng = np.random.default_rng(seed)
    return (synth.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(H)),
            synth.to_bf16_bits(0.5 + 0.1 * rng.standard_normal(H)))


def _block_gpu(lay, dev, pre, post, out=None):
    d = B.make_dims(lay.dims, lay.eps, lay.gain_per_expert)
    ws = B.alloc_block_workspace(d, lay.T)
    if out is None:
        out = torch.empty((lay.T, lay.dims["hidden"]), dtype=torch.int16, device="cuda")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.int16).cuda()
    B.block_forward(d, dev["x"], t(pre), t(post), BLOCK_EPS, B.make_weights(dev), out, ws)
    torch.cuda.synchronize()
    return out, d, ws


def assert_block_out_close(got_bits, ref_bits):
    g = G.bf16(got_bits)
    r = G.bf16(ref_bits)
    ulp = np.ldexp(1.0, np.frexp(np.abs(r))[1] - 8)
    d = np.abs(g - r)
    assert (d <= np.maximum(G.OUT_ATOL, ulp)).all(), d.max()
    rel = float(np.sqrt((d * d).mean() / max((r * r).mean(), 1e-30)))
    assert rel <= G.OUT_REL_RMS, rel


@pytest.mark.parametrize("dims,T", CASES, ids=CASE_IDS)
def test_block_matches_oracle(dims, T):
    lay = synth.make_layer(dims, T, seed=31, gain_per_expert=T % 2 == 1)
    G.log(f"dims={dims} T={T}")
    H, K, E = dims["hidden"], dims["top_k"], dims["n_experts"]
    pre, post = _gains(H, 32)
    dev = G.device_layer(lay)
    out, d, ws = _block_gpu(lay, dev, pre, post)
    v = lambda name, dt, shape: B.workspace_view(d, T, ws, name, dt, shape).cpu().numpy()
    got = dict(nf=v("norm_f32", torch.float32, (T, H)), nb=v("norm_bf16", torch.int16, (T, H)).view(np.uint16),
               f=v("layer_out", torch.int16, (T, H)).view(np.uint16), logits=v("logits", torch.float32, (T, E)),
               ids=v("ids", torch.int32, (T, K)), offsets=v("offsets", torch.int32, (E + 1,)),
               sorted=v("sorted", torch.int32, (T * K,)))
    ex = G.host_experts(dev)
    ref = oracle.block_forward(lay.dims, lay.x, pre, post, BLOCK_EPS, lay.router, lay.pooler,
                               ex["w13_codes"], ex["w13_scales"], ex["w2_codes"], ex["w2_scales"],
                               lay.gain, lay.unpooler, lay.eps, lay.gain_per_expert)
    ud = G.ulp_diff_f32(got["nf"], ref["n_f32"])
    assert ud.max() <= 1 and (ud == 0).mean() >= 0.9999
    db = np.abs(G.bf16(got["nb"]) - G.bf16(ref["n_bf16"]))
    assert (db == 0).mean() >= 0.9999 and (db <= np.ldexp(1.0, np.frexp(np.abs(G.bf16(ref["n_bf16"])))[1] - 8)).all()
    ul = G.ulp_diff_f32(got["logits"], ref["logits"])
    assert ul.max() <= 1 and (ul == 0).mean() >= 0.999
    assert np.array_equal(got["ids"], ref["ids"])
    off, sr = oracle.permute(ref["ids"], E)
    assert np.array_equal(got["offsets"], off) and np.array_equal(got["sorted"], sr)
    G.assert_out_close(got["f"], ref["f"], "layer output")
    assert_block_out_close(out.cpu().numpy(), ref["out"])


@pytest.mark.parametrize("T", [5, 1], ids=["t5", "t1_folded"])
def test_block_in_place(T):
    """out may be the residual buffer: the result is the same bit for bit
    (T = 1: the post-norm in the unpooler's last workgroup)."""
    dims = SHAPES[0][0]
    lay = synth.make_layer(dims, T, seed=33)
    pre, post = _gains(dims["hidden"], 34)
    dev = G.device_layer(lay)
    ref, _, _ = _block_gpu(lay, dev, pre, post)
    inplace = dev["x"].clone()
    dev2 = dict(dev)
    dev2["x"] = inplace
    _block_gpu(lay, dev2, pre, post, out=inplace)
    assert torch.equal(inplace, ref)


@pytest.mark.parametrize("T", [6, 1], ids=["t6", "t1_folded"])
def test_block_zero_post_gain_passes_the_residual_through(T):
    dims = SHAPES[0][0]
    lay = synth.make_layer(dims, T, seed=35)
    pre, _ = _gains(dims["hidden"], 36)
    dev = G.device_layer(lay)
    out, _, _ = _block_gpu(lay, dev, pre, np.zeros(dims["hidden"], np.uint16))
    assert torch.equal(out, dev["x"])


def test_block_real_shape_one_token(real_experts):
    """The real-shape block at T = 1, where the pre-norm runs inside the
    router + pooler launch: the pre-norm outputs, the routing, the layer's
    output and the block output against the oracle's steps composed (the
    pre-norm, the fp32 router, top-K, the routed layer on the bf16 pre-norm
    over the touched experts only, the post-norm plus the residual)."""
    lay = synth.config_layer(1)
    dims, T = lay.dims, lay.T
    H, K, E = dims["hidden"], dims["top_k"], dims["n_experts"]
    pre, post = _gains(H, 37)
    dev = G.device_layer(lay, real_experts)
    out, d, ws = _block_gpu(lay, dev, pre, post)
    v = lambda name, dt, shape: B.workspace_view(d, T, ws, name, dt, shape).cpu().numpy()
    nf_ref, nb_ref = oracle.pre_norm(lay.x, pre, BLOCK_EPS)
    ud = G.ulp_diff_f32(v("norm_f32", torch.float32, (T, H)), nf_ref)
    assert ud.max() <= 1 and (ud == 0).mean() >= 0.9999
    assert np.array_equal(v("norm_bf16", torch.int16, (T, H)).view(np.uint16), nb_ref)
    logits = oracle.router_logits_f32(nf_ref, lay.router)
    ids, w = oracle.topk(logits, K)
    assert np.array_equal(v("ids", torch.int32, (T, K)), ids)
    # the routed layer over the touched experts alone (ids renumbered 0..U-1)
    touched = np.unique(ids)
    remap = {int(e): i for i, e in enumerate(touched)}
    ex = {k: np.stack([dev[k][int(e)].cpu().numpy() for e in touched]) for k in synth.EXPERT_TENSORS}
    small = dict(dims, n_experts=len(touched))
    f_ref = oracle.latent_forward_routed(small, nb_ref, np.vectorize(remap.get)(ids).astype(np.int32), w,
                                         lay.pooler, ex["w13_codes"], ex["w13_scales"], ex["w2_codes"],
                                         ex["w2_scales"], lay.gain, lay.unpooler, lay.eps, 0)["out"]
    G.assert_out_close(v("layer_out", torch.int16, (T, H)).view(np.uint16), f_ref, "layer output")
    assert_block_out_close(out.cpu().numpy(), oracle.post_norm_residual(lay.x, f_ref, post, BLOCK_EPS))
