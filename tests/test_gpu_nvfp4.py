"""NVFP4 experts (E2M1 codes, one E4M3 scale per 16 elements, a per-tensor
fp32 scale) through the C ABI, against the oracle with the same format:
routing and grouping bit for bit, the same bars as MXFP4 for every other
step (h and route rows within 1e-2 relative RMS, y and the output within
max |delta| <= 2e-2 and relative RMS <= 1e-2)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from latent_mixture_experts_amd import binding as B
from latent_mixture_experts_amd import synth
from tests import gpu_util as G
from tests.test_gpu_parity import SHAPES, _check_all_stages

pytestmark = pytest.mark.gpu

CASES = [(synth.CONFIGS[0]["dims"], 4),   # tiny
         (SHAPES[0][0], 3),               # few tokens; L = 384: odd 128-element chunk count
         (SHAPES[4][0], 1),               # one token
         (SHAPES[0][0], 45),              # several rows per expert (streaming)
         (SHAPES[2][0], 33),              # all 256 experts
         (SHAPES[5][0], 300),             # tiled, ragged tiles
         (SHAPES[8][0], 600),             # LDS-staged tiles: full and 22-row tiles, K = 512 and 1024
         (SHAPES[9][0], 100),             # LDS-staged tiles: one partial tile per expert
         # K = 4096: four staged rows per pass, so the streaming kernels take
         # the few-rows form with 5 to 12 routes per expert (several passes;
         # token rows gathered in gate/up, rows copied straight to LDS in down)
         (dict(hidden=512, latent=4096, inter=4096, n_experts=4, top_k=2), 16)]
CASE_IDS = ["tiny", "few_tokens", "one_token", "t45", "e256", "tiled", "lds_k1024", "lds_partial",
            "few_rows_passes"]


def _nv_layer(dims, T, seed, gpe=False):
    lay = synth.make_layer(dims, T, seed=seed, gain_per_expert=gpe)
    dev = G.device_layer(lay, experts=synth.all_nvfp4_expert_bytes(lay.dims, seed, device="cuda"))
    return lay, dev


def _oracle_nv(lay, dev, **kw):
    ex = {k: dev[k].cpu().numpy() for k in synth.EXPERT_TENSORS + ("w13_global", "w2_global")}
    return oracle.latent_forward(lay.dims, lay.x, lay.router, lay.pooler, ex["w13_codes"],
                                 ex["w13_scales"], ex["w2_codes"], ex["w2_scales"], lay.gain,
                                 lay.unpooler, lay.eps, lay.gain_per_expert, fmt=oracle.NVFP4,
                                 w13_global=ex["w13_global"], w2_global=ex["w2_global"], **kw)


@pytest.mark.parametrize("dims,T", CASES, ids=CASE_IDS)
def test_nvfp4_layer_all_stages(dims, T):
    lay, dev = _nv_layer(dims, T, seed=51, gpe=T % 2 == 1)
    G.log(f"NVFP4 dims={dims} T={T}")
    d = B.make_dims(lay.dims, lay.eps, lay.gain_per_expert, B.FMT_NVFP4)
    ws = B.alloc_workspace(d, T)
    out = torch.empty((T, dims["hidden"]), dtype=torch.int16, device="cuda")
    B.latent_forward(d, dev["x"], B.make_weights(dev), out, ws)
    torch.cuda.synchronize()
    got = G.views(lay, d, ws, T)
    ref = _oracle_nv(lay, dev)
    ex = {k: dev[k].cpu().numpy() for k in synth.EXPERT_TENSORS + ("w13_global", "w2_global")}
    _check_all_stages(lay, got, ref, ex_host=ex, fmt=oracle.NVFP4)
    G.assert_out_close(out.cpu().numpy(), ref["out"])


# E4M3 scale bytes outside the synthetic range: +0 and -0, subnormals
# (exponent field 0), negative normals and the largest normal (448); no NaN
SPECIAL_E4M3 = np.array([0x00, 0x80, 0x01, 0x05, 0x07, 0xB8, 0xC3, 0x7E], dtype=np.uint8)


@pytest.mark.parametrize("dims,T", [(synth.CONFIGS[0]["dims"], 4),   # few-rows form, rows via registers
                                    (SHAPES[4][0], 1),               # one-row form, rows copied to LDS
                                    (SHAPES[0][0], 45),              # plain streaming form
                                    (SHAPES[8][0], 600)],            # LDS-staged row tiles
                         ids=["few_rows", "one_row", "plain", "row_tiles"])
def test_nvfp4_special_scale_bytes(dims, T):
    """A tenth of the E4M3 block scales replaced by zeros, subnormals,
    negative values and the largest normal: every form of the NVFP4 kernels
    (scales applied to each weight, or to per-block partial sums) against
    the oracle, whose E4M3 decode is pinned for every byte. The route rows'
    element bar is 1e-2 of the row's RMS here (5e-3 elsewhere): with a few
    blocks scaled by 448 a row's sum rests on few terms, and one bf16 ulp of
    h in such a term (the GPU's fp32 gate/up sum and the oracle's fp64 sum
    may round h to neighbouring values) is about 2^-8 of it."""
    lay, dev = _nv_layer(dims, T, seed=55)
    gen = np.random.default_rng(56)
    for k in ("w13_scales", "w2_scales"):
        sc = dev[k].cpu().numpy()
        mask = gen.random(sc.shape) < 0.1
        sc[mask] = gen.choice(SPECIAL_E4M3, size=int(mask.sum()))
        dev[k] = torch.from_numpy(sc).cuda()
    G.log(f"NVFP4 special scales dims={dims} T={T}")
    d = B.make_dims(lay.dims, lay.eps, 0, B.FMT_NVFP4)
    ws = B.alloc_workspace(d, T)
    out = torch.empty((T, dims["hidden"]), dtype=torch.int16, device="cuda")
    B.latent_forward(d, dev["x"], B.make_weights(dev), out, ws)
    torch.cuda.synchronize()
    got = G.views(lay, d, ws, T)
    ref = _oracle_nv(lay, dev)
    ex = {k: dev[k].cpu().numpy() for k in synth.EXPERT_TENSORS + ("w13_global", "w2_global")}
    _check_all_stages(lay, got, ref, ex_host=ex, fmt=oracle.NVFP4, rows_elem=1e-2)
    G.assert_out_close(out.cpu().numpy(), ref["out"])


def test_nvfp4_differs_from_mxfp4_reading_of_the_same_bytes():
    """The format flag is honoured: the NVFP4 call differs from the MXFP4 call
    whose scales are the NVFP4 bytes' first half (same code bytes)."""
    dims, T = SHAPES[0][0], 3
    lay, dev = _nv_layer(dims, T, seed=52)
    o_nv = torch.empty((T, dims["hidden"]), dtype=torch.int16, device="cuda")
    d_nv = B.make_dims(lay.dims, lay.eps, 0, B.FMT_NVFP4)
    B.latent_forward(d_nv, dev["x"], B.make_weights(dev), o_nv, B.alloc_workspace(d_nv, T))
    mx = dict(dev)
    for k in ("w13_scales", "w2_scales"):
        mx[k] = dev[k][..., : dev[k].shape[-1] // 2].contiguous()
    d_mx = B.make_dims(lay.dims, lay.eps, 0)
    o_mx = torch.empty_like(o_nv)
    B.latent_forward(d_mx, dev["x"], B.make_weights(mx), o_mx, B.alloc_workspace(d_mx, T))
    torch.cuda.synchronize()
    assert not torch.equal(o_nv, o_mx)


@pytest.mark.parametrize("dims,T", [(SHAPES[0][0], 3), (SHAPES[5][0], 300)], ids=["few_tokens", "tiled"])
def test_nvfp4_routing_replay_and_block(dims, T):
    """Routing replay of the router's own choice is bit-identical with NVFP4
    experts, and the block's layer output equals the oracle's block."""
    lay, dev = _nv_layer(dims, T, seed=53)
    d = B.make_dims(lay.dims, lay.eps, 0, B.FMT_NVFP4)
    w = B.make_weights(dev)
    ws = B.alloc_workspace(d, T)
    out = torch.empty((T, dims["hidden"]), dtype=torch.int16, device="cuda")
    B.latent_forward(d, dev["x"], w, out, ws)
    torch.cuda.synchronize()
    v = G.views(lay, d, ws, T)
    out2 = torch.empty_like(out)
    B.latent_forward_routed(d, dev["x"], torch.from_numpy(v["ids"]).cuda(),
                            torch.from_numpy(v["w"]).cuda(), w, out2, B.alloc_workspace(d, T))
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    pre, post = synth.block_gains(dims, 54)
    t16 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.int16).cuda()
    wsb = B.alloc_block_workspace(d, T)
    outb = torch.empty_like(out)
    B.block_forward(d, dev["x"], t16(pre), t16(post), 1e-6, w, outb, wsb)
    torch.cuda.synchronize()
    ex = {k: dev[k].cpu().numpy() for k in synth.EXPERT_TENSORS + ("w13_global", "w2_global")}
    ref = oracle.block_forward(lay.dims, lay.x, pre, post, 1e-6, lay.router, lay.pooler,
                               ex["w13_codes"], ex["w13_scales"], ex["w2_codes"], ex["w2_scales"],
                               lay.gain, lay.unpooler, lay.eps, 0, fmt=oracle.NVFP4,
                               w13_global=ex["w13_global"], w2_global=ex["w2_global"])
    f = B.workspace_view(d, T, wsb, "layer_out", torch.int16, (T, dims["hidden"])).cpu().numpy()
    assert np.array_equal(B.workspace_view(d, T, wsb, "ids", torch.int32, (T, dims["top_k"])).cpu().numpy(),
                          ref["ids"])
    G.assert_out_close(f.view(np.uint16), ref["f"], "layer output")
