"""The expert projections' two loops (moe_dims.expert_split_rows) through the
C ABI: in the row-tile regime, experts with at most n routes run on the
streaming kernels and the rest on the row tiles ("RadixArk team serves
Meta's Muse Spark Open on one TPU host", section "Changes to attention and
expert processing": expert work split into two loops; the page does not
say which, and here they are the two row regimes).

Skewed routing (a few hot experts, many with a handful of routes) so that
both loops have experts; the LDS-staged and the register-staged row-tile
kernels, MXFP4 and NVFP4. Every stage is held to the oracle's bar, h and
the route rows element by element from the GPU's own latent rows, with h
and the rows pre-filled with NaN (every row must be written by one of the
two loops)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from latent_mixture_experts_amd import binding as B
from latent_mixture_experts_amd import synth
from tests import gpu_util as G
from tests.test_gpu_coverage import _expert_rows_check, _nan_fill
from tests.test_gpu_parity import _check_all_stages

pytestmark = pytest.mark.gpu

CASES = [
    # LDS-staged row tiles (K = 512: multiples of 512 up to 4096)
    ("lds", dict(hidden=512, latent=512, inter=512, n_experts=64, top_k=4), 512),
    # register-staged row tiles (latent 768 is not a multiple of 512)
    ("reg", dict(hidden=512, latent=768, inter=256, n_experts=64, top_k=4), 300),
]
NV_KEYS = synth.EXPERT_TENSORS + ("w13_global", "w2_global")


def _run(lay, dev, split, fmt=B.FMT_MXFP4):
    T, L, I, K = lay.T, lay.dims["latent"], lay.dims["inter"], lay.dims["top_k"]
    d = B.make_dims(lay.dims, lay.eps, lay.gain_per_expert, fmt, expert_split_rows=split)
    ws = B.alloc_workspace(d, T)
    _nan_fill(d, T, ws, I, L, K)
    out = torch.empty((T, lay.dims["hidden"]), dtype=torch.int16, device="cuda")
    B.latent_forward(d, dev["x"], B.make_weights(dev), out, ws)
    torch.cuda.synchronize()
    got = G.views(lay, d, ws, T)
    assert np.isfinite(got["rows"]).all() and np.isfinite(G.bf16(got["h"])).all()
    return out.cpu().numpy(), got


def _both_loops(lay, got, split):
    counts = np.diff(got["offsets"])
    touched = counts[counts > 0]
    assert lay.T * lay.dims["top_k"] >= 16 * lay.dims["n_experts"]  # the row-tile regime
    if split > 0:
        assert (touched <= split).any() and (touched > split).any(), np.bincount(touched)


@pytest.mark.parametrize("split", [-1, 4, 16])
@pytest.mark.parametrize("name,dims,T", CASES, ids=[c[0] for c in CASES])
def test_two_loops_match_oracle(name, dims, T, split):
    lay = synth.make_layer(dims, T, seed=21, zipf=True, gain_per_expert=split == 4)
    G.log(f"two loops {name} dims={dims} T={T} split={split}")
    dev = G.device_layer(lay)
    out, got = _run(lay, dev, split)
    _both_loops(lay, got, split)
    ex = G.host_experts(dev)
    ref = G.oracle_full(lay, ex)
    _check_all_stages(lay, got, ref, ex_host=ex)
    G.assert_out_close(out, ref["out"])


def test_two_loops_nvfp4():
    dims, T = CASES[0][1], CASES[0][2]
    lay = synth.make_layer(dims, T, seed=22, zipf=True)
    dev = G.device_layer(lay, experts=synth.all_nvfp4_expert_bytes(lay.dims, 22, device="cuda"))
    G.log(f"two loops NVFP4 dims={dims} T={T} split=8")
    out, got = _run(lay, dev, 8, B.FMT_NVFP4)
    _both_loops(lay, got, 8)
    ex = {k: dev[k].cpu().numpy() for k in NV_KEYS}
    ref = oracle.latent_forward(lay.dims, lay.x, lay.router, lay.pooler, ex["w13_codes"],
                                ex["w13_scales"], ex["w2_codes"], ex["w2_scales"], lay.gain,
                                lay.unpooler, lay.eps, lay.gain_per_expert, fmt=oracle.NVFP4,
                                w13_global=ex["w13_global"], w2_global=ex["w2_global"])
    _check_all_stages(lay, got, ref, ex_host=ex, fmt=oracle.NVFP4)
    G.assert_out_close(out, ref["out"])


def test_two_loops_real_shape_skewed(real_experts):
    """The skewed T = 512 workload at the real shape, 16 rows against one
    loop: the same routing, every row of the three most-loaded experts and
    of three light experts against the oracle element by element, and the
    two outputs within the bar of each other."""
    lay = synth.config_layer(4)
    dev = G.device_layer(lay, real_experts)
    G.log("two loops real shape skewed T=512 split=-1")
    o1, g1 = _run(lay, dev, -1)
    G.log("two loops real shape skewed T=512 split=16")
    o2, g2 = _run(lay, dev, 16)
    _both_loops(lay, g2, 16)
    assert np.array_equal(g1["ids"], g2["ids"]) and np.array_equal(g1["sorted"], g2["sorted"])
    counts = np.diff(g2["offsets"])
    order = np.argsort(counts, kind="stable")
    light = [int(e) for e in order if 0 < counts[e] <= 16][-3:]
    heavy = [int(e) for e in order[-3:]]
    G.log(f"  light experts {light} ({counts[light].tolist()} routes), heavy {heavy}")
    _expert_rows_check(lay, dev, g2, light + heavy)
    G.assert_out_close(o2, o1, "out")
