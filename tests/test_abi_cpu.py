"""The C-ABI library without a GPU: it loads, exports every function that
include/moe.h declares, and rejects bad arguments before touching a device
(the *_validate entry points run the same checks as the compute calls)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from latent_mixture_experts_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
REAL = dict(hidden=8192, latent=4096, inter=4096, n_experts=256, top_k=8)
P = 0x10000  # fake, 16-byte aligned "device" addresses: never dereferenced


def declared_functions() -> list[str]:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert "moe_route" in names and "moe_latent_forward" in names
    lib = B.lib()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def _weights(**over):
    w = dict(router=P, pooler=P, w13_codes=P, w13_scales=P, w2_codes=P, w2_scales=P,
             norm_gain=P, unpooler=P, w13_global=None, w2_global=None)
    w.update(over)
    return B.MoeWeights(*(w[k] for k in ("router", "pooler", "w13_codes", "w13_scales",
                                          "w2_codes", "w2_scales", "norm_gain", "unpooler",
                                          "w13_global", "w2_global")))


def _fwd(d, T=4, x=P, out=P, ws=P, nbytes=None, weights=None):
    if nbytes is None:
        nbytes = B.workspace_bytes(d, max(T, 1))
    return B.lib().moe_latent_forward_validate(ctypes.byref(d), T, x, ctypes.byref(weights or _weights()),
                                               out, ws, nbytes)


def _route(d, T=4, logits=None, ws=P, nbytes=None, **p):
    args = dict(x=P, router=P, ids=P, w=P, offsets=P, sorted=P)
    args.update(p)
    if nbytes is None:
        nbytes = B.workspace_bytes(d, max(T, 1))
    return B.lib().moe_route_validate(ctypes.byref(d), T, args["x"], args["router"], args["ids"],
                                      args["w"], args["offsets"], args["sorted"], logits, ws, nbytes)


def test_valid_arguments_pass():
    d = B.make_dims(REAL)
    assert _fwd(d) == B.MOE_OK
    assert _route(d) == B.MOE_OK
    assert _route(d, logits=P) == B.MOE_OK


def test_zero_tokens_is_a_no_op():
    d = B.make_dims(REAL)
    assert _fwd(d, T=0, x=None, out=None, ws=None, nbytes=0) == B.MOE_OK
    assert _route(d, T=0, ws=None, nbytes=0) == B.MOE_OK


@pytest.mark.parametrize("field", ["router", "pooler", "w13_codes", "w13_scales", "w2_codes",
                                   "w2_scales", "norm_gain", "unpooler"])
def test_null_and_misaligned_weights(field):
    d = B.make_dims(REAL)
    assert _fwd(d, weights=_weights(**{field: None})) == B.MOE_EINVAL
    assert _fwd(d, weights=_weights(**{field: P + 8})) == B.MOE_EALIGN


def test_null_and_misaligned_buffers():
    d = B.make_dims(REAL)
    assert _fwd(d, x=None) == B.MOE_EINVAL
    assert _fwd(d, out=None) == B.MOE_EINVAL
    assert _fwd(d, ws=None) == B.MOE_EINVAL
    assert _fwd(d, x=P + 2) == B.MOE_EALIGN
    assert B.lib().moe_latent_forward_validate(ctypes.byref(d), 4, P, None, P, P, 1 << 30) == B.MOE_EINVAL
    for k in ("x", "router", "ids", "w", "offsets", "sorted"):
        assert _route(d, **{k: None}) == B.MOE_EINVAL
        assert _route(d, **{k: P + 4}) == B.MOE_EALIGN
    assert _route(d, logits=P + 4) == B.MOE_EALIGN


def _routed(d, T=4, ids=P, w=P, x=P, out=P, ws=P, nbytes=None, weights=None):
    if nbytes is None:
        nbytes = B.workspace_bytes(d, max(T, 1))
    return B.lib().moe_latent_forward_routed_validate(ctypes.byref(d), T, x, ids, w,
                                                      ctypes.byref(weights or _weights()), out, ws,
                                                      nbytes)


def test_routed_forward_arguments():
    d = B.make_dims(REAL)
    assert _routed(d) == B.MOE_OK
    assert _routed(d, weights=_weights(router=None)) == B.MOE_OK  # the router is not read
    assert _routed(d, T=0, ids=None, w=None, x=None, out=None, ws=None, nbytes=0) == B.MOE_OK
    for k in ("ids", "w", "x", "out", "ws"):
        assert _routed(d, **{k: None}) == B.MOE_EINVAL
    assert _routed(d, ids=P + 4) == B.MOE_EALIGN
    assert _routed(d, w=P + 8) == B.MOE_EALIGN
    for field in ("pooler", "w13_codes", "w13_scales", "w2_codes", "w2_scales", "norm_gain",
                  "unpooler"):
        assert _routed(d, weights=_weights(**{field: None})) == B.MOE_EINVAL
    need = B.workspace_bytes(d, 32)
    assert _routed(d, T=32, nbytes=need - 1) == B.MOE_EWORKSPACE
    assert B.lib().moe_latent_forward_routed_validate(ctypes.byref(d), 4, P, P, P, None, P, P,
                                                      1 << 30) == B.MOE_EINVAL


def _block(d, T=4, resid=P, pre=P, post=P, eps=1e-6, out=P, ws=P, nbytes=None, weights=None):
    if nbytes is None:
        nbytes = B.block_workspace_bytes(d, max(T, 1))
    return B.lib().moe_block_forward_validate(ctypes.byref(d), T, resid, pre, post, eps,
                                              ctypes.byref(weights or _weights()), out, ws, nbytes)


def test_block_forward_arguments():
    d = B.make_dims(REAL)
    assert _block(d) == B.MOE_OK
    assert _block(d, out=P) == B.MOE_OK  # out may be the residual buffer itself
    assert _block(d, T=0, resid=None, pre=None, post=None, out=None, ws=None, nbytes=0) == B.MOE_OK
    for k in ("resid", "pre", "post", "out", "ws"):
        assert _block(d, **{k: None}) == B.MOE_EINVAL
    assert _block(d, pre=P + 2) == B.MOE_EALIGN
    assert _block(d, post=P + 8) == B.MOE_EALIGN
    for eps in (-1e-6, float("nan"), float("inf")):
        assert _block(d, eps=eps) == B.MOE_EINVAL
    assert _block(d, weights=_weights(router=None)) == B.MOE_EINVAL
    need = B.block_workspace_bytes(d, 32)
    assert _block(d, T=32, nbytes=need - 1) == B.MOE_EWORKSPACE
    assert _block(d, T=32, nbytes=B.workspace_bytes(d, 32)) == B.MOE_EWORKSPACE


def test_expert_format():
    d = B.make_dims(REAL)
    assert _fwd(d) == B.MOE_OK                      # MXFP4: no global scales needed
    d = B.make_dims(REAL, expert_format=B.FMT_NVFP4)
    assert _fwd(d) == B.MOE_EINVAL                  # NVFP4 needs both per-tensor scales
    assert _fwd(d, weights=_weights(w13_global=P)) == B.MOE_EINVAL
    assert _fwd(d, weights=_weights(w13_global=P, w2_global=P)) == B.MOE_OK
    assert _fwd(d, weights=_weights(w13_global=P + 4, w2_global=P)) == B.MOE_EALIGN
    assert _routed(d, weights=_weights(w13_global=P, w2_global=P)) == B.MOE_OK
    assert _routed(d) == B.MOE_EINVAL
    assert _block(d, weights=_weights(w13_global=P, w2_global=P)) == B.MOE_OK
    d = B.make_dims(REAL, expert_format=2)
    assert _fwd(d) == B.MOE_EINVAL
    assert B.workspace_bytes(d, 4) == 0


def test_expert_split_rows():
    """-1 (one loop), 0 (the library's choice) and 1..16 are accepted; other
    values are rejected before anything is enqueued."""
    for v in (-1, 0, 1, 8, 16):
        assert _fwd(B.make_dims(REAL, expert_split_rows=v)) == B.MOE_OK
    for v in (-2, 17, 1 << 20):
        d = B.make_dims(REAL, expert_split_rows=v)
        assert _fwd(d) == B.MOE_EINVAL
        assert _routed(d) == B.MOE_EINVAL
        assert B.workspace_bytes(d, 4) == 0


def test_token_limit_of_the_32_bit_buffer_ranges():
    """h (T*K*I*2 bytes) must stay below 2^31: T <= 32767 at the real shape."""
    d = B.make_dims(REAL)
    assert _fwd(d, T=32767, nbytes=1 << 40) == B.MOE_OK
    assert _fwd(d, T=32768, nbytes=1 << 40) == B.MOE_EUNSUPPORTED
    assert B.workspace_bytes(d, 32768) == 0 and B.workspace_bytes(d, 32767) > 0
    wide = B.make_dims(dict(REAL, hidden=65536, top_k=1))  # then x (T*H*2) binds: T < 16384
    assert _fwd(wide, T=16383, nbytes=1 << 40) == B.MOE_OK
    assert _fwd(wide, T=16384, nbytes=1 << 40) == B.MOE_EUNSUPPORTED


def test_workspace_too_small():
    d = B.make_dims(REAL)
    need = B.workspace_bytes(d, 32)
    assert _fwd(d, T=32, nbytes=need - 1) == B.MOE_EWORKSPACE
    assert _route(d, T=32, nbytes=need - 1) == B.MOE_EWORKSPACE
    assert _fwd(d, T=32, nbytes=need) == B.MOE_OK


def test_workspace_size_is_monotonic_and_covers_views():
    d = B.make_dims(REAL)
    prev = 0
    block_views = ("norm_f32", "norm_bf16", "layer_out")
    for T in (1, 2, 7, 32, 100, 512, 4096):
        n = B.workspace_bytes(d, T)
        nblk = B.block_workspace_bytes(d, T)
        assert n >= prev and nblk >= n + 8 * T * REAL["hidden"]
        prev = n
        for name, which in B.VIEWS.items():
            off, nb = ctypes.c_size_t(), ctypes.c_size_t()
            assert B.lib().moe_workspace_view(ctypes.byref(d), T, which, ctypes.byref(off), ctypes.byref(nb)) == 0
            # the layer's views lie in its own workspace; the block's in the block's
            limit = nblk if name in block_views else n
            assert off.value % 256 == 0 and off.value + nb.value <= limit, (T, name)
            if name in block_views:
                assert off.value >= n - 256, (T, name)
    off, nb = ctypes.c_size_t(), ctypes.c_size_t()
    assert B.lib().moe_workspace_view(ctypes.byref(d), 4, 99, ctypes.byref(off), ctypes.byref(nb)) == B.MOE_EINVAL


def _route_sum_rule(dims: dict, T: int, nvfp4: bool) -> bool:
    """When one launch takes the post-norm, the weighted sum and the
    unpooler (include/moe.h, MOE_VIEW_ROWS_BF16): at most 16 route rows whose
    bf16 latent rows (plus 16 bytes each) fit 72 KiB, at most 16 tokens, on
    the streaming expert path (not the row-tile path, taken from 16 routes
    per expert on 256-multiple widths), and with NVFP4 experts one token."""
    L, I, E, K = dims["latent"], dims["inter"], dims["n_experts"], dims["top_k"]
    R = T * K
    tiled = R >= 16 * E and I % 256 == 0 and L % 256 == 0
    return (T <= 16 and R <= 16 and R * (2 * L + 16) <= 72 * 1024 and not tiled
            and (not nvfp4 or T == 1))


@pytest.mark.parametrize("dims", [
    REAL,
    dict(hidden=512, latent=384, inter=256, n_experts=24, top_k=6),
    dict(hidden=640, latent=640, inter=384, n_experts=16, top_k=8),
    dict(hidden=256, latent=256, inter=256, n_experts=32, top_k=1),
    dict(hidden=256, latent=256, inter=256, n_experts=32, top_k=3),
    dict(hidden=256, latent=256, inter=256, n_experts=1, top_k=1),
    dict(hidden=8192, latent=8192, inter=4096, n_experts=256, top_k=8)],
    ids=["real", "l384_k6", "l640_k8", "k1", "k3", "e1_k1", "l8192"])
@pytest.mark.parametrize("nvfp4", [False, True], ids=["mxfp4", "nvfp4"])
def test_route_sum_view_follows_its_rule(dims, nvfp4):
    """The gain-scaled bf16 route rows have a workspace view exactly when
    the route sum applies, and y keeps its own view either way (host-only:
    the view sizes are what the forward call takes)."""
    fmt = B.FMT_NVFP4 if nvfp4 else B.FMT_MXFP4
    d = B.make_dims(dims, expert_format=fmt)
    taken = []
    for T in range(1, 41):
        _, nb = B.workspace_view_range(d, T, "rows_bf16")
        _, ny = B.workspace_view_range(d, T, "y")
        assert ny == 2 * T * dims["latent"], T
        assert (nb > 0) == _route_sum_rule(dims, T, nvfp4), (T, nb)
        if nb:
            assert nb == 2 * T * dims["top_k"] * dims["latent"], T
            taken.append(T)
    if dims is REAL:
        assert taken == [1]  # eight rows of 8 KiB fit, sixteen do not


@pytest.mark.parametrize("change,code", [
    (dict(hidden=8192 + 64), B.MOE_EUNSUPPORTED),
    (dict(latent=96), B.MOE_EUNSUPPORTED),
    (dict(latent=8192 + 128), B.MOE_EUNSUPPORTED),
    (dict(inter=4096 + 32), B.MOE_EUNSUPPORTED),
    (dict(n_experts=257), B.MOE_EUNSUPPORTED),
    (dict(top_k=9), B.MOE_EUNSUPPORTED),
    (dict(n_experts=4, top_k=5), B.MOE_EUNSUPPORTED),
    (dict(hidden=0), B.MOE_EINVAL),
    (dict(top_k=0), B.MOE_EINVAL),
    (dict(n_experts=-1), B.MOE_EINVAL),
])
def test_unsupported_or_invalid_dims(change, code):
    dims = dict(REAL)
    dims.update(change)
    d = B.make_dims(dims)
    assert _fwd(d, nbytes=1 << 40) == code
    assert _route(d, nbytes=1 << 40) == code
    assert B.workspace_bytes(d, 4) == 0


def test_bad_eps_flag_and_token_count():
    d = B.make_dims(REAL, eps=float("nan"))
    assert _fwd(d, nbytes=1 << 40) == B.MOE_EINVAL
    d = B.make_dims(REAL, eps=-1.0)
    assert _fwd(d, nbytes=1 << 40) == B.MOE_EINVAL
    d = B.make_dims(REAL, gain_per_expert=2)
    assert _fwd(d, nbytes=1 << 40) == B.MOE_EINVAL
    d = B.make_dims(REAL)
    assert _fwd(d, T=-1) == B.MOE_EINVAL
    assert _fwd(d, T=1 << 25, nbytes=1 << 62) == B.MOE_EUNSUPPORTED


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert B.lib().moe_status_string(code)
    assert B.lib().moe_status_string(7) == b"unknown status"


def test_peaks_library_exports_every_declared_function():
    """The benchmark's measurement kernels (include/moe_peaks.h) load from
    their own library and reject bad arguments before any launch."""
    import ctypes

    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "moe_peaks.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))
    assert "moe_peak_copy" in names and "moe_peak_mfma_bf16" in names
    path = os.path.join(ROOT, "latent_mixture_experts_amd", "libmoe_peaks.so")
    if not os.path.exists(path):
        from latent_mixture_experts_amd import build
        build.build_peaks()
    lib = ctypes.CDLL(path)
    assert not [n for n in names if not hasattr(lib, n)]
    lib.moe_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                  ctypes.c_void_p]
    assert lib.moe_peak_copy(None, None, 16, 1, None) == -1
    assert lib.moe_peak_copy(P, P, 15, 1, None) == -1
