"""Seeded synthetic inputs for the latent MoE layer.

This module only draws random numbers with the shapes and value
distributions of the workloads; it holds none of the layer's arithmetic.
Both the CPU oracle tests and the GPU path take their inputs from here.

Two generators are used:

* Normally distributed tensors (activations, router, pooler, unpooler, norm
  gain) come from numpy's PCG64 stream seeded with ``(seed, tensor key)`` and
  are rounded to their storage type on the host.
* The packed MXFP4 expert bytes (codes and E8M0 scales, several GB at the real
  shape) come from a counter-based integer hash (Chris Wellons' "lowbias32"
  finaliser, applied twice) written with exact int64 torch operations, so the
  same bytes come out on the CPU and on the GPU, and any one expert can be
  produced on its own.

Shapes (all row-major):
  x [T][H] bf16, router [E][H] fp32, pooler [L][H] bf16, unpooler [H][L] bf16,
  gain [L] (or [E][L]) bf16,
  w13_codes [E][2I][L/2] u8, w13_scales [E][2I][L/32] u8,
  w2_codes [E][L][I/2] u8, w2_scales [E][L][I/32] u8.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field

import numpy as np
import torch

# ----------------------------------------------------------------------------
# Workloads. Distributions: activations N(0,1); router N(0, router_std);
# pooler/unpooler N(0, 1/sqrt(fan_in)); code bytes uniform over 0..255; scale
# bytes uniform over 119..123 (2^-8 .. 2^-4); gain 1 + N(0, 0.1); eps 1e-6.
# ----------------------------------------------------------------------------
REAL = dict(hidden=8192, latent=4096, inter=4096, n_experts=256, top_k=8)
TINY = dict(hidden=256, latent=128, inter=128, n_experts=16, top_k=4)

# Bias strength for the skewed workload: with this value the 16 most popular
# experts take about half of the routes at T=512 (checked by a test through
# the oracle's router).
ZIPF_S = 1.1
ZIPF_BETA = 0.93

CONFIGS = {
    0: dict(name="tiny_t4", T=4, dims=TINY, router_std=0.02, zipf=False),
    1: dict(name="decode_t1", T=1, dims=REAL, router_std=0.02, zipf=False),
    2: dict(name="verify_t32", T=32, dims=REAL, router_std=0.02, zipf=False),
    3: dict(name="prefill_t4096", T=4096, dims=REAL,
            router_std=1.0 / math.sqrt(8192), zipf=False),
    4: dict(name="skewed_t512", T=512, dims=REAL, router_std=0.02, zipf=True),
}

EPS = 1e-6
SCALE_LO, SCALE_N = 119, 5  # scale bytes uniform over 119..123

EXPERT_TENSORS = ("w13_codes", "w13_scales", "w2_codes", "w2_scales")


def expert_shape(dims: dict, name: str) -> tuple[int, int]:
    """Per-expert (rows, bytes per row) of one packed expert tensor."""
    L, I = dims["latent"], dims["inter"]
    return {
        "w13_codes": (2 * I, L // 2),
        "w13_scales": (2 * I, L // 32),
        "w2_codes": (L, I // 2),
        "w2_scales": (L, I // 32),
    }[name]


# NVFP4 experts: the same E2M1 code bytes; one E4M3 scale byte per 16
# elements (positive, exponent field 5..7, any mantissa: 0.25 .. 1.875) and
# one fp32 scale per stored tensor and expert (about 2^-6, not a power of two)
NV_SCALE_EXP_LO, NV_SCALE_EXP_N = 5, 3


def nvfp4_expert_shape(dims: dict, name: str) -> tuple[int, int]:
    rows, cols = expert_shape(dims, name)
    return (rows, cols * 2) if name.endswith("scales") else (rows, cols)


def _key(seed: int, *parts) -> int:
    text = ":".join(str(p) for p in (seed,) + parts).encode()
    return int.from_bytes(hashlib.sha256(text).digest()[:4], "little")


def _dims_tag(dims: dict) -> str:
    return "x".join(str(dims[k]) for k in ("hidden", "latent", "inter", "n_experts"))


# ---- counter-based byte generator (exact int64 arithmetic, CPU == GPU) -----
_M32 = 0xFFFFFFFF


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    # (x * c) mod 2^32 with every partial product below 2^49 (no int64 overflow)
    lo, hi = c & 0xFFFF, c >> 16
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & _M32


def _lowbias32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def counter_words(key: int, start: int, n: int, device="cpu") -> torch.Tensor:
    """n 32-bit words (in int64) for counters start .. start+n-1 of stream key."""
    idx = torch.arange(start, start + n, dtype=torch.int64, device=device) & _M32
    return _lowbias32(_lowbias32(idx) ^ (key & _M32))


def expert_bytes(dims: dict, seed: int, name: str, experts, device="cpu") -> torch.Tensor:
    """Packed bytes of tensor ``name`` for the listed experts: uint8
    [len(experts), rows, cols]. Code bytes are uniform over 0..255 (every
    nibble uniform, -0 included); scale bytes uniform over 119..123."""
    rows, cols = expert_shape(dims, name)
    per = rows * cols
    key = _key(seed, "experts", _dims_tag(dims), name)
    out = torch.empty((len(experts), rows, cols), dtype=torch.uint8, device=device)
    for i, e in enumerate(experts):
        if name.endswith("codes"):
            words = counter_words(key, int(e) * (per // 4), per // 4, device)
            b = torch.stack([(words >> s) & 0xFF for s in (0, 8, 16, 24)], dim=1)
            out[i] = b.reshape(rows, cols).to(torch.uint8)
        else:
            words = counter_words(key, int(e) * per, per, device)
            out[i] = (SCALE_LO + words % SCALE_N).reshape(rows, cols).to(torch.uint8)
    return out


def all_expert_bytes(dims: dict, seed: int, device="cpu") -> dict:
    E = dims["n_experts"]
    return {n: expert_bytes(dims, seed, n, range(E), device) for n in EXPERT_TENSORS}


def nvfp4_expert_bytes(dims: dict, seed: int, name: str, experts, device="cpu") -> torch.Tensor:
    """NVFP4 bytes of tensor ``name`` for the listed experts: codes as for
    MXFP4 (their own stream), scales [rows][cols/16] E4M3 bytes."""
    rows, cols = nvfp4_expert_shape(dims, name)
    per = rows * cols
    key = _key(seed, "nvfp4", _dims_tag(dims), name)
    out = torch.empty((len(experts), rows, cols), dtype=torch.uint8, device=device)
    for i, e in enumerate(experts):
        if name.endswith("codes"):
            words = counter_words(key, int(e) * (per // 4), per // 4, device)
            b = torch.stack([(words >> s) & 0xFF for s in (0, 8, 16, 24)], dim=1)
            out[i] = b.reshape(rows, cols).to(torch.uint8)
        else:
            words = counter_words(key, int(e) * per, per, device)
            ex = NV_SCALE_EXP_LO + (words >> 3) % NV_SCALE_EXP_N
            out[i] = ((ex << 3) | (words & 7)).reshape(rows, cols).to(torch.uint8)
    return out


def nvfp4_globals(dims: dict, seed: int) -> dict:
    """Per-tensor fp32 scales [E] of W13 and W2: 2^-6 * (1 + u/2), u in [0, 1)."""
    E = dims["n_experts"]
    r = {}
    for name in ("w13_global", "w2_global"):
        u = counter_words(_key(seed, "nvfp4", _dims_tag(dims), name), 0, E).to(torch.float64) / 2.0 ** 32
        r[name] = (2.0 ** -6 * (1.0 + u / 2)).to(torch.float32)
    return r


def all_nvfp4_expert_bytes(dims: dict, seed: int, device="cpu") -> dict:
    E = dims["n_experts"]
    r = {n: nvfp4_expert_bytes(dims, seed, n, range(E), device) for n in EXPERT_TENSORS}
    r.update({k: v.to(device) for k, v in nvfp4_globals(dims, seed).items()})
    return r


# ---- normally distributed tensors (numpy PCG64, rounded on the host) --------
def _rng(seed: int, *parts) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, _key(seed, *parts)]))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round to bf16 (nearest, ties to even) via fp32; returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Layer:
    """Dense inputs of one layer instance (numpy, host). Expert bytes are
    produced separately with :func:`expert_bytes` (large at the real shape)."""
    dims: dict
    T: int
    seed: int
    x: np.ndarray          # [T][H] uint16 (bf16 bits)
    router: np.ndarray     # [E][H] float32
    pooler: np.ndarray     # [L][H] uint16
    unpooler: np.ndarray   # [H][L] uint16
    gain: np.ndarray       # [L] or [E][L] uint16
    gain_per_expert: int = 0
    eps: float = EPS
    meta: dict = field(default_factory=dict)


def _draw_x(dims: dict, T: int, seed: int, token_set: int) -> np.ndarray:
    tag = _dims_tag(dims)
    return _rng(seed, "x", tag, T, token_set).standard_normal((T, dims["hidden"]))


def token_batch(cfg_id: int, T: int, token_set: int, seed: int = 0) -> np.ndarray:
    """The activations alone (bf16 bits [T][H]) of ``config_layer(cfg_id,
    token_set=token_set, T=T)``, without drawing the weights."""
    c = CONFIGS[cfg_id]
    x = _draw_x(c["dims"], T, seed, token_set)
    if c["zipf"]:
        x[:, c["dims"]["hidden"] - 1] = 1.0
    return to_bf16_bits(x)


def make_layer(dims: dict, T: int, seed: int = 0, router_std: float = 0.02,
               zipf: bool = False, gain_per_expert: bool = False,
               token_set: int = 0) -> Layer:
    """One seeded layer instance. ``token_set`` selects an independent draw of
    the activations only (the weights stay the same)."""
    H, L, E = dims["hidden"], dims["latent"], dims["n_experts"]
    tag = _dims_tag(dims)
    x = _draw_x(dims, T, seed, token_set)
    router = (_rng(seed, "router", tag, router_std).standard_normal((E, H))
              * router_std).astype(np.float32)
    pooler = to_bf16_bits(_rng(seed, "pooler", tag).standard_normal((L, H)) / math.sqrt(H))
    unpooler = to_bf16_bits(_rng(seed, "unpooler", tag).standard_normal((H, L)) / math.sqrt(L))
    gshape = (E, L) if gain_per_expert else (L,)
    gain = to_bf16_bits(1.0 + 0.1 * _rng(seed, "gain", tag, int(gain_per_expert))
                        .standard_normal(gshape))
    meta = {}
    if zipf:
        # Per-expert logit bias b_e = beta * ln p(rank(e)), p(r) ~ r^-s, given
        # to the router as data: input channel H-1 is 1 and router column
        # H-1 holds b_e.
        rank = _rng(seed, "zipf_rank", tag).permutation(E)
        p = (np.arange(1, E + 1, dtype=np.float64)) ** (-ZIPF_S)
        p /= p.sum()
        bias = ZIPF_BETA * np.log(p[rank])
        x[:, H - 1] = 1.0
        router[:, H - 1] = bias.astype(np.float32)
        meta["zipf_rank"] = rank
    return Layer(dims=dict(dims), T=T, seed=seed, x=to_bf16_bits(x), router=router,
                 pooler=pooler, unpooler=unpooler, gain=gain,
                 gain_per_expert=int(gain_per_expert), meta=meta)


def block_gains(dims: dict, seed: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Gains of the norms before and after the layer (bf16 bits [H]):
    1 + N(0, 0.1) and 0.5 + N(0, 0.1)."""
    H = dims["hidden"]
    tag = _dims_tag(dims)
    pre = to_bf16_bits(1.0 + 0.1 * _rng(seed, "pre_gain", tag).standard_normal(H))
    post = to_bf16_bits(0.5 + 0.1 * _rng(seed, "post_gain", tag).standard_normal(H))
    return pre, post


def config_layer(cfg_id: int, seed: int = 0, gain_per_expert: bool = False,
                 token_set: int = 0, T: int | None = None) -> Layer:
    c = CONFIGS[cfg_id]
    return make_layer(c["dims"], c["T"] if T is None else T, seed=seed,
                      router_std=c["router_std"], zipf=c["zipf"],
                      gain_per_expert=gain_per_expert, token_set=token_set)
