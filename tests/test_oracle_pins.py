"""Pins of the CPU oracle to facts that do not come from the oracle itself:
format tables, hand-derived rounding cases, exact rational arithmetic, brute
force, library routines on special cases, structured weights whose result is
known by construction, and invariants the pages state.

Pages: "Muse Spark Open on Gaudi 2" (sections "What was built", "The latent
MoE: A' with a per-expert norm", "EP and TP layout", "Correctness") and
"Soporte de dia 0 para Muse Spark Open en vLLM" (section "Arquitectura del
modelo", paragraph "MoE latente")."""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from latent_mixture_experts_amd import synth
from tests import exact

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---- number formats -----------------------------------------------------------
def test_e2m1_matches_ocp_table():
    table = exact.load_e2m1_table()
    for c in range(16):
        v = oracle.e2m1_value(c)
        assert v == table[c] and np.signbit(v) == np.signbit(table[c]), c


def test_e8m0_matches_torch_e8m0fnu_for_every_byte():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).float().double().numpy()
    got = np.array([oracle.e8m0_value(b) for b in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[0] == 2.0 ** -127 and got[127] == 1.0 and got[119] == 2.0 ** -8


def test_bf16_rounding_golden_cases():
    with open(os.path.join(exact.GOLDEN, "bf16_rounding.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            v, bits = line.split()
            assert oracle.round_bf16(float.fromhex(v)) == int(bits, 16), v


def test_bf16_rounding_matches_torch_on_fp32_values():
    # For inputs that are fp32 values, fp32 -> bf16 in torch is one rounding.
    rng = np.random.default_rng(5)
    vals = np.concatenate([
        rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 38, 3000),
        (rng.integers(0, 2 ** 16, 500).astype(np.uint32) << 16 | 0x8000).view(np.float32),  # ties
        (rng.integers(0, 2 ** 23, 500).astype(np.uint32)).view(np.float32),                   # subnormals
    ]).astype(np.float32)
    vals = vals[np.isfinite(vals)]
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.round_bf16(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_value_roundtrip():
    for bits in [0x0000, 0x8000, 0x3F80, 0x0001, 0x7F7F, 0xC2F7]:
        assert oracle.round_bf16(oracle.bf16_value(bits)) == bits


def test_mxfp4_element_layout_low_nibble_is_even_column():
    codes = np.zeros((2, 32), np.uint8)
    scales = np.full((2, 2), 127, np.uint8)
    codes[1, 5] = 0x72      # column 10 -> code 2 (1.0), column 11 -> code 7 (6.0)
    scales[1, 0] = 129      # columns 0..31 of row 1 scaled by 4
    assert oracle.mxfp4_value(codes, scales, 64, 1, 10) == 4.0
    assert oracle.mxfp4_value(codes, scales, 64, 1, 11) == 24.0
    assert oracle.mxfp4_value(codes, scales, 64, 0, 10) == 0.0


# ---- A1: router logits ---------------------------------------------------------
def test_router_logits_equal_exact_sum_rounded_to_fp32():
    rng = np.random.default_rng(11)
    T, H, E = 3, 96, 7
    x = synth.to_bf16_bits(rng.standard_normal((T, H)))
    router = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    got = oracle.router_logits(x, router)
    xf = exact.bf16_to_f64(x)
    for t in range(T):
        for e in range(E):
            s = sum(Fraction(float(xf[t, h])) * Fraction(float(router[e, h])) for h in range(H))
            assert got[t, e] == exact.fp32_of(s), (t, e)


# ---- A2: top-K ---------------------------------------------------------------------
def _brute_topk(l: np.ndarray, K: int) -> list[int]:
    """Rank of each expert = number of experts ranking before it (larger value,
    or equal value and lower id; NaN after every number)."""
    E = l.shape[0]
    rank = []
    for e in range(E):
        c = 0
        for f in range(E):
            if f == e:
                continue
            a, b = l[f], l[e]
            if np.isnan(a) and np.isnan(b):
                before = f < e
            elif np.isnan(a) or np.isnan(b):
                before = np.isnan(b)
            else:
                before = a > b or (a == b and f < e)
            c += before
        rank.append(c)
    order = sorted(range(E), key=lambda e: rank[e])
    assert sorted(rank) == list(range(E))  # a strict total order
    return order[:K]


@pytest.mark.parametrize("case", ["random", "ties", "zeros", "nan", "signed_zero", "neg_inf"])
def test_topk_matches_brute_force(case):
    rng = np.random.default_rng(3)
    T, E, K = 12, 24, 5
    if case == "random":
        l = rng.standard_normal((T, E)).astype(np.float32)
    elif case == "ties":
        l = rng.integers(-2, 3, (T, E)).astype(np.float32)
    elif case == "zeros":
        l = np.zeros((T, E), np.float32)
    elif case == "nan":
        l = rng.integers(-2, 3, (T, E)).astype(np.float32)
        l[rng.random((T, E)) < 0.4] = np.nan
    elif case == "signed_zero":
        l = np.where(rng.random((T, E)) < 0.5, -0.0, 0.0).astype(np.float32)
        l[:, ::7] = -1.0
    else:
        l = np.full((T, E), -np.inf, np.float32)
        l[:, 3] = 0.0
    ids, w = oracle.topk(l, K)
    for t in range(T):
        assert list(ids[t]) == _brute_topk(l[t], K), (case, t)
    if case == "zeros":
        assert (ids == np.arange(K)).all()


def test_topk_matches_stable_sort_on_finite_logits():
    rng = np.random.default_rng(4)
    l = rng.integers(-3, 4, (50, 64)).astype(np.float32)
    ids, _ = oracle.topk(l, 8)
    ref = torch.sort(-torch.from_numpy(l), dim=1, stable=True).indices[:, :8].numpy()
    assert np.array_equal(ids, ref)


def test_router_weights_special_cases():
    rng = np.random.default_rng(6)
    l = rng.standard_normal((200, 10)).astype(np.float32)
    # K = 2: w0 = sigmoid(l_first - l_second)
    ids, w = oracle.topk(l, 2)
    for t in range(200):
        d = float(l[t, ids[t, 0]]) - float(l[t, ids[t, 1]])
        assert w[t, 0] == np.float32(scipy.special.expit(d))
    # K = 1: weight exactly 1
    _, w1 = oracle.topk(l, 1)
    assert (w1 == 1.0).all()
    # equal logits, K a power of two: exactly 1/K
    for K in (1, 2, 4, 8):
        _, wk = oracle.topk(np.full((3, 16), 0.75, np.float32), K)
        assert (wk == np.float32(1.0 / K)).all()
    # weights sum to one and follow the selection order
    _, w8 = oracle.topk(l, 8)
    assert np.allclose(w8.sum(1), 1.0, atol=1e-6)
    assert (np.diff(w8, axis=1) <= 0).all()


# ---- A3: permutation -----------------------------------------------------------------
def test_permutation_matches_stable_argsort_and_bincount():
    rng = np.random.default_rng(8)
    for T, K, E in [(1, 8, 256), (37, 4, 16), (300, 8, 40)]:
        ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
        offsets, sr = oracle.permute(ids, E)
        flat = ids.ravel()
        assert np.array_equal(sr, np.argsort(flat, kind="stable"))
        assert np.array_equal(np.diff(offsets), np.bincount(flat, minlength=E))
        assert offsets[0] == 0 and offsets[-1] == T * K


# ---- A4 / A8: dense projections ------------------------------------------------------------
def test_linear_bf16_structured_weights():
    rng = np.random.default_rng(9)
    T, Kd, N = 3, 64, 48
    x = synth.to_bf16_bits(rng.standard_normal((T, Kd)))
    perm = rng.integers(0, Kd, N)
    pw = rng.integers(-3, 4, N)
    wf = np.zeros((N, Kd), np.float32)
    wf[np.arange(N), perm] = 2.0 ** pw
    y = oracle.linear_bf16(x, synth.to_bf16_bits(wf))
    expect = synth.to_bf16_bits(exact.bf16_to_f64(x)[:, perm] * 2.0 ** pw)  # exact products
    assert np.array_equal(y, expect)


def test_linear_bf16_equals_exact_sum_rounded_to_bf16():
    rng = np.random.default_rng(10)
    T, Kd, N = 2, 64, 9
    x = synth.to_bf16_bits(rng.standard_normal((T, Kd)))
    w = synth.to_bf16_bits(rng.standard_normal((N, Kd)) / 8)
    y = oracle.linear_bf16(x, w)
    xf, wf = exact.bf16_to_f64(x), exact.bf16_to_f64(w)
    for t in range(T):
        for n in range(N):
            s = sum(Fraction(float(xf[t, k])) * Fraction(float(wf[n, k])) for k in range(Kd))
            assert y[t, n] == exact.bf16_bits_of(s)


# ---- A5 / A6: the MXFP4 expert -----------------------------------------------------------
def _structured_expert(L, I, rng):
    """W13/W2 with one nonzero per row at a known column, a known code and a
    scale that differs per 32-column block; every other nibble is +0 or -0."""
    def build(rows, cols, col_of, code_of):
        codes = np.where(rng.random((rows, cols // 2)) < 0.5, 0x00, 0x88).astype(np.uint8)
        scales = (119 + (np.arange(rows)[:, None] + np.arange(cols // 32)[None, :]) % 5).astype(np.uint8)
        for n in range(rows):
            c, code = col_of(n), code_of(n)
            b = codes[n, c // 2]
            codes[n, c // 2] = (b & 0xF0) | code if c % 2 == 0 else (b & 0x0F) | (code << 4)
        return codes, scales
    nz = [1, 2, 3, 4, 5, 6, 7, 9, 10, 11, 12, 13, 14, 15]
    c13 = lambda n: (3 * n + 1) % L if n < I else (5 * (n - I) + 2) % L
    w13c, w13s = build(2 * I, L, c13, lambda n: nz[n % len(nz)])
    c2 = lambda m: (7 * m + 3) % I
    w2c, w2s = build(L, I, c2, lambda m: nz[(m * 5) % len(nz)])
    return (w13c, w13s, w2c, w2s), c13, c2


def test_expert_row_structured_weights():
    rng = np.random.default_rng(12)
    L, I = 64, 96
    (w13c, w13s, w2c, w2s), c13, c2 = _structured_expert(L, I, rng)
    table = exact.load_e2m1_table()

    def val(codes, scales, n, c):
        b = codes[n, c // 2]
        code = (b & 0xF) if c % 2 == 0 else (b >> 4)
        return table[code] * 2.0 ** (int(scales[n, c // 32]) - 127)

    lat = synth.to_bf16_bits(rng.standard_normal(L) * 4)
    latf = exact.bf16_to_f64(lat)
    h, row = oracle.expert_row(lat, w13c, w13s, w2c, w2s)
    g = np.array([latf[c13(n)] * val(w13c, w13s, n, c13(n)) for n in range(I)])
    u = np.array([latf[c13(I + n)] * val(w13c, w13s, I + n, c13(I + n)) for n in range(I)])
    h_expect = exact.f64_to_bf16_bits(g * scipy.special.expit(g) * u)
    hd = np.abs(h.astype(np.int64) - h_expect.astype(np.int64))
    assert hd.max() <= 1 and (hd == 0).mean() > 0.97
    # The down projection picks one h per output row: exact.
    hf = exact.bf16_to_f64(h)
    row_expect = np.array([hf[c2(m)] * val(w2c, w2s, m, c2(m)) for m in range(L)], np.float32)
    assert np.array_equal(row, row_expect)
    # gate and up are not interchangeable: swapping the halves changes h
    h2, _ = oracle.expert_row(lat, np.concatenate([w13c[I:], w13c[:I]]),
                              np.concatenate([w13s[I:], w13s[:I]]), w2c, w2s)
    assert not np.array_equal(h, h2)


def test_expert_row_random_down_projection_exact():
    rng = np.random.default_rng(13)
    L, I = 64, 64
    w13c = rng.integers(0, 256, (2 * I, L // 2), dtype=np.uint8)
    w13s = rng.integers(119, 124, (2 * I, L // 32), dtype=np.uint8)
    w2c = rng.integers(0, 256, (L, I // 2), dtype=np.uint8)
    w2s = rng.integers(119, 124, (L, I // 32), dtype=np.uint8)
    lat = synth.to_bf16_bits(rng.standard_normal(L))
    h, row = oracle.expert_row(lat, w13c, w13s, w2c, w2s)
    w2 = exact.mxfp4_dequant(w2c, w2s)
    hf = exact.bf16_to_f64(h)
    for m in range(0, L, 5):
        s = sum(Fraction(float(hf[n])) * Fraction(float(w2[m, n])) for n in range(I))
        assert row[m] == exact.fp32_of(s)
    # gate/up sums against exact rationals, then SwiGLU through scipy's expit
    w13 = exact.mxfp4_dequant(w13c, w13s)
    latf = exact.bf16_to_f64(lat)
    g = np.array([float(sum(Fraction(float(latf[l])) * Fraction(float(w13[n, l])) for l in range(L))) for n in range(I)])
    u = np.array([float(sum(Fraction(float(latf[l])) * Fraction(float(w13[I + n, l])) for l in range(L))) for n in range(I)])
    he = exact.f64_to_bf16_bits(g * scipy.special.expit(g) * u)
    assert np.abs(h.astype(np.int64) - he.astype(np.int64)).max() <= 1


# ---- NVFP4 experts (E2M1 codes, E4M3 scales per 16 elements, a per-tensor fp32 scale) ------------
def test_e4m3_matches_torch_float8_e4m3fn_for_every_byte():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().double().numpy()
    got = np.array([oracle.e4m3_value(b) for b in range(256)])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all() and nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x80] == 0.0


def _nvfp4_dequant(codes, scales, glob):
    """Whole-matrix decode with torch's E4M3 dtype and the golden E2M1 table."""
    vals = np.array(exact.load_e2m1_table())
    lo, hi = codes & 0x0F, codes >> 4
    q = np.stack([vals[lo], vals[hi]], axis=-1).reshape(codes.shape[0], -1)
    sc = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e4m3fn).double().numpy()
    return q * np.repeat(sc, 16, axis=1) * float(np.float32(glob))


def test_nvfp4_element_and_scale_layout():
    """One nonzero nibble at a time: element k of row n is nibble k % 2 of
    byte k // 2, scaled by byte k // 16 of the row's scales and the tensor's
    global scale."""
    rows, cols = 3, 64
    scales = np.array([[0x30 + 8 * j + n for j in range(cols // 16)] for n in range(rows)], np.uint8)
    glob = np.float32(0.0173)
    for n in range(rows):
        for k in (0, 1, 15, 16, 17, 47, 63):
            codes = np.zeros((rows, cols // 2), np.uint8)
            codes[n, k // 2] = 0x05 if k % 2 == 0 else 0x50  # E2M1 code 5 = 3.0
            for kk in range(cols):
                want = 3.0 * oracle.e4m3_value(int(scales[n, kk // 16])) * float(glob) if kk == k else 0.0
                assert oracle.nvfp4_value(codes, scales, glob, cols, n, kk) == want


def test_nvfp4_expert_row_matches_torch_float64():
    rng = np.random.default_rng(41)
    L, I = 64, 96
    w13c = rng.integers(0, 256, (2 * I, L // 2), dtype=np.uint8)
    w13s = ((5 + rng.integers(0, 3, (2 * I, L // 16))) << 3 | rng.integers(0, 8, (2 * I, L // 16))).astype(np.uint8)
    w2c = rng.integers(0, 256, (L, I // 2), dtype=np.uint8)
    w2s = ((5 + rng.integers(0, 3, (L, I // 16))) << 3 | rng.integers(0, 8, (L, I // 16))).astype(np.uint8)
    g13, g2 = np.float32(0.0191), np.float32(0.0227)
    lat = synth.to_bf16_bits(rng.standard_normal(L))
    h, row = oracle.expert_row_fmt(oracle.NVFP4, lat, w13c, w13s, g13, w2c, w2s, g2)
    w13 = _nvfp4_dequant(w13c, w13s, g13)
    w2 = _nvfp4_dequant(w2c, w2s, g2)
    a = exact.bf16_to_f64(lat)
    g, u = w13[:I] @ a, w13[I:] @ a
    he = exact.f64_to_bf16_bits(g * scipy.special.expit(g) * u)
    assert np.abs(h.astype(np.int64) - he.astype(np.int64)).max() <= 1 and (h == he).mean() > 0.95
    re = (w2 @ exact.bf16_to_f64(h)).astype(np.float32)
    assert np.allclose(row, re, rtol=1e-6, atol=1e-12)


def test_nvfp4_with_power_of_two_scales_equals_mxfp4():
    """E4M3 scale bytes whose value times the global scale equals the MXFP4
    block scale (the same on both 16-element halves of a 32-element block)
    give the MXFP4 row bit for bit."""
    rng = np.random.default_rng(42)
    L, I = 64, 64
    w13c = rng.integers(0, 256, (2 * I, L // 2), dtype=np.uint8)
    w2c = rng.integers(0, 256, (L, I // 2), dtype=np.uint8)
    w13s = rng.integers(119, 124, (2 * I, L // 32), dtype=np.uint8)
    w2s = rng.integers(119, 124, (L, I // 32), dtype=np.uint8)
    glob = np.float32(2.0 ** -10)
    to_e4m3 = lambda s: (np.repeat(s.astype(np.int64) - 127 + 10 + 7, 2, axis=1) << 3).astype(np.uint8)
    lat = synth.to_bf16_bits(rng.standard_normal(L))
    h1, r1 = oracle.expert_row(lat, w13c, w13s, w2c, w2s)
    h2, r2 = oracle.expert_row_fmt(oracle.NVFP4, lat, w13c, to_e4m3(w13s), glob, w2c, to_e4m3(w2s), glob)
    assert np.array_equal(h1, h2) and np.array_equal(r1, r2)


def test_nvfp4_layer_is_the_expansion_of_its_routes():
    lay = synth.config_layer(0)
    ex = {k: v.numpy() for k, v in synth.all_nvfp4_expert_bytes(lay.dims, 0).items()}
    K = lay.dims["top_k"]
    r = oracle.latent_forward(lay.dims, lay.x, lay.router, lay.pooler, ex["w13_codes"],
                              ex["w13_scales"], ex["w2_codes"], ex["w2_scales"], lay.gain,
                              lay.unpooler, lay.eps, 0, fmt=oracle.NVFP4,
                              w13_global=ex["w13_global"], w2_global=ex["w2_global"])
    for t in range(lay.T):
        for k in range(K):
            e = r["ids"][t, k]
            h, row = oracle.expert_row_fmt(oracle.NVFP4, r["lat"][t], ex["w13_codes"][e],
                                           ex["w13_scales"][e], ex["w13_global"][e],
                                           ex["w2_codes"][e], ex["w2_scales"][e], ex["w2_global"][e])
            assert np.array_equal(row, r["rows"][t * K + k]) and np.array_equal(h, r["h"][t * K + k])
    # the same codes read as MXFP4 give a different layer
    mx = {k: v.numpy() for k, v in synth.all_expert_bytes(lay.dims, 0).items()}
    r2 = oracle.latent_forward(lay.dims, lay.x, lay.router, lay.pooler, ex["w13_codes"],
                               mx["w13_scales"], ex["w2_codes"], mx["w2_scales"], lay.gain,
                               lay.unpooler, lay.eps)
    assert not np.array_equal(r["out"], r2["out"])


# ---- A7: norm and weighted sum -----------------------------------------------------------------
def test_rmsnorm_closed_forms():
    L, eps = 64, 1e-6
    gain = synth.to_bf16_bits(np.linspace(0.5, 1.5, L))
    gf = exact.bf16_to_f64(gain)
    c = 0.375
    n = oracle.rmsnorm_row(np.full(L, c, np.float32), gain, eps)
    assert np.allclose(n, gf * c / np.sqrt(c * c + eps), rtol=1e-15, atol=0)
    row = np.zeros(L, np.float32)
    row[5] = 8.0
    n = oracle.rmsnorm_row(row, gain, eps)
    assert np.allclose(n[5], gf[5] * 8.0 / np.sqrt(64.0 / L + eps), rtol=1e-15)
    assert (np.delete(n, 5) == 0).all()
    # scale invariance up to eps
    rng = np.random.default_rng(1)
    r = rng.standard_normal(L).astype(np.float32)
    assert np.allclose(oracle.rmsnorm_row(r, gain, eps), oracle.rmsnorm_row(r * 4, gain, eps), rtol=1e-5)


def test_combine_weighted_sum_closed_form():
    K, L, eps = 3, 32, 1e-6
    rows = np.stack([np.full(L, 2.0), np.full(L, -0.5), np.full(L, 4.0)]).astype(np.float32)
    w = np.array([0.5, 0.25, 0.25], np.float32)
    gain = synth.to_bf16_bits(np.ones(L))
    y = oracle.combine(rows, w, np.array([0, 1, 2], np.int32), gain, 0, eps)
    s = [2 / np.sqrt(4 + eps), -0.5 / np.sqrt(0.25 + eps), 4 / np.sqrt(16 + eps)]
    expect = 0.5 * s[0] + 0.25 * s[1] + 0.25 * s[2]
    assert (y == exact.f64_to_bf16_bits(np.full(L, expect))).all()
    # per-expert gain picks the gain row of ids[k]
    gains = synth.to_bf16_bits(np.stack([np.full(L, 1.0), np.full(L, 2.0), np.full(L, 0.5)]))
    y2 = oracle.combine(rows, w, np.array([2, 0, 1], np.int32), gains, 1, eps)
    expect2 = 0.5 * s[0] * 0.5 + 0.25 * s[1] * 1.0 + 0.25 * s[2] * 2.0
    assert (y2 == exact.f64_to_bf16_bits(np.full(L, expect2))).all()


def test_norm_of_partial_rows_differs_from_norm_of_full_row():
    """"EP and TP layout": a norm of a partial sum is wrong, so partial route
    rows must be summed before the norm. Splitting the intermediate dimension
    into quarters: the partial rows add up to the full row, but the sum of the
    normed partials is far from the normed full row."""
    rng = np.random.default_rng(14)
    L, I = 64, 128
    w13c = rng.integers(0, 256, (2 * I, L // 2), dtype=np.uint8)
    w13s = rng.integers(119, 124, (2 * I, L // 32), dtype=np.uint8)
    w2c = rng.integers(0, 256, (L, I // 2), dtype=np.uint8)
    w2s = rng.integers(119, 124, (L, I // 32), dtype=np.uint8)
    lat = synth.to_bf16_bits(rng.standard_normal(L))
    _, full = oracle.expert_row(lat, w13c, w13s, w2c, w2s)
    parts = []
    for p in range(4):
        c = w2c.copy()
        keep = np.zeros(I // 2, bool)
        keep[p * I // 8:(p + 1) * I // 8] = True
        c[:, ~keep] = 0
        parts.append(oracle.expert_row(lat, w13c, w13s, c, w2s)[1])
    assert np.allclose(sum(parts), full, rtol=1e-5, atol=1e-6)
    gain = synth.to_bf16_bits(np.ones(L))
    nf = oracle.rmsnorm_row(full, gain, 1e-6)
    npart = sum(oracle.rmsnorm_row(p, gain, 1e-6) for p in parts)
    assert np.linalg.norm(npart - nf) / np.linalg.norm(nf) > 0.1


# ---- the whole layer ----------------------------------------------------------------------------------
def _tiny(gain_per_expert=False, seed=0):
    lay = synth.config_layer(0, seed=seed, gain_per_expert=gain_per_expert)
    ex = {k: v.numpy() for k, v in synth.all_expert_bytes(lay.dims, seed).items()}
    return lay, ex


def _forward(lay, ex, x=None, router=None, **over):
    args = dict(x=lay.x if x is None else x, router=lay.router if router is None else router,
                pooler=lay.pooler, unpooler=lay.unpooler, gain=lay.gain, **ex)
    args.update(over)
    return oracle.latent_forward(lay.dims, eps=lay.eps, gain_per_expert=lay.gain_per_expert, **args)


def test_zero_input_gives_zero_output_and_lowest_ids():
    lay, ex = _tiny()
    r = _forward(lay, ex, x=np.zeros_like(lay.x))
    assert (r["out"] == 0).all() and (r["ybf"] == 0).all()
    K = lay.dims["top_k"]
    assert (r["ids"] == np.arange(K)).all() and (r["w"] == np.float32(1.0 / K)).all()


def test_norm_placement_invariant_to_expert_output_scale():
    """Doubling an expert's W2 scales doubles its route rows exactly; the
    post-expert norm removes that, so the output is unchanged (up to eps).
    Doubling the up-projection half of W13 doubles h exactly: same.
    Doubling the gate half goes through silu and must change the output."""
    lay, ex = _tiny()
    base = _forward(lay, ex)
    e = int(base["ids"][0, 0])
    I = lay.dims["inter"]

    def with_(name, rows):
        t = {k: v.copy() for k, v in ex.items()}
        t[name][e, rows] += 1
        return _forward(lay, t)

    for name, rows in [("w2_scales", slice(None)), ("w13_scales", slice(I, 2 * I))]:
        r = with_(name, rows)
        assert not np.array_equal(r["rows"], base["rows"])
        d = np.abs(exact.bf16_to_f64(r["out"]) - exact.bf16_to_f64(base["out"]))
        assert d.max() <= 1e-2 and (d == 0).mean() > 0.99, name
    r = with_("w13_scales", slice(0, I))
    d = np.abs(exact.bf16_to_f64(r["out"]) - exact.bf16_to_f64(base["out"]))
    assert d.max() > 0.05


def test_expert_relabelling_leaves_output_unchanged():
    lay, ex = _tiny()
    base = _forward(lay, ex)
    E = lay.dims["n_experts"]
    perm = np.random.default_rng(2).permutation(E)     # new id of old expert e is perm[e]
    inv = np.argsort(perm)
    router2 = lay.router[inv]
    ex2 = {k: v[inv] for k, v in ex.items()}
    r = _forward(lay, ex2, router=router2)
    assert np.array_equal(r["out"], base["out"])
    assert np.array_equal(r["ids"], perm[base["ids"]])


def test_per_route_rows_are_the_expansion_of_the_token():
    """"The latent MoE" section: every (token, route) pair is its own row.
    The oracle's route rows equal one expert_row call per (t, k) with the
    selected expert, and y is their normed, weighted sum."""
    lay, ex = _tiny(gain_per_expert=True)
    r = _forward(lay, ex)
    K = lay.dims["top_k"]
    for t in range(lay.T):
        for k in range(K):
            e = r["ids"][t, k]
            h, row = oracle.expert_row(r["lat"][t], ex["w13_codes"][e], ex["w13_scales"][e],
                                       ex["w2_codes"][e], ex["w2_scales"][e])
            assert np.array_equal(row, r["rows"][t * K + k])
            assert np.array_equal(h, r["h"][t * K + k])
        y = oracle.combine(r["rows"][t * K:(t + 1) * K], r["w"][t], r["ids"][t], lay.gain, 1, lay.eps)
        assert np.array_equal(y, r["ybf"][t])


def _torch_deq(codes, scales):
    """MXFP4 decoded in float64 from the golden E2M1 table and torch's E8M0 dtype."""
    table = torch.tensor(exact.load_e2m1_table(), dtype=torch.float64)
    c = torch.from_numpy(codes.astype(np.int64))
    v = torch.stack([table[c & 15], table[c >> 4]], dim=-1).reshape(codes.shape[0], -1)
    s = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e8m0fnu).double()
    return v * s.repeat_interleave(32, dim=1)


def _torch_ffn(lat_bits, ex, e, I):
    """FFN_e(lat) in float64 torch from exactly decoded weights; h rounded to
    bf16 (a bf16 operand of the down projection), the row left unrounded."""
    f64 = lambda b: torch.from_numpy(exact.bf16_to_f64(b))
    gu = _torch_deq(ex["w13_codes"][e], ex["w13_scales"][e]) @ f64(lat_bits)
    h = f64(exact.f64_to_bf16_bits((torch.nn.functional.silu(gu[:I]) * gu[I:]).numpy()))
    return _torch_deq(ex["w2_codes"][e], ex["w2_scales"][e]) @ h


def _reduced_layer(T, E, K, seed=3):
    dims = dict(hidden=256, latent=128, inter=128, n_experts=E, top_k=K)
    lay = synth.make_layer(dims, T, seed=seed)
    ex = {k: v.numpy() for k, v in synth.all_expert_bytes(dims, seed).items()}
    return lay, ex


def test_identity_norm_route_path_equals_fused_weighted_topk_sum():
    """"Muse Spark Open on Gaudi 2", sections "Why it needed a port" and "The
    latent MoE: A' with a per-expert norm": the stock fused MXFP4 op returns
    the router-weighted top-K sum of expert outputs; the port expands the
    routes into rows so that a norm can sit between the expert and the
    weight. With that norm replaced by the identity the two must agree:

      (1) the oracle's layer (route rows -> identity norm -> weight -> sum),
      (2) the rows computed grouped by expert through the oracle's permutation
          and scattered back to route order, then weighted and summed, and
      (3) a fused token-major sum_k w_k * FFN_{e_k}(lat[t]) in float64 torch
          over exactly decoded weights, with no permutation at all.

    (1) and (2) run the same per-row arithmetic and must agree bit for bit;
    (3) differs from them only by the fp32 rounding of each route row (one
    bf16 ulp of y at most). Pairing a weight with another route of its token,
    or dropping the weights, is checked to move y far outside that bar."""
    lay, ex = _reduced_layer(T=24, E=16, K=4)
    dims = lay.dims
    L, I, E, K = dims["latent"], dims["inter"], dims["n_experts"], dims["top_k"]
    r = _forward(lay, ex, post_norm_identity=1)
    rms = _forward(lay, ex)
    assert np.array_equal(r["rows"], rms["rows"]) and np.array_equal(r["ids"], rms["ids"])
    assert not np.array_equal(r["ybf"], rms["ybf"])   # the mode does change A7
    T = lay.T
    ids, w = r["ids"], r["w"]
    # (2) grouped by expert through the permutation, rows scattered to route order
    offsets, srt = oracle.permute(ids, E)
    rows = np.full((T * K, L), np.nan, np.float32)
    for e in range(E):
        for i in range(offsets[e], offsets[e + 1]):
            route = int(srt[i])
            _, rows[route] = oracle.expert_row(r["lat"][route // K], ex["w13_codes"][e],
                                               ex["w13_scales"][e], ex["w2_codes"][e],
                                               ex["w2_scales"][e])
    assert np.isfinite(rows).all()
    y2 = np.zeros((T, L))
    for t in range(T):
        for k in range(K):
            y2[t] += float(w[t, k]) * rows[t * K + k].astype(np.float64)
    assert np.array_equal(exact.f64_to_bf16_bits(y2.ravel()).reshape(T, L), r["ybf"])
    # (3) fused token-major sum, no permutation
    y3 = torch.zeros(T, L, dtype=torch.float64)
    for t in range(T):
        for k in range(K):
            y3[t] += float(w[t, k]) * _torch_ffn(r["lat"][t], ex, int(ids[t, k]), I)
    y3b = exact.f64_to_bf16_bits(y3.numpy().ravel()).reshape(T, L)
    d = np.abs(y3b.astype(np.int64) - r["ybf"].astype(np.int64))
    assert d.max() <= 1 and (d == 0).mean() > 0.99
    tol = np.abs(y3.numpy()).max() * 2.0 ** -7
    # the bar is sensitive: a weight paired with the wrong route, or no weights
    for bad in (np.roll(w, 1, axis=1), np.ones_like(w)):
        yb = torch.zeros(T, L, dtype=torch.float64)
        for t in range(T):
            for k in range(K):
                yb[t] += float(bad[t, k]) * _torch_ffn(r["lat"][t], ex, int(ids[t, k]), I)
        assert np.abs(yb.numpy() - exact.bf16_to_f64(r["ybf"])).max() > 10 * tol


def test_single_expert_top1_closed_form():
    """E = K = 1: every token takes expert 0 with weight exactly 1, and the
    layer reduces to out = unpool(bf16(rmsnorm(FFN(pool(x))))): a closed form
    written here in float64 torch over exactly decoded weights (rounded to
    bf16 where the layer stores bf16: latent, h, y, out)."""
    lay, ex = _reduced_layer(T=5, E=1, K=1, seed=7)
    r = _forward(lay, ex)
    assert (r["ids"] == 0).all() and (r["w"] == np.float32(1.0)).all()
    I = lay.dims["inter"]
    f64 = lambda b: torch.from_numpy(exact.bf16_to_f64(b))
    gain = f64(lay.gain)
    lat = exact.f64_to_bf16_bits((f64(lay.x) @ f64(lay.pooler).T).numpy().ravel()).reshape(r["lat"].shape)
    assert np.array_equal(lat, r["lat"])
    for t in range(lay.T):
        row = _torch_ffn(lat[t], ex, 0, I).float().double()   # route rows are fp32
        y = row / torch.sqrt((row * row).mean() + lay.eps) * gain
        ybf = exact.f64_to_bf16_bits(y.numpy())
        assert np.abs(ybf.astype(np.int64) - r["ybf"][t].astype(np.int64)).max() <= 1
        out = exact.f64_to_bf16_bits((f64(ybf) @ f64(lay.unpooler).T).numpy())
        d = np.abs(exact.bf16_to_f64(out) - exact.bf16_to_f64(r["out"][t]))
        assert d.max() <= 2e-2 and (out == r["out"][t]).mean() > 0.95


def test_token_forward_matches_latent_forward():
    lay, ex = _tiny()
    r = _forward(lay, ex)
    get = lambda e: (ex["w13_codes"][e], ex["w13_scales"][e], ex["w2_codes"][e], ex["w2_scales"][e])
    for t in range(lay.T):
        tf = oracle.token_forward(lay.dims, lay.x[t], lay.router, lay.pooler, lay.gain,
                                  lay.unpooler, lay.eps, 0, get)
        assert np.array_equal(tf["out"], r["out"][t])
        assert np.array_equal(tf["rows"], r["rows"][t * lay.dims["top_k"]:(t + 1) * lay.dims["top_k"]])


def _routed(lay, ex, ids, w, x=None):
    return oracle.latent_forward_routed(lay.dims, lay.x if x is None else x, ids, w, lay.pooler,
                                        ex["w13_codes"], ex["w13_scales"], ex["w2_codes"],
                                        ex["w2_scales"], lay.gain, lay.unpooler, lay.eps,
                                        lay.gain_per_expert)


def test_routed_with_router_choice_equals_full_layer():
    lay, ex = _tiny(gain_per_expert=True)
    base = _forward(lay, ex)
    r = _routed(lay, ex, base["ids"], base["w"])
    for k in ("out", "lat", "h", "rows", "ybf"):
        assert np.array_equal(r[k], base[k]), k


def test_routed_weights_scale_output_exactly():
    """y is linear in the router weights and the unpooler is linear in y:
    doubling every weight doubles ybf and out exactly (a power-of-two scale
    commutes with rounding), so a weight that is dropped, renormalised or
    paired with the wrong route fails."""
    lay, ex = _tiny()
    T, K, E = lay.T, lay.dims["top_k"], lay.dims["n_experts"]
    rng = np.random.default_rng(5)
    ids = rng.integers(0, E, (T, K)).astype(np.int32)
    w = rng.uniform(0.05, 1.0, (T, K)).astype(np.float32)
    a = _routed(lay, ex, ids, w)
    b = _routed(lay, ex, ids, 2 * w)
    assert np.array_equal(exact.bf16_to_f64(b["ybf"]), 2 * exact.bf16_to_f64(a["ybf"]))
    assert np.array_equal(exact.bf16_to_f64(b["out"]), 2 * exact.bf16_to_f64(a["out"]))
    # one route's weight alone: y is exactly that weight times its normed row
    w1 = np.zeros_like(w)
    w1[:, 2] = w[:, 2]
    c = _routed(lay, ex, ids, w1)
    for t in range(T):
        row = c["rows"][t * K + 2]
        nrm = oracle.rmsnorm_row(row, lay.gain, lay.eps)
        want = np.array([oracle.round_bf16(float(w1[t, 2]) * v) for v in nrm], np.uint16)
        assert np.array_equal(c["ybf"][t], want)


def test_routed_zero_weight_route_id_is_irrelevant():
    lay, ex = _tiny()
    T, K, E = lay.T, lay.dims["top_k"], lay.dims["n_experts"]
    rng = np.random.default_rng(6)
    ids = rng.integers(0, E, (T, K)).astype(np.int32)
    w = rng.uniform(0.05, 1.0, (T, K)).astype(np.float32)
    w[:, K - 1] = 0.0
    a = _routed(lay, ex, ids, w)
    ids2 = ids.copy()
    ids2[:, K - 1] = (ids[:, K - 1] + 5) % E
    b = _routed(lay, ex, ids2, w)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["ybf"], b["ybf"])
    assert not np.array_equal(a["rows"], b["rows"])


def test_routed_repeated_expert_is_one_normed_row():
    """A token listing one expert K times has K identical route rows; with
    weights summing to s, y = s * rmsnorm(row) before rounding."""
    lay, ex = _tiny()
    T, K = lay.T, lay.dims["top_k"]
    ids = np.full((T, K), 3, np.int32)
    w = np.full((T, K), 0.25, np.float32)  # K = 4: s = 1
    r = _routed(lay, ex, ids, w)
    for t in range(T):
        rows = r["rows"][t * K:(t + 1) * K]
        assert (rows == rows[0]).all()
        nrm = oracle.rmsnorm_row(rows[0], lay.gain, lay.eps)
        want = np.array([oracle.round_bf16(float(K * 0.25) * v) for v in nrm], np.uint16)
        assert np.array_equal(r["ybf"][t], want)


def test_routed_order_of_a_tokens_routes_only_reorders_the_sum():
    lay, ex = _tiny(gain_per_expert=True)
    T, K, E = lay.T, lay.dims["top_k"], lay.dims["n_experts"]
    rng = np.random.default_rng(7)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.05, 1.0, (T, K)).astype(np.float32)
    a = _routed(lay, ex, ids, w)
    perm = np.array([3, 1, 0, 2])
    b = _routed(lay, ex, ids[:, perm], w[:, perm])
    ya, yb = exact.bf16_to_f64(a["ybf"]), exact.bf16_to_f64(b["ybf"])
    ulp = np.ldexp(1.0, np.frexp(np.abs(ya))[1] - 8)
    assert (np.abs(ya - yb) <= ulp).all() and (ya == yb).mean() > 0.99


def test_routed_rejects_ids_outside_the_experts():
    lay, ex = _tiny()
    T, K, E = lay.T, lay.dims["top_k"], lay.dims["n_experts"]
    ids = np.zeros((T, K), np.int32)
    ids[1, 2] = E
    with pytest.raises(ValueError):
        _routed(lay, ex, ids, np.ones((T, K), np.float32))


# ---- the block around the layer: sandwich norms ------------------------------------------------------
def _ulp_f32(a, b):
    """Distance in fp32 units in the last place (sign-magnitude order)."""
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


def _bf16_rows(rng, T, H, scale=1.0):
    return synth.to_bf16_bits(rng.standard_normal((T, H)) * scale)


def test_pre_norm_matches_torch_rms_norm_in_float64():
    rng = np.random.default_rng(21)
    T, H = 5, 512
    x = _bf16_rows(rng, T, H)
    g = synth.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(H))
    nf, nb = oracle.pre_norm(x, g, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(exact.bf16_to_f64(x)), (H,),
                                       weight=torch.from_numpy(exact.bf16_to_f64(g)), eps=1e-6).numpy()
    ud = _ulp_f32(nf, ref.astype(np.float32))
    assert ud.max() <= 1 and (ud == 0).mean() > 0.9999
    want_b = np.array([[oracle.round_bf16(v) for v in row] for row in ref], np.uint16)
    assert (nb == want_b).mean() > 0.9999
    assert np.abs(exact.bf16_to_f64(nb) - ref).max() <= np.abs(ref).max() * 2.0 ** -8


def test_pre_norm_scale_invariant_without_eps():
    """With eps = 0, doubling the row doubles its root mean square exactly
    (sqrt(4q) = 2 sqrt(q) in IEEE arithmetic): the outputs are unchanged."""
    rng = np.random.default_rng(22)
    x = _bf16_rows(rng, 3, 256)
    g = synth.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(256))
    x2 = synth.to_bf16_bits(2.0 * exact.bf16_to_f64(x))
    a, b = oracle.pre_norm(x, g, 0.0), oracle.pre_norm(x2, g, 0.0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_post_norm_residual_closed_forms():
    rng = np.random.default_rng(23)
    T, H = 4, 384
    r = _bf16_rows(rng, T, H)
    f = _bf16_rows(rng, T, H, 0.3)
    g = synth.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(H))
    # F = 0: the residual passes through exactly
    assert np.array_equal(oracle.post_norm_residual(r, np.zeros_like(f), g, 1e-6), r)
    # residual 0: the bf16 rounding of torch's RMS norm
    out = oracle.post_norm_residual(np.zeros_like(r), f, g, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(exact.bf16_to_f64(f)), (H,),
                                       weight=torch.from_numpy(exact.bf16_to_f64(g)), eps=1e-6).numpy()
    want = np.array([[oracle.round_bf16(v) for v in row] for row in ref], np.uint16)
    assert (out == want).mean() > 0.999
    assert np.abs(exact.bf16_to_f64(out) - ref).max() <= np.abs(ref).max() * 2.0 ** -8
    # general: resid + normed f, one rounding
    out = oracle.post_norm_residual(r, f, g, 1e-6)
    want = np.array([[oracle.round_bf16(a + b) for a, b in zip(ra, rb)]
                     for ra, rb in zip(exact.bf16_to_f64(r), ref)], np.uint16)
    assert (out == want).mean() > 0.999


def test_router_logits_f32_exact_sums():
    rng = np.random.default_rng(24)
    T, H, E = 3, 64, 5
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (0.02 * rng.standard_normal((E, H))).astype(np.float32)
    got = oracle.router_logits_f32(x, wr)
    for t in range(T):
        for e in range(E):
            exact_sum = sum(Fraction(float(x[t, h])) * Fraction(float(wr[e, h])) for h in range(H))
            assert got[t, e] == np.float32(float(exact_sum))
    xb = synth.to_bf16_bits(rng.standard_normal((T, H)))
    assert np.array_equal(oracle.router_logits_f32(exact.bf16_to_f64(xb).astype(np.float32), wr),
                          oracle.router_logits(xb, wr))


def _block(lay, ex, resid, pre_gain, post_gain, block_eps=1e-6):
    return oracle.block_forward(lay.dims, resid, pre_gain, post_gain, block_eps, lay.router,
                                lay.pooler, ex["w13_codes"], ex["w13_scales"], ex["w2_codes"],
                                ex["w2_scales"], lay.gain, lay.unpooler, lay.eps,
                                lay.gain_per_expert)


def test_block_is_the_composition_of_its_steps():
    lay, ex = _tiny(gain_per_expert=True)
    rng = np.random.default_rng(25)
    H, K = lay.dims["hidden"], lay.dims["top_k"]
    pre = synth.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(H))
    post = synth.to_bf16_bits(0.5 + 0.1 * rng.standard_normal(H))
    b = _block(lay, ex, lay.x, pre, post)
    nf, nb = oracle.pre_norm(lay.x, pre, 1e-6)
    assert np.array_equal(b["n_f32"], nf) and np.array_equal(b["n_bf16"], nb)
    logits = oracle.router_logits_f32(nf, lay.router)
    ids, w = oracle.topk(logits, K)
    assert np.array_equal(b["logits"], logits) and np.array_equal(b["ids"], ids)
    f = _routed(lay, ex, ids, w, x=nb)["out"]
    assert np.array_equal(b["f"], f)
    assert np.array_equal(b["out"], oracle.post_norm_residual(lay.x, f, post, 1e-6))


def test_block_with_zero_post_gain_is_the_identity():
    lay, ex = _tiny()
    H = lay.dims["hidden"]
    pre = synth.to_bf16_bits(np.ones(H))
    b = _block(lay, ex, lay.x, pre, np.zeros(H, np.uint16))
    assert np.array_equal(b["out"], lay.x)
    assert not (b["f"] == 0).all()


def test_second_formulation_in_torch_float64():
    """The layer written as whole-matrix float64 torch operations, with MXFP4
    decoded through the golden E2M1 table and torch's E8M0 dtype."""
    lay, ex = _tiny(gain_per_expert=True)
    r = _forward(lay, ex)
    d = lay.dims
    H, L, I, E, K = d["hidden"], d["latent"], d["inter"], d["n_experts"], d["top_k"]
    f64 = lambda b: torch.from_numpy(exact.bf16_to_f64(b))
    x = f64(lay.x)
    logits = (x @ torch.from_numpy(lay.router).double().T).float()
    assert (logits.numpy() == r["logits"]).mean() > 0.99
    ids = torch.sort(-logits, dim=1, stable=True).indices[:, :K]
    assert np.array_equal(ids.numpy(), r["ids"])
    sel = torch.gather(logits, 1, ids).double()
    w = torch.softmax(sel, dim=1).float()
    assert np.allclose(w.numpy(), r["w"], rtol=2e-7, atol=0)
    lat = (x @ f64(lay.pooler).T)
    lat_b = exact.f64_to_bf16_bits(lat.numpy())
    assert np.array_equal(lat_b, r["lat"])
    table = torch.tensor(exact.load_e2m1_table(), dtype=torch.float64)

    def deq(codes, scales):
        c = torch.from_numpy(codes.astype(np.int64))
        v = torch.stack([table[c & 15], table[c >> 4]], dim=-1).reshape(codes.shape[0], -1)
        s = torch.from_numpy(scales).view(torch.float8_e8m0fnu).double()
        return v * s.repeat_interleave(32, dim=1)

    y = torch.zeros(lay.T, L, dtype=torch.float64)
    latd = f64(lat_b)
    gain = f64(lay.gain)
    for t in range(lay.T):
        for k in range(K):
            e = int(ids[t, k])
            w13 = deq(ex["w13_codes"][e], ex["w13_scales"][e])
            gu = w13 @ latd[t]
            h = f64(exact.f64_to_bf16_bits((torch.nn.functional.silu(gu[:I]) * gu[I:]).numpy()))
            row = (deq(ex["w2_codes"][e], ex["w2_scales"][e]) @ h).float().double()
            nrm = row / torch.sqrt((row * row).mean() + lay.eps) * gain[e]
            y[t] += float(r["w"][t, k]) * nrm
    ybf = exact.f64_to_bf16_bits(y.numpy())
    assert np.abs(ybf.astype(np.int64) - r["ybf"].astype(np.int64)).max() <= 1
    out = f64(ybf) @ f64(lay.unpooler).T
    diff = np.abs(out.numpy() - exact.bf16_to_f64(r["out"]))
    assert diff.max() <= 2e-2


def test_skewed_workload_routes_half_to_top16():
    """The skewed workload's bias puts about half of the routes on the 16 most
    popular experts (through the oracle's router)."""
    lay = synth.config_layer(4)
    ids, _ = oracle.topk(oracle.router_logits(lay.x, lay.router), lay.dims["top_k"])
    counts = np.sort(np.bincount(ids.ravel(), minlength=lay.dims["n_experts"]))[::-1]
    share = counts[:16].sum() / ids.size
    assert 0.45 <= share <= 0.55, share
