"""Pins for oracle.epilogue: the tanh form of GELU against the exact (erf) GELU
and its own identities, the interval bounds against brute force, the nvfp4
validity check against the oracle quantizer (accepts every quantization of a point
in the box, rejects planted changes), and the QKV scatter on a hand-made case."""
import math

import numpy as np
import pytest

from oracle.epilogue import (GELU_ARGMIN, bf16_interval, check_nvfp4_expanded, expanded_nominal_and_width,
                             gelu_interval, gelu_tanh, nvfp4_expanded_bounds, qkv_split_ref, smooth_interval)
from oracle.formats import bf16_bits_to_f32, f32_to_bf16_bits
from oracle.quant import quant_nvfp4, smooth_bf16
from oracle.reference import dequant_nvfp4
from synthetic import bf16_round

F32 = np.float32


def erf_gelu(v):
    return np.array([0.5 * x * (1.0 + math.erf(x / math.sqrt(2.0))) for x in v])


def test_gelu_tanh_tracks_exact_gelu():
    # the tanh form stays within 5e-4 of v Phi(v) everywhere (max about 4.73e-4);
    # a cubic coefficient off by 0.005, or a missing cubic term, exceeds 2e-3
    v = np.linspace(-12, 12, 48001)
    d = np.abs(gelu_tanh(v) - erf_gelu(v))
    assert d.max() < 5e-4 and d.max() > 4e-4
    for x, want in [(1.0, 0.8413447460685429), (-1.0, -0.15865525393145707), (2.0, 1.9544997361036416)]:
        assert abs(gelu_tanh(x) - want) < 5e-4


def test_gelu_tanh_is_the_tanh_form():
    # where 1 + tanh(u) keeps most digits (it is above 1e-5 for v >= -4), the
    # printed tanh form agrees to its own cancellation error
    v = np.linspace(-4, 8, 1201)
    t = 0.5 * v * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (v + 0.044715 * v ** 3)))
    assert np.allclose(gelu_tanh(v), t, rtol=1e-9, atol=0)
    # and it stays monotone and relatively accurate in the far negative tail
    w = np.linspace(-12, -6, 3001)
    g = gelu_tanh(w)
    assert np.all(np.diff(g) < 0) and np.all(g < 0)


def test_gelu_tanh_identities():
    v = np.linspace(-8, 8, 1601)
    # v/2 (1 + t(v)) - (-v)/2 (1 + t(-v)) = v for any odd t
    assert np.allclose(gelu_tanh(v) - gelu_tanh(-v), v, rtol=0, atol=1e-14)
    assert gelu_tanh(0.0) == 0.0
    h = 1e-6
    assert abs((gelu_tanh(h) - gelu_tanh(-h)) / (2 * h) - 0.5) < 1e-9
    assert gelu_tanh(30.0) == 30.0 and abs(gelu_tanh(-30.0)) < 1e-300
    # the minimum: derivative changes sign across GELU_ARGMIN, value about -0.170
    assert gelu_tanh(GELU_ARGMIN) < gelu_tanh(GELU_ARGMIN - 1e-3)
    assert gelu_tanh(GELU_ARGMIN) < gelu_tanh(GELU_ARGMIN + 1e-3)
    assert abs(gelu_tanh(GELU_ARGMIN) + 0.17004) < 1e-4


def test_gelu_interval_holds_every_point():
    rng = np.random.default_rng(4)
    ref = np.concatenate([rng.standard_normal(400) * 3, [GELU_ARGMIN, -0.7, -0.8, 0.0, 8.0, -6.0]])
    err = np.abs(rng.standard_normal(ref.size)) * 0.05
    lo, hi = gelu_interval(ref, err)
    for t in np.linspace(-1, 1, 201):
        g = gelu_tanh(ref + t * err)
        assert np.all(g >= lo) and np.all(g <= hi)
    assert np.all(hi - lo >= 0)


def test_bf16_interval_brute_force():
    rng = np.random.default_rng(5)
    c = rng.standard_normal(300) * 10.0 ** rng.integers(-3, 3, 300)
    lo, hi = c - np.abs(c) * 1e-3, c + np.abs(c) * 1e-3
    lb, hb = bf16_interval(lo, hi)
    vl, vh = bf16_bits_to_f32(lb).astype(np.float64), bf16_bits_to_f32(hb).astype(np.float64)
    for t in np.linspace(0, 1, 101):
        x = (lo + t * (hi - lo)).astype(F32)
        r = bf16_bits_to_f32(f32_to_bf16_bits(x)).astype(np.float64)
        assert np.all(r >= vl) and np.all(r <= vh)
    # the end points are reached
    assert np.array_equal(lb, f32_to_bf16_bits(lo.astype(F32))) or np.all(vl <= bf16_bits_to_f32(
        f32_to_bf16_bits(lo.astype(F32))))


def random_box(rng, R, K, ambiguous=0.02):
    x = bf16_round((rng.standard_normal((R, K)) * np.exp(rng.uniform(-3, 3, (R, 1)))).astype(F32))
    lo, hi = x.copy(), x.copy()
    # a few elements may take one of two neighbouring bf16 values
    m = rng.random((R, K)) < ambiguous
    hi[m] = hi[m] + np.where(bf16_bits_to_f32(x[m]) >= 0, 1, -1).astype(np.uint16)
    vl, vh = bf16_bits_to_f32(lo), bf16_bits_to_f32(hi)
    swap = vl > vh
    lo[swap], hi[swap] = hi[swap], lo[swap].copy()
    return x, lo, hi


def expanded(x_bits, g):
    p, bs = quant_nvfp4(x_bits, g)
    return f32_to_bf16_bits(dequant_nvfp4(p, bs, 1.0).astype(F32))


def test_check_accepts_every_quantization_in_the_box():
    rng = np.random.default_rng(6)
    R, K, g = 8, 256, F32(0.02)
    _, lo, hi = random_box(rng, R, K)
    for trial in range(20):
        pick = rng.random((R, K)) < 0.5
        x = np.where(pick, lo, hi)
        r = check_nvfp4_expanded(expanded(x, g), lo, hi, g)
        assert r["ok"], (trial, r)
    assert r["ambiguous_blocks"] > 0


def test_check_is_exact_on_a_point_and_rejects_plants():
    rng = np.random.default_rng(7)
    R, K, g = 6, 128, F32(0.01)
    x, _, _ = random_box(rng, R, K, ambiguous=0.0)
    xe = expanded(x, g)
    r = check_nvfp4_expanded(xe, x, x, g)
    assert r["ok"] and r["ambiguous_blocks"] == 0
    # one code one step up, a value off the E2M1 grid, a whole block rescaled by 2
    v = bf16_bits_to_f32(xe).astype(np.float64)
    nz = np.flatnonzero(np.abs(v[0]) > 0)[0]
    for plant in ("code", "grid", "scale"):
        w = v.copy()
        if plant == "code":
            w[0, nz] = w[0, nz] * (1.5 if abs(w[0, nz]) > 0 else 1)
        elif plant == "grid":
            w[0, nz] = w[0, nz] * 1.25
        else:
            w[1, :16] = w[1, :16] * 2
        bad = check_nvfp4_expanded(f32_to_bf16_bits(w.astype(F32)), x, x, g)
        assert not bad["ok"], plant


def test_check_with_smoothing_interval():
    rng = np.random.default_rng(8)
    R, K, g = 4, 192, F32(0.05)
    _, lo, hi = random_box(rng, R, K, ambiguous=0.05)
    lam = np.exp(rng.standard_normal(K) * 0.3).astype(F32)
    sl, sh = smooth_interval(lo, hi, lam)
    for trial in range(10):
        x = np.where(rng.random((R, K)) < 0.5, lo, hi)
        r = check_nvfp4_expanded(expanded(smooth_bf16(x, lam), g), sl, sh, g)
        assert r["ok"], (trial, r)


def test_expanded_width_covers_the_box():
    rng = np.random.default_rng(9)
    R, K, g = 4, 128, F32(0.03)
    x, lo, hi = random_box(rng, R, K, ambiguous=0.1)
    nominal, width = expanded_nominal_and_width(x, lo, hi, g)
    assert np.array_equal(f32_to_bf16_bits(nominal.astype(F32)), expanded(x, g))
    for trial in range(10):
        y = np.where(rng.random((R, K)) < 0.5, lo, hi)
        e = bf16_bits_to_f32(expanded(y, g)).astype(np.float64)
        assert np.all(np.abs(e - nominal) <= width)
    # sf range well formed
    sl, sh, _, _ = nvfp4_expanded_bounds(lo, hi, g)
    assert np.all(sl <= sh)


def test_qkv_split_hand_case():
    heads, hd, M = 2, 4, 3
    y = np.arange(M * 3 * heads * hd, dtype=np.float64).reshape(M, 3 * heads * hd)
    q, k, v = qkv_split_ref(y, heads, hd, tokens=5, offset=1)
    assert q.shape == (2, 5, 4) and np.isnan(q[:, 0]).all() and np.isnan(q[:, 4]).all()
    # token 1 + m, head h, element e of q is y[m, h hd + e]; k and v follow at +8 and +16
    assert q[1, 2, 3] == y[1, 4 + 3] and k[0, 1, 0] == y[0, 8] and v[1, 3, 2] == y[2, 16 + 4 + 2]
