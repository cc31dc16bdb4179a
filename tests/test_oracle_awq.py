"""Pins for oracle.awq (group-wise 4-bit weights with bf16 activations): exact
round trips of grid weights, zero as a grid point, the rounding error bound,
nibble order, all-zero groups, and a brute-force dot product."""
from fractions import Fraction

import numpy as np
import pytest

from oracle.awq import dequant_w4g, qlinear_w4a16_ref, quant_w4g
from oracle.formats import bf16_bits_to_f32
from oracle.quant import unpack_e2m1
from synthetic import bf16_round

F32 = np.float32


def to_bits(v):
    return bf16_round(np.asarray(v, dtype=F32))


@pytest.mark.parametrize("group", [32, 64, 128])
def test_grid_weights_round_trip(group):
    # each group holds (j - z) s for codes j, including j = 0 and j = 15, with s a
    # power of two: the rule must give back s, z and the codes exactly
    rng = np.random.default_rng(group)
    N, K = 6, 4 * group
    ng = K // group
    s = np.ldexp(1.0, rng.integers(-12, 3, size=(N, ng)))
    z = rng.integers(0, 16, size=(N, ng))
    q = rng.integers(0, 16, size=(N, ng, group))
    q[:, :, 0], q[:, :, 1] = 0, 15
    w = ((q - z[:, :, None]) * s[:, :, None]).reshape(N, K)
    packed, sb, zz = quant_w4g(to_bits(w), group)
    assert np.array_equal(bf16_bits_to_f32(sb), s.astype(F32))
    assert np.array_equal(zz, z.astype(np.uint8))
    assert np.array_equal(unpack_e2m1(packed), q.reshape(N, K).astype(np.uint8))
    assert np.array_equal(dequant_w4g(packed, sb, zz, group), w)


def test_zero_is_a_grid_point():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((8, 256)).astype(F32) * F32(0.02)
    w[rng.random(w.shape) < 0.2] = 0.0
    w[0, :64] = np.abs(w[0, :64]) + F32(0.01)     # positive-only group: range widened to 0
    w[1, :64] = -np.abs(w[1, :64]) - F32(0.01)    # negative-only group
    bits = to_bits(w)
    packed, sb, z = quant_w4g(bits, 64)
    d = dequant_w4g(packed, sb, z, 64)
    zero = bf16_bits_to_f32(bits) == 0
    assert np.all(d[zero] == 0.0)
    assert z[0, 0] == 0 and z[1, 0] == 15


@pytest.mark.parametrize("group", [32, 64, 128])
def test_rounding_error_bound(group):
    # inside the grid's span a weight is at most s/2 from its value; the span ends
    # at -z s and (15 - z) s, within s/2 (the rounding of z) plus the bf16 rounding
    # of s (15 s >= (hi - lo)(1 - 2^-8)) of the group's range
    rng = np.random.default_rng(10 + group)
    w = rng.standard_normal((16, 512)) * 0.02
    w[3] *= 1e-20
    w[4] *= 1e20
    w[5] = np.abs(w[5]) + 0.01    # groups of one sign: the span must still reach 0
    w[6] = -np.abs(w[6]) - 0.01
    bits = to_bits(w)
    w = bf16_bits_to_f32(bits).astype(np.float64)
    packed, sb, z = quant_w4g(bits, group)
    d = dequant_w4g(packed, sb, z, group)
    s = np.repeat(bf16_bits_to_f32(sb).astype(np.float64), group, axis=1)
    zz = np.repeat(z.astype(np.float64), group, axis=1)
    err = np.abs(w - d)
    inside = (w >= -zz * s) & (w <= (15 - zz) * s)
    assert np.all(err[inside] <= s[inside] * (0.5 + 2.0 ** -20))
    rng_w = np.repeat(np.maximum(w.reshape(16, -1, group).max(2), 0) - np.minimum(w.reshape(16, -1, group).min(2), 0),
                      group, axis=1)
    assert np.all(err <= s * (1.0 + 2.0 ** -20) + rng_w * 2.0 ** -8)
    assert inside.mean() > 0.9


def test_nibble_order_low_is_even():
    w = np.zeros((1, 32), F32)
    w[0, 0] = 1.0       # largest: code 15 with z = 0
    w[0, 1] = 0.5
    packed, sb, z = quant_w4g(to_bits(w), 32)
    assert z[0, 0] == 0
    assert packed[0, 0] & 0xF == 15
    assert packed[0, 0] >> 4 == int(np.rint(F32(0.5) / bf16_bits_to_f32(sb)[0, 0]))


def test_all_zero_group():
    w = np.zeros((2, 64), F32)
    w[1, 32:] = 1.0
    packed, sb, z = quant_w4g(to_bits(w), 32)
    assert sb[0, 0] == 0 and z[0, 0] == 0 and np.all(packed[0] == 0)
    assert np.all(dequant_w4g(packed, sb, z, 32)[0] == 0)


def test_gemv_brute_force():
    # y[m, n] = sum_k x[m, k] (q[n, k] - z[n, g(k)]) s[n, g(k)], summed exactly
    rng = np.random.default_rng(7)
    M, K, N, G = 3, 64, 5, 32
    x = to_bits(rng.standard_normal((M, K)))
    w = to_bits(rng.standard_normal((N, K)) * 0.02)
    packed, sb, z = quant_w4g(w, G)
    y = qlinear_w4a16_ref(x, packed, sb, z, G)
    xv = bf16_bits_to_f32(x)
    sv = bf16_bits_to_f32(sb)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                byte = int(packed[n, k // 2])
                q = (byte >> 4) if k % 2 else (byte & 15)
                acc += Fraction(float(xv[m, k])) * (q - int(z[n, k // G])) * Fraction(float(sv[n, k // G]))
            assert abs(float(acc) - y[m, n]) <= 1e-12 * max(1.0, abs(float(acc)))
