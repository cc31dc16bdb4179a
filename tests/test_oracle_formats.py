"""Pins for oracle.formats: decoders against the OCP spec points and torch's float8
type, encoders against a brute-force nearest-value search, tie and saturation tables."""
import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle.formats import (bf16_bits_to_f32, e2m1_decode, e2m1_encode, e4m3_decode,
                            e4m3_encode, f32_to_bf16_bits)


def all_finite_bf16_as_f32():
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    return f[np.isfinite(f)]


def brute_encode(a, values):
    """Nearest of ``values`` (non-negative magnitudes, indexed by code) to each |a|;
    ties go to the even code; anything above the largest value maps to it."""
    mag = np.abs(a.astype(np.float64))
    # beyond twice the largest value the nearest one cannot change; clipping keeps the
    # float64 distances below exact-representation limits
    mag = np.minimum(mag, 2 * values[-1])
    dist = np.abs(mag[:, None] - values[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    codes = np.arange(len(values))
    # among tied candidates prefer the even code (at most two candidates tie)
    even_pick = np.where(cand & (codes[None, :] % 2 == 0), codes[None, :], 10 ** 6).min(axis=1)
    any_pick = np.where(cand, codes[None, :], 10 ** 6).min(axis=1)
    return np.where(even_pick < 10 ** 6, even_pick, any_pick)


E4M3_POS = e4m3_decode(np.arange(0x7F))          # finite non-negative values, by code
E2M1_POS = e2m1_decode(np.arange(8))


def test_e4m3_decode_golden():
    for code, val in read_golden("e4m3_ocp_points.txt"):
        got = e4m3_decode(int(code, 16))
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-")


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3_decode(codes)
    nan = np.isnan(t)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(t[~nan], ours[~nan])
    assert np.array_equal(np.signbit(t[~nan]), np.signbit(ours[~nan]))


def test_e4m3_values_monotone_and_max():
    assert np.all(np.diff(E4M3_POS) > 0)
    assert E4M3_POS[-1] == 448.0 and E4M3_POS[0] == 0.0


@pytest.mark.parametrize("scale_exp", [-12, -7, 0, 3, 9])
def test_e4m3_encode_bruteforce_all_bf16(scale_exp):
    a = np.ldexp(all_finite_bf16_as_f32().astype(np.float64), scale_exp)
    a = a[np.abs(a) < 3.0e38].astype(np.float32)
    got = e4m3_encode(a)
    exp = brute_encode(a, E4M3_POS) | (np.signbit(a).astype(np.int64) << 7)
    assert np.array_equal(got.astype(np.int64), exp)


def test_e4m3_encode_bruteforce_midpoints():
    # every midpoint between neighbouring codes, and one float32 ulp either side
    mids = ((E4M3_POS[:-1] + E4M3_POS[1:]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                           np.float32([448, 448.01, 463.99, 464, 464.01, 479, 480, 1e6])])
    near = np.concatenate([near, -near])
    got = e4m3_encode(near)
    exp = brute_encode(near, E4M3_POS) | (np.signbit(near).astype(np.int64) << 7)
    assert np.array_equal(got.astype(np.int64), exp)


def test_e4m3_encode_matches_torch_unsaturated():
    rng = np.random.default_rng(7)
    a = np.concatenate([all_finite_bf16_as_f32(),
                        rng.uniform(-448, 448, 200000).astype(np.float32),
                        (rng.standard_normal(200000) * 1e-3).astype(np.float32)])
    a = a[np.abs(a) <= 448]
    t = torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(a), t)


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(e4m3_encode(vals), codes)


def test_e2m1_decode_golden():
    for code, val in read_golden("e2m1_values.txt"):
        got = e2m1_decode(int(code))
        assert got == float(val) and np.signbit(got) == val.startswith("-")


@pytest.mark.parametrize("scale_exp", [-3, 0, 2])
def test_e2m1_encode_bruteforce_all_bf16(scale_exp):
    a = np.ldexp(all_finite_bf16_as_f32().astype(np.float64), scale_exp)
    a = a[np.abs(a) < 3.0e38].astype(np.float32)
    got = e2m1_encode(a)
    exp = brute_encode(a, E2M1_POS) | (np.signbit(a).astype(np.int64) << 3)
    assert np.array_equal(got.astype(np.int64), exp)


def test_e2m1_roundtrip():
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(e2m1_encode(e2m1_decode(codes).astype(np.float32)), codes)


def test_tie_and_saturation_table():
    for fmt, val, code in read_golden("rounding_ties.txt"):
        v = np.float32([float(val)])
        got = (e4m3_encode if fmt == "e4m3" else e2m1_encode)(v)[0]
        assert got == int(code, 16), (fmt, val, hex(got))


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 100,
                        (rng.integers(0, 2 ** 31, 100000, dtype=np.uint32) & 0x7F7FFFFF).view(np.float32)])
    # exact ties: low half exactly 0x8000 with odd and even kept halves
    u = (rng.integers(0, 2 ** 15, 1000, dtype=np.uint32) << 16) | 0x8000
    x = np.concatenate([x, u.view(np.float32), -u.view(np.float32)])
    x = x[np.isfinite(x) & (np.abs(x) < 3.3e38)]
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), t)
    assert np.array_equal(bf16_bits_to_f32(t), torch.from_numpy(t.view(np.int16)).view(torch.bfloat16).float().numpy())
