"""GPU parity of the weight-only 4-bit linear (awq_w4a16) against the oracle:
bit-exact codes, scales and zero points from quant_weight_awq; qlinear_awq_w4a16
within the GEMM acceptance test (oracle.reference.check_gemm: relative Frobenius
error <= 2e-3, per element 4 bf16 ulps plus the fp32 accumulation floor
ceil(K/16) 2^-24 sum_k |x_k w_k|) on weights quantized by the oracle."""
import numpy as np
import pytest
import torch

import precision_quantized_linear_amd as qpl
from helpers import adversarial_rows, bf16_bits, host, to_dev, to_dev_bf16
from oracle.awq import dequant_w4g, quant_w4g
from oracle.formats import bf16_bits_to_f32
from oracle.reference import check_gemm
from synthetic import bf16_round, make

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def gpu_quant(w_bits, group):
    q, s, z = qpl.quant_weight_awq(to_dev_bf16(w_bits), group)
    torch.cuda.synchronize()
    return host(q), bf16_bits(s), host(z)


def assert_quant_equal(w_bits, group):
    cq, cs, cz = quant_w4g(w_bits, group)
    gq, gs, gz = gpu_quant(w_bits, group)
    assert np.array_equal(gs, cs), f"{np.count_nonzero(gs != cs)} scales differ"
    assert np.array_equal(gz, cz), f"{np.count_nonzero(gz != cz)} zero points differ"
    bad = np.argwhere(gq != cq)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("name,N,K,group", [
    ("awq_adanorm_zero", None, None, 64),        # 18432 x 3072, full size
    ("awq_adanorm_single", None, None, 32),      # 9216 x 3072
    ("awq_adanorm_zero", 37, 96, 32),
    ("awq_adanorm_zero", 5, 384, 128),
    ("awq_adanorm_zero", 1, 64, 64),
])
def test_quant_weight_awq(name, N, K, group):
    w = make(name, M=1, K=K, N=N)["w"]
    say("quant_weight_awq", name, w.shape, group)
    assert_quant_equal(w, group)


@pytest.mark.parametrize("group", [32, 64, 128])
def test_quant_weight_awq_adversarial(group):
    # zero, signed-zero, subnormal, huge and tiny rows, constant rows, random
    # finite bit patterns with spans kept finite, one-signed groups
    w = adversarial_rows(256, seed=group)
    v = bf16_bits_to_f32(w)
    big = np.abs(v) > 1e37
    w[big] = bf16_round(np.sign(v[big]) * np.float32(1e37))
    pos = bf16_round(np.abs(np.random.default_rng(group).standard_normal((2, 256))).astype(np.float32) + 0.5)
    w = np.concatenate([w, pos, pos | 0x8000])
    say("quant_weight_awq adversarial", w.shape, group)
    assert_quant_equal(w, group)


def w4a16_case(x, w, group):
    wq, ws, wz = quant_w4g(w, group)
    what = dequant_w4g(wq, ws, wz, group)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    ref, absum = xf @ what.T, np.abs(xf) @ np.abs(what).T
    y = qpl.qlinear_awq_w4a16(to_dev_bf16(x), to_dev(wq), to_dev_bf16(ws), to_dev(wz), group)
    torch.cuda.synchronize()
    return check_gemm(bf16_bits(y), ref, absum, x.shape[1])


@pytest.mark.parametrize("name,M,K,N,group", [
    ("awq_adanorm_zero", 1, None, None, 64),     # FLUX adanorm_zero, one image
    ("awq_adanorm_zero", 2, None, None, 64),     # two images (guidance batch)
    ("awq_adanorm_single", 1, None, None, 128),
    ("awq_adanorm_single", 3, None, None, 32),   # odd batch: a second pass over the weight
    ("awq_adanorm_zero", 5, 4160, 70, 64),       # K past one 4096-channel slice, ragged N
    ("awq_adanorm_zero", 1, 1056, 33, 32),       # two chunks per lane, the second partial
    ("awq_adanorm_zero", 2, 32, 1, 32),          # one group, one output
    ("awq_adanorm_zero", 1, 96, 7, 32),
    # streaming path (K <= 4096, K / group a multiple of 4): partial second chunk,
    # fewer rows than waves, an odd batch, the largest K
    ("awq_adanorm_zero", 3, 1152, 37, 32),
    ("awq_adanorm_zero", 1, 128, 3, 32),
    ("awq_adanorm_zero", 2, 4096, 1000, 128),
    ("awq_adanorm_zero", 1, 2048, 5, 64),
])
def test_qlinear_awq_w4a16(name, M, K, N, group):
    d = make(name, M=M, K=K, N=N)
    say("qlinear_awq_w4a16", name, d["x"].shape, d["w"].shape, group)
    r = w4a16_case(d["x"], d["w"], group)
    say(r)
    assert r["ok"], r


def test_qlinear_awq_w4a16_deterministic():
    d = make("awq_adanorm_zero", M=2)
    wq, ws, wz = quant_w4g(d["w"], 64)
    args = (to_dev_bf16(d["x"]), to_dev(wq), to_dev_bf16(ws), to_dev(wz), 64)
    a = bf16_bits(qpl.qlinear_awq_w4a16(*args))
    b = bf16_bits(qpl.qlinear_awq_w4a16(*args))
    assert np.array_equal(a, b)
