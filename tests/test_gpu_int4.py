"""GPU parity of the INT4 variant of the SVDQuant W4A4 linear against the oracle:
quant_act_int4 codes and scales bit-exact (also with smoothing), qlinear_int4
within the GEMM acceptance test (oracle.reference.check_gemm: relative Frobenius
error <= 2e-3, per element 4 bf16 ulps plus the fp32 accumulation floor
ceil(K/16) 2^-24 sum_k |a_k w_k|, plus the same floor on the low-rank magnitudes)
on weights quantized by the oracle."""
import numpy as np
import pytest
import torch

import precision_quantized_linear_amd as qpl
from helpers import adversarial_rows, bf16_bits, host, to_dev, to_dev_bf16
from oracle.formats import bf16_bits_to_f32
from oracle.int4 import dequant_int4, quant_int4
from oracle.quant import smooth_bf16
from oracle.reference import check_gemm, lowrank_abs, lowrank_ref
from synthetic import bf16_round, make, smooth_factors

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def assert_quant_equal(bits, lam=None):
    xr = bits if lam is None else smooth_bf16(bits, lam)
    cq, cs = quant_int4(xr)
    q, s = qpl.quant_act_int4(to_dev_bf16(bits), smooth=None if lam is None else to_dev(lam))
    torch.cuda.synchronize()
    gq, gs = host(q), host(s)
    assert np.array_equal(gs.view(np.uint32), cs.view(np.uint32)), f"{np.count_nonzero(gs != cs)} scales differ"
    bad = np.argwhere(gq != cq)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("name,M,K,smooth", [
    ("svdq_w4a4", None, None, False),     # 4608 x 3072, full size
    ("svdq_w4a4", None, None, True),
    ("svdq_w4a4", 37, 320, False),
    ("svdq_w4a4", 1, 64, True),
    ("nvfp4_mlp_down_cfg", 64, 12288, False),   # heavy tails, long rows
])
def test_quant_act_int4(name, M, K, smooth):
    d = make(name, M=M, K=K)
    lam = smooth_factors(name, K=d["K"]) if smooth else None
    say("quant_act_int4", name, d["x"].shape, "smooth" if smooth else "")
    assert_quant_equal(d["x"], lam)


def test_quant_act_int4_weight_and_adversarial():
    w = make("svdq_w4a4", M=1)["w"]
    say("quant_act_int4 weight", w.shape)
    assert_quant_equal(w)
    x = adversarial_rows(256, seed=3)
    say("quant_act_int4 adversarial", x.shape)
    assert_quant_equal(x)


def int4_case(d, rows, lam=None):
    x, w = d["x"], d["w"]
    K = x.shape[1]
    xr = x[rows] if lam is None else smooth_bf16(x[rows], lam)
    xp, xs = quant_int4(xr)
    wp, ws = quant_int4(w)
    a, b = dequant_int4(xp, xs), dequant_int4(wp, ws)
    ref, absum = a @ b.T, np.abs(a) @ np.abs(b).T
    extra = None
    kw = {}
    if "l1" in d:
        ref = ref + lowrank_ref(xr, d["l1"], d["l2"])
        extra = lowrank_abs(xr, d["l1"], d["l2"])
        kw = dict(lora_down=to_dev_bf16(d["l1"]), lora_up=to_dev_bf16(d["l2"]))
    if lam is not None:
        kw["smooth"] = to_dev(lam)
    y = qpl.qlinear_int4(to_dev_bf16(x), to_dev(wp), to_dev(ws), **kw)
    torch.cuda.synchronize()
    return check_gemm(bf16_bits(y)[rows], ref, absum, K, extra_abs=extra)


def sample_rows(M, n=64, seed=0):
    fixed = [r for r in (0, 1, 127, 128, 255, 256, M - 1, M - 2) if 0 <= r < M]
    rng = np.random.default_rng(seed)
    extra = rng.choice(M, size=n - len(fixed), replace=False)
    return np.unique(np.concatenate([fixed, extra]))


@pytest.mark.parametrize("name,M,K,N,R,smooth", [
    ("nvfp4_dit", 256, 512, 512, 0, False),     # whole tiles, persistent (8 slabs)
    ("nvfp4_dit", 300, 448, 264, 0, False),     # ragged M and N, N % 8 != 0
    ("nvfp4_dit", 1, 64, 1, 0, False),          # one group, one output: a workgroup per tile
    ("nvfp4_dit", 129, 256, 300, 0, False),     # four slabs (below the ring depth)
    ("svdq_w4a4", 300, 448, 264, None, False),  # low-rank branch (rank 32)
    ("svdq_w4a4", 37, 320, 72, None, True),     # low rank + smoothing
    ("svdq_w4a4", 130, 256, 200, 64, False),    # two 32-column groups of T
    ("svdq_w4a4", 45, 192, 200, 100, True),     # four groups (TK = 128), smoothing
    ("nvfp4_dit", 300, 400 + 48, 520, 0, True), # smoothing without the low-rank branch
    ("svdq_w4a4", 6000, 256, 200, 32, False),   # 24 rows per fused-quantizer workgroup
    ("svdq_w4a4", 5120, 320, 72, None, True),   # 20 rows per workgroup, smoothing
])
def test_qlinear_int4_small(name, M, K, N, R, smooth):
    d = make(name, M=M, K=K, N=N)
    if R:
        rng = np.random.default_rng(R)
        d["l1"] = bf16_round((rng.standard_normal((K, R)) * 0.05).astype(np.float32))
        d["l2"] = bf16_round((rng.standard_normal((R, N)) * 0.05).astype(np.float32))
    elif R == 0:
        d.pop("l1", None)
        d.pop("l2", None)
    lam = smooth_factors(name, K=d["K"]) if smooth else None
    say("qlinear_int4", name, d["M"], d["K"], d["N"], "R", d["l1"].shape[1] if "l1" in d else 0,
        "smooth" if smooth else "")
    r = int4_case(d, np.arange(d["M"]), lam)
    say(r)
    assert r["ok"], r


@pytest.mark.parametrize("name,smooth", [("svdq_w4a4", False), ("svdq_w4a4", True), ("nvfp4_dit", False)])
def test_qlinear_int4_full(name, smooth):
    # 4608 x 3072 x 3072 with rank 32, and 4608 x 3072 x 12288 (3.375 rounds of
    # 128 x 256 tiles per workgroup... 1728 tiles over 256 workgroups)
    d = make(name)
    lam = smooth_factors(name) if smooth else None
    say("qlinear_int4 full", name, d["M"], d["K"], d["N"], "smooth" if smooth else "")
    r = int4_case(d, sample_rows(d["M"]), lam)
    say(r)
    assert r["ok"], r


def test_qlinear_int4_deterministic():
    d = make("svdq_w4a4", M=256, K=512, N=256)
    wp, ws = quant_int4(d["w"])
    args = (to_dev_bf16(d["x"]), to_dev(wp), to_dev(ws))
    kw = dict(lora_down=to_dev_bf16(d["l1"]), lora_up=to_dev_bf16(d["l2"]))
    a = bf16_bits(qpl.qlinear_int4(*args, **kw))
    b = bf16_bits(qpl.qlinear_int4(*args, **kw))
    assert np.array_equal(a, b)
