"""GPU parity of the quantizers, the dequant fallback and the amax helper against the
oracle: bit-exact codes and scales (integer/byte outputs)."""
import numpy as np
import pytest
import torch

import precision_quantized_linear_amd as qpl
from helpers import (adversarial_rows, bf16_bits, host, nvfp4_workspace_parts, slab_scales_to_rows, to_dev,
                     to_dev_bf16)
from oracle.formats import bf16_bits_to_f32
from oracle.quant import (amax_bf16, calibrate_input_scale, global_scale, quant_fp8_row, quant_nvfp4,
                          smooth_bf16)
from oracle.reference import dequant_weight_fp8r, dequant_weight_nvfp4
from synthetic import bf16_round, calibration_batches, make, smooth_factors

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def gpu_fp8_row(bits):
    q, s = qpl.quant_act_fp8_row(to_dev_bf16(bits))
    torch.cuda.synchronize()
    return host(q), host(s)


def gpu_nvfp4(bits, g):
    q, s = qpl.quant_act_nvfp4(to_dev_bf16(bits), g)
    torch.cuda.synchronize()
    return host(q), host(s)


def assert_fp8_equal(bits):
    cq, cs = quant_fp8_row(bits)
    gq, gs = gpu_fp8_row(bits)
    assert np.array_equal(gs.view(np.uint32), cs.view(np.uint32)), "row scales differ"
    bad = np.argwhere(gq != cq)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}: gpu {gq[tuple(bad[0])]:#x} oracle {cq[tuple(bad[0])]:#x}"


def assert_nvfp4_equal(bits, g):
    cq, cs = quant_nvfp4(bits, g)
    gq, gs = gpu_nvfp4(bits, g)
    assert np.array_equal(gs, cs), f"{np.count_nonzero(gs != cs)} block scales differ"
    bad = np.argwhere(gq != cq)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("name,M,K", [
    ("fp8r_tiny", None, None),                 # 64 x 256
    ("fp8r_dit_n3072", None, None),            # 4608 x 3072, full size
    ("fp8r_dit_n3072", 300, 400),              # ragged: K not a multiple of 128
    ("fp8r_dit_n3072", 1, 16),                 # smallest legal shape
    ("fp8r_dit_n3072", 7, 12288),              # long rows held in registers
    ("fp8r_dit_n3072", 3, 16400),              # rows too long for registers: two-pass path
])
def test_quant_fp8_row_activations(name, M, K):
    d = make(name, M=M, K=K)
    say("quant_act_fp8_row", name, d["x"].shape)
    assert_fp8_equal(d["x"])


@pytest.mark.parametrize("name", ["fp8r_tiny", "fp8r_dit_n12288"])
def test_quant_fp8_row_weights(name):
    w = make(name, M=8)["w"]
    say("quant_act_fp8_row weight", name, w.shape)
    assert_fp8_equal(w)


@pytest.mark.parametrize("K", [16, 256, 3072])
def test_quant_fp8_row_adversarial(K):
    say("quant_act_fp8_row adversarial", K)
    assert_fp8_equal(adversarial_rows(K, seed=K))


def test_quant_fp8_row_exact_ties():
    # rows with amax 448 * 2^j: s = 2^j and bf16 values on E4M3 midpoints are exact ties
    from oracle.formats import e4m3_decode
    pos = e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    rows = []
    for j in (-4, 0, 3):
        v = np.ldexp(mids, j)
        v = v[np.abs(v) < 448 * 2.0 ** j]
        row = np.concatenate([[448 * 2.0 ** j], v, -v]).astype(np.float32)
        b = bf16_round(row)
        b = b[bf16_bits_to_f32(b) == row]
        rows.append(np.resize(b, 256))
    say("quant_act_fp8_row ties")
    assert_fp8_equal(np.stack(rows))


@pytest.mark.parametrize("name,M,K", [
    ("nvfp4_dit", None, None),                     # 4608 x 3072
    ("nvfp4_mlp_down_cfg", None, None),            # 9216 x 12288, heavy tails: saturation
    ("svdq_w4a4", 300, 400),                       # ragged
    ("nvfp4_dit", 1, 16),
])
def test_quant_nvfp4_activations(name, M, K):
    from synthetic import calibration_batches
    from oracle.quant import calibrate_input_scale
    d = make(name, M=M, K=K)
    g = calibrate_input_scale(calibration_batches(name, M=M, K=K))
    say("quant_act_nvfp4", name, d["x"].shape, "input_scale", g)
    assert_nvfp4_equal(d["x"], g)


@pytest.mark.parametrize("name", ["nvfp4_dit", "nvfp4_mlp_down_cfg", "svdq_w4a4"])
def test_quant_nvfp4_weights(name):
    w = make(name, M=8)["w"]
    g = global_scale(amax_bf16(w))
    say("quant_act_nvfp4 weight", name, w.shape, g)
    assert_nvfp4_equal(w, g)


@pytest.mark.parametrize("g", [1e-30, 1e-4, 0.01, 0.25, 3.0, 1e6, 1e37, 5e37])
def test_quant_nvfp4_adversarial(g):
    # small g saturates block scales at 448; huge g underflows them to 0 (signed-zero codes)
    say("quant_act_nvfp4 adversarial", g)
    assert_nvfp4_equal(adversarial_rows(256, seed=5), np.float32(g))


def test_quant_nvfp4_exact_ties():
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    row = np.array([6.0] + ties + [-t for t in ties] + [0.0], dtype=np.float32)
    bits = np.tile(bf16_round(row), (4, 4))
    say("quant_act_nvfp4 ties")
    assert_nvfp4_equal(bits, np.float32(0.25))


def assert_nvfp4_smoothed_equal(bits, g, lam):
    cq, cs = quant_nvfp4(smooth_bf16(bits, lam), g)
    q, sc = qpl.quant_act_nvfp4(to_dev_bf16(bits), g, smooth=to_dev(lam))
    torch.cuda.synchronize()
    gq, gs = host(q), host(sc)
    assert np.array_equal(gs, cs), f"{np.count_nonzero(gs != cs)} block scales differ"
    bad = np.argwhere(gq != cq)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("M,K", [(None, None), (300, 400), (37, 272), (1, 16)])
def test_quant_nvfp4_smoothed(M, K):
    # SVDQuant smoothing: codes of bf16(x / smooth), input_scale calibrated on smoothed batches
    d = make("svdq_w4a4", M=M, K=K)
    lam = smooth_factors("svdq_w4a4", K=d["K"])
    g = calibrate_input_scale(smooth_bf16(b, lam) for b in calibration_batches("svdq_w4a4", M=64, K=d["K"]))
    say("quant_act_nvfp4 smoothed", d["x"].shape, g)
    assert_nvfp4_smoothed_equal(d["x"], g, lam)


def test_quant_nvfp4_smoothed_adversarial():
    # factors that are powers of two, all-ones mantissas, tiny (x / smooth near the
    # top of bf16) and huge (quotients in the fp32 and bf16 subnormal range), over
    # rows with signed zeros and subnormal inputs
    K = 256
    x = adversarial_rows(K, seed=5)
    rng = np.random.default_rng(6)
    lam = np.exp(rng.uniform(-4, 4, size=K)).astype(np.float32)
    lam[0:16] = np.ldexp(1.0, rng.integers(-20, 21, size=16)).astype(np.float32)
    lam[16:32] = np.nextafter(np.ldexp(np.float32(1), rng.integers(-5, 6, size=16)).astype(np.float32),
                              np.float32(0))
    lam[32:48] = np.float32(1e-30)
    lam[48:64] = np.float32(3e37)
    lam[64:80] = np.float32(1e38)
    # quotients that overflow bf16 are outside the contract: those inputs become 1.0
    with np.errstate(over="ignore"):
        x[~np.isfinite(bf16_bits_to_f32(smooth_bf16(x, lam)))] = 0x3F80
    assert np.all(np.isfinite(bf16_bits_to_f32(smooth_bf16(x, lam))))
    for g in (1e-30, 0.01, 1e6):
        say("quant_act_nvfp4 smoothed adversarial", g)
        assert_nvfp4_smoothed_equal(x, g, lam)


def test_dequant_weight_fp8r():
    w = make("fp8r_dit_n12288", M=8, K=1024, N=333)["w"]
    wq, ws = quant_fp8_row(w)
    say("dequant_weight fp8r", wq.shape)
    out = qpl.dequant_weight(qpl.QPL_FP8R, to_dev(wq), to_dev(ws))
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(out), dequant_weight_fp8r(wq, ws))


@pytest.mark.parametrize("unit", [False, True])
def test_dequant_weight_nvfp4(unit):
    # an odd block count (129 x 65); weight_scale_2 = 1 takes the exact-product path
    w = make("nvfp4_dit", M=8, K=1040, N=129)["w"]
    g = np.float32(1.0) if unit else global_scale(amax_bf16(w))
    wp, wb = quant_nvfp4(w, g)
    say("dequant_weight nvfp4", wp.shape, "g = 1" if unit else "")
    out = qpl.dequant_weight(qpl.QPL_NVFP4, to_dev(wp), to_dev(wb), g, K=1040)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(out), dequant_weight_nvfp4(wp, wb, g))


@pytest.mark.parametrize("n", [1, 7, 8, 1000, 4608 * 3072 + 3])
def test_amax(n):
    x = bf16_round((np.random.default_rng(n).standard_normal(n) * 3).astype(np.float32))
    say("qpl_amax_bf16", n)
    a = qpl.amax_bf16(to_dev_bf16(x))
    a = qpl.amax_bf16(to_dev_bf16(x[: max(1, n // 2)]), amax=a)  # running max keeps the larger
    torch.cuda.synchronize()
    assert host(a)[0] == amax_bf16(x)


def test_quant_deterministic():
    d = make("nvfp4_dit", M=512)
    x = to_dev_bf16(d["x"])
    a = [host(t) for t in qpl.quant_act_nvfp4(x, 0.01)]
    b = [host(t) for t in qpl.quant_act_nvfp4(x, 0.01)]
    assert all(np.array_equal(p, q) for p, q in zip(a, b))


# ---- the GEMM's operands: what qlinear_nvfp4 leaves in its workspace ----
# The activation quantize inside the linear (plain, or fused with x L1 when R > 0)
# writes packed codes [M, K/2] and block scales in the GEMM's slab-major layout; the
# preparation copies the weight's block scales into that layout.  All of it must be
# bit-exact: the codes equal to quant_act_nvfp4's (signed zeros included).


def run_linear_operands(x_bits, g_in, wq, wb, lam=None, R=0, seed=0):
    M, K = x_bits.shape
    N = wq.shape[0]
    kw = {}
    if R:
        rng = np.random.default_rng(seed)
        kw["lora_down"] = to_dev_bf16(bf16_round((rng.standard_normal((K, R)) * 0.05).astype(np.float32)))
        kw["lora_up"] = to_dev_bf16(bf16_round((rng.standard_normal((R, N)) * 0.05).astype(np.float32)))
    if lam is not None:
        kw["smooth"] = to_dev(lam)
    ws = torch.zeros((qpl.qlinear_workspace_bytes(qpl.QPL_NVFP4, M, K, N, R),), dtype=torch.uint8, device="cuda")
    # a first call leaves non-zero bytes behind; the second must write every byte it owns
    ws.fill_(0xA5)
    qpl.qlinear_nvfp4(to_dev_bf16(x_bits), to_dev(wq), to_dev(wb), 1.0, g_in, workspace=ws, **kw)
    torch.cuda.synchronize()
    parts = nvfp4_workspace_parts(M, K, N, R)
    h = host(ws)
    S = parts["S"]
    xq = h[:M * K // 2].reshape(M, K // 2)
    xs, xpad = slab_scales_to_rows(h[parts["xs"]:parts["xs"] + 8 * M * S], M, K)
    wsr, wpad = slab_scales_to_rows(h[parts["ws"]:parts["ws"] + 8 * N * S], N, K)
    return xq, xs, xpad, wsr, wpad


def assert_operands_equal(x_bits, g_in, wq, wb, lam=None, R=0):
    xq, xs, xpad, wsr, wpad = run_linear_operands(x_bits, g_in, wq, wb, lam, R)
    xin = x_bits if lam is None else smooth_bf16(x_bits, lam)
    cq, cs = quant_nvfp4(xin, g_in)
    bad = np.argwhere(xq != cq)
    assert bad.size == 0, f"{len(bad)} activation code bytes differ, first at {bad[:3].tolist()}"
    bad = np.argwhere(xs != cs)
    assert bad.size == 0, f"{len(bad)} activation block scales differ, first at {bad[:3].tolist()}"
    assert not xpad.any(), "activation scale bytes past K/16 are not zero"
    assert np.array_equal(wsr, wb), "weight block scales moved wrongly"
    assert not wpad.any(), "weight scale bytes past K/16 are not zero"


def random_weight(N, K, seed):
    """Every code byte and every finite block-scale code (0..126), uniformly."""
    rng = np.random.default_rng(seed)
    return (rng.integers(0, 256, (N, K // 2)).astype(np.uint8),
            rng.integers(0, 127, (N, K // 16)).astype(np.uint8))


@pytest.mark.parametrize("name,M,K,N,smoothed,R", [
    ("nvfp4_dit", None, None, 40, False, 0),     # 4608 x 3072 activation, full size
    ("svdq_w4a4", 300, 400, 48, False, 0),       # ragged: K % 128 != 0 (a partial last scale slab)
    ("svdq_w4a4", 37, 272, 33, True, 0),         # smoothed, odd rows
    ("nvfp4_dit", 1, 16, 1, False, 0),           # one block
    ("nvfp4_dit", 64, 3072, 12288, False, 0),    # the DiT weight's scales: 1152 relay workgroups in the quantizer's launch
    ("svdq_w4a4", 64, 400, 4100, False, 0),      # ragged weight relay: K % 128 != 0, N % 256 != 0
    ("svdq_w4a4", None, None, 64, False, 32),    # the SVDQuant workload at full size, fused x L1 quantizer
    ("svdq_w4a4", None, None, 64, True, 32),     # the same with smoothing
    ("svdq_w4a4", 300, 400, 48, False, 32),      # ragged M and K
    ("svdq_w4a4", 37, 272, 33, True, 20),        # smoothed, odd rows, K % 32 == 16, rank 20
    ("svdq_w4a4", 1, 16, 1, False, 1),           # one block, rank 1
    ("svdq_w4a4", 256, 256, 16, False, 64),      # 1 row per quantizer workgroup, two T groups
    ("svdq_w4a4", 512, 208, 16, True, 100),      # 2 rows per workgroup, four T groups
    ("svdq_w4a4", 5120, 256, 16, False, 32),     # 20 rows per workgroup
    ("svdq_w4a4", 6000, 256, 16, True, 32),      # 24 rows per workgroup
    ("svdq_w4a4", 8192, 128, 16, False, 128),    # 32 rows per workgroup, rank 128
])
def test_qlinear_nvfp4_operands(name, M, K, N, smoothed, R):
    d = make(name, M=M, K=K)
    K = d["K"]
    lam = smooth_factors("svdq_w4a4", K=K) if smoothed else None
    batches = calibration_batches(name, M=64 if M is None else min(M, 512), K=K)
    if lam is not None:
        batches = (smooth_bf16(b, lam) for b in batches)
    g = calibrate_input_scale(batches)
    wq, wb = random_weight(N, K, seed=K + N)
    say("qlinear_nvfp4 operands", name, d["x"].shape, N, "R", R, "smoothed" if smoothed else "", g)
    assert_operands_equal(d["x"], g, wq, wb, lam, R)


@pytest.mark.parametrize("R", [0, 32])
@pytest.mark.parametrize("g", [1e-30, 1e-4, 0.25, 1e6, 5e37])
def test_qlinear_nvfp4_operands_adversarial(g, R):
    # block scales saturated at 448 (small g) or underflowed to 0 (huge g), signed
    # zeros, subnormal inputs, exact ties; plain and fused quantizer
    x = adversarial_rows(256, seed=7)
    wq, wb = random_weight(24, 256, seed=8)
    say("qlinear_nvfp4 operands, adversarial", x.shape, g, "R", R)
    assert_operands_equal(x, np.float32(g), wq, wb, R=R)
