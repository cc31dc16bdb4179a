"""GPU parity of qlinear_fp8r / qlinear_nvfp4 (with and without the low-rank branch)
against the oracle's float64 dequantize-then-multiply reference.

Acceptance (written in oracle.reference.check_gemm): relative Frobenius error
<= 2e-3 over the compared outputs, and per element |y - ref| <= 4 bf16 ulps of ref
plus an accumulation floor gamma * sum_k |a_k w_k|:

* nvfp4 multiplies exact f16 expansions of the codes on the f16 MFMA, whose dot
  products behave like fp32 sums: gamma = ceil(K/16) * 2^-24 (gemm_gamma).
* fp8r runs on the full-rate f8f6f4 MFMA, whose dot unit truncates products within
  groups of 8 and adds with truncation (oracle.reference.gemm_gamma_fp8_dot derives
  gamma = 7 * 2^-13 + 8 ceil(K/64) 2^-23 from that model).  The fp8r tests also
  report how many outputs the fp32 floor alone would fail and the largest error in
  bf16 ulps, and hold them to the figures measured with this kernel.

Small shapes compare every output; full-size workloads compare sampled rows (all
columns), including the first and last rows of edge tiles."""

import numpy as np
import pytest
import torch

import precision_quantized_linear_amd as qpl
from helpers import bf16_bits, to_dev, to_dev_bf16
from oracle.formats import bf16_bits_to_f32
from oracle.quant import (amax_bf16, calibrate_input_scale, global_scale, quant_fp8_row, quant_nvfp4,
                          smooth_bf16)
from oracle.reference import (check_gemm, dequant_fp8r, dequant_nvfp4, gemm_gamma_fp8_dot, lowrank_abs,
                              lowrank_ref)
from synthetic import bf16_round, calibration_batches, make, smooth_factors

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def sample_rows(M, n=64, seed=0):
    fixed = [r for r in (0, 1, 31, 32, 255, 256, M - 1, M - 2) if 0 <= r < M]
    if M <= n:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    extra = rng.choice(M, size=n - len(fixed), replace=False)
    return np.unique(np.concatenate([fixed, extra]))


def fp8r_case(d, rows):
    """The fp8r acceptance (fp8 dot-unit floor), plus the same outputs held to the
    fp32 floor alone: its failure count is reported as fails_fp32_floor."""
    x, w = d["x"], d["w"]
    K = x.shape[1]
    xq, xs = quant_fp8_row(x[rows])
    wq, ws = quant_fp8_row(w)
    a, b = dequant_fp8r(xq, xs), dequant_fp8r(wq, ws)
    ref, absum = a @ b.T, np.abs(a) @ np.abs(b).T
    y = qpl.qlinear_fp8r(to_dev_bf16(x), to_dev(wq), to_dev(ws))
    torch.cuda.synchronize()
    yb = bf16_bits(y)[rows]
    r = check_gemm(yb, ref, absum, K, gamma=gemm_gamma_fp8_dot(K))
    r["fails_fp32_floor"] = check_gemm(yb, ref, absum, K)["fails"]
    return r


def nvfp4_case(d, rows, g_in, lam=None):
    # lam: SVDQuant smoothing factors; the reference then starts from bf16(x / lam)
    x, w = d["x"], d["w"]
    K = x.shape[1]
    g_w = global_scale(amax_bf16(w))
    xr = x[rows] if lam is None else smooth_bf16(x[rows], lam)
    xp, xb = quant_nvfp4(xr, g_in)
    wp, wb = quant_nvfp4(w, g_w)
    a, b = dequant_nvfp4(xp, xb, g_in), dequant_nvfp4(wp, wb, g_w)
    ref, absum = a @ b.T, np.abs(a) @ np.abs(b).T
    extra = None
    lora = {}
    if "l1" in d:
        ref = ref + lowrank_ref(xr, d["l1"], d["l2"])
        extra = lowrank_abs(xr, d["l1"], d["l2"])
        lora = dict(lora_down=to_dev_bf16(d["l1"]), lora_up=to_dev_bf16(d["l2"]))
    if lam is not None:
        lora["smooth"] = to_dev(lam)
    y = qpl.qlinear_nvfp4(to_dev_bf16(x), to_dev(wp), to_dev(wb), g_w, g_in, **lora)
    torch.cuda.synchronize()
    return check_gemm(bf16_bits(y)[rows], ref, absum, K, extra_abs=extra)


FP8R_SHAPES = [
    ("fp8r_tiny", None, None, None),            # 64 x 256 x 512, all outputs
    ("fp8r_dit_n3072", 300, 400, 520),          # ragged M, K (not a multiple of 128) and N
    ("fp8r_dit_n3072", 512, 512, 512),          # whole tiles
    ("fp8r_dit_n3072", 1, 16, 1),               # degenerate
    ("fp8r_dit_n3072", 257, 272, 300),          # one row / column past a tile, N % 8 != 0
]


@pytest.mark.parametrize("name,M,K,N", FP8R_SHAPES)
def test_qlinear_fp8r_small(name, M, K, N):
    d = make(name, M=M, K=K, N=N)
    say("qlinear_fp8r", name, d["M"], d["K"], d["N"])
    r = fp8r_case(d, np.arange(d["M"]))
    say(r)
    assert r["ok"], r


# Measured with this kernel on the seeded workloads (deterministic): outputs that the
# fp32 floor alone fails, the largest error in bf16 ulps of the reference, and the
# outputs that pass only because of the fp8 dot-unit floor.  A change of the
# kernel's arithmetic that makes any of them worse fails here.
FP8R_RECORDED = {
    "fp8r_tiny": dict(fails_fp32_floor=17, max_ulp_err=683.4, only_floor=19),       # all 32768 outputs
    "fp8r_dit_n3072": dict(fails_fp32_floor=0, max_ulp_err=3773.9, only_floor=556),  # 256 rows x 3072
    "fp8r_dit_n12288": dict(fails_fp32_floor=0, max_ulp_err=3773.9, only_floor=2297),  # 256 rows x 12288
}


def check_recorded(name, r):
    for k, v in FP8R_RECORDED[name].items():
        if v is not None:
            assert r[k] <= v, (name, k, r[k], v)


def test_qlinear_fp8r_tiny_figures():
    # the 64 x 256 x 512 workload, every output
    d = make("fp8r_tiny")
    r = fp8r_case(d, np.arange(d["M"]))
    say("fp8r_tiny figures", {k: r[k] for k in ("fails_fp32_floor", "max_ulp_err", "only_floor", "frob")})
    assert r["ok"], r
    check_recorded("fp8r_tiny", r)


@pytest.mark.parametrize("name", ["fp8r_dit_n3072", "fp8r_dit_n12288"])
def test_qlinear_fp8r_full(name):
    # 256 sampled rows (all columns) of the 4608-row workload
    d = make(name)
    say("qlinear_fp8r full", name, d["M"], d["K"], d["N"])
    r = fp8r_case(d, sample_rows(d["M"], n=256))
    say(name, "figures", {k: r[k] for k in ("fails_fp32_floor", "max_ulp_err", "only_floor", "frob")})
    assert r["ok"], r
    check_recorded(name, r)


NVFP4_SHAPES = [
    ("nvfp4_dit", 300, 400, 520),               # K % 64 != 0: byte-wise weight loads
    ("nvfp4_dit", 512, 512, 512),
    ("nvfp4_dit", 1, 16, 1),
    ("nvfp4_mlp_down_cfg", 257, 1024, 300),
    ("svdq_w4a4", 300, 448, 264),               # low-rank branch, ragged
    ("svdq_w4a4", 256, 512, 256),
    ("svdq_w4a4", 37, 272, 72),                 # K % 32 == 16: half a k step in the fused x L1
    ("svdq_w4a4", 1, 16, 1),                    # one block, one row
]


@pytest.mark.parametrize("name,M,K,N", NVFP4_SHAPES)
def test_qlinear_nvfp4_small(name, M, K, N):
    d = make(name, M=M, K=K, N=N)
    g_in = calibrate_input_scale(calibration_batches(name, M=M, K=K))
    say("qlinear_nvfp4", name, d["M"], d["K"], d["N"], "R", d.get("R", 0))
    r = nvfp4_case(d, np.arange(d["M"]), g_in)
    assert r["ok"], r


@pytest.mark.parametrize("name", ["nvfp4_dit", "nvfp4_mlp_down_cfg", "svdq_w4a4"])
def test_qlinear_nvfp4_full(name):
    d = make(name)
    g_in = calibrate_input_scale(calibration_batches(name))
    say("qlinear_nvfp4 full", name, d["M"], d["K"], d["N"], "R", d.get("R", 0))
    r = nvfp4_case(d, sample_rows(d["M"]), g_in)
    say(r)
    assert r["ok"], r


@pytest.mark.parametrize("scheme,M,N", [("fp8r", 4608, 12288), ("nvfp4", 4608, 12288), ("fp8r", 4500, 12200),
                                         ("nvfp4", 4400, 12288), ("svdq", 4500, 12288), ("fp8r", 4608, 16384),
                                         ("nvfp4", 4500, 16384), ("fp8r", 4608, 16640), ("fp8r", 4500, 12250),
                                         ("nvfp4", 4600, 12250), ("nvfp4", 4608, 3072)])
def test_last_round_tiles(scheme, M, N):
    # 18 x 48 = 864 tiles of 256 x 256 over 256 persistent workgroups: the 96
    # tiles left for a fourth round (tile rows 16 and 17) are computed as 192 half
    # tiles of 128 x 256.  Checked: those rows and the band above them, every
    # column, at a short K.  M = 4500 leaves 20 rows in the second half of the
    # last tile row, M = 4400 none, M = 4600 rows in both halves; N = 12200 and
    # 12250 are ragged (12250: N % 8 = 2, element stores).  18 x 64 = 1152 tiles
    # leave 128 (every workgroup takes a half tile); 18 x 65 = 1170 leave 146,
    # which are computed whole; 18 x 12 = 216 fill one round.
    K = 256
    rows = np.arange(3840, M)
    if scheme == "fp8r":
        d = make("fp8r_dit_n12288", M=M, K=K, N=N)
        say("last round fp8r", M, K, N)
        r = fp8r_case(d, rows)
    else:
        name = "nvfp4_dit" if scheme == "nvfp4" else "svdq_w4a4"
        d = make(name, M=M, K=K, N=N)
        g_in = calibrate_input_scale(calibration_batches(name, M=64, K=K))
        say("last round", name, M, K, N, "R", d.get("R", 0))
        r = nvfp4_case(d, rows, g_in)
    say(r)
    assert r["ok"], r


def smoothed_scale(name, lam, K):
    return calibrate_input_scale(smooth_bf16(b, lam) for b in calibration_batches(name, M=64, K=K))


@pytest.mark.parametrize("name,M,K,N,R", [
    ("svdq_w4a4", None, None, None, None),      # full size, sampled rows
    ("svdq_w4a4", 300, 448, 264, None),         # ragged
    ("svdq_w4a4", 37, 272, 72, None),           # K % 32 == 16
    ("svdq_w4a4", 1, 16, 1, None),
    ("svdq_w4a4", 130, 256, 200, 64),           # two 32-column groups of T
    ("svdq_w4a4", 45, 208, 200, 100),           # four groups, TK = 128
    ("svdq_w4a4", 70, 320, 96, 80),             # three groups
    ("nvfp4_dit", 300, 400, 520, 0),            # smoothing without the low-rank branch
])
def test_qlinear_nvfp4_smoothed(name, M, K, N, R):
    d = make(name, M=M, K=K, N=N)
    if R:
        rng = np.random.default_rng(R)
        from synthetic import bf16_round
        d["l1"] = bf16_round((rng.standard_normal((d["K"], R)) * 0.05).astype(np.float32))
        d["l2"] = bf16_round((rng.standard_normal((R, d["N"])) * 0.05).astype(np.float32))
    lam = smooth_factors(name, K=d["K"])
    g_in = smoothed_scale(name, lam, d["K"])
    rows = sample_rows(d["M"]) if M is None else np.arange(d["M"])
    say("qlinear_nvfp4 smoothed", name, d["M"], d["K"], d["N"], "R", d["l1"].shape[1] if "l1" in d else 0)
    r = nvfp4_case(d, rows, g_in, lam)
    say(r)
    assert r["ok"], r


@pytest.mark.parametrize("R,M,K", [(1, 130, 256), (20, 130, 256), (64, 130, 256), (100, 130, 256), (128, 45, 208),
                                   (33, 17, 48), (64, 5120, 256), (32, 6000, 256), (100, 5200, 192)])
def test_qlinear_nvfp4_lowrank_ranks(R, M, K):
    # every padded rank width (32, 64, 96, 128 columns of T), ragged M and K % 32 == 16;
    # the fused quantizer with 20, 24 and 21 rows per workgroup (M = 5120, 6000, 5200)
    d = make("svdq_w4a4", M=M, K=K, N=200)
    rng = np.random.default_rng(R)
    from synthetic import bf16_round
    d["l1"] = bf16_round((rng.standard_normal((K, R)) * 0.05).astype(np.float32))
    d["l2"] = bf16_round((rng.standard_normal((R, 200)) * 0.05).astype(np.float32))
    say("qlinear_nvfp4 rank", R, M, K)
    r = nvfp4_case(d, np.arange(M), np.float32(0.01))
    assert r["ok"], r


def _scaled_bits(bits, e):
    """bf16 bit array times 2^e (exact: every scaled value stays a normal bf16)."""
    f = bf16_bits_to_f32(bits).astype(np.float64) * 2.0 ** e
    assert np.all((f == 0) | ((np.abs(f) >= 2.0 ** -126) & (np.abs(f) < 2.0 ** 127)))
    return bf16_round(f.astype(np.float32))


@pytest.mark.parametrize("target", [-126, -125, 64, 100])
def test_qlinear_nvfp4_lowrank_global_scale_edges(target):
    # input_scale * weight_scale_2 at the ends of the accepted range: x and W are
    # scaled by powers of two so the product lands in [2^target, 2^(target+1));
    # L2 carries W's factor so the low-rank term stays comparable to the 4-bit one.
    # The 4-bit product is scaled before the low-rank term joins it, so the output is
    # finite wherever the reference is, and subnormal bf16 outputs are compared too.
    M, K, N, R = 130, 256, 200, 32
    d = make("svdq_w4a4", M=M, K=K, N=N)
    g0 = float(global_scale(amax_bf16(d["x"]))) * float(global_scale(amax_bf16(d["w"])))
    shift = int(np.ceil(target - np.log2(g0)))
    ex = shift // 2
    ew = shift - ex
    d["x"], d["w"] = _scaled_bits(d["x"], ex), _scaled_bits(d["w"], ew)
    rng = np.random.default_rng(11)
    d["l1"] = bf16_round((rng.standard_normal((K, R)) * 0.05).astype(np.float32))
    d["l2"] = _scaled_bits(bf16_round((rng.standard_normal((R, N)) * 0.05).astype(np.float32)), ew)
    g_in = global_scale(amax_bf16(d["x"]))
    g = np.float32(g_in) * np.float32(global_scale(amax_bf16(d["w"])))
    assert 2.0 ** target <= g < 2.0 ** (target + 1), (g, target)
    say("qlinear_nvfp4 global scale product", g, "x 2^%d, w 2^%d" % (ex, ew))
    r = nvfp4_case(d, np.arange(M), g_in)
    say(r)
    assert r["ok"], r


def test_qlinear_one_hot_weight_fp8r():
    # W row n is one-hot at k = n (code 1.0, scale 1): y[:, n] = bf16(dec(xq[:, n]) * s_x)
    d = make("fp8r_tiny")
    x = d["x"]
    wq = np.zeros((64, 256), np.uint8)
    wq[np.arange(64), np.arange(64)] = 0x38
    ws = np.ones(64, np.float32)
    y = qpl.qlinear_fp8r(to_dev_bf16(x), to_dev(wq), to_dev(ws))
    torch.cuda.synchronize()
    xq, xs = quant_fp8_row(x)
    from oracle.formats import f32_to_bf16_bits
    exp = f32_to_bf16_bits((dequant_fp8r(xq[:, :64], xs)).astype(np.float32))
    assert np.array_equal(bf16_bits(y), exp)


def test_qlinear_deterministic():
    d = make("svdq_w4a4", M=256, K=512, N=256)
    g_w = global_scale(amax_bf16(d["w"]))
    wp, wb = quant_nvfp4(d["w"], g_w)
    args = (to_dev_bf16(d["x"]), to_dev(wp), to_dev(wb), g_w, 0.01)
    kw = dict(lora_down=to_dev_bf16(d["l1"]), lora_up=to_dev_bf16(d["l2"]))
    y1 = bf16_bits(qpl.qlinear_nvfp4(*args, **kw))
    y2 = bf16_bits(qpl.qlinear_nvfp4(*args, **kw))
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("name,M,K,N", [("nvfp4_dit", 300, 400, 520), ("svdq_w4a4", 37, 272, 72),
                                         ("nvfp4_dit", 1, 16, 1)])
def test_qlinear_nvfp4_workspace_contents_ignored(name, M, K, N):
    # K / 16 not a multiple of 8: the GEMM reads scale bytes past K / 16 in the last
    # slab of both operands' scale layouts, which the library writes as zeros.  A
    # workspace full of 0xFF (NaN as E4M3) and one full of zeros must give the same
    # bits, with and without the low-rank branch.
    d = make(name, M=M, K=K, N=N)
    R = d.get("R", 0)
    g_w = global_scale(amax_bf16(d["w"]))
    wp, wb = quant_nvfp4(d["w"], g_w)
    args = (to_dev_bf16(d["x"]), to_dev(wp), to_dev(wb), g_w, 0.01)
    kw = dict(lora_down=to_dev_bf16(d["l1"]), lora_up=to_dev_bf16(d["l2"])) if R else {}
    need = qpl.qlinear_workspace_bytes(qpl.QPL_NVFP4, d["M"], K, N, R)
    say("workspace contents", name, d["M"], K, N, "R", R)
    out = []
    for fill in (0xFF, 0x00):
        ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda")
        y = qpl.qlinear_nvfp4(*args, workspace=ws, **kw)
        torch.cuda.synchronize()
        out.append(bf16_bits(y))
    assert np.isfinite(bf16_bits_to_f32(out[0])).all()
    assert np.array_equal(out[0], out[1])


def test_fp8_dot_floor_random_codes():
    # Activations and weights are exact E4M3 values spread over the whole exponent
    # range, with row amax 448 (so the row scale is 1 and the kernel's codes are the
    # chosen values).  The per-element error of the product must stay within the
    # dot-unit floor; the fp32 floor alone is exceeded (the floor is needed).
    from oracle.formats import e4m3_decode
    from oracle.reference import gemm_gamma, ulp_bf16
    from synthetic import bf16_round
    rng = np.random.default_rng(17)
    M, N, K = 256, 256, 64
    codes = rng.integers(0, 0x7F, (M + N, K)).astype(np.uint8) | (rng.integers(0, 2, (M + N, K)).astype(np.uint8) << 7)
    codes[:, 0] = 0x7E                      # every row holds 448, so its scale is exactly 1
    vals = e4m3_decode(codes)
    xa = bf16_round(vals[:M].astype(np.float32))
    wq = codes[M:]
    y = qpl.qlinear_fp8r(to_dev_bf16(xa), to_dev(wq), to_dev(np.ones(N, np.float32)))
    torch.cuda.synchronize()
    a, b = vals[:M], vals[M:]
    ref, absum = a @ b.T, np.abs(a) @ np.abs(b).T
    yb = bf16_bits_to_f32(bf16_bits(y)).astype(np.float64)
    excess = np.maximum(np.abs(yb - ref) - 4 * ulp_bf16(ref), 0) / absum
    say("fp8 dot unit: excess error / sum|aw|: max", excess.max(), "floor", gemm_gamma_fp8_dot(K))
    assert excess.max() <= gemm_gamma_fp8_dot(K)
    assert excess.max() > gemm_gamma(K)


def test_fp8_dot_floor_cancellation():
    # Row m of x is [448, 448, 15, 15, ...] and row n of W is [448, -448, 1, 1, ...]:
    # the two large products cancel and leave 62 * 15 = 930.  The six small products in
    # the first group of eight lie 13 to 14 binades below its largest product, at the
    # group's cut, so the dot unit truncates them: the result falls short of 930 by far
    # more than fp32 summation could, and within the dot-unit floor.
    from oracle.reference import gemm_gamma, ulp_bf16
    K = 64
    x = np.full((32, K), 0x4170, np.uint16)   # bf16 15.0
    x[:, 0] = x[:, 1] = 0x43E0                # bf16 448.0
    wq = np.full((32, K), 0x38, np.uint8)      # E4M3 1.0
    wq[:, 0], wq[:, 1] = 0x7E, 0xFE            # E4M3 448, -448
    y = qpl.qlinear_fp8r(to_dev_bf16(x), to_dev(wq), to_dev(np.ones(32, np.float32)))
    torch.cuda.synchronize()
    got = bf16_bits_to_f32(bf16_bits(y)).astype(np.float64)
    ref, absum = 930.0, 2 * 448.0 * 448.0 + 62 * 15.0
    say("fp8 dot unit, cancellation: got", np.unique(got), "exact", ref)
    err = np.abs(got - ref)
    assert np.all(err > gemm_gamma(K) * absum + 4 * ulp_bf16(ref))
    assert np.all(err <= gemm_gamma_fp8_dot(K) * absum + 4 * ulp_bf16(ref))


@pytest.mark.parametrize("scheme", ["fp8r", "nvfp4"])
def test_output_past_2_31_elements(scheme):
    # M x N = 131072 x 32768 = 2^32 outputs (8 GB of bf16): the element offsets of rows past
    # 65536 exceed 2^31, so the quantizer's and the epilogue's addressing must be 64-bit.
    # K = 64 gives one or two slabs per tile, so each of the 65536 tiles has a workgroup.
    M, K, N = 131072, 64, 32768
    d = make("fp8r_dit_n3072" if scheme == "fp8r" else "nvfp4_dit", M=M, K=K, N=N)
    x, w = d["x"], d["w"]
    rows = np.unique(np.concatenate([[0, 65535, 65536, 65537, 98304, M - 2, M - 1],
                                     np.random.default_rng(3).choice(M, 25, replace=False)]))
    say("output past 2^31 elements", scheme, M, K, N)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    if scheme == "fp8r":
        xq, xs = quant_fp8_row(x[rows])
        wq, ws = quant_fp8_row(w)
        a, b = dequant_fp8r(xq, xs), dequant_fp8r(wq, ws)
        qpl.qlinear_fp8r(to_dev_bf16(x), to_dev(wq), to_dev(ws), y=y)
        gamma = gemm_gamma_fp8_dot(K)
    else:
        g_in = calibrate_input_scale(calibration_batches("nvfp4_dit", M=64, K=K))
        g_w = global_scale(amax_bf16(w))
        xp, xb = quant_nvfp4(x[rows], g_in)
        wp, wb = quant_nvfp4(w, g_w)
        a, b = dequant_nvfp4(xp, xb, g_in), dequant_nvfp4(wp, wb, g_w)
        qpl.qlinear_nvfp4(to_dev_bf16(x), to_dev(wp), to_dev(wb), g_w, g_in, y=y)
        gamma = None
    got = bf16_bits(y[torch.from_numpy(rows).cuda()])
    torch.cuda.synchronize()
    del y
    ref, absum = a @ b.T, np.abs(a) @ np.abs(b).T
    r = check_gemm(got, ref, absum, K, gamma=gamma)
    say(r)
    assert r["ok"], r
