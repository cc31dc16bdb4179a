"""GPU parity of the model-specific epilogues against the oracle (oracle.epilogue).

* GELU (tanh form) on the fp32 result of each scheme's linear: every output must lie
  in the bf16 interval that a correct fp32 evaluation of gelu(y) can round to, for
  y anywhere within the GEMM acceptance bound of the exact pre-activation; where
  that interval holds one bf16 value the output must equal it.  Relative Frobenius
  error against gelu(y_exact) <= 2e-3 (or the rounding floor of a few outputs).
* fused QKV: q, k, v hold the linear's three column parts at their head-major
  positions (gathered back, the GEMM acceptance test against the oracle), rows
  outside the written tokens stay untouched, and the values are bit-identical to
  the plain call's y.
* GELU MLP (nvfp4): h (left in the workspace) inside the GELU interval as above;
  fc2's operand, also left there, must be the nvfp4 quantization of some bf16 h in
  that interval (block by block; exact where that quantization is unique); y must
  lie within the GEMM acceptance bound of the oracle's fc2 on the oracle's own
  operand, widened by the largest effect the non-unique codes (and, with fc2's
  low-rank branch, the non-unique h) can have; and y must be bit-identical to the
  two layers run as separate calls.
"""

import numpy as np
import pytest
import torch

import precision_quantized_linear_amd as qpl
from helpers import bf16_bits, host, nvfp4_workspace_parts, slab_scales_to_rows, to_dev, to_dev_bf16
from oracle.epilogue import (bf16_interval, check_nvfp4_expanded, expanded_nominal_and_width, gelu_bf16_ref,
                             gelu_interval, gelu_tanh, pre_activation_error, qkv_split_ref, smooth_interval)
from oracle.formats import bf16_bits_to_f32, f32_to_bf16_bits
from oracle.int4 import dequant_int4, quant_int4
from oracle.quant import amax_bf16, calibrate_input_scale, global_scale, quant_fp8_row, quant_nvfp4, smooth_bf16
from oracle.reference import (FROB_ARITH, check_gemm, dequant_fp8r, dequant_nvfp4, gemm_gamma, gemm_gamma_fp8_dot,
                              lowrank_abs, lowrank_ref, ulp_bf16)
from synthetic import calibration_batches, make, smooth_factors

pytestmark = pytest.mark.gpu

F32 = np.float32


def say(*a):
    print(*a, flush=True)


def f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def sample_rows(M, n=48, seed=0):
    if M <= n:
        return np.arange(M)
    fixed = [r for r in (0, 1, 255, 256, M - 1) if 0 <= r < M]
    extra = np.random.default_rng(seed).choice(M, size=n - len(fixed), replace=False)
    return np.unique(np.concatenate([fixed, extra]))


# ---- oracle pre-activations -------------------------------------------------------

def nvfp4_pre(d, rows, g_in, lam=None, lowrank=True):
    x, w = d["x"], d["w"]
    g_w = global_scale(amax_bf16(w))
    xr = x[rows] if lam is None else smooth_bf16(x[rows], lam)
    xp, xb = quant_nvfp4(xr, g_in)
    wp, wb = quant_nvfp4(w, g_w)
    a, b = dequant_nvfp4(xp, xb, g_in), dequant_nvfp4(wp, wb, g_w)
    ref, absum, extra = a @ b.T, np.abs(a) @ np.abs(b).T, None
    kw = {}
    if lowrank and "l1" in d:
        ref = ref + lowrank_ref(xr, d["l1"], d["l2"])
        extra = lowrank_abs(xr, d["l1"], d["l2"])
        kw = dict(lora_down=to_dev_bf16(d["l1"]), lora_up=to_dev_bf16(d["l2"]))
    if lam is not None:
        kw["smooth"] = to_dev(lam)
    call = lambda **more: qpl.qlinear_nvfp4(to_dev_bf16(x), to_dev(wp), to_dev(wb), g_w, g_in, **kw, **more)  # noqa
    return ref, absum, extra, call


def fp8r_pre(d, rows):
    x, w = d["x"], d["w"]
    xq, xs = quant_fp8_row(x[rows])
    wq, ws = quant_fp8_row(w)
    a, b = dequant_fp8r(xq, xs), dequant_fp8r(wq, ws)
    call = lambda **more: qpl.qlinear_fp8r(to_dev_bf16(x), to_dev(wq), to_dev(ws), **more)  # noqa: E731
    return a @ b.T, np.abs(a) @ np.abs(b).T, None, call


def int4_pre(d, rows, lowrank=True):
    x, w = d["x"], d["w"]
    xp, xs = quant_int4(x[rows])
    wp, ws = quant_int4(w)
    a, b = dequant_int4(xp, xs), dequant_int4(wp, ws)
    ref, absum, extra, kw = a @ b.T, np.abs(a) @ np.abs(b).T, None, {}
    if lowrank and "l1" in d:
        ref = ref + lowrank_ref(x[rows], d["l1"], d["l2"])
        extra = lowrank_abs(x[rows], d["l1"], d["l2"])
        kw = dict(lora_down=to_dev_bf16(d["l1"]), lora_up=to_dev_bf16(d["l2"]))
    call = lambda **more: qpl.qlinear_int4(to_dev_bf16(x), to_dev(wp), to_dev(ws), **kw, **more)  # noqa: E731
    return ref, absum, extra, call


def check_gelu(y_bits, ref, absum, K, extra=None, gamma=None):
    err = pre_activation_error(ref, absum, K, extra, gamma)
    lo, hi = gelu_interval(ref, err)
    lb, hb = bf16_interval(lo, hi)
    y = f64(y_bits)
    bad = ~((y >= f64(lb)) & (y <= f64(hb)))
    g = gelu_tanh(ref)
    den = np.linalg.norm(g)
    frob = float(np.linalg.norm(y - g) / den)
    rounded = f64(f32_to_bf16_bits(g.astype(F32)))
    frob_limit = max(2e-3, float(np.linalg.norm(rounded - g) / den) + FROB_ARITH)
    return dict(ok=bool(not bad.any() and frob <= frob_limit and np.all(np.isfinite(y))), fails=int(bad.sum()),
                unique=float(np.mean(lb == hb)), frob=frob)


# ---- GELU ---------------------------------------------------------------------------

GELU_NVFP4 = [
    ("nvfp4_dit", 300, 448, 520, False),      # ragged M and N, N % 8 != 0
    ("svdq_w4a4", 300, 448, 264, True),       # low-rank branch
    ("svdq_w4a4", 37, 320, 72, True),         # low rank + smoothing
    ("nvfp4_dit", 1, 16, 1, False),
]


@pytest.mark.parametrize("name,M,K,N,smooth", GELU_NVFP4)
def test_gelu_nvfp4_small(name, M, K, N, smooth):
    d = make(name, M=M, K=K, N=N)
    g_in = calibrate_input_scale(calibration_batches(name, M=M, K=K))
    lam = smooth_factors(name, K=K) if smooth else None
    rows = np.arange(M)
    ref, absum, extra, call = nvfp4_pre(d, rows, g_in, lam)
    say("gelu nvfp4", name, M, K, N, "smooth" if smooth else "")
    y = call(act="gelu_tanh")
    torch.cuda.synchronize()
    r = check_gelu(bf16_bits(y)[rows], ref, absum, K, extra)
    say(r)
    assert r["ok"], r


@pytest.mark.parametrize("name", ["nvfp4_dit", "svdq_w4a4"])
def test_gelu_nvfp4_full(name):
    d = make(name)
    g_in = calibrate_input_scale(calibration_batches(name))
    rows = sample_rows(d["M"])
    ref, absum, extra, call = nvfp4_pre(d, rows, g_in)
    say("gelu nvfp4 full", name, d["M"], d["K"], d["N"])
    y = call(act="gelu_tanh")
    torch.cuda.synchronize()
    r = check_gelu(bf16_bits(y[torch.from_numpy(rows).cuda()]), ref, absum, d["K"], extra)
    say(r)
    assert r["ok"], r


@pytest.mark.parametrize("M,K,N", [(300, 400, 520), (4608, 3072, 3072)])
def test_gelu_fp8r(M, K, N):
    d = make("fp8r_dit_n3072", M=M, K=K, N=N)
    rows = sample_rows(M)
    ref, absum, extra, call = fp8r_pre(d, rows)
    say("gelu fp8r", M, K, N)
    y = call(act="gelu_tanh")
    torch.cuda.synchronize()
    r = check_gelu(bf16_bits(y[torch.from_numpy(rows).cuda()]), ref, absum, K,
                   gamma=gemm_gamma_fp8_dot(K))
    say(r)
    assert r["ok"], r


@pytest.mark.parametrize("name,M,K,N", [("svdq_w4a4", 300, 448, 264), ("nvfp4_dit", 129, 256, 300),
                                        ("svdq_w4a4", 4608, 3072, 3072)])
def test_gelu_int4(name, M, K, N):
    d = make(name, M=M, K=K, N=N)
    rows = sample_rows(M)
    ref, absum, extra, call = int4_pre(d, rows)
    say("gelu int4", name, M, K, N)
    y = call(act="gelu_tanh")
    torch.cuda.synchronize()
    r = check_gelu(bf16_bits(y[torch.from_numpy(rows).cuda()]), ref, absum, K, extra)
    say(r)
    assert r["ok"], r


# ---- fused QKV ----------------------------------------------------------------------

SENTINEL = 0x7F7F  # a bf16 bit pattern no output of these tests takes


def qkv_buffers(heads, tokens, hd):
    return [torch.full((heads, tokens, hd), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
            for _ in range(3)]


def run_qkv(scheme, d, heads, hd, tokens, off, rows):
    M, K = d["x"].shape
    if scheme == "nvfp4":
        g_in = calibrate_input_scale(calibration_batches(d["name"], M=M, K=K))
        ref, absum, extra, call = nvfp4_pre(d, rows, g_in)
        gamma = None
    elif scheme == "fp8r":
        ref, absum, extra, call = fp8r_pre(d, rows)
        gamma = gemm_gamma_fp8_dot(K)
    else:
        ref, absum, extra, call = int4_pre(d, rows)
        gamma = None
    q, k, v = qkv_buffers(heads, tokens, hd)
    plain = call()
    out = call(qkv=(q, k, v, off))
    torch.cuda.synchronize()
    assert out[0] is q
    parts = [bf16_bits(t).reshape(heads, tokens, hd) for t in (q, k, v)]
    # untouched rows keep the sentinel; written rows gather back to y
    for t in parts:
        assert np.all(t[:, :off] == SENTINEL) and np.all(t[:, off + M:] == SENTINEL)
    # the written rows hold the plain call's y at the positions of the oracle's layout
    yb = bf16_bits(plain)
    want = qkv_split_ref(f64(yb), heads, hd, tokens, off)
    for t, w in zip(parts, want):
        assert np.array_equal(f64(t[:, off:off + M]), w[:, off:off + M]), "QKV scatter differs from the plain output"
    return check_gemm(yb[rows], ref, absum, K, extra_abs=extra, gamma=gamma)


@pytest.mark.parametrize("scheme", ["nvfp4", "fp8r", "int4"])
@pytest.mark.parametrize("M,K,heads,hd,tokens,off", [(300, 448, 2, 64, 337, 37), (1, 64, 1, 8, 1, 0),
                                                     (130, 256, 3, 128, 200, 70)])
def test_qkv_small(scheme, M, K, heads, hd, tokens, off):
    N = 3 * heads * hd
    d = make("qkv_dit" if scheme != "int4" else "svdq_w4a4", M=M, K=K, N=N)
    if scheme == "fp8r":
        d = make("fp8r_dit_n3072", M=M, K=K, N=N)
    say("qkv", scheme, M, K, heads, hd, tokens, off)
    r = run_qkv(scheme, d, heads, hd, tokens, off, np.arange(M))
    say(r)
    assert r["ok"], r


def test_qkv_full_nvfp4():
    d = make("qkv_dit")
    s = d["spec"]
    say("qkv full", d["M"], d["K"], d["N"], s["heads"], s["head_dim"], s["tokens"], s["offset"])
    r = run_qkv("nvfp4", d, s["heads"], s["head_dim"], s["tokens"], s["offset"], sample_rows(d["M"]))
    say(r)
    assert r["ok"], r


# ---- GELU MLP -------------------------------------------------------------------------

def mlp_case(M, K, H, N, lr1, lr2, smooth1, smooth2, rows):
    d = make("svdq_mlp", M=M, K=K, N=H, N2=N)
    g1 = calibrate_input_scale(calibration_batches("svdq_mlp", M=M, K=K))
    lam1 = smooth_factors("svdq_mlp", K=K) if smooth1 else None
    lam2 = smooth_factors("svdq_mlp", K=H) if smooth2 else None
    ref1, absum1, extra1, _ = nvfp4_pre(d, rows, g1, lam1, lowrank=lr1)
    g_w1 = global_scale(amax_bf16(d["w"]))
    w1p, w1b = quant_nvfp4(d["w"], g_w1)
    h_nom = gelu_bf16_ref(ref1)
    h_in = h_nom if lam2 is None else smooth_bf16(h_nom, lam2)
    g2 = global_scale(amax_bf16(h_in))
    g_w2 = global_scale(amax_bf16(d["w2"]))
    w2p, w2b = quant_nvfp4(d["w2"], g_w2)
    fc1 = dict(weight=to_dev(w1p), weight_scale=to_dev(w1b), weight_scale_2=g_w1, input_scale=g1,
               smooth=None if lam1 is None else to_dev(lam1))
    if lr1:
        fc1.update(lora_down=to_dev_bf16(d["l1"]), lora_up=to_dev_bf16(d["l2"]))
    fc2 = dict(weight=to_dev(w2p), weight_scale=to_dev(w2b), weight_scale_2=g_w2, input_scale=g2,
               smooth=None if lam2 is None else to_dev(lam2))
    if lr2:
        fc2.update(lora_down=to_dev_bf16(d["l1_2"]), lora_up=to_dev_bf16(d["l2_2"]))
    x = to_dev_bf16(d["x"])
    R1, R2 = (32 if lr1 else 0), (32 if lr2 else 0)
    ws = torch.empty((qpl.qlinear_mlp_nvfp4_workspace_bytes(M, K, H, N, R1, R2),), dtype=torch.uint8, device="cuda")
    y = qpl.qlinear_mlp_nvfp4(x, fc1, fc2, workspace=ws)
    # the same two layers as separate calls
    kw1 = {k: fc1[k] for k in ("lora_down", "lora_up") if k in fc1}
    kw2 = {k: fc2[k] for k in ("lora_down", "lora_up") if k in fc2}
    h = qpl.qlinear_nvfp4(x, fc1["weight"], fc1["weight_scale"], g_w1, g1, smooth=fc1["smooth"], act="gelu_tanh",
                          **kw1)
    y2 = qpl.qlinear_nvfp4(h, fc2["weight"], fc2["weight_scale"], g_w2, g2, smooth=fc2["smooth"], **kw2)
    torch.cuda.synchronize()
    r_rows = torch.from_numpy(rows).cuda()
    # fc2's quantized input, left at the start of the workspace: packed codes, then
    # slab-major block scales; decoded here to the values e2m1(code) * dec(sf)
    parts = nvfp4_workspace_parts(M, H, N, R2)
    wsh = host(ws[:parts["xs"] + 8 * M * parts["S"]])
    hq = wsh[:M * H // 2].reshape(M, H // 2)[rows]
    hs = slab_scales_to_rows(wsh[parts["xs"]:], M, H)[0][rows]
    he_bits = f32_to_bf16_bits(dequant_nvfp4(hq, hs, 1.0).astype(F32))
    h_off = qpl.qlinear_workspace_bytes(qpl.QPL_NVFP4, M, H, N, R2)
    hw = ws[h_off:h_off + 2 * M * H].view(torch.bfloat16).view(M, H)[r_rows]
    yb = bf16_bits(y)
    same = np.array_equal(yb, bf16_bits(y2))

    # h: GELU of fc1 inside its interval
    rh = check_gelu(bf16_bits(hw), ref1, absum1, K, extra1)
    # fc2's operand: an nvfp4 quantization of some h in the GELU interval
    lo, hi = gelu_interval(ref1, pre_activation_error(ref1, absum1, K, extra1))
    hlb, hhb = bf16_interval(lo, hi)
    lb, hb = (hlb, hhb) if lam2 is None else smooth_interval(hlb, hhb, lam2)
    rq = check_nvfp4_expanded(he_bits, lb, hb, g2)

    # y against the oracle's fc2 on its nominal operand, widened by the ambiguous codes
    # (and, with fc2's low-rank branch, by the ambiguous smoothed h it reads)
    nominal, width = expanded_nominal_and_width(h_in, lb, hb, g2)
    gf = float(F32(g2))
    W2 = dequant_nvfp4(w2p, w2b, g_w2)
    ref2 = (nominal * gf) @ W2.T
    absum2 = np.abs(nominal * gf) @ np.abs(W2).T
    allow = (width * gf) @ np.abs(W2).T
    if lr2:
        ref2 = ref2 + lowrank_ref(h_in, d["l1_2"], d["l2_2"])
        lr_abs = lowrank_abs(h_in, d["l1_2"], d["l2_2"])
        dh = np.abs(f64(hb) - f64(lb))
        l1a, l2a = np.abs(f64(d["l1_2"])), np.abs(f64(d["l2_2"]))
        allow = allow + (dh @ l1a) @ l2a
        absum2 = absum2 + lr_abs
    yv = f64(yb[rows])
    err = np.abs(yv - ref2)
    floor = gemm_gamma(H) * (absum2 + allow) + allow
    # the output rounding is relative to the computed value, which the ambiguous
    # codes can move up to the allowance away from ref2
    bound = 4 * ulp_bf16(np.abs(ref2) + floor) + floor
    fails = int(np.count_nonzero(err > bound))
    den = np.linalg.norm(ref2)
    frob = float(np.linalg.norm(yv - ref2) / den)
    frob_limit = 2e-3 + float(np.linalg.norm(allow) / den)
    ok = rh["ok"] and rq["ok"] and same and fails == 0 and frob <= frob_limit
    return dict(ok=ok, h=rh, operand=rq, same_as_separate=same, fails=fails, worst=float(np.max(err / bound)),
                frob=frob, frob_limit=frob_limit)


MLP_CASES = [
    (300, 448, 512, 264, True, False, True, True),    # fc1 low rank, both smoothed, ragged M and N
    (256, 512, 512, 256, False, False, False, False), # plain BFL nvfp4 layers
    (37, 320, 272, 72, True, True, False, True),      # both low rank; H = 17 blocks of 16
    (1, 64, 16, 8, False, True, True, False),         # one hidden block, fc2 low rank
]


@pytest.mark.parametrize("M,K,H,N,lr1,lr2,smooth1,smooth2", MLP_CASES)
def test_mlp_nvfp4_small(M, K, H, N, lr1, lr2, smooth1, smooth2):
    say("mlp nvfp4", M, K, H, N, lr1, lr2, smooth1, smooth2)
    r = mlp_case(M, K, H, N, lr1, lr2, smooth1, smooth2, np.arange(M))
    say(r)
    assert r["ok"], r


def test_mlp_nvfp4_full():
    # FLUX feed-forward 4608 x 3072 -> 12288 -> 3072, both layers rank 32 and smoothed
    say("mlp nvfp4 full", 4608, 3072, 12288, 3072)
    r = mlp_case(4608, 3072, 12288, 3072, True, True, True, True, sample_rows(4608, n=32))
    say(r)
    assert r["ok"], r
