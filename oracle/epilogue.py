"""Model-specific epilogues of the quantized linear (oracle; test infrastructure only).

The Nunchaku post ("Introducing Nunchaku Lite", first paragraph) says much of the
original engine's speed comes from fused paths tied to a model's module layout,
and names fused QKV projections and fused GELU/MLP kernels; it defines neither.
The readings taken here (each listed, with its reason, in the design notes):

* GELU is the tanh form of DiT feed-forward blocks (Hendrycks and Gimpel,
  "Gaussian Error Linear Units", tanh approximation):
  gelu(v) = v / 2 * (1 + tanh(sqrt(2 / pi) * (v + 0.044715 v^3))).
  An epilogue applies it to the layer's fp32 result before the bf16 rounding:
  h = bf16(gelu(y)).
* The fused MLP is fc2(h) with h = bf16(gelu(fc1(x))).  fc2 sees h exactly as its
  own quantizer would: smoothing by fc2's factors, then nvfp4 quantization under
  fc2's input_scale.  Fusing moves that quantization into fc1's epilogue; the
  result is the two layers run one after the other.
* The fused QKV projection is one linear over the row-wise concatenation
  [W_q; W_k; W_v] whose epilogue writes the three parts of each output row to
  three tensors in the head-major layout [heads, tokens, head_dim] at a token
  offset (the layout attention reads, for the text and image tokens of a joint
  sequence).

The GPU computes y in fp32 with an unspecified summation order, so h can differ
from bf16(gelu(y_exact)) by a rounding step, and a quantization code of h can
differ with it.  The checks below therefore bound, per element, every value that
a correct computation can produce (an interval propagated through the monotone
steps: bf16 rounding, smoothing, the E4M3 block scale and the E2M1 code) and
compare exactly where that set has one member.
"""
import math

import numpy as np

from .formats import bf16_bits_to_f32, e2m1_decode, e2m1_encode, e4m3_decode, e4m3_encode, f32_to_bf16_bits
from .quant import quant_nvfp4
from .reference import dequant_nvfp4

F32 = np.float32
SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
GELU_CUBIC = 0.044715
# gelu's only minimum (gelu' = 0 near v = -0.7525, value about -0.1700; pinned by a test)
GELU_ARGMIN = -0.7525


def gelu_tanh(v):
    """The tanh form of GELU in float64, written as v / (1 + exp(-2u)) with
    u = sqrt(2 / pi) (v + 0.044715 v^3): the same function ((1 + tanh u) / 2 equals
    1 / (1 + exp(-2u))), without the cancellation of 1 + tanh(u) for large
    negative v, where the printed form loses all its digits."""
    v = np.asarray(v, dtype=np.float64)
    u = SQRT_2_OVER_PI * (v + GELU_CUBIC * v * v * v)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-2.0 * u))


def _f32_down(a):
    """Largest float32 <= a (float64 in, float64 out)."""
    f = np.asarray(a, dtype=np.float64).astype(F32)
    return np.where(f.astype(np.float64) > a, np.nextafter(f, F32(-np.inf)), f).astype(np.float64)


def _f32_up(a):
    f = np.asarray(a, dtype=np.float64).astype(F32)
    return np.where(f.astype(np.float64) < a, np.nextafter(f, F32(np.inf)), f).astype(np.float64)


def pre_activation_error(ref, abs_sum, K, extra_abs=None, gamma=None):
    """Bound on |y_fp32 - y_exact| for a layer output before its activation: the
    accumulation floor gamma sum_k |a_k w_k| (gamma defaults to the fp32 floor
    ceil(K / 16) 2^-24; the low-rank magnitudes take the fp32 floor) and two fp32
    roundings of the scale products."""
    g32 = math.ceil(K / 16) * 2.0 ** -24
    g = g32 if gamma is None else gamma
    e = g * np.asarray(abs_sum, dtype=np.float64) + 2.0 ** -22 * np.abs(ref)
    if extra_abs is not None:
        e = e + g32 * np.asarray(extra_abs, dtype=np.float64)
    return e


def gelu_eval_error(v, h):
    """Bound on the error of an fp32 evaluation of gelu at v as v / (1 + 2^t) with
    t = -2 u log2(e) computed in fp32, exp2 and a reciprocal each within a few fp32
    ulps: a relative error of t (a few ulps) moves 2^t by |t| ln 2 times it, 2 |u|
    times, so the relative error is bounded by 2^-23 (16 + 8 |u|); where 1 + 2^t
    passes 2^126 the reciprocal may flush to zero, an absolute error below
    |v| 2^-120; plus a floor below the bf16 range."""
    v = np.asarray(v, dtype=np.float64)
    u = SQRT_2_OVER_PI * (v + GELU_CUBIC * v ** 3)
    return np.abs(h) * 2.0 ** -23 * (16.0 + 8.0 * np.abs(u)) + np.abs(v) * 2.0 ** -120 + 2.0 ** -140


def gelu_interval(ref, err):
    """[lo, hi] (float64) holding gelu(t) for every t in [ref - err, ref + err],
    widened by the evaluation error.  gelu falls, then rises, with its minimum at
    GELU_ARGMIN."""
    a = np.asarray(ref, dtype=np.float64) - err
    b = np.asarray(ref, dtype=np.float64) + err
    ga, gb = gelu_tanh(a), gelu_tanh(b)
    lo = np.minimum(ga, gb)
    hi = np.maximum(ga, gb)
    inside = (a < GELU_ARGMIN + 1e-3) & (b > GELU_ARGMIN - 1e-3)
    # the true minimum is below gelu at any sampled point near it; take the value
    # at the pinned argmin minus a margin covering the argmin's uncertainty
    lo = np.where(inside, np.minimum(lo, gelu_tanh(np.float64(GELU_ARGMIN)) - 1e-6), lo)
    ev = np.maximum(gelu_eval_error(a, ga), gelu_eval_error(b, gb))
    return lo - ev, hi + ev


def bf16_interval(lo, hi):
    """bf16 bit patterns [lo_bits, hi_bits] of every bf16 value that an fp32 value
    in [lo, hi] rounds to (float32 rounding then bf16 rounding, both monotone)."""
    return f32_to_bf16_bits(_f32_down(lo).astype(F32)), f32_to_bf16_bits(_f32_up(hi).astype(F32))


def smooth_interval(lo_bits, hi_bits, smooth):
    """The monotone smoothing step bf16(x / smooth[k]) applied to both bounds."""
    lam = np.asarray(smooth, dtype=F32)
    lo = bf16_bits_to_f32(lo_bits)
    hi = bf16_bits_to_f32(hi_bits)
    return f32_to_bf16_bits((lo / lam[None, :]).astype(F32)), f32_to_bf16_bits((hi / lam[None, :]).astype(F32))


def _e2m1_value(q):
    return e2m1_decode(e2m1_encode(q.astype(F32)))


def nvfp4_expanded_bounds(lo_bits, hi_bits, g):
    """Every nvfp4 quantization (block scale rule and codes of the oracle's
    quant_nvfp4 under global scale g) of every bf16 tensor x with
    lo <= x <= hi elementwise, described per block and element.

    Returns (sf_lo, sf_hi, vlo, vhi): E4M3 block-scale codes [R, K/16] bounding the
    possible scales (positive codes order like their values), and, per candidate
    scale offset t = 0 .. max(sf_hi - sf_lo), arrays [T, R, K] of the smallest and
    largest expanded value e2m1(code) * dec(sf) an element can take under scale
    sf_lo + t (NaN where that scale is not a candidate).
    """
    lo = bf16_bits_to_f32(lo_bits).astype(np.float64)
    hi = bf16_bits_to_f32(hi_bits).astype(np.float64)
    R, K = lo.shape
    g = F32(g)
    c = F32(F32(6.0) * g)
    lob, hib = lo.reshape(R, K // 16, 16), hi.reshape(R, K // 16, 16)
    amin = np.where((lob <= 0) & (hib >= 0), 0.0, np.minimum(np.abs(lob), np.abs(hib)))
    amax = np.maximum(np.abs(lob), np.abs(hib))
    sf_lo = e4m3_encode((np.max(amin, axis=2).astype(F32) / c).astype(F32))
    sf_hi = e4m3_encode((np.max(amax, axis=2).astype(F32) / c).astype(F32))
    T = int(np.max(sf_hi.astype(np.int64) - sf_lo.astype(np.int64))) + 1 if sf_lo.size else 1
    vlo = np.full((T, R, K // 16, 16), np.nan)
    vhi = np.full((T, R, K // 16, 16), np.nan)
    for t in range(T):
        sf = sf_lo.astype(np.int64) + t
        ok = sf <= sf_hi
        sfc = np.where(ok, sf, sf_lo).astype(np.uint8)
        dsf = e4m3_decode(sfc)
        d = (dsf.astype(F32) * g).astype(F32)
        with np.errstate(divide="ignore", invalid="ignore"):
            ql = np.where(d[:, :, None] > 0, _e2m1_value((lob.astype(F32) / d[:, :, None]).astype(F32)), 0.0)
            qh = np.where(d[:, :, None] > 0, _e2m1_value((hib.astype(F32) / d[:, :, None]).astype(F32)), 0.0)
        a, b = ql * dsf[:, :, None], qh * dsf[:, :, None]
        vlo[t] = np.where(ok[:, :, None], a, np.nan)
        vhi[t] = np.where(ok[:, :, None], b, np.nan)
    return sf_lo, sf_hi, vlo.reshape(T, R, K), vhi.reshape(T, R, K)


def check_nvfp4_expanded(xe_bits, lo_bits, hi_bits, g):
    """Whether the expanded operand xe (bf16 values e2m1(code) * dec(sf), one scale
    per 16-block) is the nvfp4 quantization of some x with lo <= x <= hi: per
    block, one candidate scale must explain all 16 values, each an E2M1 value times
    dec(sf) inside its element's bounds.  Blocks whose candidate set has one member
    are compared exactly.  Returns a dict with ``ok`` and the counts."""
    xe = bf16_bits_to_f32(xe_bits).astype(np.float64)
    R, K = xe.shape
    sf_lo, sf_hi, vlo, vhi = nvfp4_expanded_bounds(lo_bits, hi_bits, g)
    T = vlo.shape[0]
    xb = xe.reshape(R, K // 16, 16)
    good = np.zeros((R, K // 16), dtype=bool)
    for t in range(T):
        a = vlo[t].reshape(R, K // 16, 16)
        b = vhi[t].reshape(R, K // 16, 16)
        sf = (sf_lo.astype(np.int64) + t).clip(0, 126).astype(np.uint8)
        dsf = e4m3_decode(sf)[:, :, None]
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.where(dsf > 0, xb / dsf, 0.0)
        on_grid = np.isin(np.abs(q), [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]) | (xb == 0)
        inside = (xb >= a) & (xb <= b) & on_grid
        good |= np.all(inside, axis=2) & ~np.isnan(a[:, :, 0])
    unique = (sf_lo == sf_hi) & np.all((vlo[0] == vhi[0]).reshape(R, K // 16, 16), axis=2)
    return dict(ok=bool(np.all(good)), bad_blocks=int(np.count_nonzero(~good)), blocks=int(good.size),
                ambiguous_blocks=int(np.count_nonzero(~unique)))


def expanded_nominal_and_width(h_bits, lo_bits, hi_bits, g):
    """The oracle's own expanded quantization of h (the nominal operand) and, per
    element, the largest distance from it to any value a correct quantization of
    an x in [lo, hi] can take (0 where the outcome is unique)."""
    packed, bs = quant_nvfp4(h_bits, g)
    nominal = dequant_nvfp4(packed, bs, 1.0)
    _, _, vlo, vhi = nvfp4_expanded_bounds(lo_bits, hi_bits, g)
    with np.errstate(invalid="ignore"):
        w = np.nanmax(np.maximum(np.abs(vlo - nominal[None]), np.abs(vhi - nominal[None])), axis=0)
    return nominal, np.nan_to_num(w)


def gelu_bf16_ref(ref):
    """bf16 bits of gelu(ref) computed in float64 and rounded once per format
    (float32, then bf16): the nominal h of the oracle."""
    return f32_to_bf16_bits(gelu_tanh(ref).astype(F32))


def qkv_split_ref(y, heads, head_dim, tokens, offset):
    """Scatter a [M, 3 heads head_dim] output into q, k, v arrays of shape
    [heads, tokens, head_dim], rows offset .. offset + M - 1 (other rows NaN)."""
    M, N = y.shape
    d = heads * head_dim
    assert N == 3 * d and offset + M <= tokens
    out = []
    for j in range(3):
        t = np.full((heads, tokens, head_dim), np.nan)
        t[:, offset:offset + M, :] = y[:, j * d:(j + 1) * d].reshape(M, heads, head_dim).transpose(1, 0, 2)
        out.append(t)
    return out
