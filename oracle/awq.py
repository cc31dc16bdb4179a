"""Weight-only 4-bit linear with 16-bit activations (oracle; test infrastructure only).

The Nunchaku post ("Introducing Nunchaku Lite", layer list) names ``awq_w4a16``:
4-bit weights, 16-bit activations, for the adaptive-normalization and modulation
projections (FLUX adanorm_single / adanorm_zero, Qwen-Image modulation), which
are memory-bound and precision-sensitive.  The post gives no format; the readings
here (each listed, with its reason, in the design notes):

* weights W [N, K] are quantized in groups of G consecutive input channels
  (G in {32, 64, 128}, K % G == 0) to unsigned 4-bit codes q in 0..15 with one
  bf16 scale s and one integer zero point z in 0..15 per group; the weight value
  is (q - z) * s.  Codes are packed two per byte, the even channel in the low
  nibble (the nvfp4 packing);
* the quantizer is the min/max rule over the group with the range widened to
  contain 0 (so that 0 is a grid point): hi = max(max w, 0), lo = min(min w, 0),
  s = bf16(fp32((hi - lo) / 15)), z = clamp(rint(-lo / s), 0, 15),
  q = clamp(rint(w / s) + z, 0, 15), fp32 arithmetic with correctly rounded
  divisions and ties to even; a group whose s is 0 gets q = z = 0;
* AWQ's activation-aware channel scaling is an offline step folded into the
  weights and the preceding operation; the layer computes y = x (W_hat)^T with
  x bf16 [M, K], accumulation in fp32 and a bf16 output.  The reference is the
  float64 product of the exactly dequantized weight.
"""
import numpy as np

from .formats import bf16_bits_to_f32, f32_to_bf16_bits
from .quant import pack_e2m1, unpack_e2m1

F32 = np.float32
GROUPS = (32, 64, 128)


def quant_w4g(w_bits, group):
    """Group-wise asymmetric 4-bit quantization of a bf16 weight [N, K].

    Returns (packed uint8 [N, K/2], scale bf16 bits uint16 [N, K/G], zero uint8 [N, K/G]).
    """
    assert group in GROUPS
    w = bf16_bits_to_f32(w_bits)
    N, K = w.shape
    assert K % group == 0
    wg = w.reshape(N, K // group, group)
    hi = np.maximum(wg.max(axis=2), F32(0))
    lo = np.minimum(wg.min(axis=2), F32(0))
    s_bits = f32_to_bf16_bits(((hi - lo).astype(F32) / F32(15)).astype(F32))
    s = bf16_bits_to_f32(s_bits)
    q = np.zeros(wg.shape, dtype=np.uint8)
    z = np.zeros(s.shape, dtype=np.uint8)
    nz = s > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        zf = np.rint((-lo[nz] / s[nz]).astype(F32))
        z[nz] = np.clip(zf, 0, 15).astype(np.uint8)
        qf = np.rint((wg[nz] / s[nz][:, None]).astype(F32)) + z[nz][:, None].astype(F32)
    q[nz] = np.clip(qf, 0, 15).astype(np.uint8)
    return pack_e2m1(q.reshape(N, K)), s_bits, z


def dequant_w4g(packed, scale_bits, zero, group):
    """float64 [N, K] = (q - z) * s per group (exact)."""
    q = unpack_e2m1(packed).astype(np.float64)
    N, K = q.shape
    s = bf16_bits_to_f32(scale_bits).astype(np.float64)
    z = np.asarray(zero, dtype=np.float64)
    v = (q.reshape(N, K // group, group) - z[:, :, None]) * s[:, :, None]
    return v.reshape(N, K)


def qlinear_w4a16_ref(x_bits, packed, scale_bits, zero, group):
    """float64 [M, N] = x (W_hat)^T with x bf16 [M, K] and the dequantized weight."""
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    return x @ dequant_w4g(packed, scale_bits, zero, group).T
