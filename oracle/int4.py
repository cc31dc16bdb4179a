"""INT4 variant of the SVDQuant W4A4 linear (oracle; test infrastructure only).

The Nunchaku post ("Introducing Nunchaku Lite", layer list) says ``svdq_w4a4`` --
4-bit weights and activations with the SVDQuant low-rank correction -- comes in
INT4 and NVFP4 variants; the NVFP4 one is the BFL nvfp4 scheme.  The post gives no
INT4 format; the readings here (each listed, with its reason, in the design notes):

* signed 4-bit codes q in -8..7 (two's complement nibbles, the even channel in the
  low nibble), one fp32 scale per group of 64 consecutive input channels, the same
  rule for activations and weights;
* symmetric rule per group: s = amax / 7 (fp32, correctly rounded);
  q = clamp(rint(x / s), -8, 7) with a correctly rounded fp32 division and ties to
  even; an all-zero group has s = 0 and codes 0;
* the layer: y = bf16(sum_g s_x[m, g] s_w[n, g] sum_{k in g} q_x q_w + (x L1) L2),
  with the same optional smoothing as the NVFP4 variant (x replaced by
  bf16(x / smooth) in both terms).  The reference is the float64 product of the
  exactly dequantized operands.
"""
import numpy as np

from .formats import bf16_bits_to_f32

F32 = np.float32
GROUP = 64


def quant_int4(x_bits):
    """Group-wise symmetric INT4 quantization of a bf16 [R, K] tensor (K % 64 == 0).

    Returns (packed uint8 [R, K/2], scale float32 [R, K/64]).
    """
    x = bf16_bits_to_f32(x_bits)
    R, K = x.shape
    assert K % GROUP == 0
    xg = x.reshape(R, K // GROUP, GROUP)
    amax = np.max(np.abs(xg), axis=2) if K else np.zeros((R, 0), F32)
    s = (amax / F32(7.0)).astype(F32)
    q = np.zeros(xg.shape, dtype=np.int8)
    nz = s > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = np.rint((xg[nz] / s[nz][:, None]).astype(F32))
    q[nz] = np.clip(qf, -8, 7).astype(np.int8)
    c = (q.reshape(R, K).astype(np.int16) & 0xF).astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8), s


def unpack_int4(packed):
    """[R, K/2] bytes -> [R, K] int8 codes (sign-extended nibbles, low nibble = even k)."""
    p = np.asarray(packed, dtype=np.uint8)
    u = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.int16)
    u[:, 0::2] = p & 0xF
    u[:, 1::2] = p >> 4
    return np.where(u >= 8, u - 16, u).astype(np.int8)


def dequant_int4(packed, scale):
    """float64 [R, K] = q * s per group (exact)."""
    q = unpack_int4(packed).astype(np.float64)
    R, K = q.shape
    s = np.asarray(scale, dtype=np.float64)
    return (q.reshape(R, K // GROUP, GROUP) * s[:, :, None]).reshape(R, K)


def qlinear_int4_ref(x_packed, x_scale, w_packed, w_scale):
    """float64 [M, N] reference of the INT4 linear on the same quantized operands."""
    return dequant_int4(x_packed, x_scale) @ dequant_int4(w_packed, w_scale).T
