"""fp8r and nvfp4 quantizers (oracle; test infrastructure only).

Follows the intro bullets of the Diffusers "BFL (fp8r / nvfp4)" guide:

* fp8r: an E4M3 ``weight`` with one fp32 ``weight_scale`` per row, and
  activations quantized per row to E4M3 at run time.
* nvfp4: packed E2M1 ``weight`` (two values per byte), E4M3 block scales per 16
  elements (``weight_scale``), a global fp32 ``weight_scale_2`` and a calibrated
  fp32 activation scale ``input_scale``.

Readings where the guide is silent (each one is listed, with its reason, in the
design notes):

* fp8r scale of a row: ``s = amax / 448`` in fp32, the same rule for weights and
  activations; codes are ``E4M3(x / s)`` with a correctly rounded fp32 division;
  an all-zero row has ``s = 0`` and signed-zero codes.
* nvfp4 with global scale ``g``: ``c = 6 * g`` (fp32, once per tensor); per
  16-block ``sf = E4M3(bmax / c)``; ``d = dec(sf) * g`` (fp32); codes
  ``E2M1(x / d)``, or signed zeros when ``d == 0``.
* Global scale of a tensor: ``amax / 2688`` in fp32 (2688 = 448 * 6 exactly);
  ``input_scale`` uses the largest amax over the calibration batches.
* Packing: byte j of a row holds element 2j in its low nibble and 2j+1 in its
  high nibble; block scales are row-major ``[rows, K/16]``.
* SVDQuant smoothing (Nunchaku post, "Background: SVDQuant and Nunchaku": the
  activation outliers are moved into the weights): the layer divides input
  channel k by a positive factor ``smooth[k]`` (the weight's column k carries the
  factor instead), ``x_hat = bf16(x / smooth[k])`` with a correctly rounded fp32
  division, and both the 4-bit path and the low-rank branch take ``x_hat``.
"""
import numpy as np

from .formats import (bf16_bits_to_f32, e2m1_encode, e4m3_decode, e4m3_encode, f32_to_bf16_bits)

F32 = np.float32


def amax_bf16(x_bits):
    """Largest magnitude of a bf16 tensor, as float32 (exact)."""
    x = bf16_bits_to_f32(x_bits)
    return F32(np.max(np.abs(x))) if x.size else F32(0.0)


def global_scale(amax):
    """nvfp4 global scale from an amax: amax / (448 * 6) in fp32."""
    return F32(F32(amax) / F32(2688.0))


def calibrate_input_scale(batches):
    """Static activation scale from calibration batches (bf16 bit arrays)."""
    return global_scale(max(amax_bf16(b) for b in batches))


def quant_fp8_row(x_bits):
    """Row-wise E4M3 quantization of a bf16 [R, K] tensor.

    Returns (codes uint8 [R, K], scale float32 [R]) with dec(codes) * scale ~ x.
    """
    x = bf16_bits_to_f32(x_bits)
    R, K = x.shape
    amax = np.max(np.abs(x), axis=1) if K else np.zeros(R, F32)
    s = (amax / F32(448.0)).astype(F32)
    codes = np.empty((R, K), dtype=np.uint8)
    nz = s > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (x[nz] / s[nz, None]).astype(F32)
    codes[nz] = e4m3_encode(q)
    codes[~nz] = np.where(np.signbit(x[~nz]), 0x80, 0x00).astype(np.uint8)
    return codes, s


def pack_e2m1(codes):
    """[R, K] E2M1 codes (0..15) -> [R, K/2] bytes: low nibble = even k."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_e2m1(packed):
    """[R, K/2] bytes -> [R, K] E2M1 codes."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def quant_nvfp4(x_bits, g):
    """NVFP4 quantization of a bf16 [R, K] tensor (K % 16 == 0) under global
    scale ``g`` (``input_scale`` for activations, ``weight_scale_2`` for weights).

    Returns (packed uint8 [R, K/2], block_scale uint8 E4M3 [R, K/16]).
    """
    x = bf16_bits_to_f32(x_bits)
    R, K = x.shape
    assert K % 16 == 0
    g = F32(g)
    c = F32(F32(6.0) * g)
    xb = x.reshape(R, K // 16, 16)
    bmax = np.max(np.abs(xb), axis=2) if K else np.zeros((R, 0), F32)
    u = (bmax / c).astype(F32)
    sf = e4m3_encode(u)
    d = (e4m3_decode(sf).astype(F32) * g).astype(F32)
    codes = np.empty(xb.shape, dtype=np.uint8)
    nz = d > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (xb[nz] / d[nz][:, None]).astype(F32)
    codes[nz] = e2m1_encode(q)
    codes[~nz] = np.where(np.signbit(xb[~nz]), 0x8, 0x0).astype(np.uint8)
    return pack_e2m1(codes.reshape(R, K)), sf


def smooth_bf16(x_bits, smooth):
    """SVDQuant smoothing of a bf16 [R, K] activation by per-channel factors.

    x_hat[r, k] = bf16_RNE(fp32(x[r, k]) / smooth[k]): one correctly rounded fp32
    division, then the round to bf16 that makes x_hat the 16-bit activation both
    branches of the layer read.  ``smooth`` is float32 [K], positive and finite.
    Returns bf16 bit patterns [R, K].
    """
    x = bf16_bits_to_f32(x_bits)
    lam = np.asarray(smooth, dtype=F32)
    assert lam.shape == (x.shape[1],)
    return f32_to_bf16_bits((x / lam[None, :]).astype(F32))
