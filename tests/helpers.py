"""Shared test helpers: numpy <-> torch bf16 bit transfers and adversarial inputs.
(No method arithmetic: only bit-pattern construction and data movement.)"""
import numpy as np
import torch


def to_dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_bits(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t):
    return t.detach().cpu().numpy()


def adversarial_rows(K, seed=0):
    """bf16 rows that stress the encoders: zero rows, signed zeros, bf16 subnormals,
    huge and tiny magnitudes, a single outlier, constant rows, random bit patterns."""
    rng = np.random.default_rng(seed)
    rows = []
    rows.append(np.zeros(K, np.uint16))                                    # all +0
    r = np.zeros(K, np.uint16); r[::3] = 0x8000; rows.append(r)            # mixed +-0
    rows.append(rng.integers(1, 0x80, K).astype(np.uint16) | (rng.integers(0, 2, K).astype(np.uint16) << 15))  # subnormals
    r = (rng.standard_normal(K) * 1e-3).astype(np.float32); r[K // 2] = 3e4
    rows.append((r.view(np.uint32) >> 16).astype(np.uint16))             # one outlier (truncated to bf16)
    rows.append(np.full(K, 0x3F80, np.uint16))                             # constant 1.0
    rows.append(np.full(K, 0xC2C8, np.uint16))                             # constant -100
    bits = rng.integers(0, 0x10000, K).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    bits[exp == 0xFF] &= 0x807F                                            # keep finite
    rows.append(bits)                                                      # random finite patterns
    r = (rng.standard_normal(K) * 1e30).astype(np.float32)
    rows.append((r.view(np.uint32) >> 16).astype(np.uint16))             # huge
    r = (rng.standard_normal(K) * 1e-30).astype(np.float32)
    rows.append((r.view(np.uint32) >> 16).astype(np.uint16))             # tiny (normal, near subnormal scale)
    r = (rng.standard_normal(K) * 2.0).astype(np.float32)
    b = (r.view(np.uint32) >> 16).astype(np.uint16)
    b[::5] = 0x0000
    b[2::5] = 0x8000
    rows.append(b)                                                         # exact +-0 among normal values
    return np.stack(rows)


def r256(b):
    return (b + 255) // 256 * 256


def nvfp4_workspace_parts(M, K, N, R=0):
    """Byte offsets of qlinear_nvfp4's workspace parts (as include/qpl.h lays them
    out): activation codes, activation block scales [S, M, 8], and the weight's
    block scales [S, N, 8] (after the low-rank parts when R > 0)."""
    S = (K + 127) // 128
    off_xs = r256(M * K // 2)
    end = off_xs + r256(8 * M * S)
    if R > 0:
        rp = (R + 31) // 32 * 32
        end += r256(2 * rp * K) + r256(2 * M * 2 * rp) + r256(2 * N * 2 * rp)
    return dict(xq=0, xs=off_xs, ws=end, S=S)


def slab_scales_to_rows(buf, rows, K):
    """uint8 [S, rows, 8] (slab-major block scales) -> ([rows, K/16] row-major, the
    bytes past K/16).  Data movement only."""
    S = (K + 127) // 128
    a = np.asarray(buf, np.uint8).reshape(S, rows, 8).transpose(1, 0, 2).reshape(rows, S * 8)
    return a[:, : K // 16], a[:, K // 16:]
