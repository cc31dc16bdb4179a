"""Host-side checks of libqpl.so that need no GPU: the library loads, exports every
entry point include/qpl.h declares, and rejects bad arguments before touching a
device (each status is forced from the host)."""
import ctypes
import os
import re

import pytest
import torch

import precision_quantized_linear_amd as qpl
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "qpl.h")
OK, NULL, SHAPE, ALIGN, ARG, WORKSPACE, DEVICE, LAUNCH = range(8)
P = ctypes.c_void_p
A = P(1 << 20)  # aligned, never dereferenced: every call below fails validation first
B = P(1 << 21)
C = P(1 << 22)
D = P(1 << 23)
MIS = P((1 << 20) + 4)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return qpl.load()


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(qpl.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(8):
        assert lib.qpl_status_str(s)
    assert lib.qpl_status_str(99) == b"unknown status"


def test_workspace_sizes(lib):
    M, K, N = 4608, 3072, 12288
    assert qpl.qlinear_workspace_bytes(qpl.QPL_FP8R, M, K, N) == M * K + M * 4
    # nvfp4: packed codes of x, its block scales slab-major [K/128, M, 8], then (R > 0)
    # L1^T, T and [L2^T | L2^T], then the weight's block scales [K/128, N, 8]
    S = K // 128
    assert qpl.qlinear_workspace_bytes(qpl.QPL_NVFP4, M, K, N) == M * K // 2 + 8 * M * S + 8 * N * S
    r = qpl.qlinear_workspace_bytes(qpl.QPL_NVFP4, M, K, 3072, 32)
    assert r == M * K // 2 + 8 * M * S + 2 * 32 * K + 2 * M * 64 + 2 * 3072 * 64 + 8 * 3072 * S
    assert qpl.qlinear_workspace_bytes(qpl.QPL_NVFP4, 4, 24, 4) == 0      # K % 16 != 0
    assert qpl.qlinear_workspace_bytes(qpl.QPL_NVFP4, 4, 32, 4, 129) == 0  # rank too large
    assert qpl.qlinear_workspace_bytes(qpl.QPL_FP8R, 4, 32, 4, 1) == 0     # fp8r has no low rank
    assert qpl.qlinear_workspace_bytes(7, 4, 32, 4) == 0
    # INT4: codes of x and W as bytes, then (R > 0) the low-rank parts, then the x and W scales
    r256 = lambda b: (b + 255) // 256 * 256  # noqa: E731
    assert qpl.qlinear_workspace_bytes(qpl.QPL_INT4, M, K, N) == (r256(M * K) + r256(N * K) + r256(4 * M * K // 64) +
                                                                 r256(4 * N * K // 64))
    assert qpl.qlinear_workspace_bytes(qpl.QPL_INT4, 4, 96, 4) == 0  # K % 64 != 0


def test_nvfp4_workspace_ragged_k(lib):
    # K = 400: ceil(400 / 128) = 4 scale slabs; every part rounded up to 256 bytes
    r256 = lambda b: (b + 255) // 256 * 256  # noqa: E731
    M, K, N = 300, 400, 520
    assert qpl.qlinear_workspace_bytes(qpl.QPL_NVFP4, M, K, N) == r256(M * K // 2) + r256(8 * M * 4) + r256(8 * N * 4)


def test_k_limits(lib):
    # 256 rows of an operand are addressed with 32-bit offsets below 2^30 (the
    # out-of-range marker): fp8r and INT4 rows are K bytes, nvfp4 rows K/2 bytes
    ws = 1 << 62
    big = (1 << 22)
    assert qpl.qlinear_workspace_bytes(qpl.QPL_FP8R, 4, big, 8) == 0
    assert qpl.qlinear_workspace_bytes(qpl.QPL_FP8R, 4, big - 16, 8) > 0
    assert qpl.qlinear_workspace_bytes(qpl.QPL_INT4, 4, big, 8) == 0
    assert qpl.qlinear_workspace_bytes(qpl.QPL_INT4, 4, big - 64, 8) > 0
    assert qpl.qlinear_workspace_bytes(qpl.QPL_NVFP4, 4, 2 * big, 8) == 0
    assert qpl.qlinear_workspace_bytes(qpl.QPL_NVFP4, 4, 2 * big - 16, 8) > 0
    # with a low-rank branch the fused quantizer stages L1^T rows of 2K bytes: K <= 2^21
    assert qpl.qlinear_workspace_bytes(qpl.QPL_NVFP4, 4, (1 << 21) + 16, 8, 32) == 0
    assert qpl.qlinear_workspace_bytes(qpl.QPL_NVFP4, 4, 1 << 21, 8, 32) > 0
    assert qpl.qlinear_workspace_bytes(qpl.QPL_INT4, 4, (1 << 21) + 64, 8, 32) == 0
    # ... and stores the activation's scales through a descriptor below 2^31 bytes
    assert qpl.qlinear_workspace_bytes(qpl.QPL_NVFP4, 1 << 17, 1 << 18, 8, 32) == 0   # 8 M K/128 = 2^31
    assert qpl.qlinear_workspace_bytes(qpl.QPL_NVFP4, (1 << 17) - 1, 1 << 18, 8, 32) > 0
    assert qpl.qlinear_workspace_bytes(qpl.QPL_INT4, 1 << 19, 1 << 16, 8, 32) == 0    # 4 M K/64 = 2^31
    assert qpl.qlinear_workspace_bytes(qpl.QPL_INT4, (1 << 19) - 1, 1 << 16, 8, 32) > 0
    # the linears refuse them before touching a device
    assert lib.qlinear_fp8r(A, 4, big, 8, B, C, D, A, ws, None) == SHAPE
    assert lib.qlinear_nvfp4(A, 4, 2 * big, 8, B, C, 1.0, 1.0, None, None, None, 0, D, A, ws, None) == SHAPE
    assert lib.qlinear_nvfp4(A, 4, (1 << 21) + 16, 8, B, C, 1.0, 1.0, None, A, B, 32, D, A, ws, None) == SHAPE
    assert lib.qlinear_int4(A, 4, big, 8, B, C, None, None, None, 0, D, A, ws, None) == SHAPE
    assert lib.qlinear_int4(A, 4, (1 << 21) + 64, 8, B, C, None, A, B, 32, D, A, ws, None) == SHAPE


def test_nvfp4_global_scale_product(lib):
    # input_scale * weight_scale_2 scales the fp32 4-bit product: a normal fp32 number
    ws = 1 << 30
    args = (A, 4, 32, 8, B, C)
    assert lib.qlinear_nvfp4(*args, 1e-20, 1e-20, None, None, None, 0, D, A, ws, None) == ARG   # 1e-40, subnormal
    assert lib.qlinear_nvfp4(*args, 1e20, 1e20, None, None, None, 0, D, A, ws, None) == ARG     # overflows
    assert lib.qlinear_nvfp4(*args, 1e-19, 1e-19, None, A, B, 4, D, A, ws, None) == ARG         # 1e-38 < 2^-126
    assert lib.qlinear_nvfp4(*args, 1e-19, 1e-18, None, A, B, 4, D, A, ws, None) != ARG         # 1e-37 is normal


def test_global_scale(lib):
    assert qpl.nvfp4_global_scale(2688.0) == 1.0
    import numpy as np
    assert qpl.nvfp4_global_scale(5.25) == float(np.float32(5.25) / np.float32(2688))


def test_quant_validation(lib):
    assert lib.quant_act_fp8_row(None, 4, 16, B, C, None) == NULL
    assert lib.quant_act_fp8_row(MIS, 4, 16, B, C, None) == ALIGN
    assert lib.quant_act_fp8_row(A, 0, 16, B, C, None) == SHAPE
    assert lib.quant_act_fp8_row(A, 4, 24, B, C, None) == SHAPE
    assert lib.quant_act_fp8_row(A, 4, 0, B, C, None) == SHAPE
    assert lib.quant_act_nvfp4(A, 4, 32, 1.0, None, None, C, None) == NULL
    for bad in (0.0, -1.0, float("inf"), float("nan"), 1e38):
        assert lib.quant_act_nvfp4(A, 4, 32, bad, None, B, C, None) == ARG, bad
    assert lib.quant_act_nvfp4(A, 4, 32, 1.0, MIS, B, C, None) == ALIGN  # smoothing factors


def test_qlinear_validation(lib):
    ws = 1 << 30
    assert lib.qlinear_fp8r(A, 4, 32, 8, B, C, D, None, ws, None) == NULL
    assert lib.qlinear_fp8r(A, 4, 32, 0, B, C, D, A, ws, None) == SHAPE
    assert lib.qlinear_fp8r(A, 4, 32, 8, B, C, D, A, 10, None) == WORKSPACE
    assert lib.qlinear_fp8r(A, 4, 32, 8, B, MIS, D, A, ws, None) == ALIGN
    # allocation-free variant: same checks, and a workspace beyond the static scratch
    assert lib.qlinear_fp8r_noalloc(A, 4, 32, 8, B, C, None, None) == NULL
    assert lib.qlinear_fp8r_noalloc(A, 4, 32, 0, B, C, D, None) == SHAPE
    assert lib.qlinear_fp8r_noalloc(A, 4, 32, 8, B, MIS, D, None) == ALIGN
    assert lib.qlinear_fp8r_noalloc(A, 9216, 3648, 8, B, C, D, None) == WORKSPACE  # 33.6 MB of codes
    args = (A, 4, 32, 8, B, C)
    assert lib.qlinear_nvfp4(*args, 1.0, 1.0, None, None, None, 0, D, A, 10, None) == WORKSPACE
    assert lib.qlinear_nvfp4(*args, 0.0, 1.0, None, None, None, 0, D, A, ws, None) == ARG
    assert lib.qlinear_nvfp4(*args, 1.0, float("nan"), None, None, None, 0, D, A, ws, None) == ARG
    assert lib.qlinear_nvfp4(*args, 1.0, 1.0, None, A, None, 4, D, A, ws, None) == NULL
    assert lib.qlinear_nvfp4(*args, 1.0, 1.0, None, A, B, 0, D, A, ws, None) == ARG
    assert lib.qlinear_nvfp4(*args, 1.0, 1.0, None, A, B, 200, D, A, ws, None) == SHAPE
    assert lib.qlinear_nvfp4(*args, 1.0, 1.0, None, MIS, B, 4, D, A, ws, None) == ALIGN
    assert lib.qlinear_nvfp4(*args, 1.0, 1.0, MIS, None, None, 0, D, A, ws, None) == ALIGN  # smoothing factors
    # INT4: K % 64, pointers, alignment, workspace, rank
    assert lib.quant_act_int4(A, 4, 96, None, B, C, None) == SHAPE
    assert lib.quant_act_int4(A, 4, 64, None, None, C, None) == NULL
    assert lib.quant_act_int4(A, 4, 64, MIS, B, C, None) == ALIGN
    assert lib.qlinear_int4(A, 4, 96, 8, B, C, None, None, None, 0, D, A, ws, None) == SHAPE
    assert lib.qlinear_int4(A, 4, 64, 8, B, C, None, None, None, 0, D, A, 10, None) == WORKSPACE
    assert lib.qlinear_int4(A, 4, 64, 8, B, C, None, A, None, 4, D, A, ws, None) == NULL
    assert lib.qlinear_int4(A, 4, 64, 8, B, C, None, A, B, 200, D, A, ws, None) == SHAPE
    assert lib.qlinear_int4(A, 4, 64, 8, B, MIS, None, None, None, 0, D, A, ws, None) == ALIGN
    # weight-only 4-bit: group size, K % group, pointers, alignment
    assert lib.quant_weight_awq(A, 4, 64, 48, B, C, D, None) == ARG
    assert lib.quant_weight_awq(A, 4, 96, 64, B, C, D, None) == SHAPE
    assert lib.quant_weight_awq(A, 4, 64, 64, B, None, D, None) == NULL
    assert lib.quant_weight_awq(A, 4, 64, 64, B, MIS, D, None) == ALIGN
    assert lib.qlinear_awq_w4a16(A, 1, 64, 8, B, C, D, 16, A, None) == ARG
    assert lib.qlinear_awq_w4a16(A, 1, 160, 8, B, C, D, 64, A, None) == SHAPE
    assert lib.qlinear_awq_w4a16(A, 0, 64, 8, B, C, D, 64, A, None) == SHAPE
    assert lib.qlinear_awq_w4a16(A, 1, 64, 8, B, C, None, 64, A, None) == NULL
    assert lib.qlinear_awq_w4a16(A, 1, 64, 8, B, C, MIS, 64, A, None) == ALIGN
    assert lib.dequant_weight(5, A, B, 1.0, 4, 32, C, None) == ARG
    assert lib.dequant_weight(1, A, B, -1.0, 4, 32, C, None) == ARG
    assert lib.dequant_weight(0, A, None, 1.0, 4, 32, C, None) == NULL
    assert lib.qpl_amax_bf16(A, 0, B, None) == SHAPE
    assert lib.qpl_amax_bf16(A, 10, P((1 << 21) + 2), None) == ALIGN


@pytest.mark.skipif(torch.cuda.is_available(), reason="forces the no-device status; a GPU is present")
def test_no_device_status(lib):
    assert lib.quant_act_fp8_row(A, 4, 16, B, C, None) == DEVICE
    assert lib.qlinear_nvfp4(A, 4, 32, 8, B, C, 1.0, 1.0, None, None, None, 0, D, A, 1 << 30, None) == DEVICE


def test_timing_collect_empty(lib):
    qpl.timing_enable(False)
    res = qpl.timing_collect()
    assert set(res) == set(qpl.KERNELS) and all(v == (0, 0.0) for v in res.values())
    assert lib.qpl_timing_collect(None, None) == NULL


def test_binding_rejects_wrong_tensors():
    x = torch.zeros((4, 32), dtype=torch.float32)
    with pytest.raises(ValueError):
        qpl.quant_act_fp8_row(x)


def epi(act=0, qkv=False, heads=2, head_dim=16, tokens=8, off=0, only_q=False):
    e = qpl.Epilogue()
    e.act = act
    if qkv or only_q:
        e.q = 1 << 24
        if not only_q:
            e.k, e.v = 1 << 25, 1 << 26
        e.heads, e.head_dim, e.tokens, e.token_offset = heads, head_dim, tokens, off
    return ctypes.byref(e)


def test_epilogue_validation(lib):
    ws = 1 << 30
    # plain descriptor: y still required; unknown activation
    assert lib.qlinear_fp8r_ex(A, 4, 32, 8, B, C, epi(), None, A, ws, None) == NULL
    assert lib.qlinear_fp8r_ex(A, 4, 32, 8, B, C, epi(act=7), D, A, ws, None) == ARG
    nv = (A, 4, 32, 96, B, C, 1.0, 1.0, None, None, None, 0)
    assert lib.qlinear_nvfp4_ex(*nv, epi(act=2), D, A, ws, None) == ARG
    # QKV: all three or none, no activation with it, shape rules (N = 3 heads head_dim)
    assert lib.qlinear_nvfp4_ex(*nv, epi(only_q=True), None, A, ws, None) == NULL
    assert lib.qlinear_nvfp4_ex(*nv, epi(act=1, qkv=True), None, A, ws, None) == ARG
    assert lib.qlinear_nvfp4_ex(*nv, epi(qkv=True, heads=3), None, A, ws, None) == SHAPE
    assert lib.qlinear_nvfp4_ex(*nv, epi(qkv=True, heads=4, head_dim=8, tokens=8), None, A, ws, None) != SHAPE
    assert lib.qlinear_nvfp4_ex(A, 4, 32, 36, B, C, 1.0, 1.0, None, None, None, 0,
                                epi(qkv=True, heads=2, head_dim=6), None, A, ws, None) == SHAPE  # not a power of two
    assert lib.qlinear_nvfp4_ex(*nv, epi(qkv=True, tokens=5, off=2), None, A, ws, None) == SHAPE  # 2 + 4 > 5
    assert lib.qlinear_nvfp4_ex(*nv, epi(qkv=True, off=-1), None, A, ws, None) == SHAPE
    e = qpl.Epilogue()
    e.q, e.k, e.v = 1 << 24, (1 << 25) + 8, 1 << 26
    e.heads, e.head_dim, e.tokens = 2, 16, 8
    assert lib.qlinear_nvfp4_ex(*nv, ctypes.byref(e), None, A, ws, None) == ALIGN
    i4 = (A, 4, 64, 96, B, C, None, None, None, 0)
    assert lib.qlinear_int4_ex(*i4, epi(qkv=True, heads=3), None, A, ws, None) == SHAPE
    assert lib.qlinear_int4_ex(*i4, epi(act=1), None, A, ws, None) == NULL


def layer(R=0, bad_scale=False, lora=False):
    L = qpl.Nvfp4Layer()
    L.weight, L.weight_scale = 1 << 20, 1 << 21
    L.weight_scale_2, L.input_scale = (0.0 if bad_scale else 1.0), 1.0
    if lora:
        L.lora_down, L.lora_up = 1 << 22, 1 << 23
    L.R = R
    return ctypes.byref(L)


def test_mlp_validation_and_workspace(lib):
    M, K, H, N = 4608, 3072, 12288, 3072
    r256 = lambda b: (b + 255) // 256 * 256  # noqa: E731
    for R1, R2 in ((0, 0), (32, 0), (32, 32)):
        fc1 = qpl.qlinear_workspace_bytes(qpl.QPL_NVFP4, M, K, H, R1)
        fc2 = qpl.qlinear_workspace_bytes(qpl.QPL_NVFP4, M, H, N, R2)
        assert qpl.qlinear_mlp_nvfp4_workspace_bytes(M, K, H, N, R1, R2) == fc2 + r256(2 * M * H) + fc1
    assert qpl.qlinear_mlp_nvfp4_workspace_bytes(4, 32, 24, 8) == 0   # H % 16 != 0
    assert qpl.qlinear_mlp_nvfp4_workspace_bytes(4, 32, 32, 8, 129) == 0
    assert qpl.qlinear_mlp_nvfp4_workspace_bytes(4, 32, 32, 8, 0, 129) == 0
    ws = 1 << 30
    assert lib.qlinear_mlp_nvfp4(A, 4, 32, 32, 8, layer(), None, D, A, ws, None) == NULL
    assert lib.qlinear_mlp_nvfp4(A, 4, 32, 32, 8, layer(), layer(bad_scale=True), D, A, ws, None) == ARG
    assert lib.qlinear_mlp_nvfp4(A, 4, 32, 32, 8, layer(R=4), layer(), D, A, ws, None) == NULL
    assert lib.qlinear_mlp_nvfp4(A, 4, 32, 32, 8, layer(), layer(R=200, lora=True), D, A, ws, None) == SHAPE
    assert lib.qlinear_mlp_nvfp4(A, 4, 32, 24, 8, layer(), layer(), D, A, ws, None) == SHAPE
    assert lib.qlinear_mlp_nvfp4(A, 4, 32, 32, 8, layer(), layer(), D, A, 100, None) == WORKSPACE
    assert lib.qlinear_mlp_nvfp4(A, 4, 32, 32, 8, layer(), layer(), MIS, A, ws, None) == ALIGN


@pytest.mark.skipif(torch.cuda.is_available(), reason="forces the no-device status; a GPU is present")
def test_epilogue_calls_reach_the_device_check(lib):
    ws = 1 << 30
    assert lib.qlinear_nvfp4_ex(A, 4, 32, 96, B, C, 1.0, 1.0, None, None, None, 0, epi(qkv=True), None, A, ws,
                                None) == DEVICE
    assert lib.qlinear_fp8r_ex(A, 4, 32, 8, B, C, epi(act=1), D, A, ws, None) == DEVICE
    assert lib.qlinear_mlp_nvfp4(A, 4, 32, 32, 8, layer(), layer(), D, A, ws, None) == DEVICE
    assert lib.qlinear_mlp_nvfp4(A, 4, 32, 32, 8, layer(R=4, lora=True), layer(R=4, lora=True), D, A, ws,
                                 None) == DEVICE
