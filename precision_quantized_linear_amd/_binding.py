"""ctypes binding of libqpl.so: argument marshalling only.

Every call forwards raw device pointers, sizes and the current HIP stream to the
C ABI declared in include/qpl.h; all arithmetic runs in the library's gfx950
kernels.  torch is used for device memory and streams only.  There is no CPU
fallback: a missing library or a non-OK status raises.
"""
import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqpl.so")

QPL_FP8R = 0
QPL_NVFP4 = 1
QPL_INT4 = 2

EXPORTS = ("quant_act_fp8_row", "quant_act_nvfp4", "qlinear_fp8r", "qlinear_nvfp4", "dequant_weight",
           "quant_weight_awq", "qlinear_awq_w4a16", "quant_act_int4", "qlinear_int4", "qlinear_fp8r_ex",
           "qlinear_nvfp4_ex", "qlinear_int4_ex", "qlinear_mlp_nvfp4", "qlinear_mlp_nvfp4_workspace_bytes",
           "qlinear_workspace_bytes", "qpl_amax_bf16", "qpl_nvfp4_global_scale", "qpl_status_str",
           "qpl_timing_enable", "qpl_timing_select", "qpl_timing_collect", "qlinear_fp8r_noalloc")

# qpl_kernel order of include/qpl.h
KERNELS = ("quant_fp8_row", "quant_nvfp4", "quant_nvfp4_linear", "gemm_fp8r", "gemm_nvfp4", "gemm_nvfp4_lowrank",
           "lowrank_prep", "dequant", "amax", "nvfp4_prep", "quant_nvfp4_lowrank", "quant_w4g", "gemv_w4a16",
           "quant_int4", "int4_expand", "gemm_int4", "quant_int4_lowrank", "gemm_epilogue")

QPL_ACT_NONE = 0
QPL_ACT_GELU_TANH = 1
_ACTS = {None: QPL_ACT_NONE, "none": QPL_ACT_NONE, "gelu_tanh": QPL_ACT_GELU_TANH}

_P, _I64, _F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float


class Epilogue(ctypes.Structure):
    """qpl_epilogue of include/qpl.h."""
    _fields_ = [("act", ctypes.c_int), ("q", _P), ("k", _P), ("v", _P), ("heads", _I64), ("head_dim", _I64),
                ("tokens", _I64), ("token_offset", _I64)]


class Nvfp4Layer(ctypes.Structure):
    """qpl_nvfp4_layer of include/qpl.h."""
    _fields_ = [("weight", _P), ("weight_scale", _P), ("weight_scale_2", _F), ("input_scale", _F),
                ("smooth", _P), ("lora_down", _P), ("lora_up", _P), ("R", _I64)]

_lib = None


class QPLError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def load():
    """Load libqpl.so (once) and declare the signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m precision_quantized_linear_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, F, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "quant_act_fp8_row": [P, I64, I64, P, P, P],
        "quant_act_nvfp4": [P, I64, I64, F, P, P, P, P],
        "qlinear_fp8r": [P, I64, I64, I64, P, P, P, P, SZ, P],
        "qlinear_nvfp4": [P, I64, I64, I64, P, P, F, F, P, P, P, I64, P, P, SZ, P],
        "dequant_weight": [ctypes.c_int, P, P, F, I64, I64, P, P],
        "quant_weight_awq": [P, I64, I64, I64, P, P, P, P],
        "qlinear_awq_w4a16": [P, I64, I64, I64, P, P, P, I64, P, P],
        "quant_act_int4": [P, I64, I64, P, P, P, P],
        "qlinear_int4": [P, I64, I64, I64, P, P, P, P, P, I64, P, P, SZ, P],
        "qpl_amax_bf16": [P, I64, P, P],
        "qlinear_fp8r_ex": [P, I64, I64, I64, P, P, P, P, P, SZ, P],
        "qlinear_nvfp4_ex": [P, I64, I64, I64, P, P, F, F, P, P, P, I64, P, P, P, SZ, P],
        "qlinear_int4_ex": [P, I64, I64, I64, P, P, P, P, P, I64, P, P, P, SZ, P],
        "qlinear_mlp_nvfp4": [P, I64, I64, I64, I64, P, P, P, P, SZ, P],
        "qlinear_fp8r_noalloc": [P, I64, I64, I64, P, P, P, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.qlinear_workspace_bytes.argtypes = [ctypes.c_int, I64, I64, I64, I64]
    lib.qlinear_workspace_bytes.restype = SZ
    lib.qlinear_mlp_nvfp4_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, I64]
    lib.qlinear_mlp_nvfp4_workspace_bytes.restype = SZ
    lib.qpl_nvfp4_global_scale.argtypes = [F]
    lib.qpl_nvfp4_global_scale.restype = F
    lib.qpl_status_str.argtypes = [ctypes.c_int]
    lib.qpl_status_str.restype = ctypes.c_char_p
    lib.qpl_timing_enable.argtypes = [ctypes.c_int]
    lib.qpl_timing_enable.restype = None
    lib.qpl_timing_select.argtypes = [ctypes.c_uint32]
    lib.qpl_timing_select.restype = None
    lib.qpl_timing_collect.argtypes = [P, P]
    lib.qpl_timing_collect.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(fn, status):
    if status != 0:
        raise QPLError(fn, status, load().qpl_status_str(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _expect(t, dtype, shape, name):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on a GPU, got "
                         f"{t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()} device={t.device}")


def _bits(t):
    """bf16 tensor -> same storage viewed as int16 (the C ABI takes the bit patterns)."""
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def quant_act_fp8_row(x, x_q=None, x_scale=None, stream=None):
    """bf16 [M,K] -> (E4M3 codes uint8 [M,K], fp32 row scales [M])."""
    M, K = x.shape
    _expect(x, torch.bfloat16, (M, K), "x")
    x_q = torch.empty((M, K), dtype=torch.uint8, device=x.device) if x_q is None else x_q
    x_scale = torch.empty((M,), dtype=torch.float32, device=x.device) if x_scale is None else x_scale
    _check("quant_act_fp8_row", load().quant_act_fp8_row(_ptr(x), M, K, _ptr(x_q), _ptr(x_scale), _stream(stream)))
    return x_q, x_scale


def quant_act_nvfp4(x, input_scale, smooth=None, x_q=None, x_block_scale=None, stream=None):
    """bf16 [M,K] -> (packed E2M1 uint8 [M,K/2], E4M3 block scales uint8 [M,K/16]);
    with smooth (float32 [K]) the quantized activation is bf16(x / smooth)."""
    M, K = x.shape
    _expect(x, torch.bfloat16, (M, K), "x")
    if smooth is not None:
        _expect(smooth, torch.float32, (K,), "smooth")
    x_q = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device) if x_q is None else x_q
    x_block_scale = (torch.empty((M, K // 16), dtype=torch.uint8, device=x.device)
                     if x_block_scale is None else x_block_scale)
    _check("quant_act_nvfp4", load().quant_act_nvfp4(_ptr(x), M, K, float(input_scale), _ptr(smooth), _ptr(x_q),
                                                      _ptr(x_block_scale), _stream(stream)))
    return x_q, x_block_scale


def qlinear_workspace_bytes(scheme, M, K, N, R=0):
    return int(load().qlinear_workspace_bytes(scheme, M, K, N, R))


def _workspace(scheme, M, K, N, R, ws, device):
    need = qlinear_workspace_bytes(scheme, M, K, N, R)
    if ws is None:
        ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def _epilogue(act, qkv, M, N, y, device):
    """(Epilogue or None, y, result): act names the activation ("gelu_tanh"); qkv is
    (q, k, v, token_offset) with q, k, v bf16 [heads, tokens, head_dim]."""
    if act not in _ACTS:
        raise ValueError(f"act: expected one of {sorted(k for k in _ACTS if k)}, got {act!r}")
    if act is None and qkv is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=device) if y is None else y
        return None, y, y
    e = Epilogue()
    e.act = _ACTS[act]
    if qkv is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=device) if y is None else y
        return e, y, y
    q, k, v, off = qkv
    heads, tokens, head_dim = q.shape
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _expect(t, torch.bfloat16, (heads, tokens, head_dim), name)
    e.q, e.k, e.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    e.heads, e.head_dim, e.tokens, e.token_offset = heads, head_dim, tokens, int(off)
    return e, None, (q, k, v)


def _ref(e):
    return None if e is None else ctypes.byref(e)


def qlinear_fp8r(x, weight, weight_scale, y=None, workspace=None, stream=None, act=None, qkv=None):
    """y[M,N] bf16 = fp8r linear of bf16 x [M,K] with E4M3 weight [N,K] and fp32 weight_scale [N].
    act="gelu_tanh" applies GELU before the rounding; qkv=(q, k, v, token_offset) writes the
    three column parts to q, k, v [heads, tokens, head_dim] instead (and returns them)."""
    M, K = x.shape
    N = weight.shape[0]
    _expect(x, torch.bfloat16, (M, K), "x")
    _expect(weight, torch.uint8, (N, K), "weight")
    _expect(weight_scale, torch.float32, (N,), "weight_scale")
    e, y, out = _epilogue(act, qkv, M, N, y, x.device)
    ws, nbytes = _workspace(QPL_FP8R, M, K, N, 0, workspace, x.device)
    if e is None:
        _check("qlinear_fp8r", load().qlinear_fp8r(_ptr(x), M, K, N, _ptr(weight), _ptr(weight_scale), _ptr(y),
                                                   _ptr(ws), nbytes, _stream(stream)))
    else:
        _check("qlinear_fp8r_ex", load().qlinear_fp8r_ex(_ptr(x), M, K, N, _ptr(weight), _ptr(weight_scale),
                                                         _ref(e), _ptr(y), _ptr(ws), nbytes, _stream(stream)))
    return out


def qlinear_fp8r_noalloc(x, weight, weight_scale, y, stream=None):
    """qlinear_fp8r into a caller-provided y [M,N] bf16 with the library's static
    device scratch as workspace: the call itself allocates nothing."""
    M, K = x.shape
    N = weight.shape[0]
    _expect(x, torch.bfloat16, (M, K), "x")
    _expect(weight, torch.uint8, (N, K), "weight")
    _expect(weight_scale, torch.float32, (N,), "weight_scale")
    _expect(y, torch.bfloat16, (M, N), "y")
    _check("qlinear_fp8r_noalloc", load().qlinear_fp8r_noalloc(_ptr(x), M, K, N, _ptr(weight), _ptr(weight_scale),
                                                               _ptr(y), _stream(stream)))
    return y


def qlinear_nvfp4(x, weight, weight_scale, weight_scale_2, input_scale, lora_down=None, lora_up=None, y=None,
                  workspace=None, stream=None, smooth=None, act=None, qkv=None):
    """y[M,N] bf16 = nvfp4 linear (+ (x L1) L2 when lora_down [K,R] / lora_up [R,N] are given);
    with smooth (float32 [K]) both terms take the smoothed activation bf16(x / smooth).
    act and qkv as in qlinear_fp8r."""
    M, K = x.shape
    N = weight.shape[0]
    _expect(x, torch.bfloat16, (M, K), "x")
    if smooth is not None:
        _expect(smooth, torch.float32, (K,), "smooth")
    _expect(weight, torch.uint8, (N, K // 2), "weight")
    _expect(weight_scale, torch.uint8, (N, K // 16), "weight_scale")
    R = 0
    if lora_down is not None:
        R = lora_down.shape[1]
        _expect(lora_down, torch.bfloat16, (K, R), "lora_down")
        _expect(lora_up, torch.bfloat16, (R, N), "lora_up")
    e, y, out = _epilogue(act, qkv, M, N, y, x.device)
    ws, nbytes = _workspace(QPL_NVFP4, M, K, N, R, workspace, x.device)
    args = (_ptr(x), M, K, N, _ptr(weight), _ptr(weight_scale), float(weight_scale_2), float(input_scale),
            _ptr(smooth), _ptr(lora_down), _ptr(lora_up), R)
    if e is None:
        _check("qlinear_nvfp4", load().qlinear_nvfp4(*args, _ptr(y), _ptr(ws), nbytes, _stream(stream)))
    else:
        _check("qlinear_nvfp4_ex", load().qlinear_nvfp4_ex(*args, _ref(e), _ptr(y), _ptr(ws), nbytes,
                                                           _stream(stream)))
    return out


def quant_act_int4(x, smooth=None, x_q=None, x_scale=None, stream=None):
    """bf16 [M,K] (K % 64 == 0) -> (packed INT4 codes uint8 [M,K/2], fp32 group scales [M,K/64])."""
    M, K = x.shape
    _expect(x, torch.bfloat16, (M, K), "x")
    if smooth is not None:
        _expect(smooth, torch.float32, (K,), "smooth")
    x_q = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device) if x_q is None else x_q
    x_scale = torch.empty((M, K // 64), dtype=torch.float32, device=x.device) if x_scale is None else x_scale
    _check("quant_act_int4", load().quant_act_int4(_ptr(x), M, K, _ptr(smooth), _ptr(x_q), _ptr(x_scale),
                                                    _stream(stream)))
    return x_q, x_scale


def qlinear_int4(x, weight, weight_scale, lora_down=None, lora_up=None, y=None, workspace=None, stream=None,
                 smooth=None, act=None, qkv=None):
    """y[M,N] bf16 = INT4 W4A4 linear (+ (x L1) L2), the INT4 variant of svdq_w4a4; act and
    qkv as in qlinear_fp8r."""
    M, K = x.shape
    N = weight.shape[0]
    _expect(x, torch.bfloat16, (M, K), "x")
    _expect(weight, torch.uint8, (N, K // 2), "weight")
    _expect(weight_scale, torch.float32, (N, K // 64), "weight_scale")
    if smooth is not None:
        _expect(smooth, torch.float32, (K,), "smooth")
    R = 0
    if lora_down is not None:
        R = lora_down.shape[1]
        _expect(lora_down, torch.bfloat16, (K, R), "lora_down")
        _expect(lora_up, torch.bfloat16, (R, N), "lora_up")
    e, y, out = _epilogue(act, qkv, M, N, y, x.device)
    ws, nbytes = _workspace(QPL_INT4, M, K, N, R, workspace, x.device)
    args = (_ptr(x), M, K, N, _ptr(weight), _ptr(weight_scale), _ptr(smooth), _ptr(lora_down), _ptr(lora_up), R)
    if e is None:
        _check("qlinear_int4", load().qlinear_int4(*args, _ptr(y), _ptr(ws), nbytes, _stream(stream)))
    else:
        _check("qlinear_int4_ex", load().qlinear_int4_ex(*args, _ref(e), _ptr(y), _ptr(ws), nbytes,
                                                         _stream(stream)))
    return out


def qlinear_mlp_nvfp4_workspace_bytes(M, K, H, N, R1=0, R2=0):
    return int(load().qlinear_mlp_nvfp4_workspace_bytes(M, K, H, N, R1, R2))


def _layer(d, rows, cols, name):
    """Nvfp4Layer from a dict with weight [rows, cols/2], weight_scale [rows, cols/16],
    weight_scale_2, input_scale and optional smooth [cols], lora_down [cols, R], lora_up [R, rows]."""
    _expect(d["weight"], torch.uint8, (rows, cols // 2), name + ".weight")
    _expect(d["weight_scale"], torch.uint8, (rows, cols // 16), name + ".weight_scale")
    L = Nvfp4Layer()
    L.weight, L.weight_scale = d["weight"].data_ptr(), d["weight_scale"].data_ptr()
    L.weight_scale_2, L.input_scale = float(d["weight_scale_2"]), float(d["input_scale"])
    if d.get("smooth") is not None:
        _expect(d["smooth"], torch.float32, (cols,), name + ".smooth")
        L.smooth = d["smooth"].data_ptr()
    if d.get("lora_down") is not None:
        R = d["lora_down"].shape[1]
        _expect(d["lora_down"], torch.bfloat16, (cols, R), name + ".lora_down")
        _expect(d["lora_up"], torch.bfloat16, (R, rows), name + ".lora_up")
        L.lora_down, L.lora_up, L.R = d["lora_down"].data_ptr(), d["lora_up"].data_ptr(), R
    return L


def qlinear_mlp_nvfp4(x, fc1, fc2, y=None, workspace=None, stream=None):
    """y [M,N] bf16 = fc2(bf16(gelu(fc1(x)))) for nvfp4 layers fc1 [H,K] and fc2 [N,H]
    given as dicts (see _layer); GELU runs in fc1's epilogue.  After the call the first
    2 M H bytes of the workspace hold fc2's expanded operand, and h follows fc2's part."""
    M, K = x.shape
    _expect(x, torch.bfloat16, (M, K), "x")
    H = fc1["weight"].shape[0]
    N = fc2["weight"].shape[0]
    l1, l2 = _layer(fc1, H, K, "fc1"), _layer(fc2, N, H, "fc2")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if y is None else y
    need = qlinear_mlp_nvfp4_workspace_bytes(M, K, H, N, l1.R, l2.R)
    ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device) if workspace is None else workspace
    _check("qlinear_mlp_nvfp4", load().qlinear_mlp_nvfp4(_ptr(x), M, K, H, N, ctypes.byref(l1), ctypes.byref(l2),
                                                         _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                                         _stream(stream)))
    return y


def quant_weight_awq(w, group=64, w_q=None, w_scale=None, w_zero=None, stream=None):
    """bf16 weight [N,K] -> (codes uint8 [N,K/2], scales bf16 [N,K/group], zero points uint8 [N,K/group])."""
    N, K = w.shape
    _expect(w, torch.bfloat16, (N, K), "w")
    G = K // group
    w_q = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device) if w_q is None else w_q
    w_scale = torch.empty((N, G), dtype=torch.bfloat16, device=w.device) if w_scale is None else w_scale
    w_zero = torch.empty((N, G), dtype=torch.uint8, device=w.device) if w_zero is None else w_zero
    _check("quant_weight_awq", load().quant_weight_awq(_ptr(w), N, K, group, _ptr(w_q), _ptr(w_scale), _ptr(w_zero),
                                                        _stream(stream)))
    return w_q, w_scale, w_zero


def qlinear_awq_w4a16(x, weight, weight_scale, weight_zero, group=64, y=None, stream=None):
    """y[M,N] bf16 = x [M,K] (bf16) times the group-wise 4-bit weight, dequantized as (q - z) s."""
    M, K = x.shape
    N = weight.shape[0]
    _expect(x, torch.bfloat16, (M, K), "x")
    _expect(weight, torch.uint8, (N, K // 2), "weight")
    _expect(weight_scale, torch.bfloat16, (N, K // group), "weight_scale")
    _expect(weight_zero, torch.uint8, (N, K // group), "weight_zero")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if y is None else y
    _check("qlinear_awq_w4a16", load().qlinear_awq_w4a16(_ptr(x), M, K, N, _ptr(weight), _ptr(weight_scale),
                                                          _ptr(weight_zero), group, _ptr(y), _stream(stream)))
    return y


def dequant_weight(scheme, weight, weight_scale, weight_scale_2=1.0, K=None, out=None, stream=None):
    """Dequantize an fp8r or nvfp4 weight to bf16 [N,K]."""
    N = weight.shape[0]
    if K is None:
        K = weight.shape[1] * (2 if scheme == QPL_NVFP4 else 1)
    out = torch.empty((N, K), dtype=torch.bfloat16, device=weight.device) if out is None else out
    _check("dequant_weight", load().dequant_weight(scheme, _ptr(weight), _ptr(weight_scale), float(weight_scale_2),
                                                   N, K, _ptr(out), _stream(stream)))
    return out


def amax_bf16(x, amax=None, stream=None):
    """Running max |x| into a device float32 [1] (initialised to 0 when not given)."""
    amax = torch.zeros((1,), dtype=torch.float32, device=x.device) if amax is None else amax
    _check("qpl_amax_bf16", load().qpl_amax_bf16(_ptr(x), x.numel(), _ptr(amax), _stream(stream)))
    return amax


def nvfp4_global_scale(amax):
    """amax / (448 * 6) in fp32 (host)."""
    return float(load().qpl_nvfp4_global_scale(float(amax)))


def timing_enable(on=True):
    """Bracket every library kernel launch with HIP events (profiling aid)."""
    load().qpl_timing_enable(1 if on else 0)


def timing_select(kinds):
    """Time only the named kernel kinds (names from KERNELS); an empty list turns timing off."""
    mask = 0
    for k in kinds:
        mask |= 1 << KERNELS.index(k)
    load().qpl_timing_select(mask)


def timing_collect():
    """Wait for the recorded events; return {kernel: (launches, total_ms)} and clear."""
    n = len(KERNELS)
    launches = (ctypes.c_int64 * n)()
    total = (ctypes.c_double * n)()
    _check("qpl_timing_collect", load().qpl_timing_collect(ctypes.cast(launches, ctypes.c_void_p),
                                                           ctypes.cast(total, ctypes.c_void_p)))
    return {k: (int(launches[i]), float(total[i])) for i, k in enumerate(KERNELS)}
