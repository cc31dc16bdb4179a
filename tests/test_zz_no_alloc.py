"""qlinear_fp8r_noalloc (the allocation-free fp8r linear) against qlinear_fp8r.

Both run the same kernels, the new entry point on the library's static device scratch
instead of a caller's workspace, so the outputs must be bit-identical.  Two calls in
a row, the second with a smaller, ragged input: the scratch keeps the first call's
contents, which must not leak into the second.  The smaller case is also held to the
oracle's fp8r acceptance, and a size beyond the scratch is refused before anything is
queued."""
import numpy as np
import pytest
import torch

import precision_quantized_linear_amd as qpl
from helpers import bf16_bits, to_dev, to_dev_bf16
from oracle.quant import quant_fp8_row
from oracle.reference import check_gemm, dequant_fp8r, gemm_gamma_fp8_dot
from synthetic import make

pytestmark = pytest.mark.gpu


def inputs(M, K, N):
    d = make("fp8r_dit_n3072", M=M, K=K, N=N)
    wq, ws = quant_fp8_row(d["w"])
    return d, to_dev_bf16(d["x"]), to_dev(wq), to_dev(ws)


def test_noalloc_matches_qlinear_fp8r_twice():
    cases = [inputs(4608, 3072, 3072), inputs(300, 400, 520)]   # 14.2 MB, then 0.12 MB of scratch
    outs = []
    for _, x, w, s in cases:
        y = torch.empty((x.shape[0], w.shape[0]), dtype=torch.bfloat16, device=x.device)
        print("qlinear_fp8r_noalloc", tuple(x.shape), w.shape[0], flush=True)
        outs.append(qpl.qlinear_fp8r_noalloc(x, w, s, y))
    torch.cuda.synchronize()
    for (_, x, w, s), y in zip(cases, outs):
        ref = qpl.qlinear_fp8r(x, w, s)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), tuple(x.shape)
    d, x, w, s = cases[1]
    xq, xs = quant_fp8_row(d["x"])
    wq, ws = quant_fp8_row(d["w"])
    a, b = dequant_fp8r(xq, xs), dequant_fp8r(wq, ws)
    r = check_gemm(bf16_bits(outs[1]), a @ b.T, np.abs(a) @ np.abs(b).T, d["K"], gamma=gemm_gamma_fp8_dot(d["K"]))
    assert r["ok"], r


def test_noalloc_refuses_beyond_scratch():
    _, x, w, s = inputs(16, 64, 8)
    big = torch.empty((9216, 3648), dtype=torch.bfloat16, device=x.device)   # 33.6 MB of codes
    wb = torch.empty((8, 3648), dtype=torch.uint8, device=x.device)
    y = torch.empty((9216, 8), dtype=torch.bfloat16, device=x.device)
    with pytest.raises(qpl.QPLError) as e:
        qpl.qlinear_fp8r_noalloc(big, wb, s, y)
    assert e.value.status == 5
