"""DiT-shaped synthetic linears (bf16 activations, bf16 weights, low-rank factors).

The workloads stand in for the transformer projections of the pipelines that the
Diffusers "BFL (fp8r / nvfp4)" guide and the Nunchaku post load; no trained
checkpoint or dataset is used.  Recipe (all draws float32 from
``numpy.random.Generator(PCG64(seed))``, then rounded to bf16 to nearest-even):

* activations X [M, K]: N(0, 1), or Student-t with 4 degrees of freedom built as
  Z / sqrt(G / 2) with Z ~ N(0, 1), G ~ Gamma(2, 1); a fixed set of outlier
  channels (columns) is multiplied by a constant;
* weights W [N, K]: N(0, 0.02);  low-rank factors L1 [K, R], L2 [R, N]: N(0, 0.05);
* the SVDQuant workload stores the residual weight W - (L1 L2)^T (rounded to bf16),
  as an SVDQuant checkpoint stores the residual beside its low-rank factors;
* calibration batches: further draws with the activation recipe and the same
  outlier channels;
* smoothing factors [K] (float32, for the SVDQuant smoothing step):
  exp(N(0, 0.25^2)), times sqrt(mult) on the outlier channels.

Seeds for workload number c: X 100c, W 100c+1, outlier channels 100c+2,
L1 100c+3, L2 100c+4, smoothing factors 100c+5, calibration batch i 100c+10+i.
"""
import numpy as np


def bf16_round(x):
    """float32 -> bf16 bit patterns (uint16), round to nearest even (finite input)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


WORKLOADS = {
    # fp8r, tiny: 4 outlier channels x20
    "fp8r_tiny": dict(c=1, scheme="fp8r", M=64, K=256, N=512, dist="normal", n_out=4, mult=20.0),
    # fp8r DiT projection: 4096 image + 512 text tokens, 1% outlier channels x10
    "fp8r_dit_n3072": dict(c=2, scheme="fp8r", M=4608, K=3072, N=3072, dist="normal", frac_out=0.01, mult=10.0),
    "fp8r_dit_n12288": dict(c=2, scheme="fp8r", M=4608, K=3072, N=12288, dist="normal", frac_out=0.01, mult=10.0),
    # nvfp4 DiT projection, activation scale calibrated on 8 batches
    "nvfp4_dit": dict(c=3, scheme="nvfp4", M=4608, K=3072, N=12288, dist="normal", frac_out=0.01, mult=10.0, n_cal=8),
    # nvfp4 MLP down-projection with a classifier-free-guidance batch (2 x 4608), heavy tails
    "nvfp4_mlp_down_cfg": dict(c=4, scheme="nvfp4", M=9216, K=12288, N=3072, dist="t4", frac_out=0.01, mult=10.0, n_cal=8),
    # SVDQuant-style W4A4: nvfp4 residual + rank-32 bf16 branch
    "svdq_w4a4": dict(c=5, scheme="nvfp4", M=4608, K=3072, N=3072, dist="normal", frac_out=0.01, mult=10.0, n_cal=8, R=32),
    # weight-only 4-bit modulation projections (one conditioning vector per image):
    # FLUX adanorm_zero 3072 -> 6 x 3072 and adanorm_single 3072 -> 3 x 3072, group 64
    "awq_adanorm_zero": dict(c=6, scheme="w4a16", M=1, K=3072, N=18432, dist="normal", frac_out=0.0, mult=1.0, G=64),
    "awq_adanorm_single": dict(c=7, scheme="w4a16", M=1, K=3072, N=9216, dist="normal", frac_out=0.0, mult=1.0, G=64),
    # FLUX double-block feed-forward (3072 -> 4 x 3072 -> 3072) as SVDQuant W4A4 layers:
    # fc1 [N, K] and fc2 [N2, N] (w2, factors l1_2 [N, R], l2_2 [R, N2]), rank 32 each
    "svdq_mlp": dict(c=8, scheme="nvfp4", M=4608, K=3072, N=12288, N2=3072, dist="normal", frac_out=0.01,
                     mult=10.0, n_cal=8, R=32),
    # FLUX attention input projection: [W_q; W_k; W_v] for 24 heads of 128 over the
    # 4096 image tokens, written after the 512 text tokens of the joint sequence
    "qkv_dit": dict(c=9, scheme="nvfp4", M=4096, K=3072, N=9216, dist="normal", frac_out=0.01, mult=10.0, n_cal=8,
                    heads=24, head_dim=128, tokens=4608, offset=512),
}


def _n_outliers(spec, K):
    if "n_out" in spec:
        return min(spec["n_out"], K)
    return int(round(spec["frac_out"] * K))


def _outlier_channels(spec, K):
    n = _n_outliers(spec, K)
    return np.sort(_rng(100 * spec["c"] + 2).choice(K, size=n, replace=False))


def _activation(spec, seed, M, K, channels):
    g = _rng(seed)
    if spec["dist"] == "normal":
        x = g.standard_normal((M, K), dtype=np.float32)
    else:
        z = g.standard_normal((M, K), dtype=np.float32)
        gam = g.standard_gamma(2.0, (M, K), dtype=np.float32)
        x = z / np.sqrt(gam / np.float32(2.0))
    if len(channels):
        x[:, channels] *= np.float32(spec["mult"])
    return bf16_round(x)


def _normal(seed, shape, std):
    return bf16_round(_rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(std))


def make(name, M=None, K=None, N=None, N2=None):
    """Inputs of workload ``name`` as bf16 bit arrays (uint16).

    M, K, N override the sizes (same recipe and seeds) for the small parity cases.
    Returns a dict: spec, M, K, N, x [M,K], w [N,K] (the residual for the
    SVDQuant workload), and l1 [K,R], l2 [R,N] when the workload has a low-rank
    branch; w2 [N2, N] for a workload with a second layer (N2 overrides its size).
    """
    spec = dict(WORKLOADS[name])
    M = spec["M"] if M is None else M
    K = spec["K"] if K is None else K
    N = spec["N"] if N is None else N
    c = spec["c"]
    ch = _outlier_channels(spec, K)
    out = dict(spec=spec, name=name, M=M, K=K, N=N, channels=ch)
    out["x"] = _activation(spec, 100 * c, M, K, ch)
    w = _normal(100 * c + 1, (N, K), 0.02)
    if "R" in spec:
        R = spec["R"]
        l1 = _normal(100 * c + 3, (K, R), 0.05)
        l2 = _normal(100 * c + 4, (R, N), 0.05)
        f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        w_res = f(w) - (f(l1) @ f(l2)).T
        out["w"] = bf16_round(w_res.astype(np.float32))
        out["l1"], out["l2"], out["R"] = l1, l2, R
    else:
        out["w"] = w
    if "N2" in spec:
        N2 = spec["N2"] if N2 is None else N2
        out["N2"] = N2
        out["w2"] = _normal(100 * c + 6, (N2, N), 0.02)
        out["l1_2"] = _normal(100 * c + 7, (N, spec["R"]), 0.05)
        out["l2_2"] = _normal(100 * c + 8, (spec["R"], N2), 0.05)
    return out


def calibration_batches(name, M=None, K=None):
    """Yield the workload's calibration batches (bf16 bit arrays [M, K]) one at a time."""
    spec = WORKLOADS[name]
    M = spec["M"] if M is None else M
    K = spec["K"] if K is None else K
    ch = _outlier_channels(spec, K)
    for i in range(spec.get("n_cal", 0)):
        yield _activation(spec, 100 * spec["c"] + 10 + i, M, K, ch)


def smooth_factors(name, K=None):
    """Positive per-channel smoothing factors float32 [K] for workload ``name``."""
    spec = WORKLOADS[name]
    K = spec["K"] if K is None else K
    lam = np.exp(_rng(100 * spec["c"] + 5).standard_normal(K, dtype=np.float32) * np.float32(0.25))
    lam = lam.astype(np.float32)
    ch = _outlier_channels(spec, K)
    if len(ch):
        lam[ch] *= np.float32(np.sqrt(spec["mult"]))
    return lam
