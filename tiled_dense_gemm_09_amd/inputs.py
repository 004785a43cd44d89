"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module only draws random numbers and stores them as f16/bf16 bit
patterns (numpy ``uint16``).  It holds none of the GEMM's arithmetic, so both
the HIP path and the CPU oracle can read the same inputs.

Recipe (NumPy ``default_rng(seed)``, PCG64; draw order A or X, then B or the
W's, then bias):

* uniform   -- i.i.d. U[-1, 1] in float64, optionally scaled, then rounded.
* int       -- i.i.d. integers uniform in {-2, ..., 2}; every FP32 partial
               sum of such products is exact, so any summation order gives
               the same bits.
* normal    -- i.i.d. N(0, sigma^2).

f16 values are rounded from float64 by ``astype(float16)`` (round to nearest
even); bf16 values go float64 -> float32 -> bf16 with round to nearest even
on the bit pattern.  The oracle reads the stored bits, so rounding during
generation never affects parity.
"""
import math

import numpy as np

F16 = 1
BF16 = 2
ACT_NONE = 0
ACT_GELU_TANH = 1


def to_bits(x, dt):
    """float64 array -> uint16 bit patterns of dtype dt (RNE)."""
    x = np.asarray(x, dtype=np.float64)
    if dt == F16:
        return x.astype(np.float16).view(np.uint16)
    if dt == BF16:
        u = x.astype(np.float32).view(np.uint32)
        u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
        return (u >> np.uint32(16)).astype(np.uint16)
    raise ValueError("unknown dtype %r" % (dt,))


def draw(rng, shape, kind, dt, scale=1.0):
    """One seeded matrix as bits."""
    if kind == "uniform":
        x = rng.uniform(-1.0, 1.0, size=shape) * scale
    elif kind == "int":
        x = rng.integers(-2, 3, size=shape).astype(np.float64) * scale
    elif kind == "normal":
        x = rng.standard_normal(size=shape) * scale
    elif kind == "bias":
        x = rng.uniform(-0.5, 0.5, size=shape) * scale
    else:
        raise ValueError(kind)
    return to_bits(x, dt)


def problem(dt, M, N, K, seed, kind="uniform", bias=False, act=ACT_NONE, a_scale=1.0,
            b_scale=1.0, bias_kind="bias"):
    """A generic seeded GEMM problem: dict with dt, M, N, K, A, B, bias, act."""
    rng = np.random.default_rng(seed)
    A = draw(rng, (M, K), kind, dt, a_scale)
    B = draw(rng, (K, N), kind, dt, b_scale)
    bv = draw(rng, (N,), bias_kind, dt) if bias else None
    return dict(dt=dt, M=M, N=N, K=K, A=A, B=B, bias=bv, act=act)


def qkv_problem(dt, M, N, K, seed, kind="normal", x_scale=1.0, w_scale=None):
    """X[M,K] and three W[K,N] for the horizontally fused projection."""
    rng = np.random.default_rng(seed)
    if w_scale is None:
        w_scale = 1.0 / math.sqrt(K) if kind == "normal" else 1.0
    X = draw(rng, (M, K), kind, dt, x_scale)
    Ws = [draw(rng, (K, N), kind, dt, w_scale) for _ in range(3)]
    return dict(dt=dt, M=M, N=N, K=K, X=X, W=Ws)


# ------------------------------------------- block-scaled 8-bit operands

FP8_E4M3, FP8_E5M2 = 0, 1
_FP8_MAX = {FP8_E4M3: 448.0, FP8_E5M2: 57344.0}


def to_fp8(x, fmt):
    """float64 array -> 8-bit float bytes (OCP e4m3 / e5m2, round to nearest
    even through torch's float8 conversion of the float32 value)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.float8_e4m3fn if fmt == FP8_E4M3 else torch.float8_e5m2)
    return t.view(torch.uint8).numpy().copy()


def mx_quantize(x, fmt):
    """Rows of x [R, K] -> (bytes [R, K], e8m0 scales [K/32, R]).  Each row's
    32-element k-block gets the smallest power of two 2^(e - 127) that brings
    its largest magnitude within the format's largest finite value (the
    microscaling recipe); the block is divided by it and rounded."""
    R, K = x.shape
    peak = np.abs(x).reshape(R, K // 32, 32).max(axis=2)
    e = np.ceil(np.log2(np.maximum(peak, 1e-30) / _FP8_MAX[fmt])).astype(np.int64) + 127
    e = np.clip(e, 1, 254)
    q = to_fp8(x / np.repeat(np.ldexp(1.0, e - 127), 32, axis=1), fmt)
    return q, np.ascontiguousarray(e.T.astype(np.uint8))


def mx_problem(fmt_a, fmt_b, M, N, K, seed, kind="normal", bias=False, act=ACT_NONE, dt=BF16):
    """A [M,K] and B [N,K] 8-bit operands with e8m0 scales SA [K/32,M] and
    SB [K/32,N].  kind "normal": A ~ N(0,1), B ~ N(0, 1/K), quantized per
    32-block; kind "int": entries in {-2..2} and scales 2^-2..2^2, so every
    FP32 partial sum is exact in any order (|sum| < 2^20, step 2^-4)."""
    rng = np.random.default_rng(seed)
    if kind == "int":
        A = to_fp8(rng.integers(-2, 3, (M, K)), fmt_a)
        Bt = to_fp8(rng.integers(-2, 3, (N, K)), fmt_b)
        SA = rng.integers(125, 130, (K // 32, M)).astype(np.uint8)
        SB = rng.integers(125, 130, (K // 32, N)).astype(np.uint8)
    else:
        A, SA = mx_quantize(rng.standard_normal((M, K)), fmt_a)
        Bt, SB = mx_quantize(rng.standard_normal((N, K)) / math.sqrt(K), fmt_b)
    bv = draw(rng, (N,), "int" if kind == "int" else "bias", dt) if bias else None
    return dict(fmt_a=fmt_a, fmt_b=fmt_b, M=M, N=N, K=K, A=A, SA=SA, B=Bt, SB=SB, bias=bv,
                act=act, dt=dt)


# --------------------------------------------------------------- attention

def attention_problem(dt, B, H, S, D, seed, kind="normal", causal=False):
    """Q, K, V [B, H, S, D] bit patterns: i.i.d. N(0, 1) (kind "normal"), or
    integers in {-2..2} (kind "int")."""
    rng = np.random.default_rng(seed)
    Q = draw(rng, (B, H, S, D), kind, dt)
    K = draw(rng, (B, H, S, D), kind, dt)
    V = draw(rng, (B, H, S, D), kind, dt)
    return dict(dt=dt, B=B, H=H, S=S, D=D, Q=Q, K=K, V=V, causal=causal)


# The five workloads.  Config names follow their shapes.
CONFIGS = {
    # f16 256^3, U[-1,1]; integer variant {-2..2}
    "f16_256": dict(dt=F16, M=256, N=256, K=256, kind="uniform", seed=1, int_seed=101),
    # f16 1024^3, U[-1,1] (the TileLang example's shape)
    "f16_1024": dict(dt=F16, M=1024, N=1024, K=1024, kind="uniform", seed=2, int_seed=102),
    # f16 4096^3, GELU_tanh(A.B + bias); A, B = K^(-1/4) * U[-1,1] = U[-1,1]/8
    "f16_4096_gelu": dict(dt=F16, M=4096, N=4096, K=4096, kind="uniform", seed=3,
                          int_seed=103, bias=True, act=ACT_GELU_TANH, a_scale=4096 ** -0.25,
                          b_scale=4096 ** -0.25),
    # bf16 QKV: X[8192,4096] ~ N(0,1), W_{q,k,v}[4096,4096] ~ N(0, 1/4096)
    "bf16_qkv": dict(dt=BF16, M=8192, N=4096, K=4096, kind="normal", seed=4, int_seed=104,
                     qkv=True),
    # bf16 decode-shaped M=16, N=K=8192: X ~ N(0,1), W ~ N(0, 1/8192)
    "bf16_skinny": dict(dt=BF16, M=16, N=8192, K=8192, kind="normal", seed=5, int_seed=105,
                        a_scale=1.0, b_scale=8192 ** -0.5),
    # bf16 8192^3, same distributions as the skinny case
    "bf16_8192": dict(dt=BF16, M=8192, N=8192, K=8192, kind="normal", seed=6, int_seed=106,
                      a_scale=1.0, b_scale=8192 ** -0.5),
}


def config_problem(name, integer=False):
    """The seeded inputs of one named workload (integer=True: entries in {-2..2})."""
    c = CONFIGS[name]
    seed = c["int_seed"] if integer else c["seed"]
    kind = "int" if integer else c["kind"]
    if c.get("qkv"):
        return qkv_problem(c["dt"], c["M"], c["N"], c["K"], seed, kind)
    if integer:
        return problem(c["dt"], c["M"], c["N"], c["K"], seed, "int", bias=c.get("bias", False),
                       act=ACT_NONE, bias_kind="int")
    return problem(c["dt"], c["M"], c["N"], c["K"], seed, kind, bias=c.get("bias", False),
                   act=c.get("act", ACT_NONE), a_scale=c.get("a_scale", 1.0),
                   b_scale=c.get("b_scale", 1.0))
