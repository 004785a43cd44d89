"""CPU oracle for the tiled dense GEMM (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``tg_oracle.c`` -- a plain
double-precision triple loop with its own f16/bf16 codecs -- through ctypes,
and shares nothing with the HIP library.

All matrices cross this boundary as raw 16-bit patterns (numpy ``uint16``),
so the oracle reads exactly the stored f16/bf16 values.

Every function here is pinned by ``tests/test_oracle_pins.py`` against
properties fixed by mathematics (identity, permutations, exact small-integer
products, brute force with rational arithmetic, codec round trips, GELU
identities); none is pinned only by itself.
"""
import ctypes
import os
import subprocess

import numpy as np

F16 = 1
BF16 = 2
ACT_NONE = 0
ACT_GELU_TANH = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tg_oracle.c")
_LIB = os.path.join(_HERE, "libtg_oracle.so")
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64


def build(force=False):
    """Compile tg_oracle.c with gcc (no HIP headers, no GPU code)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-D_DEFAULT_SOURCE", "-ffp-contract=off", "-fopenmp",
            "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        lib.tgo_gemm.argtypes = [_I, _L, _L, _L, _P, _L, _P, _L, _P, _I, _P, _P, _L, _L, _L, _I]
        lib.tgo_gemm_sample.argtypes = [_I, _L, _L, _L, _P, _L, _P, _L, _P, _I, _L, _P, _P, _P,
                                        _P, _I]
        lib.tgo_gemm_ex.argtypes = [_I, _L, _L, _L, _P, _L, _P, _L, _I, _P, _I, _P, _L, _P, _P,
                                    _L, _L, _L, _I]
        lib.tgo_gemm_ex_sample.argtypes = [_I, _L, _L, _L, _P, _L, _P, _L, _I, _P, _I, _P, _L,
                                           _L, _P, _P, _P, _P, _I]
        lib.tgo_gemm_mx.argtypes = [_I, _I, _L, _L, _L, _P, _L, _P, _L, _P, _L, _P, _L, _P, _I,
                                    _I, _P, _P, _L, _L, _L, _I]
        lib.tgo_decode_fp8_array.argtypes = [_I, _L, _P, _P]
        lib.tgo_attention.argtypes = [_I, _L, _L, _L, _L, _P, _P, _P, ctypes.c_double, _I, _P,
                                      _P, _P, _I]
        lib.tgo_gemm_qkv.argtypes = [_I, _L, _L, _L, _P, _L, _P, _P, _P, _L, _P, _P, _P, _P, _P,
                                     _P, _L, _L, _L, _I]
        lib.tgo_decode_array.argtypes = [_I, _L, _P, _P]
        lib.tgo_encode_array.argtypes = [_I, _L, _P, _P]
        lib.tgo_gelu_array.argtypes = [_L, _P, _P]
        lib.tgo_max_threads.restype = _I
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _bits(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs are uint16 bit patterns, got %s" % a.dtype)
    return a


def max_threads():
    return _load().tgo_max_threads()


def decode(dt, bits):
    """f16/bf16 bit patterns -> float64 values."""
    bits = _bits(bits)
    out = np.empty(bits.shape, np.float64)
    if _load().tgo_decode_array(dt, bits.size, _ptr(bits), _ptr(out)):
        raise ValueError("bad dtype")
    return out


def encode(dt, x):
    """float64 -> f16/bf16 bits, round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    if _load().tgo_encode_array(dt, x.size, _ptr(x), _ptr(out)):
        raise ValueError("bad dtype")
    return out


def gelu_tanh(x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.float64)
    _load().tgo_gelu_array(x.size, _ptr(x), _ptr(out))
    return out


def gemm(dt, A, B, bias=None, act=ACT_NONE, rows=None, threads=0):
    """C = round(act(A.B + bias)) on rows [r0, r1) (all rows by default).

    Returns (f64, bits): the unrounded double result and its RNE bits, both
    of shape [r1 - r0, N].
    """
    A, B = _bits(A), _bits(B)
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    if bias is not None:
        bias = _bits(bias)
        if bias.shape != (N,):
            raise ValueError("bias must be [N]")
    r0, r1 = (0, M) if rows is None else rows
    f64 = np.zeros((M, N), np.float64) if rows is None else np.zeros((M, N), np.float64)
    bits = np.zeros((M, N), np.uint16)
    rc = _load().tgo_gemm(dt, M, N, K, _ptr(A), K, _ptr(B), N, _ptr(bias), act, _ptr(f64),
                          _ptr(bits), N, r0, r1, threads)
    if rc:
        raise ValueError("oracle rejected the arguments")
    return f64[r0:r1], bits[r0:r1]


def gemm_sample(dt, A, B, ii, jj, bias=None, act=ACT_NONE, threads=0):
    """The elements (ii[s], jj[s]) of round(act(A.B + bias)); returns (f64, bits)."""
    A, B = _bits(A), _bits(B)
    M, K = A.shape
    _, N = B.shape
    if bias is not None:
        bias = _bits(bias)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    f64 = np.empty(ii.shape, np.float64)
    bits = np.empty(ii.shape, np.uint16)
    rc = _load().tgo_gemm_sample(dt, M, N, K, _ptr(A), K, _ptr(B), N, _ptr(bias), act, ii.size,
                                 _ptr(ii), _ptr(jj), _ptr(f64), _ptr(bits), threads)
    if rc:
        raise ValueError("oracle rejected the arguments")
    return f64, bits


def _ex_operands(A, B, trans_b, bias, R):
    A, B = _bits(A), _bits(B)
    M, K = A.shape
    if trans_b:
        N, K2 = B.shape
    else:
        K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    if bias is not None:
        bias = _bits(bias)
        if bias.shape != (N,):
            raise ValueError("bias must be [N]")
    if R is not None:
        R = _bits(R)
        if R.shape != (M, N):
            raise ValueError("residual must be [M,N]")
    return A, B, bias, R, M, N, K


def gemm_ex(dt, A, B, trans_b=False, bias=None, act=ACT_NONE, R=None, rows=None, threads=0):
    """C = round(act(A.opB + bias) + R) on rows [r0, r1); opB = B ([K,N]) or
    the transpose of B stored [N,K] when trans_b.  Returns (f64, bits)."""
    A, B, bias, R, M, N, K = _ex_operands(A, B, trans_b, bias, R)
    r0, r1 = (0, M) if rows is None else rows
    f64 = np.zeros((M, N), np.float64)
    bits = np.zeros((M, N), np.uint16)
    rc = _load().tgo_gemm_ex(dt, M, N, K, _ptr(A), K, _ptr(B), K if trans_b else N,
                             int(bool(trans_b)), _ptr(bias), act, _ptr(R), N, _ptr(f64),
                             _ptr(bits), N, r0, r1, threads)
    if rc:
        raise ValueError("oracle rejected the arguments")
    return f64[r0:r1], bits[r0:r1]


def gemm_ex_sample(dt, A, B, ii, jj, trans_b=False, bias=None, act=ACT_NONE, R=None, threads=0):
    """The elements (ii[s], jj[s]) of gemm_ex; returns (f64, bits)."""
    A, B, bias, R, M, N, K = _ex_operands(A, B, trans_b, bias, R)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    f64 = np.empty(ii.shape, np.float64)
    bits = np.empty(ii.shape, np.uint16)
    rc = _load().tgo_gemm_ex_sample(dt, M, N, K, _ptr(A), K, _ptr(B), K if trans_b else N,
                                    int(bool(trans_b)), _ptr(bias), act, _ptr(R), N, ii.size,
                                    _ptr(ii), _ptr(jj), _ptr(f64), _ptr(bits), threads)
    if rc:
        raise ValueError("oracle rejected the arguments")
    return f64, bits


FP8_E4M3, FP8_E5M2, E8M0 = 0, 1, 2


def decode_fp8(fmt, x):
    """8-bit floats (FP8_E4M3 / FP8_E5M2) or e8m0 scales (E8M0) to double."""
    x = np.ascontiguousarray(x, dtype=np.uint8)
    out = np.empty(x.shape, np.float64)
    _load().tgo_decode_fp8_array(fmt, x.size, _ptr(x), _ptr(out))
    return out


def gemm_mx(fmt_a, fmt_b, A, SA, B, SB, bias=None, act=ACT_NONE, dt=BF16, rows=None, threads=0):
    """Block-scaled 8-bit GEMM: A [M,K] and B [N,K] bytes, SA [K/32,M] and
    SB [K/32,N] e8m0 bytes; C = round_dt(act(sum_k a*sa * b*sb + bias)).
    Returns (f64, bits) for rows [r0, r1)."""
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    SA = np.ascontiguousarray(SA, dtype=np.uint8)
    SB = np.ascontiguousarray(SB, dtype=np.uint8)
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K or K % 32 or SA.shape != (K // 32, M) or SB.shape != (K // 32, N):
        raise ValueError("operand shapes do not match")
    if bias is not None:
        bias = _bits(bias)
        if bias.shape != (N,):
            raise ValueError("bias must be [N]")
    r0, r1 = (0, M) if rows is None else rows
    f64 = np.zeros((M, N), np.float64)
    bits = np.zeros((M, N), np.uint16)
    rc = _load().tgo_gemm_mx(fmt_a, fmt_b, M, N, K, _ptr(A), K, _ptr(SA), M, _ptr(B), K,
                             _ptr(SB), N, _ptr(bias), act, dt, _ptr(f64), _ptr(bits), N, r0, r1,
                             threads)
    if rc:
        raise ValueError("oracle rejected the arguments")
    return f64[r0:r1], bits[r0:r1]


def attention(dt, Q, K, V, causal=False, scale=None, threads=0):
    """Softmax(scale Q K^T + mask) V for Q, K, V [B, H, S, D] bit arrays;
    scale defaults to 1/sqrt(D).  Returns (f64, bits, lse)."""
    Q, K, V = _bits(Q), _bits(K), _bits(V)
    if Q.ndim != 4 or K.shape != Q.shape or V.shape != Q.shape:
        raise ValueError("Q, K, V must share one [B, H, S, D] shape")
    B, H, S, D = Q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    f64 = np.zeros(Q.shape, np.float64)
    bits = np.zeros(Q.shape, np.uint16)
    lse = np.zeros((B, H, S), np.float64)
    rc = _load().tgo_attention(dt, B, H, S, D, _ptr(Q), _ptr(K), _ptr(V), float(scale),
                               int(bool(causal)), _ptr(f64), _ptr(bits), _ptr(lse), threads)
    if rc:
        raise ValueError("oracle rejected the arguments")
    return f64, bits, lse


def gemm_qkv(dt, X, Wq, Wk, Wv, rows=None, threads=0):
    """Three independent GEMMs X.W_t; returns [(f64, bits)] * 3."""
    X = _bits(X)
    Ws = [_bits(w) for w in (Wq, Wk, Wv)]
    M, K = X.shape
    N = Ws[0].shape[1]
    r0, r1 = (0, M) if rows is None else rows
    f = [np.zeros((M, N), np.float64) for _ in range(3)]
    b = [np.zeros((M, N), np.uint16) for _ in range(3)]
    rc = _load().tgo_gemm_qkv(dt, M, N, K, _ptr(X), K, _ptr(Ws[0]), _ptr(Ws[1]), _ptr(Ws[2]), N,
                              _ptr(f[0]), _ptr(f[1]), _ptr(f[2]), _ptr(b[0]), _ptr(b[1]),
                              _ptr(b[2]), N, r0, r1, threads)
    if rc:
        raise ValueError("oracle rejected the arguments")
    return [(f[t][r0:r1], b[t][r0:r1]) for t in range(3)]
