"""Pins for the CPU oracle: each check ties it to something other than itself.

The oracle is the plain definition of the tiled GEMM's result (the TileLang
article, section 4: C = A.B with an f32 accumulator and an f16 output; "TileIR":
epilogue fusion of bias + activation and horizontal QKV fusion).  These tests
fix it with mathematics and independent code:

* codecs against NumPy's float16 and torch's bfloat16 conversions, and
  against the defining property of round-to-nearest-even (checked with exact
  rational arithmetic), over every 16-bit pattern and random doubles;
* the GEMM against identities, permutations, closed forms, exact integer
  products, rational brute force on tiny inputs, and a float64 library
  product;
* GELU_tanh against its odd-part identity, its asymptotes and an exactly
  solvable point (tanh(ln 3) = 4/5);
* the 8-bit float and e8m0 decoders against torch's float8 types over every
  pattern; the block-scaled GEMM against the f16 GEMM (unit scales), a closed
  form for the scales and rational brute force;
* attention against uniform weights (Q = 0), the causal first row (= V[0]),
  pure-Python brute force, a NumPy cross-check and the invariance of the
  softmax to a common shift of the keys;
* the epilogue order (bias before activation, residual after it), QKV =
  three GEMMs, the transposed-operand form against brute force and against
  the same operand stored the other way, and independence of the thread
  count and of row subsets.

A plausible slip in the oracle -- a dropped term, a wrong sign or index, a
transposed operand, a wrong rounding direction or constant -- fails one of
them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tiled_dense_gemm_09_amd import inputs

F16, BF16 = oracle.F16, oracle.BF16
ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def bits_of(dt, values):
    return oracle.encode(dt, np.asarray(values, np.float64))


def is_nan_bits(dt, b):
    b = np.asarray(b).astype(np.uint32)
    if dt == F16:
        return ((b & 0x7C00) == 0x7C00) & ((b & 0x03FF) != 0)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


# ------------------------------------------------------------------ codecs

def test_f16_decode_matches_numpy_on_every_pattern():
    got = oracle.decode(F16, ALL)
    ref = ALL.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert math.copysign(1.0, got[0x8000]) == -1.0


def test_bf16_decode_matches_torch_on_every_pattern():
    torch = pytest.importorskip("torch")
    ref = torch.from_numpy(ALL.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    got = oracle.decode(BF16, ALL)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("dt", [F16, BF16])
def test_roundtrip_every_pattern(dt):
    vals = oracle.decode(dt, ALL)
    back = oracle.encode(dt, vals)
    nan = is_nan_bits(dt, ALL)
    assert np.array_equal(back[~nan], ALL[~nan])
    canon = 0x7E00 if dt == F16 else 0x7FC0
    assert np.all(back[nan] == canon)


def test_f16_encode_matches_numpy_on_random_doubles_and_ties():
    rng = np.random.default_rng(7)
    mags = np.exp2(rng.uniform(-30, 17, size=400_000))
    x = mags * rng.choice([-1.0, 1.0], size=mags.size)
    # every midpoint between consecutive finite positive f16 values (exact ties)
    pos = ALL[(ALL < 0x7C00)].astype(np.uint16)
    v = oracle.decode(F16, pos)
    mids = (v[:-1] + v[1:]) / 2.0
    x = np.concatenate([x, mids, -mids, [65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -25, 2.0 ** -26]])
    got = oracle.encode(F16, x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def _nearest_even_ok(dt, x, b):
    """b is the RNE encoding of x: no finite neighbour is nearer, ties go to even."""
    fx = Fraction(float(x))
    vb = oracle.decode(dt, np.array([b], np.uint16))[0]
    if math.isinf(vb):
        return True  # overflow checks live in a separate test
    d0 = abs(fx - Fraction(vb))
    for nb in (int(b) - 1, int(b) + 1):
        vn = oracle.decode(dt, np.array([nb & 0xFFFF], np.uint16))[0]
        if math.isnan(vn) or math.isinf(vn):
            continue
        dn = abs(fx - Fraction(vn))
        if dn < d0:
            return False
        if dn == d0 and (int(b) & 1):
            return False
    return True


@pytest.mark.parametrize("dt", [F16, BF16])
def test_encode_is_round_to_nearest_even(dt):
    rng = np.random.default_rng(11)
    hi = 15 if dt == F16 else 120
    lo = -26 if dt == F16 else -134
    mags = np.exp2(rng.uniform(lo, hi, size=3000))
    # doubles with bits below the target precision (not representable in f32 either)
    x = mags * (1.0 + rng.uniform(0, 1e-9, size=mags.size)) * rng.choice([-1.0, 1.0], mags.size)
    got = oracle.encode(dt, x)
    for xi, bi in zip(x, got):
        assert _nearest_even_ok(dt, xi, bi), (dt, xi, hex(int(bi)))


def test_bf16_encode_matches_torch_on_float32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    x32 = (rng.standard_normal(300_000) * np.exp2(rng.uniform(-40, 40, 300_000))).astype(np.float32)
    # exact bf16 ties: a bf16 value plus half an ulp
    base = oracle.decode(BF16, rng.integers(0x0080, 0x7F00, 20000).astype(np.uint16))
    ties = (base + np.abs(base) * 2.0 ** -8).astype(np.float32)
    x32 = np.concatenate([x32, ties, -ties])
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.encode(BF16, x32.astype(np.float64))
    assert np.array_equal(got, ref)


def test_overflow_and_specials():
    assert oracle.encode(F16, np.array([65520.0]))[0] == 0x7C00  # rounds up to inf
    assert oracle.encode(F16, np.array([65519.0]))[0] == 0x7BFF
    assert oracle.encode(F16, np.array([-np.inf]))[0] == 0xFC00
    assert oracle.encode(BF16, np.array([3.5e38]))[0] == 0x7F80
    assert oracle.encode(F16, np.array([-0.0]))[0] == 0x8000
    assert oracle.encode(F16, np.array([2.0 ** -25]))[0] == 0x0000  # tie to even (zero)
    assert oracle.encode(F16, np.array([3 * 2.0 ** -25]))[0] == 0x0002  # tie to even


# -------------------------------------------------------------------- GEMM

def rand_bits(dt, shape, seed):
    return inputs.draw(np.random.default_rng(seed), shape, "uniform", dt)


@pytest.mark.parametrize("dt", [F16, BF16])
def test_identity_is_exact(dt):
    A = rand_bits(dt, (19, 23), 1)
    I_k = bits_of(dt, np.eye(23))
    I_m = bits_of(dt, np.eye(19))
    _, c = oracle.gemm(dt, A, I_k)
    assert np.array_equal(c, A)
    _, c = oracle.gemm(dt, I_m, A)
    assert np.array_equal(c, A)


@pytest.mark.parametrize("dt", [F16, BF16])
def test_permutations_are_exact(dt):
    rng = np.random.default_rng(3)
    A = rand_bits(dt, (7, 11), 2)
    p = rng.permutation(11)
    P = np.zeros((11, 11))
    P[p, np.arange(11)] = 1.0  # (A.P)[:, j] = A[:, p[j]]
    _, c = oracle.gemm(dt, A, bits_of(dt, P))
    assert np.array_equal(c, A[:, p])
    q = rng.permutation(7)
    Q = np.zeros((7, 7))
    Q[np.arange(7), q] = 1.0  # (Q.A)[i, :] = A[q[i], :]
    _, c = oracle.gemm(dt, bits_of(dt, Q), A)
    assert np.array_equal(c, A[q, :])


@pytest.mark.parametrize("shape", [(4, 4, 4), (3, 5, 2), (1, 1, 1), (2, 3, 7)])
@pytest.mark.parametrize("dt", [F16, BF16])
def test_brute_force_rational(dt, shape):
    M, N, K = shape
    A = rand_bits(dt, (M, K), 10 + M)
    B = rand_bits(dt, (K, N), 20 + N)
    av = oracle.decode(dt, A)
    bv = oracle.decode(dt, B)
    f64, bits = oracle.gemm(dt, A, B)
    for i in range(M):
        for j in range(N):
            exact = sum((Fraction(float(av[i, k])) * Fraction(float(bv[k, j])) for k in range(K)),
                        Fraction(0))
            bound = sum(abs(float(av[i, k]) * float(bv[k, j])) for k in range(K)) * K * 2.0 ** -52
            assert abs(Fraction(float(f64[i, j])) - exact) <= Fraction(bound)
            # the rounded output is a nearest representable value to the exact sum
            vb = Fraction(float(oracle.decode(dt, bits[i:i + 1, j])[0]))
            for nb in (int(bits[i, j]) - 1, int(bits[i, j]) + 1):
                vn = float(oracle.decode(dt, np.array([nb & 0xFFFF], np.uint16))[0])
                if math.isfinite(vn) and ((vn >= 0) == (float(vb) >= 0) or vn == 0):
                    assert abs(Fraction(vn) - exact) >= abs(vb - exact) - Fraction(bound)


@pytest.mark.parametrize("dt", [F16, BF16])
def test_small_integers_exact(dt):
    rng = np.random.default_rng(5)
    M, N, K = 9, 13, 700
    a = rng.integers(-2, 3, (M, K))
    b = rng.integers(-2, 3, (K, N))
    exact = a @ b  # int64, independent integer arithmetic
    f64, bits = oracle.gemm(dt, bits_of(dt, a), bits_of(dt, b))
    assert np.array_equal(f64, exact.astype(np.float64))
    # rounding of the exact integer: check the nearest-even property directly
    for i in range(M):
        for j in range(N):
            assert _nearest_even_ok(dt, float(exact[i, j]), bits[i, j])


def test_integer_outputs_above_f16_exact_range():
    # |sum| > 2048 needs rounding in f16: ones(1,K).ones(K,1) = K for K = 2049..2051
    for K in (2049, 2050, 2051, 4095):
        _, bits = oracle.gemm(F16, bits_of(F16, np.ones((1, K))), bits_of(F16, np.ones((K, 1))))
        assert bits[0, 0] == np.float16(K).view(np.uint16)


@pytest.mark.parametrize("dt", [F16, BF16])
def test_closed_forms(dt):
    M, N, K = 6, 10, 37
    f64, _ = oracle.gemm(dt, bits_of(dt, np.ones((M, K))), bits_of(dt, np.ones((K, N))))
    assert np.all(f64 == K)
    # rank one: u (M x 1) times v (1 x N) gives u_i v_j
    u = np.arange(1, M + 1, dtype=np.float64)
    v = np.arange(-5, N - 5, dtype=np.float64)
    f64, _ = oracle.gemm(dt, bits_of(dt, u[:, None]), bits_of(dt, v[None, :]))
    assert np.array_equal(f64, np.outer(u, v))
    # B = e_j selects column j of A
    A = rand_bits(dt, (M, K), 4)
    E = np.zeros((K, 1))
    E[13, 0] = 1.0
    _, bits = oracle.gemm(dt, A, bits_of(dt, E))
    assert np.array_equal(bits[:, 0], A[:, 13])


@pytest.mark.parametrize("dt", [F16, BF16])
def test_float64_library_crosscheck(dt):
    A = rand_bits(dt, (33, 129), 8)
    B = rand_bits(dt, (129, 65), 9)
    f64, _ = oracle.gemm(dt, A, B)
    ref = oracle.decode(dt, A) @ oracle.decode(dt, B)
    scale = np.abs(oracle.decode(dt, A)) @ np.abs(oracle.decode(dt, B))
    assert np.all(np.abs(f64 - ref) <= 1e-12 * scale)


def test_nonsquare_transposition_is_caught():
    # A.B for A[2,3], B[3,4] against hand-written integer entries
    A = np.array([[1, 2, 0], [0, -1, 3]], np.float64)
    B = np.array([[1, 0, 2, -1], [0, 1, 1, 0], [2, 0, 0, 1]], np.float64)
    want = np.array([[1, 2, 4, -1], [6, -1, -1, 3]], np.float64)
    f64, _ = oracle.gemm(F16, bits_of(F16, A), bits_of(F16, B))
    assert np.array_equal(f64, want)


def test_thread_count_and_row_subsets_do_not_change_bits():
    A = rand_bits(BF16, (64, 300), 30)
    B = rand_bits(BF16, (300, 40), 31)
    bias = rand_bits(BF16, (40,), 32)
    f1, b1 = oracle.gemm(BF16, A, B, bias, oracle.ACT_GELU_TANH, threads=1)
    f8, b8 = oracle.gemm(BF16, A, B, bias, oracle.ACT_GELU_TANH, threads=8)
    assert np.array_equal(b1, b8) and np.array_equal(f1, f8)
    fs, bs = oracle.gemm(BF16, A, B, bias, oracle.ACT_GELU_TANH, rows=(17, 45))
    assert np.array_equal(bs, b1[17:45]) and np.array_equal(fs, f1[17:45])


def test_sample_matches_full():
    A = rand_bits(F16, (50, 70), 40)
    B = rand_bits(F16, (70, 90), 41)
    bias = rand_bits(F16, (90,), 42)
    f, b = oracle.gemm(F16, A, B, bias, oracle.ACT_GELU_TANH)
    rng = np.random.default_rng(0)
    ii = rng.integers(0, 50, 300)
    jj = rng.integers(0, 90, 300)
    fs, bs = oracle.gemm_sample(F16, A, B, ii, jj, bias, oracle.ACT_GELU_TANH)
    assert np.array_equal(fs, f[ii, jj]) and np.array_equal(bs, b[ii, jj])


# ---------------------------------------------------------------- epilogue

def test_bias_only():
    N = 33
    bias = rand_bits(F16, (N,), 50)
    _, bits = oracle.gemm(F16, bits_of(F16, np.zeros((5, 8))), rand_bits(F16, (8, N), 51), bias)
    assert np.all(bits == bias[None, :])
    # K = 0: the empty sum is zero, C = bias
    _, bits = oracle.gemm(F16, np.zeros((3, 0), np.uint16), np.zeros((0, N), np.uint16), bias)
    assert np.all(bits == bias[None, :])


def test_integer_bias_is_per_column_and_exact():
    rng = np.random.default_rng(6)
    a = rng.integers(-2, 3, (4, 50))
    b = rng.integers(-2, 3, (50, 6))
    bias = np.array([-3, 0, 1, 2, 7, -8], np.float64)
    f64, _ = oracle.gemm(BF16, bits_of(BF16, a), bits_of(BF16, b), bits_of(BF16, bias))
    assert np.array_equal(f64, (a @ b).astype(np.float64) + bias[None, :])


def test_gelu_odd_part_identity_and_zero():
    x = np.linspace(-12, 12, 4801)
    g = oracle.gelu_tanh(x)
    gm = oracle.gelu_tanh(-x)
    # tanh is odd, so gelu(x) - gelu(-x) = x exactly in real arithmetic
    assert np.all(np.abs((g - gm) - x) <= 4e-16 * np.maximum(1.0, np.abs(x)) * 4)
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0


def test_gelu_asymptotes():
    g = oracle.gelu_tanh(np.array([10.0, -10.0, 30.0, -30.0]))
    assert abs(g[0] - 10.0) < 1e-12 and abs(g[1]) < 1e-12
    assert g[2] == 30.0 and g[3] == 0.0


def _gelu_tanh_decimal(x):
    """0.5 x (1 + tanh(u)) at 200 significant digits, tanh from exp:
    tanh(u) = (e^(2u) - 1) / (e^(2u) + 1).  With that many digits the
    cancellation in 1 + tanh(u) for very negative u costs nothing."""
    import decimal
    with decimal.localcontext() as ctx:
        ctx.prec = 200
        D = decimal.Decimal
        X = D(x)
        # pi to 60 digits (only its first ~20 matter for a double result)
        pi = D("3.14159265358979323846264338327950288419716939937510582097494")
        c = (D(2) / pi).sqrt()
        u = c * (X + D("0.044715") * X ** 3)
        e2u = (2 * u).exp()
        tanh = (e2u - 1) / (e2u + 1)
        return float(D("0.5") * X * (1 + tanh))


def test_gelu_against_high_precision_including_the_far_negative_tail():
    # points where the double tanh form would cancel (x < -6.4) and ordinary ones
    xs = [-9.5, -9.0, -8.0, -7.0, -6.5, -6.0, -5.0, -3.0, -1.25, -0.5, 0.5, 1.0, 2.5, 5.0, 8.0]
    g = oracle.gelu_tanh(np.array(xs))
    for x, v in zip(xs, g):
        ref = _gelu_tanh_decimal(x)
        assert ref != 0.0
        # rounding u = c (x + 0.044715 x^3) in double costs ~|u| ulps of exp(-2u)
        u = math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)
        assert abs(v - ref) <= 2.0 ** -52 * (8 + 6 * abs(u)) * abs(ref), (x, v, ref)


def test_gelu_at_an_exactly_solvable_point():
    # With c = sqrt(2/pi): if c (x + 0.044715 x^3) = ln 3 then tanh = 4/5 and
    # gelu(x) = 0.5 x (1 + 4/5) = 0.9 x.  Solve for x by bisection.
    c = math.sqrt(2.0 / math.pi)
    target = math.log(3.0)
    lo, hi = 0.0, 3.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if c * (mid + 0.044715 * mid ** 3) < target:
            lo = mid
        else:
            hi = mid
    x = 0.5 * (lo + hi)
    g = oracle.gelu_tanh(np.array([x, -x]))
    assert abs(g[0] - 0.9 * x) < 1e-14
    assert abs(g[1] - (-0.1 * x)) < 1e-14  # 0.5 (-x) (1 - 4/5)


def test_epilogue_adds_bias_before_activation():
    one = bits_of(F16, np.ones((1, 1)))
    bias = bits_of(F16, np.array([1.0]))
    f64, _ = oracle.gemm(F16, one, one, bias, oracle.ACT_GELU_TANH)
    assert f64[0, 0] == oracle.gelu_tanh(np.array([2.0]))[0]
    assert f64[0, 0] != oracle.gelu_tanh(np.array([1.0]))[0] + 1.0


# ------------------------------------------- extended form: opB and residual

@pytest.mark.parametrize("dt", [F16, BF16])
def test_transposed_operand_brute_force(dt):
    # B stored [N,K]: output (i, j) is the sum over k of A[i][k] * B[j][k]
    M, N, K = 3, 4, 5
    A = rand_bits(dt, (M, K), 41)
    Bt = rand_bits(dt, (N, K), 42)
    av, bv = oracle.decode(dt, A), oracle.decode(dt, Bt)
    f64, _ = oracle.gemm_ex(dt, A, Bt, trans_b=True)
    for i in range(M):
        for j in range(N):
            exact = sum((Fraction(float(av[i, k])) * Fraction(float(bv[j, k])) for k in range(K)),
                        Fraction(0))
            bound = sum(abs(float(av[i, k]) * float(bv[j, k])) for k in range(K)) * K * 2.0 ** -52
            assert abs(Fraction(float(f64[i, j])) - exact) <= Fraction(bound)


@pytest.mark.parametrize("dt", [F16, BF16])
def test_transposed_storage_gives_the_same_bits(dt):
    p = inputs.problem(dt, 37, 53, 29, seed=43, bias=True, act=inputs.ACT_GELU_TANH)
    Bt = np.ascontiguousarray(p["B"].T)   # the same operand stored [N,K]
    f1, b1 = oracle.gemm(dt, p["A"], p["B"], p["bias"], oracle.ACT_GELU_TANH)
    f2, b2 = oracle.gemm_ex(dt, p["A"], Bt, trans_b=True, bias=p["bias"], act=oracle.ACT_GELU_TANH)
    assert np.array_equal(b1, b2) and np.array_equal(f1, f2)
    # and a non-square transposed read is not a plain one
    with pytest.raises(ValueError):
        oracle.gemm_ex(dt, p["A"], Bt, trans_b=False)


@pytest.mark.parametrize("dt", [F16, BF16])
def test_residual_integer_exact(dt):
    rng = np.random.default_rng(44)
    a = rng.integers(-2, 3, (9, 31))
    b = rng.integers(-2, 3, (31, 7))
    r = rng.integers(-40, 41, (9, 7))
    bias = rng.integers(-3, 4, 7)
    f64, bits = oracle.gemm_ex(dt, bits_of(dt, a), bits_of(dt, b), bias=bits_of(dt, bias),
                               R=bits_of(dt, r))
    ref = (a @ b + bias[None, :] + r).astype(np.float64)
    assert np.array_equal(f64, ref)
    assert np.array_equal(bits, bits_of(dt, ref))


def test_residual_is_added_after_the_activation():
    one = bits_of(F16, np.ones((1, 1)))
    two = bits_of(F16, 2.0 * np.ones((1, 1)))
    f64, _ = oracle.gemm_ex(F16, one, two, act=oracle.ACT_GELU_TANH, R=one)
    g2 = oracle.gelu_tanh(np.array([2.0]))[0]
    assert f64[0, 0] == g2 + 1.0
    assert f64[0, 0] != oracle.gelu_tanh(np.array([3.0]))[0]


def test_residual_only_when_k_is_zero():
    bias = rand_bits(F16, (6,), 46)
    R = rand_bits(F16, (4, 6), 47)
    f64, _ = oracle.gemm_ex(F16, np.zeros((4, 0), np.uint16), np.zeros((0, 6), np.uint16),
                            bias=bias, act=oracle.ACT_GELU_TANH, R=R)
    g = oracle.gelu_tanh(oracle.decode(F16, bias))
    assert np.array_equal(f64, g[None, :] + oracle.decode(F16, R))


def test_ex_sample_matches_full():
    p = inputs.problem(BF16, 40, 70, 33, seed=48, bias=True, act=inputs.ACT_GELU_TANH)
    Bt = np.ascontiguousarray(p["B"].T)
    R = rand_bits(BF16, (40, 70), 49)
    f, b = oracle.gemm_ex(BF16, p["A"], Bt, trans_b=True, bias=p["bias"],
                          act=oracle.ACT_GELU_TANH, R=R)
    ii = np.array([0, 39, 17, 5, 22]); jj = np.array([0, 69, 3, 44, 60])
    fs, bs = oracle.gemm_ex_sample(BF16, p["A"], Bt, ii, jj, trans_b=True, bias=p["bias"],
                                   act=oracle.ACT_GELU_TANH, R=R)
    assert np.array_equal(fs, f[ii, jj]) and np.array_equal(bs, b[ii, jj])


# -------------------------------------- block-scaled 8-bit GEMM (e8m0 scales)

ALL8 = np.arange(256, dtype=np.uint8)


@pytest.mark.parametrize("fmt,tname", [(oracle.FP8_E4M3, "float8_e4m3fn"),
                                       (oracle.FP8_E5M2, "float8_e5m2")])
def test_fp8_decode_matches_torch_on_every_pattern(fmt, tname):
    torch = pytest.importorskip("torch")
    ref = torch.from_numpy(ALL8.copy()).view(getattr(torch, tname)).to(torch.float64).numpy()
    got = oracle.decode_fp8(fmt, ALL8)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e8m0_decode_is_a_power_of_two():
    got = oracle.decode_fp8(oracle.E8M0, ALL8)
    assert np.isnan(got[255])
    for e in range(255):
        assert got[e] == math.ldexp(1.0, e - 127)


def _fp8_bits(fmt, rng, shape):
    """Random finite 8-bit patterns (NaN and infinity patterns redrawn)."""
    v = rng.integers(0, 256, shape).astype(np.uint8)
    d = oracle.decode_fp8(fmt, v)
    bad = ~np.isfinite(d)
    while bad.any():
        v[bad] = rng.integers(0, 256, int(bad.sum())).astype(np.uint8)
        d = oracle.decode_fp8(fmt, v)
        bad = ~np.isfinite(d)
    return v


@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 1), (0, 1)])
def test_mx_with_unit_scales_is_the_f16_gemm(fa, fb):
    # every e4m3 / e5m2 value is an f16 value, so with scales 2^0 the
    # block-scaled product must be the (pinned) f16 GEMM of the decoded values
    rng = np.random.default_rng(50 + fa + 2 * fb)
    M, N, K = 7, 9, 96
    A = _fp8_bits(fa, rng, (M, K))
    Bt = _fp8_bits(fb, rng, (N, K))
    SA = np.full((K // 32, M), 127, np.uint8)
    SB = np.full((K // 32, N), 127, np.uint8)
    f1, b1 = oracle.gemm_mx(fa, fb, A, SA, Bt, SB, dt=F16)
    a16 = bits_of(F16, oracle.decode_fp8(fa, A))
    b16 = bits_of(F16, oracle.decode_fp8(fb, Bt).T)
    f2, b2 = oracle.gemm(F16, a16, b16)
    assert np.array_equal(f1, f2) and np.array_equal(b1, b2)


def test_mx_block_scales_closed_form():
    # A = B = 1: C[i][j] = sum over k-blocks b of 32 * 2^(sa[b][i] - 127) * 2^(sb[b][j] - 127)
    M, N, K = 3, 4, 128
    one = 0x38  # e4m3 1.0
    A = np.full((M, K), one, np.uint8)
    Bt = np.full((N, K), one, np.uint8)
    SA = np.array([[127 + b + i for i in range(M)] for b in range(K // 32)], np.uint8)
    SB = np.array([[125 + (b * j) % 3 for j in range(N)] for b in range(K // 32)], np.uint8)
    f64, _ = oracle.gemm_mx(0, 0, A, SA, Bt, SB)
    for i in range(M):
        for j in range(N):
            ref = sum(32 * 2.0 ** (int(SA[b, i]) - 127) * 2.0 ** (int(SB[b, j]) - 127)
                      for b in range(K // 32))
            assert f64[i, j] == ref


def test_mx_brute_force_rational_nonsquare():
    rng = np.random.default_rng(52)
    M, N, K = 2, 3, 64
    A = _fp8_bits(0, rng, (M, K))
    Bt = _fp8_bits(1, rng, (N, K))
    SA = rng.integers(120, 134, (K // 32, M)).astype(np.uint8)
    SB = rng.integers(120, 134, (K // 32, N)).astype(np.uint8)
    f64, _ = oracle.gemm_mx(0, 1, A, SA, Bt, SB)
    av, bv = oracle.decode_fp8(0, A), oracle.decode_fp8(1, Bt)
    for i in range(M):
        for j in range(N):
            exact = sum((Fraction(float(av[i, k])) * Fraction(2) ** (int(SA[k // 32, i]) - 127) *
                         Fraction(float(bv[j, k])) * Fraction(2) ** (int(SB[k // 32, j]) - 127)
                         for k in range(K)), Fraction(0))
            bound = sum(abs(float(av[i, k]) * float(bv[j, k])) * 2.0 ** (int(SA[k // 32, i]) +
                        int(SB[k // 32, j]) - 254) for k in range(K)) * K * 2.0 ** -52
            assert abs(Fraction(float(f64[i, j])) - exact) <= Fraction(bound)


# --------------------------------------------------------------- attention

def _att_decode(dt, x):
    return oracle.decode(dt, x)


@pytest.mark.parametrize("causal", [False, True])
def test_attention_uniform_weights_when_q_is_zero(causal):
    p = inputs.attention_problem(BF16, 1, 2, 9, 16, seed=60)
    Q = np.zeros_like(p["Q"])
    f64, _, lse = oracle.attention(BF16, Q, p["K"], p["V"], causal=causal)
    V = _att_decode(BF16, p["V"])
    for i in range(9):
        n = i + 1 if causal else 9
        assert np.allclose(f64[:, :, i], V[:, :, :n].mean(axis=2), rtol=1e-14, atol=1e-15)
        assert np.allclose(lse[:, :, i], math.log(n), rtol=1e-15)


def test_attention_causal_first_row_is_v0():
    p = inputs.attention_problem(F16, 2, 3, 7, 8, seed=61)
    f64, bits, lse = oracle.attention(F16, p["Q"], p["K"], p["V"], causal=True)
    assert np.array_equal(f64[:, :, 0], _att_decode(F16, p["V"])[:, :, 0])
    assert np.array_equal(bits[:, :, 0], p["V"][:, :, 0])
    q0 = _att_decode(F16, p["Q"])[:, :, 0]
    k0 = _att_decode(F16, p["K"])[:, :, 0]
    assert np.allclose(lse[:, :, 0], (q0 * k0).sum(-1) / math.sqrt(8), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_attention_brute_force_python(causal):
    # pure-Python floats and math.exp, independent of the oracle's C
    p = inputs.attention_problem(BF16, 1, 2, 5, 3, seed=62)
    f64, _, lse = oracle.attention(BF16, p["Q"], p["K"], p["V"], causal=causal, scale=0.7)
    Q, K, V = (_att_decode(BF16, p[n]).tolist() for n in ("Q", "K", "V"))
    for h in range(2):
        for i in range(5):
            keys = range(i + 1) if causal else range(5)
            sc = [0.7 * sum(Q[0][h][i][d] * K[0][h][j][d] for d in range(3)) for j in keys]
            m = max(sc)
            w = [math.exp(x - m) for x in sc]
            tot = sum(w)
            for d in range(3):
                ref = sum(w[t] * V[0][h][j][d] for t, j in enumerate(keys)) / tot
                assert abs(f64[0, h, i, d] - ref) <= 1e-13 * max(1.0, abs(ref))
            assert abs(lse[0, h, i] - (m + math.log(tot))) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_attention_numpy_crosscheck(causal):
    p = inputs.attention_problem(F16, 2, 2, 64, 16, seed=63)
    f64, _, lse = oracle.attention(F16, p["Q"], p["K"], p["V"], causal=causal)
    Q, K, V = (_att_decode(F16, p[n]) for n in ("Q", "K", "V"))
    s = np.einsum("bhid,bhjd->bhij", Q, K) / 4.0
    if causal:
        s = np.where(np.tril(np.ones((64, 64), bool)), s, -np.inf)
    w = np.exp(s - s.max(-1, keepdims=True))
    ref = np.einsum("bhij,bhjd->bhid", w / w.sum(-1, keepdims=True), V)
    assert np.allclose(f64, ref, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, np.log(np.exp(s - s.max(-1, keepdims=True)).sum(-1)) +
                       s.max(-1), rtol=1e-13)


def test_attention_is_invariant_to_a_common_key_shift():
    # adding one vector w to every key row adds q.w to every score of query q:
    # the softmax weights, hence O, do not change; lse shifts by scale q.w
    p = inputs.attention_problem(BF16, 1, 1, 12, 8, seed=64, kind="int")
    w = np.array([1, -2, 0, 1, 2, -1, 0, 1], np.float64)
    K2 = bits_of(BF16, _att_decode(BF16, p["K"]) + w)
    f1, _, l1 = oracle.attention(BF16, p["Q"], p["K"], p["V"])
    f2, _, l2 = oracle.attention(BF16, p["Q"], K2, p["V"])
    assert np.allclose(f1, f2, rtol=1e-13, atol=1e-14)
    qw = _att_decode(BF16, p["Q"])[0, 0] @ w
    assert np.allclose(l2[0, 0] - l1[0, 0], qw / math.sqrt(8), rtol=1e-12, atol=1e-12)


def test_qkv_is_three_gemms():
    p = inputs.qkv_problem(BF16, 24, 40, 56, seed=9)
    outs = oracle.gemm_qkv(BF16, p["X"], *p["W"])
    for t in range(3):
        f, b = oracle.gemm(BF16, p["X"], p["W"][t])
        assert np.array_equal(outs[t][1], b) and np.array_equal(outs[t][0], f)


def test_inputs_are_deterministic_and_shaped():
    p1 = inputs.config_problem("f16_256")
    p2 = inputs.config_problem("f16_256")
    assert np.array_equal(p1["A"], p2["A"]) and np.array_equal(p1["B"], p2["B"])
    assert p1["A"].shape == (256, 256) and p1["A"].dtype == np.uint16
    q = inputs.config_problem("f16_256", integer=True)
    vals = np.unique(oracle.decode(F16, q["A"]))
    assert set(vals.tolist()) == {-2.0, -1.0, 0.0, 1.0, 2.0}
    c3 = inputs.CONFIGS["f16_4096_gelu"]
    assert c3["a_scale"] == 0.125 and c3["b_scale"] == 0.125
