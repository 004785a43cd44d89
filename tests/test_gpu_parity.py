"""GPU parity: every entry point of libtg.so against the CPU oracle.

Bar: |gpu - oracle| <= 1e-2 + 5e-3 |oracle| per element on random inputs
(oracle = unrounded double), and bit-exact equality with the oracle's
round-to-nearest-even bits on inputs with entries in {-2..2}, where every
FP32 partial sum is exact in any order.

Sizes: every configured workload, including the full-size ones in the
launch configuration the benchmark times (f16 4096^3 + GELU, the bf16 QKV
projection, bf16 M = 16 and 8192^3), is compared element by element over its
whole output, random and integer variants alike; only the two problems past
2^31 elements are compared on sampled outputs.
Ragged shapes use padded pitches whose padding holds NaN, so any read past
the logical bounds would show up, and outputs carry NaN canaries around the
written region.
"""
import sys

import numpy as np
import pytest

import oracle
import util
from tiled_dense_gemm_09_amd import inputs

pytestmark = pytest.mark.gpu

F16, BF16 = inputs.F16, inputs.BF16
NAN_BITS = {F16: 0x7E00, BF16: 0x7FC0}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def tg():
    import torch
    assert torch.cuda.is_available()
    from tiled_dense_gemm_09_amd import tg as _tg
    return _tg


def dev_problem(p):
    dt = p["dt"]
    A = util.to_dev(p["A"], dt)
    B = util.to_dev(p["B"], dt)
    bias = util.to_dev(p["bias"], dt) if p.get("bias") is not None else None
    return A, B, bias


def run(tg, p):
    import torch
    A, B, bias = dev_problem(p)
    act = "gelu_tanh" if p["act"] == inputs.ACT_GELU_TANH else "none"
    C = tg.gemm(A, B, bias=bias, act=act)
    torch.cuda.synchronize()
    return util.to_bits(C), tg.last_kernel()


# ------------------------------------------------------------ small configs

@pytest.mark.parametrize("name", ["f16_256", "f16_1024"])
def test_small_config_random_full(tg, name):
    p = inputs.config_problem(name)
    say("case", name, "random", p["M"], p["N"], p["K"])
    bits, kern = run(tg, p)
    f64, rbits = oracle.gemm(p["dt"], p["A"], p["B"])
    err = util.check_tol(p["dt"], bits, f64, name, ref_bits=rbits)
    say("  kernel", kern, "max abs err", err)


@pytest.mark.parametrize("name,expect", [("f16_256", "async_64x64x32_s4_splitk2"),
                                         ("f16_1024", "async_64x64x32_s4")])
def test_small_config_automatic_split_k(tg, monkeypatch, name, expect):
    # the same workloads with TG_SPLITK=0: 256^3 (16 tiles of 64 x 64) splits
    # K in two, 1024^3 (256 tiles) fills the chip unsplit; integer inputs
    # bit-exact, random inputs within the tolerance
    monkeypatch.setenv("TG_SPLITK", "0")
    for integer in (True, False):
        p = inputs.config_problem(name, integer=integer)
        say("case", name, "automatic split-K", "integer" if integer else "random")
        bits, kern = run(tg, p)
        assert kern == expect, kern
        f64, rbits = oracle.gemm(p["dt"], p["A"], p["B"])
        if integer:
            util.check_exact(bits, rbits, name + " split-K")
        else:
            util.check_tol(p["dt"], bits, f64, name + " split-K", ref_bits=rbits)


MEDIUM_M_SPLIT_CASES = [
    # (dt, M, N, K, trans_b, splits): grids well short of a wave with a long
    # K split it by default (64 x 64 tiles here, the split count the
    # launch-time model takes)
    (F16, 64, 4096, 4096, False, 4),
    (BF16, 128, 2048, 2048, False, 4),
    (F16, 96, 1000, 3072, False, 6),     # partial last row and column tiles
    (BF16, 64, 2048, 4096, True, None),  # B stored [N,K]
]


@pytest.mark.parametrize("case", MEDIUM_M_SPLIT_CASES, ids=lambda c: "%dx%dx%d%s" % (
    c[1], c[2], c[3], "_bt" if c[4] else ""))
def test_medium_m_default_split_k(tg, case):
    # integer inputs bit-exact; random inputs with bias and GELU within the
    # tolerance, and the same bits on a second call (the partials are added
    # in split order, not in arrival order)
    dt, M, N, K, trans_b, splits = case
    for integer in (True, False):
        kind = "int" if integer else "normal"
        p = inputs.problem(dt, M, N, K, seed=M + N + K + integer, kind=kind, bias=True,
                           act=inputs.ACT_NONE if integer else inputs.ACT_GELU_TANH,
                           bias_kind="int" if integer else "bias",
                           b_scale=1.0 if integer else 1.0 / np.sqrt(K))
        say("case medium-M split-K", dt, M, N, K, "B [N,K]" if trans_b else "B [K,N]", kind)
        bits, kern = run_ex(tg, p, trans_b)
        say("  kernel", kern)
        if splits is None:
            assert "_splitk" in kern, kern
        else:
            assert kern.endswith("_splitk%d" % splits), kern
        f64, rbits = oracle.gemm(dt, p["A"], p["B"], p["bias"], p["act"])
        if integer:
            util.check_exact(bits, rbits, "medium-M split-K integer")
        else:
            util.check_tol(dt, bits, f64, "medium-M split-K", ref_bits=rbits)
            again, _ = run_ex(tg, p, trans_b)
            util.check_exact(again, bits, "medium-M split-K repeat")


@pytest.mark.parametrize("name", ["f16_256", "f16_1024"])
def test_small_config_integer_exact(tg, name):
    p = inputs.config_problem(name, integer=True)
    say("case", name, "integer", p["M"], p["N"], p["K"])
    bits, _ = run(tg, p)
    _, ref = oracle.gemm(p["dt"], p["A"], p["B"])
    util.check_exact(bits, ref, name)


def test_tileLang_tiling_config_runs(tg, monkeypatch):
    # 1024^3 with a 128 x 128 tile (the pages' starting tiling) must agree too
    monkeypatch.setenv("TG_FORCE_CONFIG", "tiled_128x128x64_w2x2")
    p = inputs.config_problem("f16_1024", integer=True)
    bits, kern = run(tg, p)
    assert kern == "tiled_128x128x64_w2x2"
    _, ref = oracle.gemm(p["dt"], p["A"], p["B"])
    util.check_exact(bits, ref, "1024 forced 128x128")


# --------------------------------------------------------------- epilogue

def test_bias_gelu_medium_full(tg):
    p = inputs.problem(F16, 512, 768, 640, seed=31, bias=True, act=inputs.ACT_GELU_TANH,
                       a_scale=0.2, b_scale=0.2)
    say("case bias+gelu 512x768x640")
    bits, _ = run(tg, p)
    f64, rbits = oracle.gemm(F16, p["A"], p["B"], p["bias"], oracle.ACT_GELU_TANH)
    util.check_tol(F16, bits, f64, "bias+gelu", ref_bits=rbits)


def test_gelu_config_full_output(tg):
    # f16 4096^3 + bias + GELU, every one of the 16.8 M outputs against the oracle
    p = inputs.config_problem("f16_4096_gelu")
    say("case f16_4096_gelu full", p["M"], p["N"], p["K"])
    bits, kern = run(tg, p)
    say("  kernel", kern)
    assert kern == "async_256x256x32p_s4_mfma16", kern
    f64, rbits = oracle.gemm(F16, p["A"], p["B"], p["bias"], oracle.ACT_GELU_TANH)
    util.check_tol(F16, bits, f64, "f16_4096_gelu", ref_bits=rbits)


def test_gelu_config_integer_bias_exact_full(tg):
    p = inputs.config_problem("f16_4096_gelu", integer=True)
    assert p["act"] == inputs.ACT_NONE and p["bias"] is not None
    say("case f16_4096 integer + bias, full")
    bits, kern = run(tg, p)
    assert kern == "async_256x256x32p_s4_mfma16", kern
    _, ref = oracle.gemm(F16, p["A"], p["B"], p["bias"])
    util.check_exact(bits, ref, "f16_4096 integer+bias")


# -------------------------------------------------------------------- QKV

def run_qkv(tg, q):
    import torch
    X = util.to_dev(q["X"], q["dt"])
    Ws = [util.to_dev(w, q["dt"]) for w in q["W"]]
    outs = tg.gemm_qkv(X, *Ws)
    torch.cuda.synchronize()
    return X, Ws, [util.to_bits(o) for o in outs]


def test_qkv_medium_full_and_equal_to_three_gemms(tg):
    import torch
    q = inputs.qkv_problem(BF16, 384, 512, 320, seed=41)
    say("case qkv 384x512x320")
    X, Ws, outs = run_qkv(tg, q)
    refs = oracle.gemm_qkv(BF16, q["X"], *q["W"])
    for t in range(3):
        util.check_tol(BF16, outs[t], refs[t][0], "qkv[%d]" % t, ref_bits=refs[t][1])
        single = util.to_bits(tg.gemm(X, Ws[t]))
        torch.cuda.synchronize()
        util.check_exact(outs[t], single, "qkv[%d] vs tg_gemm" % t)


def test_qkv_config_full_output(tg):
    # bf16 X[8192,4096] x three W[4096,4096], all 3 x 33.6 M outputs
    q = inputs.config_problem("bf16_qkv")
    say("case bf16_qkv full", q["M"], q["N"], q["K"])
    _, _, outs = run_qkv(tg, q)
    assert tg.last_kernel() == "async_256x256x32p_s4_mfma16", tg.last_kernel()
    refs = oracle.gemm_qkv(BF16, q["X"], *q["W"])
    for t in range(3):
        util.check_tol(BF16, outs[t], refs[t][0], "qkv config [%d]" % t, ref_bits=refs[t][1])


def test_qkv_config_integer_exact_full(tg):
    q = inputs.config_problem("bf16_qkv", integer=True)
    say("case bf16_qkv integer, full")
    _, _, outs = run_qkv(tg, q)
    refs = oracle.gemm_qkv(BF16, q["X"], *q["W"])
    for t in range(3):
        util.check_exact(outs[t], refs[t][1], "qkv integer [%d]" % t)


# ------------------------------------------------------------------ skinny

def test_skinny_config_full(tg):
    p = inputs.config_problem("bf16_skinny")
    say("case bf16_skinny", p["M"], p["N"], p["K"])
    bits, kern = run(tg, p)
    say("  kernel", kern)
    assert kern.startswith("skinny")
    f64, rbits = oracle.gemm(BF16, p["A"], p["B"])
    util.check_tol(BF16, bits, f64, "skinny", ref_bits=rbits)


def test_skinny_config_integer_exact_and_deterministic(tg):
    p = inputs.config_problem("bf16_skinny", integer=True)
    bits, _ = run(tg, p)
    bits2, _ = run(tg, p)
    _, ref = oracle.gemm(BF16, p["A"], p["B"])
    util.check_exact(bits, ref, "skinny integer")
    util.check_exact(bits2, bits, "skinny repeat")


@pytest.mark.parametrize("integer", [False, True])
def test_skinny_32_rows_full_size(tg, integer):
    # the benchmark's M = 32 line: bf16 32 x 8192 x 8192, every output checked
    p = inputs.problem(BF16, 32, 8192, 8192, seed=5400 + integer, kind="int" if integer else "normal",
                       b_scale=1.0 if integer else 8192 ** -0.5)
    say("case skinny 32x8192x8192", "integer" if integer else "")
    bits, kern = run(tg, p)
    say("  kernel", kern)
    assert kern.startswith("skinny_stream") and kern.endswith("_m32")
    f64, rbits = oracle.gemm(BF16, p["A"], p["B"])
    if integer:
        util.check_exact(bits, rbits, "skinny 32 rows integer")
    else:
        util.check_tol(BF16, bits, f64, "skinny 32 rows", ref_bits=rbits)


SKINNY_COLS_CASES = [
    # (dt, M, N, K): the column-tile small-M kernel (TG_SKINNY_COLS=1): N a
    # multiple of 32 with at least 128 tiles, K of 256; M = 16 and M < 16
    (BF16, 16, 8192, 8192),
    (F16, 5, 4096, 1024),
    (BF16, 1, 6144, 2048),
]


@pytest.mark.parametrize("dt,M,N,K", SKINNY_COLS_CASES)
def test_skinny_cols_kernel(tg, monkeypatch, dt, M, N, K):
    # integer operands with bias and residual: bit-exact; random operands
    # with bias, GELU and residual: within the tolerance
    monkeypatch.setenv("TG_SKINNY_COLS", "1")
    for integer in (True, False):
        p = inputs.problem(dt, M, N, K, seed=800 + M + integer, kind="int" if integer else "normal",
                           b_scale=1.0 if integer else K ** -0.5, bias=True,
                           bias_kind="int" if integer else "bias",
                           act=inputs.ACT_NONE if integer else inputs.ACT_GELU_TANH)
        R = inputs.draw(np.random.default_rng(801 + N), (M, N), "int" if integer else "uniform",
                        dt)
        say("case skinny cols", dt, M, N, K, "integer" if integer else "random")
        bits, kern = run_ex(tg, p, False, R)
        say("  kernel", kern)
        assert kern.startswith("skinny_cols_bn32_split1"), kern
        f64, rbits = oracle.gemm_ex(dt, p["A"], p["B"], bias=p["bias"], act=p["act"], R=R)
        if integer:
            util.check_exact(bits, rbits, "skinny cols integer")
        else:
            util.check_tol(dt, bits, f64, "skinny cols", ref_bits=rbits)


def test_skinny_matches_tiled_on_integers(tg, monkeypatch):
    p = inputs.problem(BF16, 16, 2048, 4096, seed=51, kind="int")
    a, ka = run(tg, p)
    monkeypatch.setenv("TG_FORCE_CONFIG", "tiled_64x64x64_w2x2")
    b, kb = run(tg, p)
    assert ka.startswith("skinny") and kb.startswith("tiled")
    util.check_exact(a, b, "skinny vs tiled")


# Both column widths of the streaming small-M kernel, forced, on shapes with
# one split, a few splits and more than eight (a second combine round), with
# M below 16 (rows past M are clamped on load and never stored).
SKINNY_FORCED = [
    # bn, dt, M, N, K, splits ("" = the planner's choice)
    (128, BF16, 16, 2048, 4096, ""), (128, F16, 7, 1024, 4096, "1"),
    (128, BF16, 16, 4096, 5120, "10"), (128, F16, 1, 384, 1536, ""),
    (256, BF16, 16, 2048, 4096, ""), (256, F16, 9, 1024, 4096, "1"),
    (256, BF16, 16, 2048, 8192, "11"),
    # 16 < M <= 32: two 16-row blocks
    (128, BF16, 32, 2048, 4096, ""), (128, F16, 17, 1024, 4096, "1"),
    (128, BF16, 32, 4096, 5120, "10"), (256, BF16, 24, 2048, 8192, "11"),
    (256, F16, 32, 1024, 4096, "1"),
]


@pytest.mark.parametrize("bn,dt,M,N,K,splits", SKINNY_FORCED)
@pytest.mark.parametrize("integer", [False, True])
def test_skinny_stream_widths(tg, monkeypatch, bn, dt, M, N, K, splits, integer):
    monkeypatch.setenv("TG_SKINNY_BN", str(bn))
    monkeypatch.setenv("TG_SKINNY_SPLITS", splits)
    seed = 5000 + bn + M + N // 128 + K // 512 + (7 if integer else 0)
    p = inputs.problem(dt, M, N, K, seed=seed, kind="int" if integer else "normal",
                       b_scale=1.0 if integer else K ** -0.5)
    say("case skinny bn", bn, "splits", splits or "auto", dt, M, N, K, "integer" if integer else "")
    bits, kern = run(tg, p)
    say("  kernel", kern)
    assert kern.startswith("skinny_stream_bn%d_" % bn)
    assert kern.endswith("_m32") == (M > 16)
    if splits:
        assert ("_split%sx" % splits) in kern
    f64, rbits = oracle.gemm(dt, p["A"], p["B"])
    if integer:
        util.check_exact(bits, rbits, "skinny bn%d integer" % bn)
    else:
        util.check_tol(dt, bits, f64, "skinny bn%d" % bn, ref_bits=rbits)


@pytest.mark.parametrize("bn", [128, 256])
@pytest.mark.parametrize("M", [13, 29])
def test_skinny_stream_epilogue(tg, monkeypatch, bn, M):
    """Bias, GELU_tanh and a residual through the split-K combine."""
    import torch
    monkeypatch.setenv("TG_SKINNY_BN", str(bn))
    dt, N, K = BF16, 2048, 4096
    p = inputs.problem(dt, M, N, K, seed=5200 + bn + M, kind="normal", b_scale=K ** -0.5,
                       bias=True, act=inputs.ACT_GELU_TANH)
    R = inputs.draw(np.random.default_rng(5300 + bn + M), (M, N), "uniform", dt)
    A, B, bias = dev_problem(p)
    Rd = util.to_dev(R, dt)
    C = tg.gemm(A, B, bias=bias, act="gelu_tanh", residual=Rd)
    torch.cuda.synchronize()
    kern = tg.last_kernel()
    say("case skinny epilogue bn", bn, "kernel", kern)
    assert kern.startswith("skinny_stream_bn%d_" % bn) and "_split1x" not in kern
    f64, rbits = oracle.gemm_ex(dt, p["A"], p["B"], bias=p["bias"], act=oracle.ACT_GELU_TANH, R=R)
    util.check_tol(dt, util.to_bits(C), f64, "skinny epilogue bn%d" % bn, ref_bits=rbits)


# ----------------------------------------------------------- 8192^3 square

def test_square_8192_full_output(tg):
    # bf16 8192^3, every one of the 67 M outputs against the oracle
    p = inputs.config_problem("bf16_8192")
    say("case bf16_8192 full", p["M"], p["N"], p["K"])
    bits, kern = run(tg, p)
    say("  kernel", kern)
    assert kern == "async_256x256x32p_s4_mfma16", kern
    f64, rbits = oracle.gemm(BF16, p["A"], p["B"])
    util.check_tol(BF16, bits, f64, "bf16_8192", ref_bits=rbits)


def test_output_past_2_to_the_31_elements(tg):
    # 98304 x 32768 outputs (3.2e9 elements, 6 GiB): element offsets pass
    # 2^31 (and byte offsets 2^32), so any 32-bit index arithmetic in the
    # 256 x 256 kernel would wrap; integer inputs and bias, sampled outputs
    # on both sides of offset 2^31, bit-exact
    import torch
    M, N, K = 98304, 32768, 256
    p = inputs.problem(F16, M, N, K, seed=210, kind="int", bias=True, bias_kind="int")
    say("case large output", M, N, K)
    A, B, bias = dev_problem(p)
    C = torch.empty((M, N), dtype=torch.float16, device="cuda")
    tg.gemm(A, B, out=C, bias=bias)
    torch.cuda.synchronize()
    kern = tg.last_kernel()
    say("  kernel", kern)
    assert kern.startswith("async_256x256")
    ii, jj = util.sample_indices(M, N, 1000, seed=211)
    extra = [(65535, N - 1), (65536, 0), (65536, 1), (M - 1, N - 1), (M - 1, 0), (80000, 12345)]
    ii = np.concatenate([ii, [e[0] for e in extra]]).astype(np.int64)
    jj = np.concatenate([jj, [e[1] for e in extra]]).astype(np.int64)
    got = util.to_bits(C[torch.from_numpy(ii).cuda(), torch.from_numpy(jj).cuda()])
    del C
    _, ref = oracle.gemm_sample(F16, p["A"], p["B"], ii, jj, p["bias"])
    util.check_exact(got, ref, "large output")


def test_small_m_weight_past_2_to_the_31_elements(tg):
    # W of 8192 x 393216 bf16 (3.2e9 elements, 6 GiB) streamed by the small-M
    # kernel: row offsets k * ldb pass 2^31.  W is drawn on the device from a
    # seeded generator (integers in {-2..2}); the oracle gets the same values
    # of 64 sampled columns, including the last ones, and checks every row
    import torch
    M, N, K = 16, 393216, 8192
    say("case small M, large W", M, N, K)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(220)
    W = torch.randint(-2, 3, (K, N), generator=gen, dtype=torch.int8, device="cuda")
    W = W.to(torch.bfloat16)
    x = inputs.problem(BF16, M, 64, K, seed=221, kind="int")["A"]
    X = util.to_dev(x, BF16)
    Y = tg.gemm(X, W)
    torch.cuda.synchronize()
    kern = tg.last_kernel()
    say("  kernel", kern)
    assert kern.startswith("skinny_stream")
    rng = np.random.default_rng(222)
    jj = np.unique(np.concatenate([rng.integers(0, N, 56), [0, 1, N - 256, N - 129, N - 8,
                                                            N - 2, N - 1, 270000]]))
    jt = torch.from_numpy(jj).cuda()
    wsub = util.to_bits(W[:, jt].contiguous())
    got = util.to_bits(Y[:, jt].contiguous())
    del W
    _, ref = oracle.gemm(BF16, x, wsub)
    util.check_exact(got, ref, "small M, large W")


def test_square_8192_integer_exact_full(tg):
    p = inputs.config_problem("bf16_8192", integer=True)
    say("case bf16_8192 integer, full")
    bits, kern = run(tg, p)
    assert kern == "async_256x256x32p_s4_mfma16", kern
    _, ref = oracle.gemm(BF16, p["A"], p["B"])
    util.check_exact(bits, ref, "bf16_8192 integer")


# ------------------------------------------------------- ragged and edges

def padded(bits, ld, dt):
    """Copy a [R, C] bit matrix into a [R, ld] buffer whose padding is NaN."""
    R, C = bits.shape
    buf = np.full((R, ld), NAN_BITS[dt], np.uint16)
    buf[:, :C] = bits
    return buf


def round8(x):
    return max(8, (x + 7) // 8 * 8)


RAGGED = [
    (F16, 1, 1, 1), (F16, 4, 4, 4), (BF16, 129, 257, 31), (F16, 17, 300, 100),
    (BF16, 300, 17, 1000), (F16, 255, 511, 129), (BF16, 64, 64, 64), (F16, 520, 264, 72),
    (BF16, 16, 1000, 777), (F16, 5, 513, 4100), (BF16, 1, 4096, 300), (F16, 33, 2000, 520),
]


@pytest.mark.parametrize("dt,M,N,K", RAGGED)
@pytest.mark.parametrize("integer", [False, True])
def test_ragged_shapes_with_poisoned_padding(tg, dt, M, N, K, integer):
    import torch
    say("case ragged", dt, M, N, K, "integer" if integer else "random")
    p = inputs.problem(dt, M, N, K, seed=M * 7 + N * 3 + K, kind="int" if integer else "uniform",
                       bias=not integer, act=inputs.ACT_NONE if integer else inputs.ACT_GELU_TANH)
    lda, ldb, ldc = round8(K + 3), round8(N + 5), round8(N + 9)
    Abuf = util.to_dev(padded(p["A"], lda, dt), dt)
    Bbuf = util.to_dev(padded(p["B"], ldb, dt), dt)
    # output buffer with two extra canary rows below M
    Cbuf = util.to_dev(np.full((M + 2, ldc), NAN_BITS[dt], np.uint16), dt)
    bias = util.to_dev(p["bias"], dt) if p["bias"] is not None else None
    A, B, C = Abuf[:, :K], Bbuf[:, :N], Cbuf[:M, :N]
    tg.gemm(A, B, out=C, bias=bias, act="none" if integer else "gelu_tanh")
    torch.cuda.synchronize()
    say("  kernel", tg.last_kernel())
    full = util.to_bits(Cbuf)
    f64, ref = oracle.gemm(dt, p["A"], p["B"], p["bias"], p["act"])
    if integer:
        util.check_exact(full[:M, :N], ref, "ragged exact")
    else:
        util.check_tol(dt, full[:M, :N], f64, "ragged", ref_bits=ref)
    assert np.all(full[:M, N:] == NAN_BITS[dt]), "wrote into the pitch padding"
    assert np.all(full[M:, :] == NAN_BITS[dt]), "wrote below the last row"


def test_unaligned_operands_take_the_reported_element_wise_kernel(tg):
    import torch
    dt = F16
    p = inputs.problem(dt, 70, 90, 50, seed=61, bias=True, act=inputs.ACT_GELU_TANH)
    Abuf = util.to_dev(padded(p["A"], 51, dt), dt)  # pitch 51: not a multiple of 8
    A = Abuf[:, :50]
    B = util.to_dev(p["B"], dt)
    bias = util.to_dev(p["bias"], dt)
    C = tg.gemm(A, B, bias=bias, act="gelu_tanh")
    torch.cuda.synchronize()
    assert tg.last_kernel().endswith("_unaligned"), tg.last_kernel()
    f64, rbits = oracle.gemm(dt, p["A"], p["B"], p["bias"], oracle.ACT_GELU_TANH)
    util.check_tol(dt, util.to_bits(C), f64, "unaligned", ref_bits=rbits)
    # B stored [N,K] with an odd pitch stays on the reported scalar fallback
    Bt = util.to_dev(padded(np.ascontiguousarray(p["B"].T), 51, dt), dt)[:, :50]
    C2 = tg.gemm(A, Bt.t(), bias=bias, act="gelu_tanh")
    torch.cuda.synchronize()
    assert tg.last_kernel().startswith("generic_fma (unaligned"), tg.last_kernel()
    util.check_tol(dt, util.to_bits(C2), f64, "generic", ref_bits=rbits)


UNALIGNED_CASES = [
    # (dt, M, N, K, pitch pads of A, B, C, output offset in elements): odd
    # and even pitches off the 8-element grid, an output starting one
    # element into its buffer, every tile size of the chooser, a residual
    # with its own (odd) pitch
    (F16, 255, 257, 129, (1, 3, 5), 0),
    (BF16, 1000, 1000, 1000, (0, 0, 0), 1),
    (F16, 513, 1025, 777, (2, 6, 1), 0),
]


@pytest.mark.parametrize("dt,M,N,K,pads,off", UNALIGNED_CASES)
def test_unaligned_pitches_integer_exact(tg, dt, M, N, K, pads, off):
    # operands and output carved out of padded buffers whose pitches are not
    # multiples of 8 elements, or an output that starts off the 16-byte
    # grid; integer inputs, bias and residual: bit-exact.  Padding holds NaN
    # so a read past the logical bounds shows.
    import torch
    p = inputs.problem(dt, M, N, K, seed=230 + M, kind="int", bias=True, bias_kind="int")
    R = inputs.draw(np.random.default_rng(231 + N), (M, N), "int", dt, 8.0)
    lda, ldb, ldc = K + pads[0], N + pads[1], N + pads[2]
    A = util.to_dev(padded(p["A"], lda, dt), dt)[:, :K]
    B = util.to_dev(padded(p["B"], ldb, dt), dt)[:, :N]
    bias = util.to_dev(p["bias"], dt)
    Cbuf = util.to_dev(np.full(M * ldc + 1, NAN_BITS[dt], np.uint16), dt)
    C = Cbuf[off:off + M * ldc].view(M, ldc)[:, :N]
    Rd = util.to_dev(R, dt)
    say("case unaligned", dt, M, N, K, "pitches", lda, ldb, ldc, "C offset", off)
    tg.gemm(A, B, out=C, bias=bias, residual=Rd)
    torch.cuda.synchronize()
    kern = tg.last_kernel()
    say("  kernel", kern)
    assert kern.endswith("_unaligned"), kern
    _, ref = oracle.gemm_ex(dt, p["A"], p["B"], bias=p["bias"], R=R)
    util.check_exact(util.to_bits(C), ref, "unaligned " + kern)
    # nothing written outside the logical output
    full = util.to_bits(Cbuf)
    inside = np.zeros(full.shape, bool)
    for i in range(M):
        inside[off + i * ldc: off + i * ldc + N] = True
    assert np.all(full[~inside] == NAN_BITS[dt]), "write outside the output"


STAGED_CASES = [
    # (dt, M, N, K, pitch pads of A, B, C, output offset in elements, B
    # stored [N,K], bias offset in elements, residual read from the output):
    # problems of at least 2^30 multiply-adds with operands off the 16-byte
    # grid, staged through aligned, zero-padded copies.  N off the 8 grid and
    # an output one element into its buffer (output staged and copied back;
    # K padded to 264 for the masked 256 x 256 loop); only A off the grid
    # (the kernel writes C itself; K padded to 1152 for 128 x 128 tiles);
    # B stored [N,K] with an odd pitch; a bias 2 bytes past an 8-byte
    # boundary with the residual read from the output itself
    (BF16, 4095, 4095, 263, (0, 0, 0), 1, False, 0, False),
    (F16, 2000, 2056, 1030, (1, 0, 0), 0, False, 0, False),
    (F16, 1536, 1000, 2047, (0, 0, 0), 0, True, 0, False),
    (BF16, 1100, 1003, 1024, (0, 0, 2), 0, False, 1, True),
]


@pytest.mark.parametrize("dt,M,N,K,pads,off,trans_b,boff,inplace", STAGED_CASES)
def test_off_grid_operands_staged_integer_exact(tg, dt, M, N, K, pads, off, trans_b, boff,
                                                inplace):
    # NaN in every pitch padding and around the output: the staged copies
    # must read only the logical operands, the copy back write only the
    # logical output.  Integer inputs, bias and residual: bit-exact.
    import torch
    p = inputs.problem(dt, M, N, K, seed=240 + M, kind="int", bias=True, bias_kind="int")
    R = inputs.draw(np.random.default_rng(241 + N), (M, N), "int", dt, 8.0)
    lda, ldc = K + pads[0], N + pads[2]
    A = util.to_dev(padded(p["A"], lda, dt), dt)[:, :K]
    if trans_b:
        ldb = K + pads[1]
        B = util.to_dev(padded(np.ascontiguousarray(p["B"].T), ldb, dt), dt)[:, :K].t()
    else:
        ldb = N + pads[1]
        B = util.to_dev(padded(p["B"], ldb, dt), dt)[:, :N]
    bbuf = util.to_dev(np.concatenate([np.full(boff, NAN_BITS[dt], np.uint16), p["bias"]]), dt)
    bias = bbuf[boff:]
    Cbuf = util.to_dev(np.full(M * ldc + 1, NAN_BITS[dt], np.uint16), dt)
    C = Cbuf[off:off + M * ldc].view(M, ldc)[:, :N]
    if inplace:
        C.copy_(util.to_dev(R, dt))
        Rd = C
    else:
        Rd = util.to_dev(R, dt)
    say("case staged", dt, M, N, K, "pitches", lda, ldb, ldc, "C offset", off,
        "B[N,K]" if trans_b else "", "bias offset", boff, "in place" if inplace else "")
    tg.gemm(A, B, out=C, bias=bias, residual=Rd)
    torch.cuda.synchronize()
    kern = tg.last_kernel()
    say("  kernel", kern)
    assert kern.endswith("_staged"), kern
    _, ref = oracle.gemm_ex(dt, p["A"], p["B"], bias=p["bias"], R=R)
    util.check_exact(util.to_bits(C), ref, "staged " + kern)
    full = util.to_bits(Cbuf)
    inside = np.zeros(full.shape, bool)
    for i in range(M):
        inside[off + i * ldc: off + i * ldc + N] = True
    assert np.all(full[~inside] == NAN_BITS[dt]), "write outside the output"


def test_off_grid_operands_staged_on_stream_k_integer_exact(tg, monkeypatch):
    # A with an odd pitch on a problem whose 256 x 256 tiles leave a partial
    # wave (9 x 16 tiles; TG_STREAMK=2 takes it although each workgroup gets
    # fewer than 16 K quads): the staged copies feed the stream-K kernel.
    import torch
    monkeypatch.setenv("TG_STREAMK", "2")
    dt, M, N, K = F16, 2049, 4096, 1023
    p = inputs.problem(dt, M, N, K, seed=250, kind="int", bias=True, bias_kind="int")
    R = inputs.draw(np.random.default_rng(251), (M, N), "int", dt, 8.0)
    A = util.to_dev(padded(p["A"], K, dt), dt)
    B = util.to_dev(p["B"], dt)
    bias, Rd = util.to_dev(p["bias"], dt), util.to_dev(R, dt)
    say("case staged stream-K", dt, M, N, K)
    C = tg.gemm(A, B, bias=bias, residual=Rd)
    torch.cuda.synchronize()
    kern = tg.last_kernel()
    say("  kernel", kern)
    assert kern == "async_256x256x32_s4_mfma16_streamk_staged", kern
    _, ref = oracle.gemm_ex(dt, p["A"], p["B"], bias=p["bias"], R=R)
    util.check_exact(util.to_bits(C), ref, "staged stream-K")


REALIGN_CASES = [
    # (dt, M, N, K, pitch pads of A, B, C, W offset, C offset (elements),
    # split count forced or 0, random or integer inputs): small M with W,
    # X or Y off the 16-byte grid, taken by the realigning streaming kernel.
    # An odd vocabulary width at M = 1, 16 and 32 (unsplit, 419 tiles); an
    # odd W pitch with W starting 3 elements into its buffer; every operand
    # odd (X copied, K cut inside a slab); only Y off the grid; three tiles
    # with K split 5 ways (320 deep: a short last chunk); forced split counts
    (BF16, 1, 50257, 4096, (0, 0, 0), 0, 0, 0, "int"),
    (F16, 16, 50257, 4096, (0, 0, 0), 0, 1, 0, "int"),
    (BF16, 32, 50257, 2048, (0, 0, 0), 0, 0, 0, "normal"),
    (BF16, 32, 4099, 1024, (0, 2, 1), 3, 0, 0, "int"),
    (F16, 17, 1000, 1000, (3, 5, 0), 1, 0, 0, "int"),
    (BF16, 16, 4095, 4095, (0, 0, 0), 0, 0, 0, "int"),
    (F16, 5, 4096, 4096, (0, 0, 1), 0, 0, 0, "int"),
    (BF16, 8, 300, 320, (0, 1, 0), 7, 0, 0, "int"),
    (F16, 16, 2001, 2048, (0, 0, 0), 0, 0, 1, "int"),
    (BF16, 24, 2001, 2048, (0, 0, 0), 0, 0, 3, "normal"),
    (F16, 16, 2001, 2112, (0, 0, 0), 5, 0, 7, "int"),
    # 257 to 511 tiles of 120 columns: 64-column tiles (501, the last one
    # 3 columns wide), W 5 elements into its buffer, Y one element in
    (F16, 16, 32003, 1024, (0, 3, 0), 5, 1, 0, "int"),
]


@pytest.mark.parametrize("dt,M,N,K,pads,woff,off,splits,kind", REALIGN_CASES)
def test_small_m_off_grid_realigned(tg, monkeypatch, dt, M, N, K, pads, woff, off, splits, kind):
    # NaN in every pitch padding, before W and around the output: the
    # aligned pieces read past a row's last column feed only columns that
    # are never stored, and rows past K read as zero.  Bias, GELU and a
    # residual with its own odd pitch; bit-exact on integer inputs, within
    # the tolerance on normal ones.
    import torch
    if splits:
        monkeypatch.setenv("TG_SKINNY_SPLITS", str(splits))
    else:
        monkeypatch.delenv("TG_SKINNY_SPLITS", raising=False)
    monkeypatch.delenv("TG_FORCE_CONFIG", raising=False)
    act = oracle.ACT_GELU_TANH if kind == "normal" else oracle.ACT_NONE
    p = inputs.problem(dt, M, N, K, seed=260 + M + N, kind=kind, bias=True,
                       bias_kind="int" if kind == "int" else "bias")
    R = inputs.draw(np.random.default_rng(261 + N), (M, N), "int", dt, 8.0)
    lda, ldb, ldc = K + pads[0], N + pads[1], N + pads[2]
    A = util.to_dev(padded(p["A"], lda, dt), dt)[:, :K]
    wflat = np.concatenate([np.full(woff, NAN_BITS[dt], np.uint16),
                            padded(p["B"], ldb, dt).reshape(-1)])
    B = util.to_dev(wflat, dt)[woff:].view(K, ldb)[:, :N]
    bias = util.to_dev(p["bias"], dt)
    Rd = util.to_dev(padded(R, N + 3, dt), dt)[:, :N]
    Cbuf = util.to_dev(np.full(M * ldc + 1, NAN_BITS[dt], np.uint16), dt)
    C = Cbuf[off:off + M * ldc].view(M, ldc)[:, :N]
    say("case realign", dt, M, N, K, "pitches", lda, ldb, ldc, "W offset", woff, "C offset", off,
        "splits", splits or "planned", kind)
    tg.gemm(A, B, out=C, bias=bias, act="gelu_tanh" if act else "none", residual=Rd)
    torch.cuda.synchronize()
    kern = tg.last_kernel()
    say("  kernel", kern)
    assert kern.startswith("skinny_realign_bn"), kern
    if N == 32003:
        assert kern.startswith("skinny_realign_bn64_"), kern
    if splits:  # the planner keeps a forced count within the K chunks
        assert ("_split1x" in kern) == (splits == 1), kern
    assert ("_m32" in kern) == (M > 16), kern
    assert ("_xstaged" in kern) == (lda % 8 != 0 or K % 64 != 0), kern
    f64, ref = oracle.gemm_ex(dt, p["A"], p["B"], bias=p["bias"], act=act, R=R)
    got = util.to_bits(C)
    if kind == "int":
        util.check_exact(got, ref, "realign " + kern)
    else:
        util.check_tol(dt, got, f64, "realign " + kern, ref_bits=ref)
    full = util.to_bits(Cbuf)
    inside = np.zeros(full.shape, bool)
    for i in range(M):
        inside[off + i * ldc: off + i * ldc + N] = True
    assert np.all(full[~inside] == NAN_BITS[dt]), "write outside the output"


NK_CASES = [
    # (dt, M, N, K, pitch pads of A, B (rows of the [N,K] store), C, split
    # count forced or 0, random or integer inputs): small M with B stored
    # [N,K], 16-byte aligned rows, whole rows staged through LDS.
    # M = 1, 16, 32 at 8192 and an odd vocabulary width; K cut inside a
    # 16-byte piece (1001, 777: the last piece masked) with X copied or read
    # in place; Y with an odd pitch; forced split counts
    (BF16, 1, 8192, 8192, (0, 0, 0), 0, "int"),
    (F16, 16, 50257, 4096, (0, 0, 0), 0, "int"),
    (BF16, 32, 4096, 4096, (0, 0, 3), 0, "normal"),
    (F16, 17, 1000, 1001, (0, 7, 0), 0, "int"),
    (BF16, 5, 300, 777, (7, 7, 1), 0, "int"),
    (F16, 16, 2048, 2048, (0, 0, 0), 1, "int"),
    (BF16, 24, 2000, 3000, (8, 8, 0), 3, "normal"),
]


@pytest.mark.parametrize("dt,M,N,K,pads,splits,kind", NK_CASES)
def test_small_m_b_stored_nk(tg, monkeypatch, dt, M, N, K, pads, splits, kind):
    # NaN in every pitch padding and around the output; bias, GELU and a
    # residual with an odd pitch; bit-exact on integer inputs, within the
    # tolerance on normal ones
    import torch
    if splits:
        monkeypatch.setenv("TG_SKINNY_SPLITS", str(splits))
    else:
        monkeypatch.delenv("TG_SKINNY_SPLITS", raising=False)
    monkeypatch.delenv("TG_FORCE_CONFIG", raising=False)
    act = oracle.ACT_GELU_TANH if kind == "normal" else oracle.ACT_NONE
    p = inputs.problem(dt, M, N, K, seed=280 + M + N, kind=kind, bias=True,
                       bias_kind="int" if kind == "int" else "bias",
                       b_scale=1.0 if kind == "int" else K ** -0.5)
    R = inputs.draw(np.random.default_rng(281 + N), (M, N), "int", dt, 8.0)
    lda, ldb, ldc = K + pads[0], K + pads[1], N + pads[2]
    A = util.to_dev(padded(p["A"], lda, dt), dt)[:, :K]
    B = util.to_dev(padded(np.ascontiguousarray(p["B"].T), ldb, dt), dt)[:, :K].t()
    bias = util.to_dev(p["bias"], dt)
    Rd = util.to_dev(padded(R, N + 3, dt), dt)[:, :N]
    Cbuf = util.to_dev(np.full((M, ldc), NAN_BITS[dt], np.uint16), dt)
    C = Cbuf[:, :N]
    say("case B[N,K] small M", dt, M, N, K, "pitches", lda, ldb, ldc, "splits",
        splits or "planned", kind)
    tg.gemm(A, B, out=C, bias=bias, act="gelu_tanh" if act else "none", residual=Rd)
    torch.cuda.synchronize()
    kern = tg.last_kernel()
    say("  kernel", kern)
    assert kern.startswith("skinny_nk_bn128_split"), kern
    if splits:
        assert ("_split1x" in kern) == (splits == 1), kern
    assert ("_m32" in kern) == (M > 16), kern
    assert ("_xstaged" in kern) == (lda % 8 != 0 or K % 64 != 0), kern
    f64, ref = oracle.gemm_ex(dt, p["A"], p["B"], bias=p["bias"], act=act, R=R)
    got = util.to_bits(C)
    if kind == "int":
        util.check_exact(got, ref, "B[N,K] small M " + kern)
    else:
        util.check_tol(dt, got, f64, "B[N,K] small M " + kern, ref_bits=ref)
    assert np.all(util.to_bits(Cbuf)[:, N:] == NAN_BITS[dt]), "wrote into the pitch padding"


def test_realigned_kernel_forced_on_aligned_operands_matches_streaming(tg, monkeypatch):
    # TG_FORCE_CONFIG=skinny_realign runs the realigning kernel on aligned
    # operands too (every row offset 0); integer inputs: the same bits as
    # the streaming kernel and the oracle
    import torch
    dt, M, N, K = BF16, 16, 4096, 2048
    p = inputs.problem(dt, M, N, K, seed=270, kind="int", bias=True, bias_kind="int")
    A, B, bias = util.to_dev(p["A"], dt), util.to_dev(p["B"], dt), util.to_dev(p["bias"], dt)
    monkeypatch.delenv("TG_FORCE_CONFIG", raising=False)
    C1 = tg.gemm(A, B, bias=bias)
    torch.cuda.synchronize()
    k1 = tg.last_kernel()
    monkeypatch.setenv("TG_FORCE_CONFIG", "skinny_realign")
    C2 = tg.gemm(A, B, bias=bias)
    torch.cuda.synchronize()
    k2 = tg.last_kernel()
    say("  kernels", k1, "|", k2)
    assert k1.startswith("skinny_stream") and k2.startswith("skinny_realign"), (k1, k2)
    _, ref = oracle.gemm(dt, p["A"], p["B"], p["bias"])
    util.check_exact(util.to_bits(C1), ref, "streaming")
    util.check_exact(util.to_bits(C2), ref, "realign forced")


PARTIAL64_CASES = [
    # (dt, M, N, K, B stored [N,K]): M (and N) off the 64 grid with more than
    # an eighth of the last tile idle, taken by the 64-row tiles on either B
    # layout: one row tile under 64 rows, 100 and 200 rows, N under one tile
    (BF16, 48, 4096, 1024, False),
    (F16, 48, 4096, 1024, True),
    (F16, 100, 1000, 512, True),
    (BF16, 200, 264, 384, False),
    (F16, 33, 56, 256, True),
    (BF16, 1000, 200, 256, True),
]


@pytest.mark.parametrize("dt,M,N,K,trans_b", PARTIAL64_CASES)
def test_partial_64_tiles_integer_exact(tg, monkeypatch, dt, M, N, K, trans_b):
    # NaN in the pitch padding of every operand and around the output: the
    # clamped copies of a partial tile read only inside the operands and the
    # stores stop at M and N.  Integer inputs, bias and residual: bit-exact.
    import torch
    monkeypatch.delenv("TG_FORCE_CONFIG", raising=False)
    p = inputs.problem(dt, M, N, K, seed=290 + M + N, kind="int", bias=True, bias_kind="int")
    R = inputs.draw(np.random.default_rng(291 + M), (M, N), "int", dt, 8.0)
    A = util.to_dev(padded(p["A"], K + 8, dt), dt)[:, :K]
    if trans_b:
        B = util.to_dev(padded(np.ascontiguousarray(p["B"].T), K + 8, dt), dt)[:, :K].t()
    else:
        B = util.to_dev(padded(p["B"], N + 8, dt), dt)[:, :N]
    bias, Rd = util.to_dev(p["bias"], dt), util.to_dev(R, dt)
    Cbuf = util.to_dev(np.full((M + 2, N + 8), NAN_BITS[dt], np.uint16), dt)
    say("case partial 64 tiles", dt, M, N, K, "B[N,K]" if trans_b else "B[K,N]")
    tg.gemm(A, B, out=Cbuf[:M, :N], bias=bias, residual=Rd)
    torch.cuda.synchronize()
    kern = tg.last_kernel()
    say("  kernel", kern)
    assert kern.startswith("async_64x"), kern
    _, ref = oracle.gemm_ex(dt, p["A"], p["B"], bias=p["bias"], R=R)
    full = util.to_bits(Cbuf)
    util.check_exact(full[:M, :N], ref, "partial 64 tiles " + kern)
    assert np.all(full[:M, N:] == NAN_BITS[dt]) and np.all(full[M:] == NAN_BITS[dt]), \
        "write outside the output"


def test_k_zero_gives_activated_bias(tg):
    import torch
    dt = BF16
    bias_bits = inputs.draw(np.random.default_rng(3), (40,), "bias", dt)
    bias = util.to_dev(bias_bits, dt)
    A = torch.empty((24, 0), dtype=torch.bfloat16, device="cuda")
    B = torch.empty((0, 40), dtype=torch.bfloat16, device="cuda")
    C = tg.gemm(A, B, bias=bias, act="gelu_tanh")
    torch.cuda.synchronize()
    f64, rbits = oracle.gemm(dt, np.zeros((24, 0), np.uint16), np.zeros((0, 40), np.uint16),
                         bias_bits, oracle.ACT_GELU_TANH)
    util.check_tol(dt, util.to_bits(C), f64, "K=0", ref_bits=rbits)


# ------------------------------------------------- async tile configurations

ASYNC_CONFIGS = ["async_256x256x32_s4_mfma16_w8", "async_256x256x32_s4_mfma16",
                 "async_128x128x32_s4_mfma16", "async_128x128x64_s4_mfma16",
                 "async_256x256x32_s4", "async_128x128x32_s4", "async_64x128x32_s4",
                 "async_64x64x32_s4"]


@pytest.mark.parametrize("cfg", ASYNC_CONFIGS)
@pytest.mark.parametrize("dt", [F16, BF16])
def test_async_config_integer_bias_exact(tg, monkeypatch, cfg, dt):
    # 512 x 768 x 384: several tiles in both directions for every tile size,
    # a K loop of 12 steps (three trips round the four stages), integer bias
    monkeypatch.setenv("TG_FORCE_CONFIG", cfg)
    p = inputs.problem(dt, 512, 768, 384, seed=61 + dt, kind="int", bias=True,
                       bias_kind="int")
    say("case", cfg, "dt", dt, "integer + bias 512x768x384")
    bits, kern = run(tg, p)
    assert kern == cfg
    _, ref = oracle.gemm(dt, p["A"], p["B"], p["bias"])
    util.check_exact(bits, ref, cfg)


@pytest.mark.parametrize("cfg", ASYNC_CONFIGS)
def test_async_config_bias_gelu_random(tg, monkeypatch, cfg):
    monkeypatch.setenv("TG_FORCE_CONFIG", cfg)
    p = inputs.problem(F16, 256, 512, 640, seed=71, bias=True, act=inputs.ACT_GELU_TANH,
                       a_scale=0.2, b_scale=0.2)
    say("case", cfg, "bias+gelu 256x512x640")
    bits, kern = run(tg, p)
    assert kern == cfg
    f64, rbits = oracle.gemm(F16, p["A"], p["B"], p["bias"], oracle.ACT_GELU_TANH)
    util.check_tol(F16, bits, f64, cfg, ref_bits=rbits)


@pytest.mark.parametrize("dt", [F16, BF16])
def test_192_tiles_integer_bias_exact(tg, monkeypatch, dt):
    # 576 x 768 x 384: 3 x 4 tiles of 192 x 192 (384-byte B rows with their
    # own swizzle, 96 x 96 wave tiles, 192-byte epilogue rows), 12 K steps
    monkeypatch.setenv("TG_FORCE_CONFIG", "async_192x192x32_s4_mfma16")
    p = inputs.problem(dt, 576, 768, 384, seed=63 + dt, kind="int", bias=True,
                       bias_kind="int")
    say("case 192 x 192 tiles dt", dt, "integer + bias 576x768x384")
    bits, kern = run(tg, p)
    assert kern == "async_192x192x32_s4_mfma16", kern
    _, ref = oracle.gemm(dt, p["A"], p["B"], p["bias"])
    util.check_exact(bits, ref, kern)


def test_192_tiles_bias_gelu_random(tg, monkeypatch):
    monkeypatch.setenv("TG_FORCE_CONFIG", "async_192x192x32_s4_mfma16")
    p = inputs.problem(F16, 384, 576, 640, seed=73, bias=True, act=inputs.ACT_GELU_TANH,
                       a_scale=0.2, b_scale=0.2)
    say("case 192 x 192 tiles bias+gelu 384x576x640")
    bits, kern = run(tg, p)
    assert kern == "async_192x192x32_s4_mfma16", kern
    f64, rbits = oracle.gemm(F16, p["A"], p["B"], p["bias"], oracle.ACT_GELU_TANH)
    util.check_tol(F16, bits, f64, kern, ref_bits=rbits)


def test_192_tiles_chosen_for_3072_outputs(tg):
    # 3072 x 3072 outputs: 144 tiles of 256 x 256 (a partial wave, too short
    # a K share per workgroup for stream-K) but 256 of 192 x 192; every output
    # compared with the oracle
    import torch
    dt = BF16
    p = inputs.problem(dt, 3072, 3072, 1024, seed=74, kind="int", bias=True, bias_kind="int")
    say("case 192 x 192 tiles chosen, 3072x3072x1024")
    bits, kern = run(tg, p)
    assert kern == "async_192x192x32_s4_mfma16", kern
    _, ref = oracle.gemm(dt, p["A"], p["B"], p["bias"])
    util.check_exact(bits, ref, kern)


def test_async_small_tile_qkv(tg, monkeypatch):
    # N = 384 is a multiple of 128 but not of 256: the 128 x 128 tiles serve it
    q = inputs.qkv_problem(BF16, 256, 384, 256, seed=81, kind="int")
    say("case qkv 256x384x256 small tiles")
    monkeypatch.setenv("TG_FORCE_CONFIG", "async_128x128x32_s4")
    _, _, outs = run_qkv(tg, q)
    assert tg.last_kernel() == "async_128x128x32_s4"
    for t in range(3):
        _, ref = oracle.gemm(BF16, q["X"], q["W"][t])
        util.check_exact(outs[t], ref, "qkv small tiles [%d]" % t)


# ------------------------------------------- split-K for under-filled grids

SPLIT_CASES = [
    # (dt, M, N, K, config, splits): 24 and 6 tiles of 128 x 128, 6 and 2 tiles
    # of 64 x 128; 8 splits of 128, 4 of 256, 2 of 512, 3 of 128
    (F16, 512, 768, 1024, "async_128x128x32_s4", 8),
    (BF16, 512, 768, 1024, "async_128x128x32_s4", 4),
    (F16, 256, 384, 1024, "async_128x128x32_s4", 2),
    (BF16, 192, 256, 512, "async_64x128x32_s4", 4),
    (F16, 128, 128, 384, "async_64x128x32_s4", 3),
    (BF16, 192, 320, 1024, "async_64x64x32_s4", 8),
    (F16, 1000, 384, 1024, "async_128x128x32_s4", 4),   # partial last row tile
    # the 16x16x32 128 x 128 tiles: 64-deep steps in 4 splits of 512 k and
    # (partial last row tile) 2 of 512; 32-deep steps in 3 splits of 512
    (F16, 512, 768, 2048, "async_128x128x64_s4_mfma16", 4),
    (BF16, 1000, 384, 1024, "async_128x128x64_s4_mfma16", 2),
    (BF16, 384, 512, 1536, "async_128x128x32_s4_mfma16", 3),
]


def forced_split(monkeypatch, cfg, splits):
    monkeypatch.setenv("TG_FORCE_CONFIG", cfg)
    monkeypatch.setenv("TG_SPLITK", str(splits))
    return "%s_splitk%d" % (cfg, splits)


@pytest.mark.parametrize("trans_b", [False, True])
@pytest.mark.parametrize("dt,M,N,K,cfg,splits", SPLIT_CASES)
def test_split_k_integer_exact(tg, monkeypatch, dt, M, N, K, cfg, splits, trans_b):
    # integer operands, bias and residual: every FP32 partial sum is exact, so
    # the ordered sum of the splits must reproduce the oracle's bits
    name = forced_split(monkeypatch, cfg, splits)
    p = inputs.problem(dt, M, N, K, seed=140 + splits + M, kind="int", bias=True,
                       bias_kind="int")
    R = inputs.draw(np.random.default_rng(141 + N), (M, N), "int", dt, 8.0)
    say("case split-K integer", dt, M, N, K, name, "B[N,K]" if trans_b else "B[K,N]")
    bits, kern = run_ex(tg, p, trans_b, R)
    assert kern == name
    _, ref = oracle.gemm_ex(dt, p["A"], np.ascontiguousarray(p["B"].T) if trans_b else p["B"],
                            trans_b=trans_b, bias=p["bias"], R=R)
    util.check_exact(bits, ref, name)


@pytest.mark.parametrize("dt,M,N,K,cfg,splits", SPLIT_CASES[:4] + SPLIT_CASES[-3:])
def test_split_k_bias_gelu_random_and_repeatable(tg, monkeypatch, dt, M, N, K, cfg, splits):
    # random operands: within the tolerance, and the same bits on every call
    # (the splits are added in split order whatever order they finish in)
    name = forced_split(monkeypatch, cfg, splits)
    p = inputs.problem(dt, M, N, K, seed=150 + splits, bias=True, act=inputs.ACT_GELU_TANH,
                       a_scale=0.2, b_scale=0.2)
    say("case split-K gelu", dt, M, N, K, name)
    bits, kern = run(tg, p)
    assert kern == name
    f64, rbits = oracle.gemm(dt, p["A"], p["B"], p["bias"], oracle.ACT_GELU_TANH)
    util.check_tol(dt, bits, f64, name, ref_bits=rbits)
    for _ in range(3):
        again, _ = run(tg, p)
        assert np.array_equal(again, bits), "split-K result changed between calls"


def test_split_k_qkv_and_more_than_one_wave(tg, monkeypatch):
    # three outputs in one launch (18 tiles x 4 splits), then 256 tiles x 2
    # splits = 512 workgroups, then the first shape again: the tile counters
    # must come back to zero after every launch
    name = forced_split(monkeypatch, "async_128x128x32_s4", 4)
    q = inputs.qkv_problem(BF16, 256, 384, 512, seed=161, kind="int")
    say("case split-K qkv 256x384x512 x3")
    _, _, outs = run_qkv(tg, q)
    assert tg.last_kernel() == name
    for t in range(3):
        _, ref = oracle.gemm(BF16, q["X"], q["W"][t])
        util.check_exact(outs[t], ref, "split-K qkv [%d]" % t)
    monkeypatch.setenv("TG_SPLITK", "2")
    p = inputs.problem(F16, 2048, 2048, 256, seed=162, kind="int")
    say("case split-K 2048x2048x256, 512 workgroups")
    bits, kern = run(tg, p)
    assert kern == "async_128x128x32_s4_splitk2"
    _, ref = oracle.gemm(F16, p["A"], p["B"])
    util.check_exact(bits, ref, kern)
    monkeypatch.setenv("TG_SPLITK", "4")
    _, _, outs = run_qkv(tg, q)
    for t in range(3):
        _, ref = oracle.gemm(BF16, q["X"], q["W"][t])
        util.check_exact(outs[t], ref, "split-K qkv again [%d]" % t)


def test_split_k_qkv_on_16x16x32_tiles(tg, monkeypatch):
    # three outputs of the 16x16x32 128 x 128 tiles in one split launch:
    # forced (64-deep steps, 2 x 3 x 3 tiles x 4 splits), then the default
    # dispatch of a small-M QKV with long K, which the launch-time model
    # splits; integer operands, bit-exact
    name = forced_split(monkeypatch, "async_128x128x64_s4_mfma16", 4)
    q = inputs.qkv_problem(BF16, 256, 384, 1024, seed=163, kind="int")
    say("case split-K qkv on 64-deep 128 x 128 tiles 256x384x1024 x3")
    _, _, outs = run_qkv(tg, q)
    assert tg.last_kernel() == name, tg.last_kernel()
    for t in range(3):
        _, ref = oracle.gemm(BF16, q["X"], q["W"][t])
        util.check_exact(outs[t], ref, "16x16x32 split-K qkv [%d]" % t)
    monkeypatch.delenv("TG_FORCE_CONFIG")
    monkeypatch.delenv("TG_SPLITK")
    q = inputs.qkv_problem(F16, 128, 1024, 4096, seed=164, kind="int")
    say("case default qkv 128x1024x4096 x3")
    _, _, outs = run_qkv(tg, q)
    kern = tg.last_kernel()
    say("  kernel", kern)
    assert "_splitk" in kern, kern
    for t in range(3):
        _, ref = oracle.gemm(F16, q["X"], q["W"][t])
        util.check_exact(outs[t], ref, "default split qkv [%d]" % t)


def test_split_paths_replay_in_graphs(tg, monkeypatch):
    # both split-K paths keep per-tile counters that each launch leaves at
    # zero, so a captured call replays correctly with no reset; eager calls
    # between the replays share the same counters and workspace
    import torch
    cases = [
        (F16, 256, 320, 1024, {"TG_FORCE_CONFIG": "async_64x64x32_s4", "TG_SPLITK": "4"},
         "async_64x64x32_s4_splitk4"),
        (BF16, 16, 4096, 4096, {}, "skinny_stream"),
    ]
    for dt, M, N, K, env, kern in cases:
        for k, v in env.items():
            monkeypatch.setenv(k, v)
        p = inputs.problem(dt, M, N, K, seed=200 + M, kind="int", bias=True, bias_kind="int")
        A, B, bias = dev_problem(p)
        C = torch.empty((M, N), dtype=torch.float16 if dt == F16 else torch.bfloat16,
                        device="cuda")
        tg.gemm(A, B, out=C, bias=bias)  # allocates the workspace outside the capture
        torch.cuda.synchronize()
        assert tg.last_kernel().startswith(kern), tg.last_kernel()
        _, ref = oracle.gemm(dt, p["A"], p["B"], p["bias"])
        util.check_exact(util.to_bits(C), ref, kern + " eager")
        say("case graph replay", kern, M, N, K)
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g):
                tg.gemm(A, B, out=C, bias=bias)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for i in range(4):
            C.zero_()
            g.replay()
            torch.cuda.synchronize()
            util.check_exact(util.to_bits(C), ref, "%s replay %d" % (kern, i))
            tg.gemm(A, B, out=C, bias=bias)
            torch.cuda.synchronize()
            util.check_exact(util.to_bits(C), ref, "%s eager after replay %d" % (kern, i))
        for k in env:
            monkeypatch.delenv(k)


def test_split_k_off_and_unsplittable_k(tg, monkeypatch):
    # TG_SPLITK=1 keeps the forced tile unsplit; a K that no split count
    # divides into multiples of 128 (K = 128) runs unsplit too
    import torch
    monkeypatch.setenv("TG_FORCE_CONFIG", "async_64x128x32_s4")
    monkeypatch.setenv("TG_SPLITK", "1")
    a = torch.zeros((256, 256), dtype=torch.float16, device="cuda")
    tg.gemm(a, a)
    assert tg.last_kernel() == "async_64x128x32_s4"
    monkeypatch.setenv("TG_SPLITK", "4")
    b = torch.zeros((256, 128), dtype=torch.float16, device="cuda")
    tg.gemm(b, torch.zeros((128, 256), dtype=torch.float16, device="cuda"))
    assert tg.last_kernel() == "async_64x128x32_s4"
    torch.cuda.synchronize()


# ---------------- partial last row tile on the 256 x 256 (16x16x32) kernels

RAGGED_M_CASES = [
    # (dt, M, N, K, config): on the 16x16x32 kernels the last row tile holds
    # 1, 131, 184 and 255 rows (at most M/8 padding rows), both wave rows
    # partly or wholly outside
    (F16, 2049, 512, 256, "async_256x256x32_s4_mfma16"),
    (BF16, 1923, 768, 384, "async_256x256x32_s4_mfma16"),
    (F16, 3000, 512, 512, "async_256x256x32_s4_mfma16"),
    (BF16, 2303, 256, 256, "async_256x256x32_s4_mfma16_w8"),
    # 192 x 192 tiles: a last row tile of 140 rows (the second wave row
    # holds 44)
    (F16, 1100, 384, 256, "async_192x192x32_s4_mfma16"),
    # 128 x 128 tiles: a last row tile of 76 rows (the second wave row holds
    # 12)
    (BF16, 1100, 384, 256, "async_128x128x32_s4_mfma16"),
    (F16, 1100, 384, 512, "async_128x128x64_s4_mfma16"),
    # the 32x32x16 kernel: last row tiles of 152, 104, 24 and 30 rows
    (BF16, 2200, 256, 256, "async_256x256x32_s4"),
    (F16, 1000, 384, 256, "async_128x128x32_s4"),
    (BF16, 600, 256, 384, "async_64x128x32_s4"),
    (F16, 350, 320, 256, "async_64x64x32_s4"),
]


@pytest.mark.parametrize("trans_b", [False, True])
@pytest.mark.parametrize("dt,M,N,K,cfg", RAGGED_M_CASES)
def test_partial_row_tile_integer_exact(tg, monkeypatch, dt, M, N, K, cfg, trans_b):
    # integer operands, bias and residual: bit-exact; the output sits in a
    # buffer with 8 extra rows of NaN that must stay untouched
    import torch
    monkeypatch.setenv("TG_FORCE_CONFIG", cfg)
    p = inputs.problem(dt, M, N, K, seed=240 + M, kind="int", bias=True, bias_kind="int")
    R = inputs.draw(np.random.default_rng(241 + N), (M, N), "int", dt, 8.0)
    A = util.to_dev(p["A"], dt)
    Bd = util.to_dev(np.ascontiguousarray(p["B"].T) if trans_b else p["B"], dt)
    b = Bd.t() if trans_b else Bd
    bias = util.to_dev(p["bias"], dt)
    Cbuf = util.to_dev(np.full((M + 8, N), NAN_BITS[dt], np.uint16), dt)
    C = Cbuf[:M]
    say("case partial row tile", dt, M, N, K, cfg, "B[N,K]" if trans_b else "B[K,N]")
    tg.gemm(A, b, out=C, bias=bias, residual=util.to_dev(R, dt))
    torch.cuda.synchronize()
    assert tg.last_kernel() == cfg, tg.last_kernel()
    _, ref = oracle.gemm_ex(dt, p["A"], np.ascontiguousarray(p["B"].T) if trans_b else p["B"],
                            trans_b=trans_b, bias=p["bias"], R=R)
    full = util.to_bits(Cbuf)
    util.check_exact(full[:M], ref, "partial row tile")
    assert np.all(full[M:] == NAN_BITS[dt]), "rows past M were written"


RAGGED_N_CASES = [
    # (dt, M, N, K, config): N a multiple of 8 leaving a partial last column
    # tile of at most N/8 padding columns; the last case is ragged in M too
    (F16, 512, 2000, 256, "async_256x256x32_s4_mfma16"),
    (BF16, 384, 1096, 256, "async_192x192x32_s4_mfma16"),
    (F16, 256, 1000, 256, "async_128x128x32_s4_mfma16"),
    (BF16, 384, 1000, 512, "async_128x128x64_s4_mfma16"),
    (BF16, 256, 2200, 384, "async_256x256x32_s4"),
    (F16, 256, 1000, 256, "async_128x128x32_s4"),
    (BF16, 192, 600, 512, "async_64x128x32_s4"),
    (F16, 128, 360, 256, "async_64x64x32_s4"),
    (BF16, 1000, 1000, 256, "async_128x128x32_s4"),
]


@pytest.mark.parametrize("trans_b", [False, True])
@pytest.mark.parametrize("dt,M,N,K,cfg", RAGGED_N_CASES)
def test_partial_column_tile_integer_exact(tg, monkeypatch, dt, M, N, K, cfg, trans_b):
    # integer operands, bias and residual: bit-exact; the output's rows carry
    # 8 extra columns of NaN that must stay untouched
    import torch
    monkeypatch.setenv("TG_FORCE_CONFIG", cfg)
    p = inputs.problem(dt, M, N, K, seed=260 + N, kind="int", bias=True, bias_kind="int")
    R = inputs.draw(np.random.default_rng(261 + M), (M, N), "int", dt, 8.0)
    A = util.to_dev(p["A"], dt)
    Bd = util.to_dev(np.ascontiguousarray(p["B"].T) if trans_b else p["B"], dt)
    b = Bd.t() if trans_b else Bd
    bias = util.to_dev(p["bias"], dt)
    Cbuf = util.to_dev(np.full((M, N + 8), NAN_BITS[dt], np.uint16), dt)
    C = Cbuf[:, :N]
    say("case partial column tile", dt, M, N, K, cfg, "B[N,K]" if trans_b else "B[K,N]")
    tg.gemm(A, b, out=C, bias=bias, residual=util.to_dev(R, dt))
    torch.cuda.synchronize()
    assert tg.last_kernel() == cfg, tg.last_kernel()
    _, ref = oracle.gemm_ex(dt, p["A"], np.ascontiguousarray(p["B"].T) if trans_b else p["B"],
                            trans_b=trans_b, bias=p["bias"], R=R)
    full = util.to_bits(Cbuf)
    util.check_exact(full[:, :N], ref, "partial column tile")
    assert np.all(full[:, N:] == NAN_BITS[dt]), "columns past N were written"


def test_partial_column_tile_split_k_and_qkv(tg, monkeypatch):
    import torch
    monkeypatch.setenv("TG_FORCE_CONFIG", "async_128x128x32_s4")
    monkeypatch.setenv("TG_SPLITK", "2")
    p = inputs.problem(BF16, 256, 1000, 1024, seed=270, kind="int", bias=True, bias_kind="int")
    say("case partial column tile split-K 256x1000x1024")
    bits, kern = run(tg, p)
    assert kern == "async_128x128x32_s4_splitk2", kern
    _, ref = oracle.gemm(BF16, p["A"], p["B"], p["bias"])
    util.check_exact(bits, ref, "partial column tile split-K")
    monkeypatch.delenv("TG_SPLITK")
    q = inputs.qkv_problem(BF16, 512, 1000, 256, seed=271, kind="int")
    say("case partial column tile qkv 512x1000x256 x3")
    _, _, outs = run_qkv(tg, q)
    assert tg.last_kernel() == "async_128x128x32_s4"
    for t in range(3):
        _, ref = oracle.gemm(BF16, q["X"], q["W"][t])
        util.check_exact(outs[t], ref, "partial column tile qkv [%d]" % t)


KMASK_CASES = [
    # (dt, M, N, K, forced configuration or None): K a multiple of 8 off the
    # 128 grid on the 256 x 256 16x16x32 tiles (chosen with a full wave of
    # them, or forced): the whole 128-deep quads on the unmasked loop, then
    # the last quad with the k past K read as zeros; K below one quad (72)
    # runs the masked quad alone
    (F16, 4000, 4000, 1000, None),
    (BF16, 4096, 3840, 2000, None),
    (BF16, 512, 512, 200, "async_256x256x32_s4_mfma16"),
    (F16, 512, 512, 72, "async_256x256x32_s4_mfma16"),
    (BF16, 768, 512, 4040, "async_256x256x32_s4_mfma16"),
    (F16, 576, 576, 200, "async_192x192x32_s4_mfma16"),
    (BF16, 384, 384, 200, "async_128x128x32_s4_mfma16"),
    # 64-deep steps: K below one quad of 256 (the masked quad alone), and
    # two whole quads plus a masked one
    (F16, 384, 384, 200, "async_128x128x64_s4_mfma16"),
    (BF16, 256, 512, 1000, "async_128x128x64_s4_mfma16"),
]


@pytest.mark.parametrize("trans_b", [False, True])
@pytest.mark.parametrize("dt,M,N,K,force", KMASK_CASES)
def test_k_off_the_loop_grid_integer_exact(tg, monkeypatch, dt, M, N, K, force, trans_b):
    # A and B sit in buffers whose pitch padding holds NaN: the kernels must
    # read only k < K.  Integer operands, bias and residual: bit-exact.
    import torch
    if force:
        monkeypatch.setenv("TG_FORCE_CONFIG", force)
    p = inputs.problem(dt, M, N, K, seed=280 + K, kind="int", bias=True, bias_kind="int")
    R = inputs.draw(np.random.default_rng(281 + M), (M, N), "int", dt, 8.0)
    A = util.to_dev(padded(p["A"], K + 8, dt), dt)[:, :K]
    if trans_b:
        b = util.to_dev(padded(np.ascontiguousarray(p["B"].T), K + 8, dt), dt)[:, :K].t()
    else:
        b = util.to_dev(padded(p["B"], N + 8, dt), dt)[:, :N]
    bias = util.to_dev(p["bias"], dt)
    say("case K off the grid", dt, M, N, K, "B[N,K]" if trans_b else "B[K,N]", force or "")
    C = tg.gemm(A, b, bias=bias, residual=util.to_dev(R, dt))
    torch.cuda.synchronize()
    kern = tg.last_kernel()
    say("  kernel", kern)
    assert kern.startswith("async_") and not kern.endswith("_kpad"), kern
    if force:
        assert kern == force, kern
    _, ref = oracle.gemm_ex(dt, p["A"], np.ascontiguousarray(p["B"].T) if trans_b else p["B"],
                            trans_b=trans_b, bias=p["bias"], R=R)
    util.check_exact(util.to_bits(C), ref, "K off the grid " + kern)


def test_k_off_the_loop_grid_gelu_random(tg):
    p = inputs.problem(BF16, 4096, 4096, 2000, seed=290, bias=True, act=inputs.ACT_GELU_TANH,
                       a_scale=0.1, b_scale=0.1)
    say("case K off the grid, gelu 4096 x 4096 x 2000")
    bits, kern = run(tg, p)
    assert kern.startswith("async_") and not kern.endswith("_kpad"), kern
    f64, rbits = oracle.gemm(BF16, p["A"], p["B"], p["bias"], oracle.ACT_GELU_TANH)
    util.check_tol(BF16, bits, f64, "K off the grid, gelu", ref_bits=rbits)


KPAD_CASES = [
    # (dt, M, N, K): K off the 8-element grid (pitches padded to it) on
    # problems of >= 2^30 multiply-adds: A and B are copied with K rounded
    # up to 128 and zeros in the added entries
    (F16, 1000, 1200, 1004),
    (BF16, 2000, 2000, 1995),
]


def test_k_dispatch_off_the_grids(tg):
    # 4096 x 4096 outputs (a full wave of 256 x 256 tiles): K = 520, the
    # masked loop (120 padded k, fewer than K); K = 36: 92 padded k would be
    # more than K, the tiled kernel; K = 1004 (off the 8-element grid, 20
    # padded k): K padding; K = 524 (116 padded k, more than K / 8): the tiled
    # kernel.  1536 x 2048 outputs (48 tiles of 256 x 256, 192 of 128 x
    # 128): K = 1000 masked on the 128 x 128 16x16x32 tiles; 768 x 2048 (96
    # of them, under half a wave): K = 1000 padded instead
    import torch
    for (M, N), K, ld, expect in (((4096, 4096), 520, 520, "async_256x256x32_s4_mfma16"),
                                  ((4096, 4096), 36, 40, "tiled_"),
                                  ((4096, 4096), 1004, 1008, "_kpad"),
                                  ((4096, 4096), 524, 528, "tiled_"),
                                  ((1536, 2048), 1000, 1000, "async_128x128x32_s4_mfma16"),
                                  ((768, 2048), 1000, 1000, "_kpad")):
        a = torch.zeros((M, ld), dtype=torch.float16, device="cuda")[:, :K]
        b = torch.zeros((K, N), dtype=torch.float16, device="cuda")
        tg.gemm(a, b)
        kern = tg.last_kernel()
        assert kern == expect or kern.startswith(expect) or kern.endswith(expect), (K, kern)
    torch.cuda.synchronize()


@pytest.mark.parametrize("trans_b", [False, True])
@pytest.mark.parametrize("dt,M,N,K", KPAD_CASES)
def test_k_padded_to_the_loop_integer_exact(tg, dt, M, N, K, trans_b):
    # A and B sit in buffers whose pitch padding holds NaN: the padded copies
    # must read only k < K.  Integer operands, bias and residual: bit-exact.
    import torch
    p = inputs.problem(dt, M, N, K, seed=280 + K, kind="int", bias=True, bias_kind="int")
    R = inputs.draw(np.random.default_rng(281 + M), (M, N), "int", dt, 8.0)
    ldk = round8(K + 8)
    A = util.to_dev(padded(p["A"], ldk, dt), dt)[:, :K]
    if trans_b:
        b = util.to_dev(padded(np.ascontiguousarray(p["B"].T), ldk, dt), dt)[:, :K].t()
    else:
        b = util.to_dev(padded(p["B"], N + 8, dt), dt)[:, :N]
    bias = util.to_dev(p["bias"], dt)
    say("case K padded", dt, M, N, K, "B[N,K]" if trans_b else "B[K,N]")
    C = tg.gemm(A, b, bias=bias, residual=util.to_dev(R, dt))
    torch.cuda.synchronize()
    kern = tg.last_kernel()
    say("  kernel", kern)
    assert kern.endswith("_kpad"), kern
    _, ref = oracle.gemm_ex(dt, p["A"], np.ascontiguousarray(p["B"].T) if trans_b else p["B"],
                            trans_b=trans_b, bias=p["bias"], R=R)
    util.check_exact(util.to_bits(C), ref, "K padded " + kern)


def test_partial_row_tile_gelu_random_and_qkv(tg, monkeypatch):
    # M = 1200: 5 row tiles, 80 padding rows (at most M / 8 are allowed)
    import torch
    monkeypatch.setenv("TG_FORCE_CONFIG", "async_256x256x32_s4_mfma16")
    p = inputs.problem(BF16, 1200, 512, 640, seed=250, bias=True, act=inputs.ACT_GELU_TANH,
                       a_scale=0.2, b_scale=0.2)
    say("case partial row tile gelu 1200x512x640")
    bits, kern = run(tg, p)
    assert kern == "async_256x256x32_s4_mfma16"
    f64, rbits = oracle.gemm(BF16, p["A"], p["B"], p["bias"], oracle.ACT_GELU_TANH)
    util.check_tol(BF16, bits, f64, "partial row tile gelu", ref_bits=rbits)
    q = inputs.qkv_problem(BF16, 1200, 256, 256, seed=251, kind="int")
    say("case partial row tile qkv 1200x256x256 x3")
    _, _, outs = run_qkv(tg, q)
    assert tg.last_kernel() == "async_256x256x32_s4_mfma16"
    for t in range(3):
        _, ref = oracle.gemm(BF16, q["X"], q["W"][t])
        util.check_exact(outs[t], ref, "partial row tile qkv [%d]" % t)


def test_projection_with_ragged_token_count(tg):
    # X[3000, 4096] . W[4096, 11008]: a token count off the tile grid with
    # model dimensions on it takes the 256 x 256 kernel by itself
    import torch
    p = inputs.problem(BF16, 3000, 11008, 4096, seed=252, kind="normal", b_scale=1 / 64)
    say("case projection 3000x11008x4096")
    bits, kern = run(tg, p)
    # 12 x 43 = 516 tiles: two whole waves plus 4 tiles, so stream-K
    assert kern == "async_256x256x32_s4_mfma16_streamk", kern
    f64, rbits = oracle.gemm(BF16, p["A"], p["B"])
    util.check_tol(BF16, bits, f64, "projection", ref_bits=rbits)


# ------------------------------- extended epilogue: residual and B stored [N,K]

def run_ex(tg, p, trans_b, R=None, Rin_place=False):
    """C = act(A.opB + bias) + R through tg_gemm_ex; returns (bits, kernel)."""
    import torch
    dt = p["dt"]
    A = util.to_dev(p["A"], dt)
    Bd = util.to_dev(np.ascontiguousarray(p["B"].T) if trans_b else p["B"], dt)
    b = Bd.t() if trans_b else Bd
    bias = util.to_dev(p["bias"], dt) if p.get("bias") is not None else None
    act = "gelu_tanh" if p["act"] == inputs.ACT_GELU_TANH else "none"
    if Rin_place:
        C = util.to_dev(R, dt)
        tg.gemm(A, b, out=C, bias=bias, act=act, residual=C)
    else:
        res = util.to_dev(R, dt) if R is not None else None
        C = tg.gemm(A, b, bias=bias, act=act, residual=res)
    torch.cuda.synchronize()
    return util.to_bits(C), tg.last_kernel()


EX_SHAPES = [
    # (dt, M, N, K, force): every kernel family with a residual
    (F16, 512, 768, 384, "async_256x256x32_s4"),
    (BF16, 768, 512, 256, "async_256x256x32_s4_mfma16"),
    (F16, 512, 512, 512, "async_256x256x32_s4_mfma16_w8"),
    (F16, 384, 576, 256, "async_192x192x32_s4_mfma16"),
    (BF16, 384, 256, 384, "async_128x128x32_s4_mfma16"),
    (F16, 256, 384, 768, "async_128x128x64_s4_mfma16"),
    (BF16, 256, 384, 256, "async_128x128x32_s4"),
    (F16, 192, 256, 512, "async_64x128x32_s4"),
    (BF16, 192, 320, 384, "async_64x64x32_s4"),   # N a multiple of 64, not of 128
    (BF16, 300, 170, 200, None),          # ragged: tiled kernel (B [K,N]) / generic (B [N,K])
    (F16, 16, 1024, 2048, None),          # small M: streaming split-K kernel / B [N,K] kernel
    (BF16, 5, 520, 777, None),            # small M, ragged: realigning kernel / generic
    (F16, 64, 128, 96, "generic"),
]


@pytest.mark.parametrize("trans_b", [False, True])
@pytest.mark.parametrize("dt,M,N,K,force", EX_SHAPES)
def test_residual_and_transposed_b_integer_exact(tg, monkeypatch, dt, M, N, K, force, trans_b):
    if force:
        monkeypatch.setenv("TG_FORCE_CONFIG", force)
    p = inputs.problem(dt, M, N, K, seed=90 + M + N, kind="int", bias=True, bias_kind="int")
    R = inputs.draw(np.random.default_rng(91 + K), (M, N), "int", dt, 8.0)
    say("case ex integer", dt, M, N, K, force, "B[N,K]" if trans_b else "B[K,N]")
    bits, kern = run_ex(tg, p, trans_b, R)
    say("  kernel", kern)
    if force and force.startswith("async"):
        assert kern == force
    if trans_b and not (force or "").startswith("async"):
        # B stored [N,K] with pitch K: the small-M kernel when the rows are
        # on the 16-byte grid, else the reported fallback
        small = not force and M <= 32 and N >= 256 and K >= 256 and K % 8 == 0
        assert kern.startswith("skinny_nk" if small else "generic"), kern
    _, ref = oracle.gemm_ex(dt, p["A"], np.ascontiguousarray(p["B"].T) if trans_b else p["B"],
                            trans_b=trans_b, bias=p["bias"], R=R)
    util.check_exact(bits, ref, "ex %s" % kern)


@pytest.mark.parametrize("trans_b", [False, True])
@pytest.mark.parametrize("dt,M,N,K,force", EX_SHAPES[:8])
def test_residual_and_transposed_b_gelu_random(tg, monkeypatch, dt, M, N, K, force, trans_b):
    if force:
        monkeypatch.setenv("TG_FORCE_CONFIG", force)
    p = inputs.problem(dt, M, N, K, seed=95 + M, bias=True, act=inputs.ACT_GELU_TANH,
                       a_scale=0.25, b_scale=0.25)
    R = inputs.draw(np.random.default_rng(96 + N), (M, N), "uniform", dt)
    say("case ex gelu", dt, M, N, K, force, "B[N,K]" if trans_b else "B[K,N]")
    bits, kern = run_ex(tg, p, trans_b, R)
    Bo = np.ascontiguousarray(p["B"].T) if trans_b else p["B"]
    f64, rbits = oracle.gemm_ex(dt, p["A"], Bo, trans_b=trans_b, bias=p["bias"],
                                act=oracle.ACT_GELU_TANH, R=R)
    util.check_tol(dt, bits, f64, "ex gelu %s" % kern, ref_bits=rbits)


@pytest.mark.parametrize("force", ["async_128x128x32_s4", None])
def test_in_place_residual(tg, monkeypatch, force):
    if force:
        monkeypatch.setenv("TG_FORCE_CONFIG", force)
    for (M, N, K) in ((256, 384, 256), (16, 1024, 1024)):
        p = inputs.problem(BF16, M, N, K, seed=97, kind="int", bias=True, bias_kind="int")
        R = inputs.draw(np.random.default_rng(98), (M, N), "int", BF16, 4.0)
        say("case in-place residual", M, N, K, force)
        bits, kern = run_ex(tg, p, False, R, Rin_place=True)
        _, ref = oracle.gemm_ex(BF16, p["A"], p["B"], bias=p["bias"], R=R)
        util.check_exact(bits, ref, "in place %s" % kern)


def test_transposed_b_full_size(tg):
    # the headline shape with the weight stored [N,K] and a residual, every
    # output against the oracle
    p = inputs.config_problem("f16_4096_gelu")
    R = inputs.draw(np.random.default_rng(99), (p["M"], p["N"]), "uniform", F16)
    say("case 4096 B[N,K] + residual")
    bits, kern = run_ex(tg, p, True, R)
    assert kern == "async_256x256x32p_s4_mfma16", kern
    f64, rbits = oracle.gemm_ex(F16, p["A"], np.ascontiguousarray(p["B"].T), trans_b=True,
                                bias=p["bias"], act=oracle.ACT_GELU_TANH, R=R)
    util.check_tol(F16, bits, f64, "4096 B[N,K] + residual", ref_bits=rbits)


# -------------------------------------- block-scaled 8-bit GEMM (e8m0 scales)

def run_mx(tg, p, out_dtype=None):
    import torch
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    bias = util.to_dev(p["bias"], p["dt"]) if p.get("bias") is not None else None
    names = {inputs.FP8_E4M3: "e4m3", inputs.FP8_E5M2: "e5m2"}
    C = tg.gemm_mx(dev(p["A"]), dev(p["SA"]), dev(p["B"]), dev(p["SB"]), names[p["fmt_a"]],
                   names[p["fmt_b"]], bias=bias,
                   act="gelu_tanh" if p["act"] == inputs.ACT_GELU_TANH else "none",
                   out_dtype=util.torch_dtype(p["dt"]))
    torch.cuda.synchronize()
    return util.to_bits(C), tg.last_kernel()


MX_FORMATS = [(0, 0), (1, 1), (0, 1), (1, 0)]


@pytest.mark.parametrize("fa,fb", MX_FORMATS)
@pytest.mark.parametrize("M,N,K", [(512, 768, 512), (100, 72, 96)])
def test_mx_integer_exact(tg, fa, fb, M, N, K):
    # entries in {-2..2}, scales 2^-2..2^2: every FP32 partial sum is exact
    p = inputs.mx_problem(fa, fb, M, N, K, seed=120 + 2 * fa + fb, kind="int", bias=True,
                          dt=BF16 if fa == fb else F16)
    say("case mx integer", fa, fb, M, N, K)
    bits, kern = run_mx(tg, p)
    say("  kernel", kern)
    assert kern.startswith("mx_256x256" if M % 256 == 0 and N % 256 == 0 else "mx_generic")
    _, ref = oracle.gemm_mx(fa, fb, p["A"], p["SA"], p["B"], p["SB"], p["bias"], dt=p["dt"])
    util.check_exact(bits, ref, "mx %s" % kern)


@pytest.mark.parametrize("fa,fb", MX_FORMATS[:3])
def test_mx_random_bias_gelu(tg, fa, fb):
    p = inputs.mx_problem(fa, fb, 512, 512, 1024, seed=130 + fa + fb, bias=True,
                          act=inputs.ACT_GELU_TANH)
    say("case mx random bias+gelu", fa, fb)
    bits, kern = run_mx(tg, p)
    assert kern.startswith("mx_256x256")
    f64, rbits = oracle.gemm_mx(fa, fb, p["A"], p["SA"], p["B"], p["SB"], p["bias"],
                                oracle.ACT_GELU_TANH, dt=BF16)
    util.check_tol(BF16, bits, f64, "mx random", ref_bits=rbits)


def test_mx_generic_matches_fast_path(tg, monkeypatch):
    p = inputs.mx_problem(0, 0, 256, 256, 512, seed=140)
    fast, k1 = run_mx(tg, p)
    monkeypatch.setenv("TG_FORCE_CONFIG", "generic")
    slow, k2 = run_mx(tg, p)
    assert k1.startswith("mx_256x256") and k2.startswith("mx_generic")
    f64, rbits = oracle.gemm_mx(0, 0, p["A"], p["SA"], p["B"], p["SB"], dt=BF16)
    util.check_tol(BF16, fast, f64, "mx fast", ref_bits=rbits)
    util.check_tol(BF16, slow, f64, "mx generic", ref_bits=rbits)


def test_mx_full_size_rows(tg):
    # 4096^3, e4m3 x e4m3 with microscaled N(0,1) data; whole rows checked
    p = inputs.mx_problem(0, 0, 4096, 4096, 4096, seed=150, bias=True)
    say("case mx 4096^3")
    bits, kern = run_mx(tg, p)
    assert kern.startswith("mx_256x256")
    for r0 in (0, 2047, 4092):
        f64, rbits = oracle.gemm_mx(0, 0, p["A"], p["SA"], p["B"], p["SB"], p["bias"], dt=BF16,
                                    rows=(r0, r0 + 4))
        util.check_tol(BF16, bits[r0:r0 + 4], f64, "mx 4096 rows %d" % r0, ref_bits=rbits)


# -------------------------------------------------------- fused attention

def run_attn(tg, p, lse=True):
    import torch
    q, k, v = (util.to_dev(p[n], p["dt"]) for n in ("Q", "K", "V"))
    out, l = tg.attention(q, k, v, causal=p["causal"], lse=True)
    torch.cuda.synchronize()
    return util.to_bits(out), l.cpu().numpy().astype(np.float64), tg.last_kernel()


# P is rounded to the input dtype before the P.V product (as FlashAttention
# does); the oracle keeps P in double, so O is compared within the
# tolerance only, not for correct rounding.
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dt", [F16, BF16])
@pytest.mark.parametrize("B,H,S,D", [(1, 2, 256, 128), (2, 3, 384, 128), (1, 2, 200, 64)])
def test_attention_random(tg, dt, causal, B, H, S, D):
    p = inputs.attention_problem(dt, B, H, S, D, seed=170 + S + dt, causal=causal)
    say("case attention", dt, B, H, S, D, "causal" if causal else "full")
    bits, lse, kern = run_attn(tg, p)
    say("  kernel", kern)
    assert kern.startswith("attn_fwd_256x64" if D == 128 and S % 256 == 0 else
                           "attn_fwd_128x64" if D == 128 and S % 128 == 0 else "attn_generic")
    f64, _, lse_ref = oracle.attention(dt, p["Q"], p["K"], p["V"], causal=causal)
    util.check_tol(dt, bits, f64, "attention %s" % kern)
    assert np.max(np.abs(lse - lse_ref)) < 2e-3
    if causal:
        # row 0 attends to key 0 alone: O = V[0] exactly
        assert np.array_equal(bits[:, :, 0], p["V"][:, :, 0])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S", [512, 384])
def test_attention_rising_scores(tg, causal, S):
    # key j scaled by 1 + j/24: row maxima keep rising along the sequence, so
    # the running reference is raised (and O, l rescaled) on many tiles, not
    # only the first
    p = inputs.attention_problem(BF16, 1, 2, S, 128, seed=185 + S, causal=causal)
    k = util.decode(BF16, p["K"]) * (1.0 + np.arange(S) / 24.0)[None, None, :, None]
    p["K"] = inputs.to_bits(k, BF16)
    bits, lse, kern = run_attn(tg, p)
    assert kern.startswith("attn_fwd")
    f64, _, lse_ref = oracle.attention(BF16, p["Q"], p["K"], p["V"], causal=causal)
    util.check_tol(BF16, bits, f64, "attention rising scores")
    assert np.all(np.abs(lse - lse_ref) < 1e-3 + 1e-4 * np.abs(lse_ref))


@pytest.mark.parametrize("causal", [False, True])
def test_attention_block_sizes_agree_bitwise(tg, monkeypatch, causal):
    # every wave runs the same tiles in the same order whether its workgroup
    # holds 128 or 256 queries (tiles above a wave's causal diagonal are exact
    # no-ops, skipped or not), so the two kernels give the same bits
    p = inputs.attention_problem(BF16, 2, 2, 768, 128, seed=187, causal=causal)
    a, la, ka = run_attn(tg, p)
    monkeypatch.setenv("TG_ATTN_BM", "128")
    b, lb, kb = run_attn(tg, p)
    assert ka.startswith("attn_fwd_256x64") and kb.startswith("attn_fwd_128x64"), (ka, kb)
    util.check_exact(a, b, "attention 256 vs 128 queries per workgroup")
    assert np.array_equal(la, lb)
    f64, _, _ = oracle.attention(BF16, p["Q"], p["K"], p["V"], causal=causal)
    util.check_tol(BF16, a, f64, "attention block sizes")


def test_attention_uniform_integer_values(tg):
    # Q = 0: every weight is exactly 1, O = mean of the V rows it can see
    p = inputs.attention_problem(BF16, 1, 2, 256, 128, seed=180, kind="int", causal=True)
    p["Q"] = np.zeros_like(p["Q"])
    bits, lse, _ = run_attn(tg, p)
    f64, rbits, lse_ref = oracle.attention(BF16, p["Q"], p["K"], p["V"], causal=True)
    util.check_tol(BF16, bits, f64, "uniform attention", ref_bits=rbits)
    assert np.allclose(lse, lse_ref, atol=1e-5)


def test_attention_generic_matches_fast_path(tg, monkeypatch):
    p = inputs.attention_problem(F16, 1, 2, 256, 128, seed=181, causal=True)
    fast, l1, k1 = run_attn(tg, p)
    monkeypatch.setenv("TG_FORCE_CONFIG", "generic")
    slow, l2, k2 = run_attn(tg, p)
    assert k1.startswith("attn_fwd") and k2.startswith("attn_generic")
    f64, _, lse_ref = oracle.attention(F16, p["Q"], p["K"], p["V"], causal=True)
    util.check_tol(F16, fast, f64, "attn fast")
    util.check_tol(F16, slow, f64, "attn generic")


@pytest.mark.parametrize("causal", [False, True])
def test_attention_full_size_heads(tg, causal):
    # the benchmark shape: batch 4, 16 heads, 4096 tokens, head dim 128;
    # heads (0, 0) and (3, 15) checked in full against the oracle
    p = inputs.attention_problem(BF16, 4, 16, 4096, 128, seed=190, causal=causal)
    say("case attention 4x16x4096x128", "causal" if causal else "full")
    bits, lse, kern = run_attn(tg, p)
    assert kern.startswith("attn_fwd")
    for (b, h) in ((0, 0), (3, 15)):
        sub = {n: p[n][b:b + 1, h:h + 1] for n in ("Q", "K", "V")}
        f64, _, lse_ref = oracle.attention(BF16, sub["Q"], sub["K"], sub["V"], causal=causal)
        util.check_tol(BF16, bits[b:b + 1, h:h + 1], f64, "attention head %d,%d" % (b, h))
        assert np.max(np.abs(lse[b:b + 1, h:h + 1] - lse_ref)) < 2e-3


# ------------------------------------------------------------ edge cases

def test_mx_k_zero_gives_activated_bias(tg):
    import torch
    p = inputs.mx_problem(0, 0, 40, 24, 0, seed=210, bias=True, act=inputs.ACT_GELU_TANH)
    bits, kern = run_mx(tg, p)
    assert kern.startswith("mx_generic")
    f64, rbits = oracle.gemm_mx(0, 0, p["A"], p["SA"], p["B"], p["SB"], p["bias"],
                                oracle.ACT_GELU_TANH, dt=BF16)
    util.check_tol(BF16, bits, f64, "mx K=0", ref_bits=rbits)


@pytest.mark.parametrize("S,D", [(1, 128), (7, 32), (129, 128)])
def test_attention_tiny_and_ragged(tg, S, D):
    for causal in (False, True):
        p = inputs.attention_problem(F16, 1, 3, S, D, seed=211 + S, causal=causal)
        bits, lse, kern = run_attn(tg, p)
        assert kern.startswith("attn_generic")
        f64, _, lse_ref = oracle.attention(F16, p["Q"], p["K"], p["V"], causal=causal)
        util.check_tol(F16, bits, f64, "attention S=%d D=%d" % (S, D))
        assert np.max(np.abs(lse - lse_ref)) < 2e-3


def test_transposed_b_k_zero(tg):
    # K = 0 with B given as [N,K] (TG_OP_T): C = act(bias) + R
    import torch
    dt = BF16
    bias = inputs.draw(np.random.default_rng(212), (24,), "bias", dt)
    R = inputs.draw(np.random.default_rng(213), (8, 24), "uniform", dt)
    bd, Rd = util.to_dev(bias, dt), util.to_dev(R, dt)
    C = torch.empty((8, 24), dtype=torch.bfloat16, device="cuda")
    tg.gemm_ex_ptr(dt, 8, 24, 0, 0, 0, 0, 0, tg.OP_T, C.data_ptr(), 24,
                   bias=bd.data_ptr(), act=1, R=Rd.data_ptr(), ldr=24)
    torch.cuda.synchronize()
    f64, rbits = oracle.gemm_ex(dt, np.zeros((8, 0), np.uint16), np.zeros((24, 0), np.uint16),
                                trans_b=True, bias=bias, act=oracle.ACT_GELU_TANH, R=R)
    util.check_tol(dt, util.to_bits(C), f64, "B[N,K] K=0", ref_bits=rbits)


def test_small_m_dispatch_bounds(tg):
    # M <= 32 streams W: the split-K streaming kernel when it fits, the
    # realigning one for other shapes with N and K of at least 256; larger M
    # (one partial 64-row tile at M = 33), or narrower shapes, take the
    # asynchronous tiles
    import torch
    w = torch.zeros((8192, 8192), dtype=torch.bfloat16, device="cuda")
    for M, expect in ((16, "skinny_stream"), (32, "skinny_stream"), (33, "async_64x")):
        x = torch.zeros((M, 8192), dtype=torch.bfloat16, device="cuda")
        tg.gemm(x, w)
        assert tg.last_kernel().startswith(expect), (M, tg.last_kernel())
    x = torch.zeros((20, 1000), dtype=torch.bfloat16, device="cuda")
    tg.gemm(x, torch.zeros((1000, 1000), dtype=torch.bfloat16, device="cuda"))
    assert tg.last_kernel().startswith("skinny_realign"), tg.last_kernel()
    tg.gemm(x, torch.zeros((1000, 200), dtype=torch.bfloat16, device="cuda"))
    assert not tg.last_kernel().startswith("skinny"), tg.last_kernel()
    torch.cuda.synchronize()


def test_dispatch_choices(tg, monkeypatch):
    import torch
    a = torch.zeros((4096, 4096), dtype=torch.float16, device="cuda")
    tg.gemm(a, a)
    assert tg.last_kernel().startswith(("tiled_256x256", "async_256x256"))
    x = torch.zeros((16, 8192), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((8192, 8192), dtype=torch.bfloat16, device="cuda")
    tg.gemm(x, w)
    assert tg.last_kernel().startswith("skinny")
    c = torch.zeros((2048, 2048), dtype=torch.float16, device="cuda")
    tg.gemm(c, c)
    assert tg.last_kernel() == "async_128x128x32_s4"
    # under-filled grids: the configuration of least modelled time, 64 x 64
    # tiles at 1024^3 (256 tiles) and 256^3, 128 x 128 at 2048^3, 64 x 128
    # for 1024 x 2048 x 2048; no split at these K (TG_SPLITK=0: enough
    # splits for one wave of workgroups)
    b = torch.zeros((1024, 1024), dtype=torch.float16, device="cuda")
    tg.gemm(b, b)
    assert tg.last_kernel() == "async_64x64x32_s4"
    d = torch.zeros((256, 256), dtype=torch.float16, device="cuda")
    tg.gemm(d, d)
    assert tg.last_kernel() == "async_64x64x32_s4"
    e = torch.zeros((1024, 2048), dtype=torch.float16, device="cuda")
    tg.gemm(e, c)
    assert tg.last_kernel() == "async_64x128x32_s4"
    # partial last row tiles: 144 tiles of 256 x 256 (more than half a wave,
    # not a whole one) against 242 of 192 x 192, which fill their wave
    # better: the 192 x 192 tiles; stream-K with TG_STREAMK=2; never the
    # forced-only 8-wave variant
    f = torch.zeros((2049, 4096), dtype=torch.float16, device="cuda")
    g = torch.zeros((4096, 4096), dtype=torch.float16, device="cuda")
    tg.gemm(f, g)
    assert tg.last_kernel() == "async_192x192x32_s4_mfma16", tg.last_kernel()
    monkeypatch.setenv("TG_STREAMK", "2")
    tg.gemm(f, g)
    assert tg.last_kernel() == "async_256x256x32_s4_mfma16_streamk", tg.last_kernel()
    monkeypatch.delenv("TG_STREAMK")
    # whole waves (4096^3: 256 tiles) stay data-parallel, on the pair-staged loop
    tg.gemm(g, g)
    assert tg.last_kernel() == "async_256x256x32p_s4_mfma16", tg.last_kernel()
    # below a full wave of 256 x 256 tiles the launch-time model picks the
    # tile and the split count: 64 x 4096 x 4096 in four splits of 64 x 64
    # tiles; 128 x 4096 x 14336 split as well; TG_SPLITK=1 turns it off
    h = torch.zeros((64, 4096), dtype=torch.float16, device="cuda")
    tg.gemm(h, g)
    assert tg.last_kernel() == "async_64x64x32_s4_splitk4", tg.last_kernel()
    i = torch.zeros((128, 14336), dtype=torch.float16, device="cuda")
    j = torch.zeros((14336, 4096), dtype=torch.float16, device="cuda")
    tg.gemm(i, j)
    assert "_splitk" in tg.last_kernel(), tg.last_kernel()
    monkeypatch.setenv("TG_SPLITK", "1")
    tg.gemm(h, g)
    assert tg.last_kernel() == "async_64x64x32_s4", tg.last_kernel()
    monkeypatch.setenv("TG_SPLITK", "0")
    tg.gemm(b, b)
    assert tg.last_kernel() == "async_64x64x32_s4"
    tg.gemm(d, d)
    assert tg.last_kernel() == "async_64x64x32_s4_splitk2"
    monkeypatch.delenv("TG_SPLITK")
    torch.cuda.synchronize()


def test_invalid_arguments_raise(tg):
    import torch
    a = torch.zeros((8, 8), dtype=torch.float16, device="cuda")
    with pytest.raises(tg.TgError):
        tg.gemm(a, a, out=a)  # output overlaps the inputs


PAIR_CASES = [
    # (dt, M, N, K, integer, B stored [N,K]): the pair-staged 256 x 256 loop,
    # both B layouts: whole tiles, 4 and 2 pairs of 64 k; partial last row
    # and column tiles (600 rows, 520 columns); a single four-step round
    (F16, 512, 768, 1024, True, True),
    (BF16, 512, 512, 512, True, True),
    (BF16, 600, 520, 512, True, True),
    (F16, 768, 512, 128, True, True),
    (F16, 768, 512, 384, False, True),
    (F16, 512, 768, 1024, True, False),
    (BF16, 512, 512, 512, True, False),
    (BF16, 600, 520, 512, True, False),
    (F16, 768, 512, 128, True, False),
    (BF16, 768, 512, 384, False, False),
]


@pytest.mark.parametrize("dt,M,N,K,integer,trans_b", PAIR_CASES)
def test_pair_staged_loop(tg, monkeypatch, dt, M, N, K, integer, trans_b):
    monkeypatch.setenv("TG_FORCE_CONFIG", "async_256x256x32p_s4_mfma16")
    kind = "int" if integer else "normal"
    p = inputs.problem(dt, M, N, K, seed=1500 + M + K, kind=kind, bias=True,
                       bias_kind="int" if integer else "bias",
                       act=inputs.ACT_NONE if integer else inputs.ACT_GELU_TANH,
                       b_scale=1.0 if integer else K ** -0.5)
    R = inputs.draw(np.random.default_rng(1501 + N), (M, N), "int", dt, 4.0) if integer else None
    say("case pair-staged loop", dt, M, N, K, kind, "B[N,K]" if trans_b else "B[K,N]")
    bits, kern = run_ex(tg, p, trans_b, R)
    assert kern == "async_256x256x32p_s4_mfma16", kern
    B = np.ascontiguousarray(p["B"].T) if trans_b else p["B"]
    f64, rbits = oracle.gemm_ex(dt, p["A"], B, trans_b=trans_b, bias=p["bias"], act=p["act"],
                                R=R)
    if integer:
        util.check_exact(bits, rbits, "pair-staged loop")
    else:
        util.check_tol(dt, bits, f64, "pair-staged loop", ref_bits=rbits)


def test_leading_dimension_past_32_bit_lane_offsets(tg):
    # 256 rows of A at a pitch of 2^23 + 64 elements span more than 4 GiB,
    # past the 32-bit lane offsets of the 16x16x32 kernels' copies: the
    # 32x32x16 kernels take it, exact on integer operands
    import torch
    M, N, K, lda = 256, 512, 512, (1 << 23) + 64
    Ab = inputs.draw(np.random.default_rng(1601), (M, K), "int", BF16, 4.0)
    Bb = inputs.draw(np.random.default_rng(1602), (K, N), "int", BF16, 4.0)
    say("case lda 2^23 + 64", M, N, K)
    big = torch.zeros((M, lda), dtype=torch.bfloat16, device="cuda")
    big[:, :K] = util.to_dev(Ab, BF16)
    C = tg.gemm(big[:, :K], util.to_dev(Bb, BF16))
    torch.cuda.synchronize()
    kern = tg.last_kernel()
    assert "mfma16" not in kern, kern
    _, ref = oracle.gemm(BF16, Ab, Bb)
    util.check_exact(util.to_bits(C), ref, "lda 2^23 + 64")
    del big


def test_pair_staged_loop_dispatch(tg):
    # taken unforced with a full wave of 256 x 256 tiles and K a multiple of
    # 128, B in either layout; K off that grid keeps the masked 32-deep loop
    import torch
    a = torch.zeros((4096, 1024), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((4096, 1024), dtype=torch.bfloat16, device="cuda")
    tg.gemm(a, w.t())
    assert tg.last_kernel() == "async_256x256x32p_s4_mfma16", tg.last_kernel()
    tg.gemm(a[:, :1000], w[:, :1000].t())
    assert tg.last_kernel() == "async_256x256x32_s4_mfma16", tg.last_kernel()
    tg.gemm(a, w.t().contiguous())
    assert tg.last_kernel() == "async_256x256x32p_s4_mfma16", tg.last_kernel()
    tg.gemm(a[:, :1000], w.t().contiguous()[:1000])
    assert tg.last_kernel() == "async_256x256x32_s4_mfma16", tg.last_kernel()
    torch.cuda.synchronize()
