"""GPU parity of stream-K on the 256 x 256 16x16x32 tiles: problems whose
tile count leaves a partial last wave run a persistent grid in which whole
waves stay data-parallel and the last tiles are split by K across the
workgroups, the last piece in adding every piece in K order ("TIRx",
section 4.3: work partitioning decided at run time; "Beyond Hand-Written
CUDA", section 2: the tile scheduler stage).

Integer operands: bit-exact against the oracle and against the same call
with stream-K off.  Random operands: within the tolerance, and the same bits
on every run (the pieces are added in a fixed order whatever order they
finish in).  By default stream-K takes only shapes whose share of K per
workgroup is at least 2048; the small shapes here set TG_STREAMK=2, which
takes them too, so the same kernel paths are exercised at a fraction of the
oracle's cost."""
import numpy as np
import pytest

import oracle
import util
from tiled_dense_gemm_09_amd import inputs

pytestmark = pytest.mark.gpu

F16, BF16 = inputs.F16, inputs.BF16
SK = "async_256x256x32_s4_mfma16_streamk"


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def tg():
    import torch
    assert torch.cuda.is_available()
    from tiled_dense_gemm_09_amd import tg as _tg
    return _tg


# (dt, M, N, K, B stored [N,K]): every tile split (144 tiles, fewer than a
# wave but at least half of one), two whole waves plus a partial one (576 tiles: 256 data-parallel,
# 320 split), a piece of one quad (K = 256), partial last row and column
# tiles, and B stored [N,K]
CASES = [
    (F16, 3072, 3072, 512, False),
    (BF16, 9216, 4096, 256, False),
    (F16, 3000, 2600, 384, False),
    (BF16, 4352, 4096, 640, True),
    (F16, 2049, 4096, 1024, True),
]


def run(tg, dt, A, B, trans_b, bias=None, act="none", R=None):
    import torch
    Ad = util.to_dev(A, dt)
    Bd = util.to_dev(np.ascontiguousarray(B.T), dt).t() if trans_b else util.to_dev(B, dt)
    bd = util.to_dev(bias, dt) if bias is not None else None
    Rd = util.to_dev(R, dt) if R is not None else None
    C = tg.gemm(Ad, Bd, bias=bd, act=act, residual=Rd)
    torch.cuda.synchronize()
    return util.to_bits(C), tg.last_kernel()


@pytest.mark.parametrize("dt,M,N,K,trans_b", CASES)
def test_stream_k_integer_exact_and_equal_to_data_parallel(tg, monkeypatch, dt, M, N, K,
                                                           trans_b):
    monkeypatch.setenv("TG_STREAMK", "2")
    p = inputs.problem(dt, M, N, K, seed=1000 + M + K, kind="int", bias=True, bias_kind="int")
    R = inputs.draw(np.random.default_rng(1001 + N), (M, N), "int", dt, 4.0)
    say("case stream-K integer", dt, M, N, K, "B[N,K]" if trans_b else "")
    bits, kern = run(tg, dt, p["A"], p["B"], trans_b, p["bias"], R=R)
    say("  kernel", kern)
    assert kern == SK, kern
    _, ref = oracle.gemm_ex(dt, p["A"], p["B"], bias=p["bias"], R=R)
    util.check_exact(bits, ref, "stream-K integer")
    monkeypatch.setenv("TG_STREAMK", "0")
    bits_dp, kern_dp = run(tg, dt, p["A"], p["B"], trans_b, p["bias"], R=R)
    assert kern_dp != SK, kern_dp
    util.check_exact(bits_dp, bits, "stream-K vs " + kern_dp)


@pytest.mark.parametrize("dt,M,N,K,trans_b", CASES[:3])
def test_stream_k_random_bias_gelu_and_repeatable(tg, monkeypatch, dt, M, N, K, trans_b):
    monkeypatch.setenv("TG_STREAMK", "2")
    p = inputs.problem(dt, M, N, K, seed=1100 + M, kind="normal", b_scale=K ** -0.5, bias=True,
                       act=inputs.ACT_GELU_TANH)
    say("case stream-K random", dt, M, N, K)
    bits, kern = run(tg, dt, p["A"], p["B"], trans_b, p["bias"], act="gelu_tanh")
    assert kern == SK, kern
    f64, rbits = oracle.gemm(dt, p["A"], p["B"], p["bias"], oracle.ACT_GELU_TANH)
    util.check_tol(dt, bits, f64, "stream-K random", ref_bits=rbits)
    for i in range(3):
        again, _ = run(tg, dt, p["A"], p["B"], trans_b, p["bias"], act="gelu_tanh")
        util.check_exact(again, bits, "stream-K repeat %d" % i)


def test_stream_k_qkv(tg, monkeypatch):
    # three outputs of 18 x 5 tiles each: 270 tiles, one wave plus 14
    import torch
    monkeypatch.setenv("TG_STREAMK", "2")
    q = inputs.qkv_problem(BF16, 4608, 1280, 512, seed=1200, kind="int")
    say("case stream-K qkv")
    X = util.to_dev(q["X"], BF16)
    outs = tg.gemm_qkv(X, *[util.to_dev(w, BF16) for w in q["W"]])
    torch.cuda.synchronize()
    assert tg.last_kernel() == SK, tg.last_kernel()
    refs = oracle.gemm_qkv(BF16, q["X"], *q["W"])
    for t in range(3):
        util.check_exact(util.to_bits(outs[t]), refs[t][1], "stream-K qkv [%d]" % t)


def test_stream_k_replays_from_a_graph_with_eager_calls_between(tg, monkeypatch):
    # the tile counters are left at zero by every launch, so a captured call
    # replays with no reset, and eager calls between the replays share them
    import torch
    monkeypatch.setenv("TG_STREAMK", "2")
    dt, M, N, K = F16, 3072, 3072, 512
    p = inputs.problem(dt, M, N, K, seed=1300, kind="int", bias=True, bias_kind="int")
    A, B = util.to_dev(p["A"], dt), util.to_dev(p["B"], dt)
    bias = util.to_dev(p["bias"], dt)
    C = torch.empty((M, N), dtype=torch.float16, device="cuda")
    tg.gemm(A, B, out=C, bias=bias)  # workspace allocated outside the capture
    torch.cuda.synchronize()
    assert tg.last_kernel() == SK, tg.last_kernel()
    _, ref = oracle.gemm(dt, p["A"], p["B"], p["bias"])
    util.check_exact(util.to_bits(C), ref, "eager")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            tg.gemm(A, B, out=C, bias=bias)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i in range(3):
        C.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        util.check_exact(util.to_bits(C), ref, "replay %d" % i)
        C.fill_(float("nan"))
        tg.gemm(A, B, out=C, bias=bias)
        torch.cuda.synchronize()
        util.check_exact(util.to_bits(C), ref, "eager after replay %d" % i)


def test_stream_k_full_size_shapes_off_the_wave(tg, monkeypatch):
    # bf16 3584^3 (196 tiles, fewer than a wave, 22 quads per workgroup;
    # split only with TG_STREAMK=2) and 6144^3 (576 tiles: two waves whole,
    # 64 + 256 split, by default), every output against the oracle
    for n in (3584, 6144):
        monkeypatch.setenv("TG_STREAMK", "2" if n == 3584 else "1")
        p = inputs.problem(BF16, n, n, n, seed=1400 + n, kind="normal", b_scale=n ** -0.5)
        say("case stream-K %d^3" % n)
        bits, kern = run(tg, BF16, p["A"], p["B"], False)
        assert kern == SK, kern
        f64, rbits = oracle.gemm(BF16, p["A"], p["B"])
        util.check_tol(BF16, bits, f64, "stream-K %d^3" % n, ref_bits=rbits)


def test_stream_k_default_threshold(tg):
    # by default only grids of a whole wave or more split their short last
    # wave: 3000 x 11008 x 4096 (two waves + 4 tiles) takes stream-K; short
    # of a wave the grid stays whole: 3072^3 and 2049 x 4096 x 4096 (144
    # tiles of 256, 256 and 242 of 192) on 192 x 192 tiles, 3584^3 (196 of
    # 256, 361 of 192) on a partly filled wave of 256 x 256 tiles, where the
    # 32x32x16 kernel measured faster than the 16x16x32 one (83 against 87
    # us)
    import torch
    for (M, N, K), expect in (((3072, 3072, 3072), "async_192x192x32_s4_mfma16"),
                              ((3000, 11008, 4096), SK),
                              ((2049, 4096, 4096), "async_192x192x32_s4_mfma16"),
                              ((3584, 3584, 3584), "async_256x256x32_s4")):
        a = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
        b = torch.zeros((K, N), dtype=torch.bfloat16, device="cuda")
        tg.gemm(a, b)
        assert tg.last_kernel() == expect, ((M, N, K), tg.last_kernel())
    torch.cuda.synchronize()
