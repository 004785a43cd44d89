"""GPU checks of the C ABI's boundary rules that need a device: calls that
would have to grow the library's workspace while their stream is captured
into a graph, and argument views the binding must refuse before anything is
launched."""
import numpy as np
import pytest

import oracle
import util
from tiled_dense_gemm_09_amd import inputs

pytestmark = pytest.mark.gpu

F16, BF16 = inputs.F16, inputs.BF16
NOT_SUPPORTED = 2


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def tg():
    import torch
    assert torch.cuda.is_available()
    from tiled_dense_gemm_09_amd import tg as _tg
    return _tg


def capture(fn):
    """Capture fn() (plus a small marker kernel, so the graph is never empty)
    on a side stream; returns the graph, the marker tensor and whatever fn
    raised."""
    import torch
    mark = torch.zeros(16, device="cuda")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    raised = None
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            mark.add_(1.0)
            try:
                fn()
            except Exception as e:  # noqa: BLE001 -- inspected by the caller
                raised = e
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g, mark, raised


def test_cold_k_padding_call_under_capture_takes_a_kernel_without_workspace(tg):
    # K off the 8-element grid on a large problem normally copies A and B
    # into the workspace with K padded.  When the workspace would have to
    # grow during a capture, the call runs the tiled kernel (no workspace)
    # instead; the graph then replays correctly, with eager work between the
    # replays.
    import torch
    w0 = tg.workspace_bytes()
    n = 1024
    while 16384 + 4 * n * (n + 128) + 256 <= w0:
        n *= 2
    if n > 8192:
        pytest.skip("workspace already %d bytes" % w0)
    M, N, K = n, n, n + 4  # K rounds up to n + 128: 124 padded k, at most K / 8
    p = inputs.problem(F16, M, N, K, seed=700, kind="int", bias=True, bias_kind="int")
    # A in a buffer whose pitch (n + 8) is a multiple of 8, NaN in the padding
    abuf = np.full((M, n + 8), 0x7E00, np.uint16)
    abuf[:, :K] = p["A"]
    A, B = util.to_dev(abuf, F16)[:, :K], util.to_dev(p["B"], F16)
    bias = util.to_dev(p["bias"], F16)
    C = torch.empty((M, N), dtype=torch.float16, device="cuda")
    say("case cold K padding under capture", M, N, K, "workspace", w0)
    g, mark, raised = capture(lambda: tg.gemm(A, B, out=C, bias=bias))
    assert raised is None, raised
    kern = tg.last_kernel()
    say("  kernel", kern)
    assert kern.startswith("tiled_") and "stream capture" in kern, kern
    assert tg.workspace_bytes() == w0
    rows = [0, 1, M // 2, M - 1]
    refs = [oracle.gemm(F16, p["A"], p["B"], p["bias"], rows=(r, r + 1))[1] for r in rows]
    for i in range(3):
        C.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = util.to_bits(C)
        for r, ref in zip(rows, refs):
            util.check_exact(got[r:r + 1], ref, "replay %d row %d" % (i, r))
        tg.gemm(A, B, out=C, bias=bias)  # eager: now grows the workspace, K padded
        torch.cuda.synchronize()
        assert tg.last_kernel().endswith("_kpad"), tg.last_kernel()
        got = util.to_bits(C)
        for r, ref in zip(rows, refs):
            util.check_exact(got[r:r + 1], ref, "eager %d row %d" % (i, r))
    assert float(mark[0]) == 3.0
    assert tg.workspace_bytes() > w0


def test_cold_model_split_under_capture_runs_unsplit():
    # 128 x 4096 x 14336: the launch-time model splits K.  In a fresh process
    # (no workspace yet) a captured call would have to allocate it: it runs
    # the same tiles unsplit instead and says so, and the graph replays the
    # exact result; the same call made eagerly afterwards splits.  Integer
    # operands: every sum is exact in FP32, so the unsplit replay, the split
    # eager call and an FP32 reference round to the same bits.
    import json
    import os
    import subprocess
    import sys
    code = r"""
import json, torch
from tiled_dense_gemm_09_amd import tg
g0 = torch.Generator().manual_seed(702)
A = torch.randint(-2, 3, (128, 14336), generator=g0).to(torch.bfloat16).cuda()
B = torch.randint(-2, 3, (14336, 4096), generator=g0).to(torch.bfloat16).cuda()
C = torch.full((128, 4096), float("nan"), dtype=torch.bfloat16, device="cuda")
w0 = tg.workspace_bytes()
g = torch.cuda.CUDAGraph()
side = torch.cuda.Stream()
side.wait_stream(torch.cuda.current_stream())
with torch.cuda.stream(side):
    with torch.cuda.graph(g):
        tg.gemm(A, B, out=C)
torch.cuda.current_stream().wait_stream(side)
torch.cuda.synchronize()
k_cap = tg.last_kernel()
w1 = tg.workspace_bytes()
g.replay()
torch.cuda.synchronize()
rep = C.clone()
C.fill_(float("nan"))
tg.gemm(A, B, out=C)
torch.cuda.synchronize()
ref = (A.float() @ B.float()).to(torch.bfloat16)
print(json.dumps({"w0": w0, "w1": w1, "w2": tg.workspace_bytes(), "captured": k_cap,
                  "eager": tg.last_kernel(),
                  "replay_eq_eager": bool(torch.equal(rep.view(torch.int16), C.view(torch.int16))),
                  "eager_eq_ref": bool(torch.equal(C.view(torch.int16), ref.view(torch.int16)))}))
"""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                       timeout=100)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    say("  ", d)
    assert d["w0"] == 0 and d["w1"] == 0, d
    assert d["captured"].endswith("(unsplit: stream capture)"), d
    assert "_splitk" in d["eager"] and d["w2"] > 0, d
    assert d["replay_eq_eager"] and d["eager_eq_ref"], d


def test_cold_staged_call_under_capture_takes_the_element_wise_kernel(tg):
    # operands off the 16-byte grid on a large problem are normally staged
    # through aligned copies in the workspace; when the workspace would have
    # to grow during a capture, the call runs the tiled kernel with
    # element-wise loads and stores (no workspace) and says so; the graph
    # replays correctly, and the same call made eagerly afterwards is staged
    import torch
    w0 = tg.workspace_bytes()
    n = 1025
    while 16384 + 2 * (n * (n + 7) * 2 + n * (n + 7)) + 256 <= w0:
        n = 2 * n + 1
    if n > 8193:
        pytest.skip("workspace already %d bytes" % w0)
    M, N, K = n, n, n  # odd pitches: every operand off the grid
    p = inputs.problem(BF16, M, N, K, seed=702, kind="int", bias=True, bias_kind="int")
    A, B = util.to_dev(p["A"], BF16), util.to_dev(p["B"], BF16)
    bias = util.to_dev(p["bias"], BF16)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    say("case cold staged call under capture", M, N, K, "workspace", w0)
    g, mark, raised = capture(lambda: tg.gemm(A, B, out=C, bias=bias))
    assert raised is None, raised
    kern = tg.last_kernel()
    say("  kernel", kern)
    assert "_unaligned" in kern and "not staged: stream capture" in kern, kern
    assert tg.workspace_bytes() == w0
    rows = [0, M // 2, M - 1]
    refs = [oracle.gemm(BF16, p["A"], p["B"], p["bias"], rows=(r, r + 1))[1] for r in rows]
    for i in range(2):
        C.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = util.to_bits(C)
        for r, ref in zip(rows, refs):
            util.check_exact(got[r:r + 1], ref, "replay %d row %d" % (i, r))
        tg.gemm(A, B, out=C, bias=bias)
        torch.cuda.synchronize()
        assert tg.last_kernel().endswith("_staged"), tg.last_kernel()
        got = util.to_bits(C)
        for r, ref in zip(rows, refs):
            util.check_exact(got[r:r + 1], ref, "eager %d row %d" % (i, r))
    assert float(mark[0]) == 2.0
    assert tg.workspace_bytes() > w0


def test_cold_split_k_call_under_capture_launches_nothing(tg, monkeypatch):
    # a split-K call whose workspace would have to grow inside a capture
    # returns TG_ERROR_NOT_SUPPORTED, says why, and captures no launch: the
    # replayed graph leaves the output untouched.  The same call made eagerly
    # afterwards grows the workspace and is exact.
    import torch
    monkeypatch.setenv("TG_FORCE_CONFIG", "async_128x128x32_s4")
    monkeypatch.setenv("TG_SPLITK", "8")
    w0 = tg.workspace_bytes()
    n = 1024
    while 16384 + 8 * n * n * 4 <= w0:
        n *= 2
    if n > 8192:
        pytest.skip("workspace already %d bytes" % w0)
    M, N, K = n, n, 1024
    p = inputs.problem(BF16, M, N, K, seed=701, kind="int")
    A, B = util.to_dev(p["A"], BF16), util.to_dev(p["B"], BF16)
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    say("case cold split-K under capture", M, N, K, "workspace", w0)
    g, mark, raised = capture(lambda: tg.gemm(A, B, out=C))
    assert isinstance(raised, tg.TgError) and raised.status == NOT_SUPPORTED, raised
    assert "stream capture" in tg.last_kernel(), tg.last_kernel()
    assert tg.workspace_bytes() == w0
    g.replay()
    torch.cuda.synchronize()
    assert float(mark[0]) == 1.0
    assert bool(torch.isnan(C).all()), "the failed call launched something"
    tg.gemm(A, B, out=C)
    torch.cuda.synchronize()
    assert tg.last_kernel() == "async_128x128x32_s4_splitk8", tg.last_kernel()
    assert tg.workspace_bytes() > w0
    got = util.to_bits(C)
    for r in (0, M // 3, M - 1):
        _, ref = oracle.gemm(BF16, p["A"], p["B"], rows=(r, r + 1))
        util.check_exact(got[r:r + 1], ref, "eager split-K row %d" % r)


def test_overlapping_views_and_host_bias_are_refused(tg):
    # a broadcast row (stride 0) or rows that overlap would make the library
    # read or write a full pitch per row past the allocation; a host bias is
    # not a device pointer.  All are refused in the binding, before any call.
    import torch
    K, N = 256, 256
    row = torch.zeros((1, K), dtype=torch.float16, device="cuda")
    b = torch.zeros((K, N), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError, match="overlapping rows"):
        tg.gemm(row.expand(64, K), b)
    flat = torch.zeros(64 * K, dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError, match="overlapping rows"):
        tg.gemm(flat.as_strided((64, K), (K // 2, 1)), b)
    out = torch.zeros((1, N), dtype=torch.float16, device="cuda").expand(64, N)
    a = torch.zeros((64, K), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError, match="overlapping rows"):
        tg.gemm(a, b, out=out)
    with pytest.raises(ValueError, match="device"):
        tg.gemm(a, b, bias=torch.zeros(N, dtype=torch.float16))
    with pytest.raises(ValueError, match="device"):
        tg.gemm(a, b, residual=torch.zeros((64, N), dtype=torch.float16))
    x = torch.zeros((64, K), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((1, N), dtype=torch.bfloat16, device="cuda").expand(K, N)
    with pytest.raises(ValueError, match="overlapping rows"):
        tg.gemm_qkv(x, w, w, w)
    a8 = torch.zeros((256, 256), dtype=torch.uint8, device="cuda")
    s8 = torch.full((8, 256), 127, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="device"):
        tg.gemm_mx(a8, s8, a8, s8, bias=torch.zeros(256, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="overlapping rows"):
        tg.gemm_mx(torch.zeros((1, 256), dtype=torch.uint8, device="cuda").expand(256, 256), s8,
                   a8, s8)
    torch.cuda.synchronize()


def test_log_prints_each_choice_and_the_model_estimates():
    # TG_LOG is read once per process: a child process with TG_LOG=2 prints
    # the chosen kernel and the launch-time model's estimate of every
    # candidate (a grid short of a wave of 256 x 256 tiles)
    import os
    import subprocess
    import sys
    code = ("import torch\n"
            "from tiled_dense_gemm_09_amd import tg\n"
            "x = torch.zeros((256, 4096), dtype=torch.bfloat16, device='cuda')\n"
            "w = torch.zeros((4096, 4096), dtype=torch.bfloat16, device='cuda')\n"
            "tg.gemm(x, w)\n"
            "torch.cuda.synchronize()\n"
            "print(tg.last_kernel())\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, TG_LOG="2")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, env=env, capture_output=True,
                       text=True, timeout=100)
    assert r.returncode == 0, r.stderr[-2000:]
    chosen = r.stdout.strip().splitlines()[-1]
    estimates = [l for l in r.stderr.splitlines() if l.startswith("[tg] model 256x4096x4096:")]
    assert len(estimates) >= 4, r.stderr[-2000:]
    assert "[tg] kernel: " + chosen in r.stderr, (chosen, r.stderr[-2000:])
    assert any(chosen.split("_splitk")[0] + "," in l for l in estimates), (chosen, estimates)


@pytest.mark.parametrize("trans_b", [False, True])
def test_pair_staged_kernel_replays_in_a_graph(tg, trans_b):
    # a full wave of 256 x 256 tiles takes the pair-staged loop, which needs
    # no workspace: captured, then replayed three times with the eager call
    # between the replays, every result equal to the oracle's on sampled rows
    import torch
    M, N, K = 4096, 4096, 512
    p = inputs.problem(BF16, M, N, K, seed=710 + int(trans_b), kind="int", bias=True,
                       bias_kind="int")
    A = util.to_dev(p["A"], BF16)
    Bd = util.to_dev(np.ascontiguousarray(p["B"].T) if trans_b else p["B"], BF16)
    B = Bd.t() if trans_b else Bd
    bias = util.to_dev(p["bias"], BF16)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    say("case pair-staged kernel in a graph", M, N, K, "B[N,K]" if trans_b else "B[K,N]")
    g, mark, raised = capture(lambda: tg.gemm(A, B, out=C, bias=bias))
    assert raised is None, raised
    assert tg.last_kernel() == "async_256x256x32p_s4_mfma16", tg.last_kernel()
    rows = [0, 1, 255, 256, M // 2 + 3, M - 1]
    refs = [oracle.gemm(BF16, p["A"], p["B"], p["bias"], rows=(r, r + 1))[1] for r in rows]
    for i in range(3):
        C.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = util.to_bits(C)
        for r, ref in zip(rows, refs):
            util.check_exact(got[r:r + 1], ref, "replay %d row %d" % (i, r))
        C.fill_(float("nan"))
        tg.gemm(A, B, out=C, bias=bias)
        torch.cuda.synchronize()
        assert tg.last_kernel() == "async_256x256x32p_s4_mfma16", tg.last_kernel()
        got = util.to_bits(C)
        for r, ref in zip(rows, refs):
            util.check_exact(got[r:r + 1], ref, "eager %d row %d" % (i, r))
    assert float(mark[0]) == 3.0
