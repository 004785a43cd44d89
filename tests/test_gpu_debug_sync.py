"""The synchronising build against the library, on every kernel family.

libtg_debugsync.so is the library's sources compiled with TG_DEBUG_SYNC:
every partial wait of a copy pipeline (direct global-to-LDS copies in flight
while earlier stages are read) waits for all outstanding memory operations
instead, and every pipeline barrier waits for them first.  Both builds do
the same arithmetic in the same order, so their outputs must be equal bit
for bit.  A difference means that in the library some wave read an LDS stage
before every copy into it had landed, or a copy refilled a stage that a wave
was still reading: a race the parity tests can miss when its timing window
rarely opens.  Operands are random normals, not integers, so a stale or
half-written stage changes the result bits.
"""
import pytest

pytestmark = pytest.mark.gpu

ENV_KEYS = ("TG_FORCE_CONFIG", "TG_SPLITK", "TG_STREAMK", "TG_SKINNY_COLS", "TG_SKINNY_BN",
            "TG_SKINNY_SPLITS", "TG_SKINNY_REGS", "TG_ATTN_BM")


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def libs():
    import torch
    assert torch.cuda.is_available()
    from tiled_dense_gemm_09_amd import tg
    return tg, tg.lib, tg.load_library(tg.DEBUG_SYNC_PATH)


def rnd(shape, dt, gen, scale=1.0):
    import torch
    return (torch.randn(shape, generator=gen, device="cuda") * scale).to(dt)


def gemm_case(M, N, K, dt="f16", bias=True, act="gelu_tanh", bt=False, a_pad=0, b_pad=0,
              residual=False):
    """Inputs for tg.gemm, drawn once (A and B carved out of buffers a_pad and
    b_pad elements wider than their rows); the returned function runs the
    call."""
    import torch

    def setup(gen):
        t = torch.float16 if dt == "f16" else torch.bfloat16
        a = rnd((M, K + a_pad), t, gen)[:, :K]
        if bt:
            b = rnd((N, K), t, gen, K ** -0.5).t()
        else:
            b = rnd((K, N + b_pad), t, gen, K ** -0.5)[:, :N]
        bb = rnd((N,), t, gen) if bias else None
        r = rnd((M, N), t, gen) if residual else None
        return lambda tg: [tg.gemm(a, b, bias=bb, act=act, residual=r)]
    return setup


def qkv_case(M, N, K):
    import torch

    def setup(gen):
        x = rnd((M, K), torch.bfloat16, gen)
        w = [rnd((K, N), torch.bfloat16, gen, K ** -0.5) for _ in range(3)]
        return lambda tg: list(tg.gemm_qkv(x, *w))
    return setup


def mx_case(M, N, K, fmt="e4m3"):
    import torch

    def setup(gen):
        # a [M,K] and b [N,K]: 8-bit codes away from NaN (e4m3: magnitude
        # codes below 0x7e), signed for a; scales [K/32, M] and [K/32, N] near 2^0
        a = torch.randint(0, 0x7E, (M, K), generator=gen, device="cuda", dtype=torch.int32)
        a = (a | (torch.randint(0, 2, (M, K), generator=gen, device="cuda",
                                dtype=torch.int32) << 7)).to(torch.uint8)
        b = torch.randint(0, 0x7E, (N, K), generator=gen, device="cuda",
                          dtype=torch.int32).to(torch.uint8)
        sa = torch.randint(120, 128, (K // 32, M), generator=gen, device="cuda",
                           dtype=torch.int32).to(torch.uint8)
        sb = torch.randint(120, 128, (K // 32, N), generator=gen, device="cuda",
                           dtype=torch.int32).to(torch.uint8)
        bias = rnd((N,), torch.bfloat16, gen)
        return lambda tg: [tg.gemm_mx(a, sa, b, sb, fmt, fmt, bias=bias, act="gelu_tanh")]
    return setup


def attn_case(B, H, S, D, causal):
    import torch

    def setup(gen):
        q, k, v = (rnd((B, H, S, D), torch.bfloat16, gen) for _ in range(3))
        return lambda tg: list(tg.attention(q, k, v, causal=causal, lse=True))
    return setup


# (id, environment, inputs, expected kernel-name prefix)
CASES = [
    ("async16p_4096_gelu", {}, gemm_case(4096, 4096, 1024), "async_256x256x32p_s4_mfma16"),
    ("async16_bt_bf16", {"TG_FORCE_CONFIG": "async_256x256x32_s4_mfma16"},
     gemm_case(512, 512, 2048, "bf16", bt=True), "async_256x256x32_s4_mfma16"),
    ("async16p_bt_residual", {"TG_FORCE_CONFIG": "async_256x256x32p_s4_mfma16"},
     gemm_case(512, 768, 1024, "bf16", bt=True, residual=True), "async_256x256x32p_s4_mfma16"),
    ("async16_residual", {"TG_FORCE_CONFIG": "async_256x256x32_s4_mfma16"},
     gemm_case(512, 768, 1024, residual=True), "async_256x256x32_s4_mfma16"),
    ("async16_kmask", {}, gemm_case(4096, 4096, 1000), "async_256x256x32_s4_mfma16"),
    ("async16_streamk", {"TG_STREAMK": "2"}, gemm_case(3072, 3072, 1024, "bf16"),
     "async_256x256x32_s4_mfma16_streamk"),
    ("async16_192", {}, gemm_case(3072, 3072, 1024, "bf16"), "async_192x192x32_s4_mfma16"),
    ("async16_192_bt_kmask", {"TG_FORCE_CONFIG": "async_192x192x32_s4_mfma16"},
     gemm_case(576, 768, 1000, bt=True, residual=True), "async_192x192x32_s4_mfma16"),
    ("async16_128_bt_kmask", {"TG_FORCE_CONFIG": "async_128x128x32_s4_mfma16"},
     gemm_case(384, 512, 1000, bt=True, residual=True), "async_128x128x32_s4_mfma16"),
    ("async16_128k64_kmask", {"TG_FORCE_CONFIG": "async_128x128x64_s4_mfma16"},
     gemm_case(384, 512, 1000, residual=True), "async_128x128x64_s4_mfma16"),
    ("async16_w8", {"TG_FORCE_CONFIG": "async_256x256x32_s4_mfma16_w8"},
     gemm_case(512, 512, 1024), "async_256x256x32_s4_mfma16_w8"),
    ("async32_256", {"TG_FORCE_CONFIG": "async_256x256x32_s4"},
     gemm_case(512, 512, 1024, "bf16"), "async_256x256x32_s4"),
    ("async32_128", {"TG_FORCE_CONFIG": "async_128x128x32_s4"}, gemm_case(512, 512, 1024),
     "async_128x128x32_s4"),
    ("async32_64x128_bt", {"TG_FORCE_CONFIG": "async_64x128x32_s4"},
     gemm_case(256, 384, 1024, "bf16", bt=True), "async_64x128x32_s4"),
    ("async32_64", {"TG_FORCE_CONFIG": "async_64x64x32_s4"}, gemm_case(256, 256, 1024),
     "async_64x64x32_s4"),
    ("async32_splitk", {"TG_FORCE_CONFIG": "async_128x128x32_s4", "TG_SPLITK": "4"},
     gemm_case(512, 512, 2048, "bf16"), "async_128x128x32_s4_splitk4"),
    ("kpad", {}, gemm_case(2048, 2048, 1028, a_pad=4), "async_128x128x32_s4_kpad"),
    ("tiled_256", {"TG_FORCE_CONFIG": "tiled_256x256x64_w2x2"}, gemm_case(512, 512, 512),
     "tiled_256x256x64_w2x2"),
    ("tiled_128_edges", {"TG_FORCE_CONFIG": "tiled_128x128x64_w2x2"},
     gemm_case(200, 136, 520, "bf16"), "tiled_128x128x64_w2x2"),
    ("tiled_unaligned", {}, gemm_case(300, 264, 264, a_pad=3, b_pad=3), "tiled_"),
    ("staged", {}, gemm_case(1100, 1003, 1024, "bf16", b_pad=1), "async_"),
    ("generic_bt", {"TG_FORCE_CONFIG": "generic"}, gemm_case(64, 96, 80, bt=True),
     "generic_fma"),
    ("skinny_bn128", {}, gemm_case(16, 2048, 2048, "bf16", bias=False, act="none"),
     "skinny_stream_bn128"),
    ("skinny_bn256", {"TG_SKINNY_BN": "256"}, gemm_case(16, 4096, 2048, "bf16"),
     "skinny_stream_bn256"),
    ("skinny_m32", {}, gemm_case(32, 2048, 2048), "skinny_stream_bn128"),
    ("skinny_registers", {"TG_SKINNY_REGS": "1"}, gemm_case(16, 1000, 1024), "skinny_bn"),
    ("skinny_cols", {"TG_SKINNY_COLS": "1"}, gemm_case(16, 4096, 2048, "bf16"), "skinny_cols"),
    ("skinny_realign", {}, gemm_case(16, 4099, 2048, "bf16", b_pad=3), "skinny_realign"),
    ("skinny_nk", {}, gemm_case(16, 4096, 4096, "bf16", bt=True), "skinny_nk"),
    ("skinny_nk_m32_tail", {}, gemm_case(24, 1000, 1000, bt=True, residual=True), "skinny_nk"),
    ("skinny_realign_m32_xstaged", {}, gemm_case(24, 1500, 1000, a_pad=3, b_pad=1, residual=True),
     "skinny_realign"),
    ("qkv", {}, qkv_case(1024, 1024, 1024), "async"),
    ("mx_e4m3", {}, mx_case(1024, 1024, 1024), "mx_256x256x64_s4"),
    ("attention_full", {}, attn_case(1, 2, 1024, 128, False), "attn"),
    ("attention_causal", {}, attn_case(1, 2, 1024, 128, True), "attn"),
]


@pytest.mark.parametrize("cid,env,setup,prefix", CASES, ids=[c[0] for c in CASES])
def test_synchronising_build_gives_the_same_bits(libs, monkeypatch, cid, env, setup, prefix):
    import torch
    tg, lib, dbg = libs
    for k in ENV_KEYS:
        monkeypatch.delenv(k, raising=False)
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(sum(map(ord, cid)))
    run = setup(gen)
    say("case", cid, env)
    outs = {}
    for name, handle in (("library", lib), ("synchronising", dbg)):
        monkeypatch.setattr(tg, "lib", handle)
        got = run(tg)
        torch.cuda.synchronize()
        outs[name] = ([t.detach().clone() for t in got], tg.last_kernel())
    monkeypatch.setattr(tg, "lib", lib)
    (ref, kern), (chk, kern_dbg) = outs["library"], outs["synchronising"]
    say("  kernel", kern, "|", kern_dbg)
    assert kern.startswith(prefix), kern
    assert kern_dbg == kern
    for i, (a, b) in enumerate(zip(ref, chk)):
        av = a.contiguous().view(torch.int8) if a.element_size() == 1 else \
            a.contiguous().view(torch.int16 if a.element_size() == 2 else torch.int32)
        bv = b.contiguous().view(av.dtype)
        diff = int((av != bv).sum())
        assert diff == 0, "%s output %d: %d of %d elements differ between the builds" % (
            cid, i, diff, av.numel())
