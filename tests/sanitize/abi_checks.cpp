// Host-side checks of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (built host-only, run on the CPU, no GPU).
//
// tg_api.cpp is compiled with the sanitizers and linked with the stubs
// below in place of the kernel files' launchers: every call made here must
// be rejected, or be a no-op, before any kernel is chosen or launched, so a
// stub that runs aborts the check.  The calls cover the argument validation
// (NULL pointers, negative, huge and overflowing sizes and pitches,
// overlapping outputs, unknown enums) and the host-side helpers, including
// arguments at the edges of their ranges.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "tg.h"
#include "tg_launch.h"

// line of the check being evaluated and the index of the table row, for
// the report of a stub that runs
static int g_line = 0, g_case = -1;

namespace tg {
[[noreturn]] static void reached(const char *what)
{
    fprintf(stderr,
            "check failed: %s reached from a call that should launch nothing (line %d, case %d)\n",
            what, g_line, g_case);
    abort();
}
int num_tile_configs() { reached("num_tile_configs"); }
const TileConfig &tile_config(int) { reached("tile_config"); }
hipError_t launch_tiled(int, int, int, const GemmArgs &, int, hipStream_t) { reached("launch_tiled"); }
bool tiled_unaligned(const GemmArgs &) { reached("tiled_unaligned"); }
hipError_t launch_generic(int, int, const GemmArgs &, hipStream_t) { reached("launch_generic"); }
int num_async_configs() { reached("num_async_configs"); }
const char *async_config_name(int) { reached("async_config_name"); }
bool async_forced_only(int) { reached("async_forced_only"); }
bool async_mfma16(int) { reached("async_mfma16"); }
bool async_pairs(int) { reached("async_pairs"); }
int async_tile_m(int) { reached("async_tile_m"); }
int async_tile_n(int) { reached("async_tile_n"); }
int async_k_step(int) { reached("async_k_step"); }
bool async_eligible(const GemmArgs &, int, bool) { reached("async_eligible"); }
int async_tiles_m(const GemmArgs &, int) { reached("async_tiles_m"); }
int async_tiles_n(const GemmArgs &, int) { reached("async_tiles_n"); }
int plan_async_splits(const GemmArgs &, int, int) { reached("plan_async_splits"); }
size_t async_ws_floats(const GemmArgs &, int, int) { reached("async_ws_floats"); }
hipError_t launch_async(int, int, int, const GemmArgs &, int, int, float *, int *, hipStream_t)
{
    reached("launch_async");
}
SkPlan plan_stream_k(const GemmArgs &, int, int, bool) { reached("plan_stream_k"); }
size_t stream_k_ws_floats(const SkPlan &) { reached("stream_k_ws_floats"); }
hipError_t launch_async_sk(int, int, int, const GemmArgs &, int, const SkPlan &, float *, int *,
                           hipStream_t)
{
    reached("launch_async_sk");
}
bool mx_fast_eligible(const MxArgs &) { reached("mx_fast_eligible"); }
hipError_t launch_mx(int, int, const MxArgs &, int, hipStream_t) { reached("launch_mx"); }
hipError_t launch_mx_generic(int, int, const MxArgs &, hipStream_t) { reached("launch_mx_generic"); }
bool attn_fast_eligible(const AttnArgs &, int) { reached("attn_fast_eligible"); }
int attn_block_m(const AttnArgs &, int) { reached("attn_block_m"); }
hipError_t launch_attn(int, bool, int, const AttnArgs &, hipStream_t) { reached("launch_attn"); }
hipError_t launch_attn_generic(int, bool, const AttnArgs &, int, hipStream_t)
{
    reached("launch_attn_generic");
}
hipError_t launch_pad_copy(const unsigned short *, int64_t, int, int, unsigned short *, int, int,
                           hipStream_t)
{
    reached("launch_pad_copy");
}
hipError_t launch_unpad_copy(const unsigned short *, int, unsigned short *, int64_t, int, int,
                             hipStream_t)
{
    reached("launch_unpad_copy");
}
SkinnyPlan plan_skinny(int, int, int) { reached("plan_skinny"); }
SkinnyPlan plan_skinny_realign(int, int, int, int) { reached("plan_skinny_realign"); }
SkinnyPlan plan_skinny_nk(int, int, int, int) { reached("plan_skinny_nk"); }
size_t skinny_ws_floats(const SkinnyPlan &, int, int) { reached("skinny_ws_floats"); }
hipError_t launch_skinny(int, int, const GemmArgs &, const SkinnyPlan &, float *, int *, hipStream_t)
{
    reached("launch_skinny");
}
} // namespace tg

static int failures = 0;
#define EXPECT(cond)                                                                             \
    do {                                                                                         \
        g_line = __LINE__;                                                                       \
        if (!(cond)) {                                                                           \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);                   \
            ++failures;                                                                          \
        }                                                                                        \
    } while (0)

// Fake device addresses: never dereferenced on the host, only compared.
static void *P(uint64_t a) { return reinterpret_cast<void *>(a); }
static const uint64_t A0 = 0x7F0000000000ull, B0 = 0x7F0010000000ull, C0 = 0x7F0020000000ull,
                      R0 = 0x7F0030000000ull, S0 = 0x7F0040000000ull, T0 = 0x7F0050000000ull;
static const int64_t BIG = (int64_t)1 << 62, HUGE_ = INT64_MAX;

int main()
{
    const tg_dtype F16 = TG_DTYPE_F16;
    // plain GEMM: every kind of invalid argument
    struct Case {
        int dt;
        int64_t M, N, K, lda, ldb, ldc;
        uint64_t A, B, C;
    } cases[] = {
        {7, 64, 64, 32, 32, 64, 64, A0, B0, C0},        // unknown dtype
        {1, -1, 64, 32, 32, 64, 64, A0, B0, C0},        // negative size
        {1, 64, -5, 32, 32, 64, 64, A0, B0, C0},
        {1, 64, 64, -32, 32, 64, 64, A0, B0, C0},
        {1, (int64_t)1 << 31, 64, 32, 32, 64, 64, A0, B0, C0}, // size past 2^31
        {1, 64, 64, HUGE_, HUGE_, 64, 64, A0, B0, C0},
        {1, 64, 64, 32, 31, 64, 64, A0, B0, C0},        // short pitches
        {1, 64, 64, 32, 32, 63, 64, A0, B0, C0},
        {1, 64, 64, 32, 32, 64, 63, A0, B0, C0},
        {1, 64, 64, 32, -1, 64, 64, A0, B0, C0},        // negative pitch
        {1, 64, 64, 32, 32, 64, 64, 0, B0, C0},         // NULL pointers
        {1, 64, 64, 32, 32, 64, 64, A0, 0, C0},
        {1, 64, 64, 32, 32, 64, 64, A0, B0, 0},
        {1, 64, 64, 32, 32, 64, 64, A0, B0, A0 + 64},   // C overlaps A
        {1, 64, 64, 32, 32, 64, 64, A0, B0, B0 + 2048}, // C overlaps B
        // pitches whose row extents overflow 64-bit arithmetic
        {1, 64, 64, 32, BIG, 64, 64, A0, B0, C0},
        {1, 64, 64, 32, 32, BIG, 64, A0, B0, C0},
        {1, 64, 64, 32, 32, 64, BIG, A0, B0, C0},
        {1, ((int64_t)1 << 31) - 1, 64, 32, HUGE_ / 2, 64, 64, A0, B0, C0},
        {1, 64, ((int64_t)1 << 31) - 1, 32, 32, HUGE_, HUGE_, A0, B0, C0},
        // an output at the top of the address space: its extent wraps
        {1, 64, 64, 32, 32, 64, 64, A0, B0, UINT64_MAX - 64},
    };
    for (const Case &c : cases) {
        g_case = (int)(&c - cases);
        EXPECT(tg_gemm((tg_dtype)c.dt, c.M, c.N, c.K, P(c.A), c.lda, P(c.B), c.ldb, P(c.C), c.ldc,
                       nullptr) == TG_ERROR_INVALID_VALUE);
        EXPECT(tg_gemm_bias_act((tg_dtype)c.dt, c.M, c.N, c.K, P(c.A), c.lda, P(c.B), c.ldb,
                                P(S0), TG_ACT_GELU_TANH, P(c.C), c.ldc,
                                nullptr) == TG_ERROR_INVALID_VALUE);
        EXPECT(tg_gemm_bias_act_noalloc((tg_dtype)c.dt, c.M, c.N, c.K, P(c.A), c.lda, P(c.B),
                                        c.ldb, nullptr, TG_ACT_NONE, P(c.C), c.ldc,
                                        nullptr) == TG_ERROR_INVALID_VALUE);
        EXPECT(tg_gemm_ex((tg_dtype)c.dt, c.M, c.N, c.K, P(c.A), c.lda, P(c.B), c.ldb, TG_OP_N,
                          nullptr, TG_ACT_NONE, nullptr, 0, P(c.C), c.ldc,
                          nullptr) == TG_ERROR_INVALID_VALUE);
    }
    // bias, activation, residual and operand-form errors
    EXPECT(tg_gemm_bias_act(F16, 64, 64, 32, P(A0), 32, P(B0), 64, P(S0 + 1), TG_ACT_NONE, P(C0),
                            64, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_gemm_bias_act(F16, 64, 64, 32, P(A0), 32, P(B0), 64, nullptr, (tg_act)9, P(C0), 64,
                            nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_gemm_bias_act(F16, 64, 64, 32, P(A0), 32, P(B0), 64, P(C0 + 8), TG_ACT_NONE, P(C0),
                            64, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_gemm_ex(F16, 64, 64, 32, P(A0), 32, P(B0), 32, (tg_op)5, nullptr, TG_ACT_NONE,
                      nullptr, 0, P(C0), 64, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_gemm_ex(F16, 64, 64, 32, P(A0), 32, P(B0), 31, TG_OP_T, nullptr, TG_ACT_NONE,
                      nullptr, 0, P(C0), 64, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_gemm_ex(F16, 64, 64, 32, P(A0), 32, P(B0), 32, TG_OP_T, nullptr, TG_ACT_NONE,
                      P(R0 + 1), 64, P(C0), 64, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_gemm_ex(F16, 64, 64, 32, P(A0), 32, P(B0), 32, TG_OP_T, nullptr, TG_ACT_NONE,
                      P(C0 + 128), 64, P(C0), 64, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_gemm_ex(F16, 64, 64, 32, P(A0), 32, P(B0), 32, TG_OP_T, nullptr, TG_ACT_NONE,
                      P(R0), BIG, P(C0), 64, nullptr) == TG_ERROR_INVALID_VALUE);
    // QKV: outputs overlapping each other or the weights
    EXPECT(tg_gemm_qkv(F16, 64, 64, 32, P(A0), 32, P(B0), P(B0 + 8192), P(B0 + 16384), 64, P(C0),
                       P(C0 + 4096), P(C0 + 16384), 64, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_gemm_qkv(F16, 64, 64, 32, P(A0), 32, P(B0), P(B0 + 8192), P(B0 + 16384), 64, P(C0),
                       P(B0 + 8192), P(C0 + 65536), 64, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_gemm_qkv(F16, 64, 64, 32, P(A0), 32, P(B0), nullptr, P(B0 + 16384), 64, P(C0),
                       P(C0 + 16384), P(C0 + 65536), 64, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_gemm_qkv(F16, 64, 64, 32, P(A0), 32, P(B0), P(B0 + 8192), P(B0 + 16384), BIG,
                       P(C0), P(C0 + 16384), P(C0 + 65536), 64, nullptr) == TG_ERROR_INVALID_VALUE);
    // no-ops: nothing is chosen or launched
    EXPECT(tg_gemm(F16, 0, 64, 32, P(A0), 32, P(B0), 64, P(C0), 64, nullptr) == TG_SUCCESS);
    EXPECT(tg_gemm(F16, 64, 0, 32, nullptr, 32, nullptr, 64, nullptr, 64, nullptr) == TG_SUCCESS);
    EXPECT(strcmp(tg_last_kernel(), "none") == 0);
    EXPECT(tg_gemm_ex(F16, 0, 64, 64, P(A0), 64, P(B0), 64, TG_OP_T, nullptr, TG_ACT_NONE, P(C0),
                      64, P(C0), 64, nullptr) == TG_SUCCESS);
    // block-scaled GEMM
    struct MxCase {
        int fa, fb, odt;
        int64_t M, N, K, lda, ldsa, ldb, ldsb, ldc;
        uint64_t A, SA, B, SB, C;
    } mx[] = {
        {3, 0, 2, 256, 256, 64, 64, 256, 64, 256, 256, A0, S0, B0, T0, C0},
        {0, 0, 7, 256, 256, 64, 64, 256, 64, 256, 256, A0, S0, B0, T0, C0},
        {0, 0, 2, 256, 256, 48, 64, 256, 64, 256, 256, A0, S0, B0, T0, C0},
        {0, 0, 2, 256, 256, 64, 63, 256, 64, 256, 256, A0, S0, B0, T0, C0},
        {0, 0, 2, 256, 256, 64, 64, 255, 64, 256, 256, A0, S0, B0, T0, C0},
        {0, 0, 2, 256, 256, 64, 64, 256, 64, 256, 256, A0, 0, B0, T0, C0},
        {0, 0, 2, 256, 256, 64, 64, 256, 64, 256, 256, A0, S0, B0, T0, A0 + 128},
        {0, 0, 2, 256, 256, 64, BIG, 256, 64, 256, 256, A0, S0, B0, T0, C0},
        {0, 0, 2, 256, 256, 64, 64, BIG, 64, 256, 256, A0, S0, B0, T0, C0},
        {0, 0, 2, 256, 256, 64, 64, 256, 64, 256, BIG, A0, S0, B0, T0, C0},
        {0, 0, 2, -256, 256, 64, 64, 256, 64, 256, 256, A0, S0, B0, T0, C0},
        {0, 0, 2, 256, 256, HUGE_ / 32 * 32, HUGE_, 256, HUGE_, 256, 256, A0, S0, B0, T0, C0},
    };
    g_case = -1;
    for (const MxCase &c : mx)
        if ((g_case = (int)(&c - mx)) >= 0)
            EXPECT(tg_gemm_mx((tg_fp8_format)c.fa, (tg_fp8_format)c.fb, c.M, c.N, c.K, P(c.A), c.lda,
                          P(c.SA), c.ldsa, P(c.B), c.ldb, P(c.SB), c.ldsb, nullptr, TG_ACT_NONE,
                          (tg_dtype)c.odt, P(c.C), c.ldc, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_gemm_mx(TG_FP8_E4M3, TG_FP8_E4M3, 0, 256, 64, P(A0), 64, P(S0), 0, P(B0), 64, P(T0),
                      256, nullptr, TG_ACT_NONE, TG_DTYPE_BF16, P(C0), 256, nullptr) == TG_SUCCESS);
    // attention
    EXPECT(tg_attention_fwd((tg_dtype)5, 1, 1, 128, 128, P(A0), P(B0), P(R0), P(C0), nullptr,
                            0.f, 0, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_attention_fwd(F16, -1, 1, 128, 128, P(A0), P(B0), P(R0), P(C0), nullptr, 0.f, 0,
                            nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_attention_fwd(F16, 1, 1, 128, 256, P(A0), P(B0), P(R0), P(C0), nullptr, 0.f, 0,
                            nullptr) == TG_ERROR_NOT_SUPPORTED);
    EXPECT(tg_attention_fwd(F16, BIG, BIG, BIG, 128, P(A0), P(B0), P(R0), P(C0), nullptr, 0.f, 0,
                            nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_attention_fwd(F16, (int64_t)1 << 20, (int64_t)1 << 20, 128, 128, P(A0), P(B0),
                            P(R0), P(C0), nullptr, 0.f, 0, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_attention_fwd(F16, 1, 2, 128, 128, P(A0), P(B0), P(R0), P(A0 + 256), nullptr, 0.f,
                            1, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_attention_fwd(F16, 1, 2, 128, 128, P(A0), P(B0), P(R0), P(C0), (float *)(C0 + 64),
                            0.f, 1, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_attention_fwd(F16, 0, 2, 128, 128, nullptr, nullptr, nullptr, nullptr, nullptr, 0.f,
                            0, nullptr) == TG_SUCCESS);
    // diagnostics and host helpers over their ranges and past them
    for (int s = -3; s < 10; ++s)
        EXPECT(tg_status_string((tg_status)s) != nullptr);
    EXPECT(strcmp(tg_status_string((tg_status)99), "TG_UNKNOWN_STATUS") == 0);
    int64_t mat, tm, tn;
    for (int64_t tiles_m : {1, 3, 7, 16, 33})
        for (int64_t tiles_n : {1, 2, 5, 16, 31})
            for (int64_t n_mat : {1, 3})
                for (int64_t g : {1, 4, 8, 64}) {
                    const int64_t total = tiles_m * tiles_n * n_mat;
                    for (int64_t b = -2; b < total + 2; ++b) {
                        const int rc = tg_schedule_tile(tiles_m, tiles_n, n_mat, g, b, &mat, &tm,
                                                        &tn);
                        EXPECT((rc == 0) == (b >= 0 && b < total));
                        if (rc == 0)
                            EXPECT(mat >= 0 && mat < n_mat && tm >= 0 && tm < tiles_m &&
                                   tn >= 0 && tn < tiles_n);
                    }
                }
    EXPECT(tg_schedule_tile(0, 4, 1, 4, 0, &mat, &tm, &tn) == -1);
    EXPECT(tg_schedule_tile(BIG, BIG, 1, 4, 0, &mat, &tm, &tn) == -1);
    EXPECT(tg_schedule_tile(1 << 20, 1 << 20, 3, 4, 5, &mat, &tm, &tn) == -1);
    EXPECT(tg_schedule_tile(4, 4, 1, HUGE_, 3, &mat, &tm, &tn) == -1 ||
           (tm >= 0 && tm < 4 && tn >= 0 && tn < 4));
    for (int layout = -1; layout < 8; ++layout)
        for (int64_t r : {(int64_t)-1, (int64_t)0, (int64_t)5, (int64_t)1 << 40, HUGE_})
            EXPECT(tg_lds_swizzle(layout, r) >= -1);
    for (int64_t cols : {8, 64, 128, 256})
        for (int64_t row = 0; row < 64; ++row)
            EXPECT(tg_lds_offset(cols, row, cols - 1) >= 0);
    for (int64_t v : {(int64_t)-1, (int64_t)0, (int64_t)7, BIG, HUGE_})
        EXPECT(tg_in_bounds(16, 16, v, 0) == (v >= 0 && v < 16));
    if (failures)
        fprintf(stderr, "%d check(s) failed\n", failures);
    else
        printf("abi host checks passed\n");
    return failures ? 1 : 0;
}
