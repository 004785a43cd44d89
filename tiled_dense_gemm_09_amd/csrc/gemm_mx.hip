// gemm_mx.hip -- block-scaled 8-bit GEMM on the gfx950 scaled matrix cores.
//
//   C = act( sum_k a(A[m][k]) 2^(SA[k/32][m] - 127) * b(B[n][k]) 2^(SB[k/32][n] - 127)
//            + bias[n] )
//
// with 8-bit float operands (OCP e4m3 or e5m2) and one e8m0 power-of-two
// scale per 32 consecutive k of each row of A and each column of B: the
// low-precision block-scaled GEMM of "TIRx", section 6 (FP8 with e8m0
// block-wise scaling), with the block of 32 along K that the OCP
// microscaling formats and the gfx950 scaled MFMA use.  FP32 accumulation,
// FP32 epilogue, one rounding to the 16-bit output type.
//
// Mapping onto gfx950:
//  - v_mfma_scale_f32_32x32x64_f8f6f4 (64 k per instruction, two 32-blocks):
//    lane l supplies row l % 32 of its operand as 32 bytes and one e8m0
//    byte.  Measured on gfx950: bytes 0-15 of every lane are k-block 0 (lane
//    half h holding k 16h .. 16h+15) and bytes 16-31 are k-block 1 (k 32 +
//    16h ..); block 0 is scaled by the scale bytes of the lanes 0-31 and
//    block 1 by those of lanes 32-63.  So lane half h reads 16-byte granules
//    h and 2 + h of the 64-byte row and supplies the scale of block h.
//  - Both operands are K-contiguous ([M,K] and [N,K]), so both are staged
//    the same way: 64-byte rows (one 64-deep step) copied straight into LDS
//    with 16-byte direct-to-LDS loads, granule c of row r at c ^ swz_a(r),
//    and read back with 128-bit reads (two per 32-byte operand).  A step is
//    64 bytes per row, as in the 16-bit kernels' 32-deep steps, so the tile
//    traffic per step and per MFMA cycle is the same.
//  - Scales are stored block-major ([K/32][M]: the M scales of one k-block
//    are contiguous), so each step's 2 x 256 scales of A and of B are four
//    contiguous 256-byte runs, copied into LDS by 16 lanes of each wave
//    alongside the tiles (the scale tensor's layout is part of the kernel's
//    contract, as the pages note for block-scaled GEMMs).
//  - Four stages, copies three steps ahead, one barrier per step, the
//    epilogue restaged through LDS (tg_pipeline.h), as in gemm_async.hip.
#include <type_traits>
#include <utility>

#include "tg_device.h"
#include "tg_launch.h"
#include "tg_pipeline.h"

namespace tg {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int MX_BM = 256, MX_BN = 256, MX_BK = 64, MX_NT = 256, MX_STAGES = 4;
constexpr int MX_A_BYTES = MX_BM * MX_BK;                  // [256][64] bytes
constexpr int MX_B_BYTES = MX_BN * MX_BK;                  // [256][64] bytes
constexpr int MX_S_OFF = MX_A_BYTES + MX_B_BYTES;          // scales: A blk 0, A blk 1, B blk 0, B blk 1
constexpr int MX_STAGE = MX_S_OFF + 1024;
constexpr int MX_COPIES = 9; // per wave per step: 4 A, 4 B tile copies and one scale run

// f(std::integral_constant<int, q>) for q = 0 .. N-1, so that q can feed an
// instruction's immediate operands
template <int... Q, class F>
__device__ __forceinline__ void static_for_seq(std::integer_sequence<int, Q...>, F &&f)
{
    (f(std::integral_constant<int, Q>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_seq(std::make_integer_sequence<int, N>{}, f);
}

} // namespace

template <int DT, int ACT, int FA, int FB>
__global__ __launch_bounds__(MX_NT, 1) void gemm_mx_kernel(MxArgs p, int tiles_m, int tiles_n,
                                                           int group_m)
{
    __shared__ __attribute__((aligned(1024))) unsigned char st0[MX_STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char st1[MX_STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char st2[MX_STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char st3[MX_STAGE];
    auto stage = [&](auto sidx) -> unsigned char * {
        constexpr int S = decltype(sidx)::value;
        if constexpr (S == 0)
            return st0;
        else if constexpr (S == 1)
            return st1;
        else if constexpr (S == 2)
            return st2;
        else
            return st3;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave >> 1, wave_n = wave & 1; // 2 x 2 waves of 128 x 128
    const int h = lane >> 5;                         // which 32-k half of a step the lane holds

    const TileCoord tc = schedule_tile(tiles_m, tiles_n, 1, group_m, blockIdx.x);
    const int m0 = tc.tm * MX_BM, n0 = tc.tn * MX_BN;
    const int KT = p.K / MX_BK;

    // ---- copy plan.  Tile copy q (0..15) fills rows 16q..16q+15 of the A
    // or B tile; lane -> (row 16q + lane/4, granule lane%4).  Wave w issues
    // copies 4w..4w+3 of each, and scale run w: the 256 scales of k-block
    // 2 kt + (w & 1) of A (w < 2) or B (w >= 2), 4 bytes per lane with the
    // 4-byte direct-to-LDS load (lane l's bytes land at M0 + 4 l).
    const unsigned char *ga[4];
    const unsigned char *gb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 16 * (wave * 4 + i) + (lane >> 2);
        const int c = (lane & 3) ^ swz_a(r);
        ga[i] = p.A + (int64_t)(m0 + r) * p.lda + c * 16;
        gb[i] = p.B + (int64_t)(n0 + r) * p.ldb + c * 16;
    }
    const unsigned char *gs = (wave < 2 ? p.SA + m0 : p.SB + n0) + 4 * lane +
                              (wave & 1) * (wave < 2 ? p.ldsa : p.ldsb);
    const int64_t s_step = 2 * (wave < 2 ? p.ldsa : p.ldsb); // two k-blocks per step

    // The copies are inline assembly so that the compiler's own wait
    // insertion stays out of the pipeline; wait_vmcnt covers them.
    auto copy = [&](int kt, unsigned char *st, int c) {
        const unsigned lds = (unsigned)(uintptr_t)(lds_void *)st;
        if (c < 4) {
            asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(ga[c] + kt * MX_BK),
                         "{m0}"(lds + (wave * 4 + c) * 1024)
                         : "memory");
        } else if (c < 8) {
            asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gb[c - 4] + kt * MX_BK),
                         "{m0}"(lds + MX_A_BYTES + (wave * 4 + c - 4) * 1024)
                         : "memory");
        } else {
            asm volatile("global_load_lds_dword %0, off" ::"v"(gs + kt * s_step),
                         "{m0}"(lds + MX_S_OFF + wave * 256)
                         : "memory");
        }
    };
    auto issue = [&](int kt, unsigned char *st) {
#pragma unroll
        for (int c = 0; c < MX_COPIES; ++c)
            copy(kt, st, c);
    };

    // ---- accumulators start at bias[n] (or 0); lane l of block (i, j)
    // holds columns n = 32 j + 8 g + 4 (l / 32) + {0..3} in registers 4g..4g+3
    f32x16 acc[4][4];
    if (p.bias != nullptr) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const u32x2 braw = *reinterpret_cast<const u32x2 *>(
                    p.bias + n0 + wave_n * 128 + j * 32 + g * 8 + (lane >> 5) * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float b = from_bits<DT>((unsigned short)(braw[e >> 1] >> (16 * (e & 1))));
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[i][j][4 * g + e] = b;
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[i][j][r] = 0.f;
    }

    // ---- fragment addressing (byte offsets within a stage).  Operand block
    // i of A: row wave_m*128 + 32i + lane%32, granules h and 2 + h (k
    // 16h..16h+15 of the step's first 32-block and of its second); its
    // scale: the step's A block h, same row.
    int a_off[4][2], b_off[4][2], sa_off[4], sb_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ra = wave_m * 128 + 32 * i + (lane & 31);
        const int rb = wave_n * 128 + 32 * i + (lane & 31);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            a_off[i][t] = ra * 64 + (((2 * t + h) ^ swz_a(ra)) * 16);
            b_off[i][t] = MX_A_BYTES + rb * 64 + (((2 * t + h) ^ swz_a(rb)) * 16);
        }
        sa_off[i] = MX_S_OFF + h * 256 + ra;
        sb_off[i] = MX_S_OFF + 512 + h * 256 + rb;
    }

    // sa / sb hold the four scale bytes of the wave's four A (B) blocks in
    // one register; each MFMA picks its byte with op_sel
    struct Frag {
        i32x8 a[4], b[4];
        int sa, sb;
    };
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    // piece q of a fragment set: 0..15 the 128-bit operand reads (A blocks
    // then B blocks, two halves each, straight into the halves of the
    // 8-register MFMA operands), 16..23 the scale bytes
    auto read_piece = [&](Frag &f, const unsigned char *st, int q) {
        if (q < 16) {
            const int blk = (q & 7) >> 1, t = q & 1;
            const int off = q < 8 ? a_off[blk][t] : b_off[blk][t];
            const i32x4 v = *reinterpret_cast<const i32x4 *>(st + off);
            i32x8 &dst = q < 8 ? f.a[blk] : f.b[blk];
            if (t == 0)
                dst.lo = v;
            else
                dst.hi = v;
        } else if (q < 20) {
            const int v = st[sa_off[q - 16]];
            f.sa = q == 16 ? v : (f.sa | (v << (8 * (q - 16))));
        } else {
            const int v = st[sb_off[q - 20]];
            f.sb = q == 20 ? v : (f.sb | (v << (8 * (q - 20))));
        }
    };
    auto read = [&](Frag &f, const unsigned char *st) {
#pragma unroll
        for (int q = 0; q < 24; ++q)
            read_piece(f, st, q);
    };
    auto mma_one = [&](const Frag &f, auto qc) {
        constexpr int q = decltype(qc)::value, i = q >> 2, j = q & 3;
        // src0 = B (its rows become the MFMA rows = output columns n), src1 = A;
        // scale bytes j of f.sb and i of f.sa
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[j], f.a[i], acc[i][j], FB,
                                                                    FA, j, f.sb, i, f.sa);
    };

    // ---- pipeline.  Step k:
    //     wait for this wave's copies of step k+1 and its reads of stage k,
    //     barrier (everybody's copies of k+1 landed; stage k is free)
    //     16 MFMAs of step k, interleaved with the reads of step k+1's
    //     fragments from stage k+1 (three per MFMA in the first half, so they
    //     are done long before the next wait) and the copies of step k+4
    //     into stage k
    // Copies have three steps to land; the loop is unrolled by the stage
    // count so every stage is named statically; past the last step the
    // copies repeat the last tile and the reads reread a stage (harmless).
    Frag f0, f1;
    auto step = [&](int kt, auto sidx, Frag &fc, Frag &fn) {
        constexpr int S = decltype(sidx)::value;
        unsigned char *cur = stage(sidx);
        unsigned char *nxt = stage(std::integral_constant<int, (S + 1) % 4>{});
        wait_vmcnt<2 * MX_COPIES>();
        __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0)
        stage_barrier();
        const int kc = min(kt + 4, KT - 1);
        static_for<16>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            mma_one(fc, qc);
            if constexpr (q < 8) {
                read_piece(fn, nxt, 3 * q);
                read_piece(fn, nxt, 3 * q + 1);
                read_piece(fn, nxt, 3 * q + 2);
            }
            if constexpr (q >= 4 && q < 4 + MX_COPIES)
                copy(kc, cur, q - 4);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    issue(0, st0);
    issue(1, st1);
    issue(2, st2);
    issue(3, st3);
    wait_vmcnt<3 * MX_COPIES>();
    stage_barrier();
    read(f0, st0);
    for (int kt = 0; kt < KT; kt += 4) {
        step(kt, std::integral_constant<int, 0>{}, f0, f1);
        step(kt + 1, std::integral_constant<int, 1>{}, f1, f0);
        step(kt + 2, std::integral_constant<int, 2>{}, f0, f1);
        step(kt + 3, std::integral_constant<int, 3>{}, f1, f0);
    }
    // every copy has landed and every read is done: the LDS is free
    wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    stage_barrier();

    unsigned char *ep = wave == 0 ? st0 : wave == 1 ? st1 : wave == 2 ? st2 : st3;
    restaged_epilogue<DT, ACT, 4, 4, false>(
        acc, ep, lane, p.C + (int64_t)(m0 + wave_m * 128) * p.ldc + n0 + wave_n * 128, p.ldc,
        nullptr, 0);
}

// ---------------------------------------------------------------------------
// Fallback for any shape (K a multiple of 32): one thread per output, the
// 8-bit values and scales decoded from their bit layouts, FP32 FMA over k.

namespace {

// OCP 8-bit floats: e4m3 (bias 7, no infinities, S.1111.111 = NaN) and e5m2
// (bias 15, IEEE-style specials), decoded from the bits.
template <int FMT>
__device__ __forceinline__ float fp8_value(unsigned x)
{
    const float sgn = (x & 0x80u) ? -1.f : 1.f;
    if constexpr (FMT == 0) {
        const int e = (x >> 3) & 15, f = x & 7;
        if (e == 15 && f == 7)
            return __builtin_nanf("");
        return sgn * (e == 0 ? __builtin_ldexpf((float)f, -9) : __builtin_ldexpf(8.f + f, e - 10));
    } else {
        const int e = (x >> 2) & 31, f = x & 3;
        if (e == 31)
            return f ? __builtin_nanf("") : sgn * __builtin_inff();
        return sgn * (e == 0 ? __builtin_ldexpf((float)f, -16) : __builtin_ldexpf(4.f + f, e - 17));
    }
}

__device__ __forceinline__ float e8m0_value(unsigned e)
{
    return e == 0xFFu ? __builtin_nanf("") : __builtin_ldexpf(1.f, (int)e - 127);
}

} // namespace

template <int DT, int ACT, int FA, int FB>
__global__ __launch_bounds__(256) void gemm_mx_generic_kernel(MxArgs p)
{
    const int64_t n = (int64_t)blockIdx.x * 16 + (threadIdx.x & 15);
    if (n >= p.N)
        return;
    for (int64_t m = (int64_t)blockIdx.y * 16 + (threadIdx.x >> 4); m < p.M;
         m += (int64_t)gridDim.y * 16) {
        float acc = p.bias != nullptr ? from_bits<DT>(p.bias[n]) : 0.f;
        for (int kb = 0; kb < p.K / 32; ++kb) {
            const float s = e8m0_value(p.SA[(int64_t)kb * p.ldsa + m]) *
                            e8m0_value(p.SB[(int64_t)kb * p.ldsb + n]);
            float part = 0.f;
            for (int k = 32 * kb; k < 32 * kb + 32; ++k)
                part = __builtin_fmaf(fp8_value<FA>(p.A[m * p.lda + k]),
                                      fp8_value<FB>(p.B[n * p.ldb + k]), part);
            acc = __builtin_fmaf(part, s, acc);
        }
        p.C[m * p.ldc + n] = to_bits<DT>(activate<ACT>(acc));
    }
}

bool mx_fast_eligible(const MxArgs &a)
{
    auto al16 = [](const void *q) { return ((uintptr_t)q & 15u) == 0; };
    return a.M % MX_BM == 0 && a.N % MX_BN == 0 && a.K % (MX_STAGES * MX_BK) == 0 && a.K > 0 &&
           al16(a.A) && al16(a.B) && al16(a.SA) && al16(a.SB) && al16(a.C) &&
           ((uintptr_t)a.bias & 7u) == 0 && a.lda % 16 == 0 && a.ldb % 16 == 0 &&
           a.ldsa % 16 == 0 && a.ldsb % 16 == 0 && a.ldc % 8 == 0;
}

#define TG_MX_DISPATCH(KERNEL, GRID, BLOCK, ...)                                                  \
    do {                                                                                         \
        const int code = ((dt == DT_F16) ? 0 : 8) | ((act == ACT_GELU) ? 4 : 0) | (a.fmt_a << 1) | \
                         a.fmt_b;                                                                \
        switch (code) {                                                                          \
        case 0: hipLaunchKernelGGL((KERNEL<DT_F16, ACT_NONE, 0, 0>), GRID, BLOCK, 0, s, __VA_ARGS__); break; \
        case 1: hipLaunchKernelGGL((KERNEL<DT_F16, ACT_NONE, 0, 1>), GRID, BLOCK, 0, s, __VA_ARGS__); break; \
        case 2: hipLaunchKernelGGL((KERNEL<DT_F16, ACT_NONE, 1, 0>), GRID, BLOCK, 0, s, __VA_ARGS__); break; \
        case 3: hipLaunchKernelGGL((KERNEL<DT_F16, ACT_NONE, 1, 1>), GRID, BLOCK, 0, s, __VA_ARGS__); break; \
        case 4: hipLaunchKernelGGL((KERNEL<DT_F16, ACT_GELU, 0, 0>), GRID, BLOCK, 0, s, __VA_ARGS__); break; \
        case 5: hipLaunchKernelGGL((KERNEL<DT_F16, ACT_GELU, 0, 1>), GRID, BLOCK, 0, s, __VA_ARGS__); break; \
        case 6: hipLaunchKernelGGL((KERNEL<DT_F16, ACT_GELU, 1, 0>), GRID, BLOCK, 0, s, __VA_ARGS__); break; \
        case 7: hipLaunchKernelGGL((KERNEL<DT_F16, ACT_GELU, 1, 1>), GRID, BLOCK, 0, s, __VA_ARGS__); break; \
        case 8: hipLaunchKernelGGL((KERNEL<DT_BF16, ACT_NONE, 0, 0>), GRID, BLOCK, 0, s, __VA_ARGS__); break; \
        case 9: hipLaunchKernelGGL((KERNEL<DT_BF16, ACT_NONE, 0, 1>), GRID, BLOCK, 0, s, __VA_ARGS__); break; \
        case 10: hipLaunchKernelGGL((KERNEL<DT_BF16, ACT_NONE, 1, 0>), GRID, BLOCK, 0, s, __VA_ARGS__); break; \
        case 11: hipLaunchKernelGGL((KERNEL<DT_BF16, ACT_NONE, 1, 1>), GRID, BLOCK, 0, s, __VA_ARGS__); break; \
        case 12: hipLaunchKernelGGL((KERNEL<DT_BF16, ACT_GELU, 0, 0>), GRID, BLOCK, 0, s, __VA_ARGS__); break; \
        case 13: hipLaunchKernelGGL((KERNEL<DT_BF16, ACT_GELU, 0, 1>), GRID, BLOCK, 0, s, __VA_ARGS__); break; \
        case 14: hipLaunchKernelGGL((KERNEL<DT_BF16, ACT_GELU, 1, 0>), GRID, BLOCK, 0, s, __VA_ARGS__); break; \
        default: hipLaunchKernelGGL((KERNEL<DT_BF16, ACT_GELU, 1, 1>), GRID, BLOCK, 0, s, __VA_ARGS__); break; \
        }                                                                                        \
    } while (0)

hipError_t launch_mx(int dt, int act, const MxArgs &a, int group_m, hipStream_t s)
{
    const int tiles_m = a.M / MX_BM, tiles_n = a.N / MX_BN;
    const dim3 grid(tiles_m * tiles_n), block(MX_NT);
    TG_MX_DISPATCH(gemm_mx_kernel, grid, block, a, tiles_m, tiles_n, group_m);
    return hipGetLastError();
}

hipError_t launch_mx_generic(int dt, int act, const MxArgs &a, hipStream_t s)
{
    const int64_t gy = ((int64_t)a.M + 15) / 16;
    const dim3 grid((a.N + 15) / 16, (unsigned)(gy < 65535 ? gy : 65535)), block(256);
    TG_MX_DISPATCH(gemm_mx_generic_kernel, grid, block, a);
    return hipGetLastError();
}

#undef TG_MX_DISPATCH

} // namespace tg
