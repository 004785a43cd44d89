// gemm_tiled.hip -- the tiled MFMA GEMM for gfx950.
//
// One workgroup computes one BM x BN tile of C (or of one of the three QKV
// outputs).  The structure is the tile loop of the pages: clear an FP32
// accumulator, march over K in BK-deep steps, at each step stage an A tile
// and a B tile and run a tile multiply-accumulate, then apply the epilogue
// while the accumulator is still in registers and store the tile ("TileIR",
// the matmul inner loop and epilogue fusion; "Beyond Hand-Written CUDA",
// section 4, the pipelined FP16 GEMM with shared-memory tiles and a float32
// fragment).
//
// gfx950 mapping:
//  - Global -> registers: 128-bit loads.  A rows are K-contiguous and are
//    loaded as 16-byte chunks.  B[K,N] is N-contiguous, but the MFMA wants 8
//    consecutive k of one column per lane, so every thread loads an 8 x 8
//    block of B (8 k-rows of 8 columns) and transposes it in registers;
//    A and B then sit in LDS with the same K-contiguous row layout.
//  - Two LDS stages: the loads for step k+1 are in flight while step k runs
//    its MFMAs; one barrier per step ("Beyond Hand-Written CUDA", section 5:
//    LDS footprint = stages x (A tile + B tile); 2 x (256 + 256) x 72 x 2 B =
//    144 KiB of the 160 KiB per CU for the largest tile).
//  - LDS rows are padded by 8 elements (16 bytes), which makes the 128-bit
//    fragment reads conflict-free (see lds_offset_bytes).
//  - v_mfma_f32_16x16x32_{f16,bf16} with B as the first operand and A as
//    the second, so the accumulator holds C transposed: each lane owns 4
//    consecutive columns of one row, stored as one 64-bit write.
//  - Workgroup -> tile through schedule_tile (XCD-aware, grouped).
//  - Every load and store is guarded by logical bounds; interior tiles take
//    the 128-bit path, edge chunks fall back to element accesses.
#include <type_traits>

#include "tg_device.h"
#include "tg_launch.h"

namespace tg {

namespace {

template <bool EDGE, bool UNAL = false>
__device__ __forceinline__ u32x4 load_row_chunk(const unsigned short *base, int64_t ld, int rows,
                                                int cols, int r, int c)
{
    // 8 consecutive elements (r, c..c+7) of a rows x cols row-major matrix;
    // out-of-bounds elements read as zero.  EDGE = false: the caller has
    // established that the whole chunk is in bounds.  UNAL: the chunk need
    // not be 16-byte aligned, so every element is loaded on its own.
    if (!UNAL && (!EDGE || (r < rows && c + 8 <= cols)))
        return *reinterpret_cast<const u32x4 *>(base + (int64_t)r * ld + c);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < rows && c < cols) {
        const unsigned short *p = base + (int64_t)r * ld;
        unsigned short e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            e[i] = (c + i < cols) ? p[c + i] : (unsigned short)0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = (unsigned int)e[2 * i] | ((unsigned int)e[2 * i + 1] << 16);
    }
    return v;
}

} // namespace

// Operand staging registers of one K-step: CA chunks of A and CB 8x8 blocks of B.
template <int CA, int CB>
struct Stage {
    u32x4 a[CA];
    u32x4 b[CB][8];
};

template <int DT, int BM, int BN, int BK, int WM, int WN, int ACT, bool EDGE, bool UNAL>
__device__ __forceinline__ void tile_body(const GemmArgs &p, int m0, int n0,
                                          const unsigned short *Bm, unsigned short *Cm,
                                          unsigned short *smem)
{
    constexpr int NT = 64 * WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN; // wave tile
    constexpr int FM = TM / 32, FN = TN / 32; // 32x32 MFMA blocks per wave
    constexpr int PA = lds_pitch(BK);         // LDS row pitch in elements
    constexpr int KC = BK / 8;                // 16-byte chunks per K-row
    constexpr int CA = BM * KC / NT;          // A chunks per thread per step
    constexpr int NBLK = KC * (BN / 8);       // 8x8 B blocks per step
    constexpr int CB = (NBLK + NT - 1) / NT;  // B blocks per thread per step
    constexpr int A_ELEMS = BM * PA, B_ELEMS = BN * PA;
    static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "wave tile");
    static_assert(BK % 16 == 0 && BK >= 64, "BK: whole MFMA steps, 8 k-blocks per row");
    static_assert((BM * KC) % NT == 0 && NT % KC == 0, "A chunk mapping");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_m = wave / WN, wave_n = wave % WN;
    const int M = p.M, N = p.N, K = p.K;

    // A staging: chunk (row, kc) with kc fixed per thread.
    const int a_kc = tid % KC;
    const int a_row0 = tid / KC;
    // B staging: block b -> (kb = b % KC, nb = b / KC); lanes of one wave
    // cover all kb for 8 column blocks, which keeps both the global rows
    // (128-byte segments) and the transposed LDS writes conflict-free.
    using St = Stage<CA, CB>;

    // Interior tiles load through buffer resources: one per-thread VGPR
    // offset per operand, the per-chunk offsets in scalar registers, and the
    // resource base advanced by one K-step at a time (so offsets stay far
    // below 2^32).  Edge tiles use predicated element-wise loads.
    const int va = (a_row0 * (int)p.lda + a_kc * 8) * 2;
    int vb[CB];
#pragma unroll
    for (int j = 0; j < CB; ++j) {
        const int b = tid + j * NT;
        vb[j] = ((b % KC) * 8 * (int)p.ldb + (b / KC) * 8) * 2;
    }

    auto load = [&](St &r, int kt) {
        const int kbase = kt * BK;
        if constexpr (!EDGE) {
            const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(p.A + (int64_t)m0 * p.lda + kbase), (short)0, 0x7FFFFFFF, 0x00020000);
            const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(Bm + (int64_t)kbase * p.ldb + n0), (short)0, 0x7FFFFFFF, 0x00020000);
#pragma unroll
            for (int i = 0; i < CA; ++i)
                r.a[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       ra, va, i * (NT / KC) * (int)p.lda * 2, 0));
#pragma unroll
            for (int j = 0; j < CB; ++j) {
                const int b = tid + j * NT;
                if (NBLK % NT == 0 || b < NBLK) {
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        r.b[j][i] = __builtin_bit_cast(
                            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, vb[j],
                                                                         i * (int)p.ldb * 2, 0));
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < CA; ++i)
                r.a[i] = load_row_chunk<true, UNAL>(p.A, p.lda, M, K,
                                                    m0 + a_row0 + i * (NT / KC), kbase + a_kc * 8);
#pragma unroll
            for (int j = 0; j < CB; ++j) {
                const int b = tid + j * NT;
                if (NBLK % NT == 0 || b < NBLK) {
                    const int kb = b % KC, nb = b / KC;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        r.b[j][i] = load_row_chunk<true, UNAL>(Bm, p.ldb, K, N,
                                                               kbase + kb * 8 + i, n0 + nb * 8);
                }
            }
        }
    };

    auto store = [&](const St &r, int buf) {
        unsigned short *As = smem + buf * (A_ELEMS + B_ELEMS);
        unsigned short *Bs = As + A_ELEMS;
#pragma unroll
        for (int i = 0; i < CA; ++i)
            *reinterpret_cast<u32x4 *>(As + (a_row0 + i * (NT / KC)) * PA + a_kc * 8) = r.a[i];
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            const int b = tid + j * NT;
            if (NBLK % NT == 0 || b < NBLK) {
                const int kb = b % KC, nb = b / KC;
                // r.b[j][i] = row k_i, columns c = 0..7 (two per dword).  Column c
                // over k_0..k_7 is dword e = (k_{2e}, k_{2e+1}) of that column.
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    u32x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const unsigned int x = r.b[j][2 * e][c >> 1];
                        const unsigned int y = r.b[j][2 * e + 1][c >> 1];
                        o[e] = (c & 1) ? ((x >> 16) | (y & 0xFFFF0000u))
                                       : ((x & 0xFFFFu) | (y << 16));
                    }
                    *reinterpret_cast<u32x4 *>(Bs + (nb * 8 + c) * PA + kb * 8) = o;
                }
            }
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.f;

    const int lrow = lane & 31;     // operand row / column of this lane
    const int lk = (lane >> 5) * 8; // its 8 k-values within a 16-deep step

    // One K-step from LDS stage `buf`.  The fragments of the next 16-deep
    // sub-step are read before the MFMAs of the current one are issued, and a
    // scheduling barrier after each sub-step keeps the compiler from hoisting
    // further reads (which would cost registers the staging buffers need).
    auto compute = [&](int buf) {
        const unsigned short *As = smem + buf * (A_ELEMS + B_ELEMS);
        const unsigned short *Bs = As + A_ELEMS;
        u32x4 af[2][FM], bf[2][FN];
        auto read = [&](int kk, int slot) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[slot][i] = *reinterpret_cast<const u32x4 *>(
                    As + (wave_m * TM + i * 32 + lrow) * PA + kk * 16 + lk);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[slot][j] = *reinterpret_cast<const u32x4 *>(
                    Bs + (wave_n * TN + j * 32 + lrow) * PA + kk * 16 + lk);
        };
        read(0, 0);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int cur = kk & 1;
            if (kk + 1 < BK / 16)
                read(kk + 1, cur ^ 1);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = mfma32x32x16<DT>(bf[cur][j], af[cur][i], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Two LDS stages, one register stage: the loads of tile k+1 are issued
    // before the MFMAs of tile k and written to the other LDS stage after
    // them; one barrier per K-step.
    const int KT = (K + BK - 1) / BK;
    if (KT > 0) {
        St r0;
        load(r0, 0);
        store(r0, 0);
        __syncthreads();
        for (int kt = 0; kt < KT; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < KT)
                load(r0, kt + 1);
            compute(cur);
            __builtin_amdgcn_sched_barrier(0);
            if (kt + 1 < KT)
                store(r0, cur ^ 1);
            __syncthreads();
        }
    }

    // Epilogue on the register accumulator.  With B as the first MFMA operand
    // the 32x32 accumulator block is C transposed: lane l holds row
    // m = l % 32 and, in registers 4g..4g+3, the 4 consecutive columns
    // n = 8g + 4 (l / 32) + {0,1,2,3}.
    auto epilogue = [&](auto has_bias) {
        constexpr bool HB = decltype(has_bias)::value;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = m0 + wave_m * TM + i * 32 + lrow;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n = n0 + wave_n * TN + j * 32 + g * 8 + (lane >> 5) * 4;
                    float v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float x = acc[i][j][4 * g + r];
                        if constexpr (HB) {
                            if (!EDGE || n + r < N)
                                x += from_bits<DT>(p.bias[n + r]);
                        }
                        v[r] = activate<ACT>(x);
                    }
                    if (!EDGE || m < M) {
                        if (p.R != nullptr)
                            add_residual<DT, 4, !UNAL>(p.R, p.ldr, m, n, N, v);
                        unsigned short *cp = Cm + (int64_t)m * p.ldc + n;
                        if (!UNAL && (!EDGE || n + 4 <= N)) {
                            u32x2 o = {pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3])};
                            *reinterpret_cast<u32x2 *>(cp) = o;
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (n + r < N)
                                    cp[r] = to_bits<DT>(v[r]);
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    if (p.bias != nullptr)
        epilogue(std::true_type{});
    else
        epilogue(std::false_type{});
}

// EDGE = false: every tile of the grid is interior (M, N, K are multiples of
// the tile and the pitches fit 32-bit buffer offsets), so no predicate is
// evaluated anywhere.  EDGE = true: every load and store is bounds-checked.
// UNAL (with EDGE): operands, pitches or the output are not 16-byte aligned
// (only 2-byte), so every global load and store moves one element; the MFMA
// loop and the LDS layout are unchanged.  The host picks the variant per
// launch; keeping them in separate kernels keeps the register allocation of
// the fast path unaffected by the predicated ones.
template <int DT, int BM, int BN, int BK, int WM, int WN, int ACT, bool EDGE, bool UNAL>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_tiled_kernel(GemmArgs p, int tiles_m,
                                                                   int tiles_n, int group_m)
{
    constexpr int PA = lds_pitch(BK);
    __shared__ __attribute__((aligned(16))) unsigned short smem[2 * (BM + BN) * PA];

    const TileCoord tc = schedule_tile(tiles_m, tiles_n, p.n_mat, group_m, blockIdx.x);
    const int m0 = tc.tm * BM, n0 = tc.tn * BN;
    const unsigned short *Bm = tc.mat == 0 ? p.B[0] : (tc.mat == 1 ? p.B[1] : p.B[2]);
    unsigned short *Cm = tc.mat == 0 ? p.C[0] : (tc.mat == 1 ? p.C[1] : p.C[2]);
    tile_body<DT, BM, BN, BK, WM, WN, ACT, EDGE, UNAL>(p, m0, n0, Bm, Cm, smem);
}

// ------------------------------------------------------------------ configs

static const TileConfig kConfigs[] = {
    {256, 256, 64, 2, 2, "tiled_256x256x64_w2x2"},
    {256, 128, 64, 2, 2, "tiled_256x128x64_w2x2"},
    {128, 128, 64, 2, 2, "tiled_128x128x64_w2x2"},
    {64, 64, 64, 2, 2, "tiled_64x64x64_w2x2"},
};

int num_tile_configs() { return (int)(sizeof(kConfigs) / sizeof(kConfigs[0])); }
const TileConfig &tile_config(int i) { return kConfigs[i]; }

bool tiled_unaligned(const GemmArgs &a)
{
    auto mis = [](const void *q) { return ((uintptr_t)q & 15u) != 0; };
    bool u = a.lda % 8 != 0 || a.ldb % 8 != 0 || a.ldc % 8 != 0 || mis(a.A) ||
             (a.R != nullptr && (a.ldr % 8 != 0 || mis(a.R)));
    for (int t = 0; t < a.n_mat; ++t)
        u = u || mis(a.B[t]) || mis(a.C[t]);
    return u;
}

template <int DT, int BM, int BN, int BK, int WM, int WN>
static hipError_t launch_cfg(int act, const GemmArgs &a, int group_m, hipStream_t s)
{
    const int tiles_m = (a.M + BM - 1) / BM;
    const int tiles_n = (a.N + BN - 1) / BN;
    const int blocks = tiles_m * tiles_n * a.n_mat;
    dim3 grid(blocks), block(64 * WM * WN);
    const bool unal = tiled_unaligned(a);
    const bool interior = !unal && a.M % BM == 0 && a.N % BN == 0 && a.K % BK == 0 &&
                          a.lda < (1 << 22) && a.ldb < (1 << 22);
#define TG_LAUNCH(ACT_, EDGE_, UNAL_)                                                            \
    hipLaunchKernelGGL((gemm_tiled_kernel<DT, BM, BN, BK, WM, WN, ACT_, EDGE_, UNAL_>), grid,    \
                       block, 0, s, a, tiles_m, tiles_n, group_m)
    if (act == ACT_GELU) {
        if (unal)
            TG_LAUNCH(ACT_GELU, true, true);
        else if (interior)
            TG_LAUNCH(ACT_GELU, false, false);
        else
            TG_LAUNCH(ACT_GELU, true, false);
    } else {
        if (unal)
            TG_LAUNCH(ACT_NONE, true, true);
        else if (interior)
            TG_LAUNCH(ACT_NONE, false, false);
        else
            TG_LAUNCH(ACT_NONE, true, false);
    }
#undef TG_LAUNCH
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_dt(int cfg, int act, const GemmArgs &a, int group_m, hipStream_t s)
{
    switch (cfg) {
    case 0: return launch_cfg<DT, 256, 256, 64, 2, 2>(act, a, group_m, s);
    case 1: return launch_cfg<DT, 256, 128, 64, 2, 2>(act, a, group_m, s);
    case 2: return launch_cfg<DT, 128, 128, 64, 2, 2>(act, a, group_m, s);
    case 3: return launch_cfg<DT, 64, 64, 64, 2, 2>(act, a, group_m, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_tiled(int cfg, int dt, int act, const GemmArgs &a, int group_m,
                        hipStream_t stream)
{
    return dt == DT_F16 ? launch_dt<DT_F16>(cfg, act, a, group_m, stream)
                        : launch_dt<DT_BF16>(cfg, act, a, group_m, stream);
}

} // namespace tg
