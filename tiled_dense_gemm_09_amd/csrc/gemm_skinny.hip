// gemm_skinny.hip -- the small-M path (M <= 16), bound by HBM bandwidth.
//
// For a decode-shaped product Y[M,N] = X[M,K] . W[K,N] with M <= 16 the
// arithmetic intensity is about M flop per byte of W, far below the ridge
// point, so the kernel's only job is to stream W from HBM exactly once with
// many loads in flight ("TileIR": moving data is the biggest barrier;
// in-flight fetches cost footprint).
//
// Work split: workgroup (tile_n, split) owns 256 columns of W and one
// K-chunk.  It walks its chunk in 64 x 256 slabs (32 KiB), keeping DEPTH
// slabs of 128-bit loads in flight in registers.  Each slab is transposed in
// registers into the K-contiguous LDS layout the MFMA reads (the same layout
// as the square kernel's B tile) and multiplied with the 16 rows of X on
// v_mfma_f32_16x16x32 (rows of X beyond M are zero).
//
// Split-K reduction: each workgroup writes its FP32 partial [16 x 256] to a
// workspace and bumps a per-column-tile counter; the workgroup that arrives
// last sums the partials in split order 0, 1, ..., S-1 (so the result does
// not depend on arrival order), applies bias + activation, rounds, stores Y,
// and resets the counter to zero for the next call.
#include <cstdlib>

#include "tg_device.h"
#include "tg_launch.h"

namespace tg {

namespace {

constexpr int SK_BN = 256;  // columns per workgroup
constexpr int SK_BK = 64;   // slab depth
constexpr int SK_NT = 256;  // threads
constexpr int SK_PA = lds_pitch(SK_BK);
constexpr int SK_DEPTH = 4; // slabs of loads in flight per thread

__device__ __forceinline__ u32x4 ld_chunk(const unsigned short *base, int64_t ld, int rows,
                                          int cols, int r, int c)
{
    if (r < rows && c + 8 <= cols)
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

struct Slot {
    u32x4 w[8]; // 8 k-rows x 8 columns of W
    u32x4 x[2]; // X fragments for the slab's two 32-deep MFMA steps
};

} // namespace

// EDGE = false: N is a multiple of 256 and every split's K-range a multiple
// of DEPTH slabs, so the kernel runs branch-free on buffer loads (rows of X
// at or beyond M read as zero through the buffer range check on the
// per-lane offset).  EDGE = true: every chunk is bounds-checked.
template <int DT, int ACT, int DEPTH, bool EDGE>
__global__ __launch_bounds__(SK_NT, 2) void gemm_skinny_kernel(GemmArgs p, int k_chunk,
                                                               int splits, float *ws,
                                                               int *counters)
{
    __shared__ __attribute__((aligned(16))) unsigned short smem[2 * SK_BN * SK_PA];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int tile_n = blockIdx.x / splits;
    const int split = blockIdx.x - tile_n * splits;
    const int n0 = tile_n * SK_BN;
    const int M = p.M, N = p.N, K = p.K;
    const int kbeg = split * k_chunk;
    const int kend = min(K, kbeg + k_chunk);
    const int slabs = (kend - kbeg + SK_BK - 1) / SK_BK;
    const unsigned short *W = p.B[0];

    // this thread's 8x8 block of every slab: kb = tid % 8, nb = tid / 8
    const int kb = tid & 7, nb = tid >> 3;
    // X fragment: row (lane % 16), 8 k starting at (lane / 16) * 8
    const int xr = lane & 15, xk = (lane >> 4) * 8;

    // fast path: W through a resource based at (kbeg, n0), X through one
    // whose range ends after row M-1 (so rows >= M load zeros)
    const int vw = (kb * 8 * (int)p.ldb + nb * 8) * 2;
    const int vx = (xr * (int)p.lda + kbeg + xk) * 2;

    auto load = [&](Slot &s, int slab) {
        const int k0 = kbeg + slab * SK_BK;
        if constexpr (!EDGE) {
            const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(W + (int64_t)k0 * p.ldb + n0), (short)0, 0x7FFFFFFF, 0x00020000);
            const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
                (void *)p.A, (short)0, M * (int)p.lda * 2, 0x00020000);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                s.w[i] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, vw, i * (int)p.ldb * 2, 0));
#pragma unroll
            for (int h = 0; h < 2; ++h)
                s.x[h] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               rx, vx + (slab * SK_BK + h * 32) * 2, 0, 0));
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                s.w[i] = ld_chunk(W, p.ldb, kend, N, k0 + kb * 8 + i, n0 + nb * 8);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = k0 + h * 32 + xk;
                s.x[h] = ld_chunk(p.A, p.lda, M, kend, xr, k);
            }
        }
    };

    auto store = [&](const Slot &s, int buf) {
        unsigned short *Ws = smem + buf * (SK_BN * SK_PA);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const unsigned int x = s.w[2 * e][c >> 1];
                const unsigned int y = s.w[2 * e + 1][c >> 1];
                o[e] = (c & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
            }
            *reinterpret_cast<u32x4 *>(Ws + (nb * 8 + c) * SK_PA + kb * 8) = o;
        }
    };

    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const u32x4 (&x)[2], int buf) {
        const unsigned short *Ws = smem + buf * (SK_BN * SK_PA);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = wave * 64 + j * 16 + (lane & 15);
                const u32x4 wf = *reinterpret_cast<const u32x4 *>(Ws + n * SK_PA + h * 32 + xk);
                acc[j] = mfma16x16x32<DT>(wf, x[h], acc[j]);
            }
        }
    };

    // DEPTH slabs of loads stay in flight: slot d holds slab s0 + d; it is
    // written to LDS, reloaded with slab s0 + d + DEPTH, and the MFMAs of
    // slab s0 + d run after the barrier.
    Slot slot[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
        if (EDGE ? d < slabs : true)
            load(slot[d], d);

    for (int s0 = 0; s0 < slabs; s0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int s = s0 + d;
            if (EDGE && s >= slabs)
                break;
            const int buf = s & 1;
            store(slot[d], buf);
            u32x4 x[2] = {slot[d].x[0], slot[d].x[1]};
            if (s + DEPTH < slabs)
                load(slot[d], s + DEPTH);
            __syncthreads();
            compute(x, buf);
        }
    }

    // Partial result: lane holds Y[m = lane % 16][n .. n+3] for 4 column blocks.
    const int m = lane & 15;
    if (splits == 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + wave * 64 + j * 16 + (lane >> 4) * 4;
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float x = acc[j][r];
                if (p.bias != nullptr && n + r < N)
                    x += from_bits<DT>(p.bias[n + r]);
                v[r] = activate<ACT>(x);
            }
            if (m < M) {
                if (p.R != nullptr)
                    add_residual<DT, 4>(p.R, p.ldr, m, n, N, v);
                unsigned short *cp = p.C[0] + (int64_t)m * p.ldc + n;
                if (n + 4 <= N) {
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
        return;
    }

    // workspace layout: ws[(split * 16 + m) * 256 * n_tiles + n] (FP32, N padded to tiles)
    const int64_t ws_ld = (int64_t)gridDim.x / splits * SK_BN;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int nl = wave * 64 + j * 16 + (lane >> 4) * 4;
        float *dst = ws + ((int64_t)split * 16 + m) * ws_ld + n0 + nl;
        *reinterpret_cast<f32x4 *>(dst) = acc[j];
    }
    // Release this thread's partials at device scope (the XCDs' L2 caches are
    // not coherent with each other), then count the split in.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (tid == 0) {
        const int old = __hip_atomic_fetch_add(&counters[tile_n], 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old == splits - 1);
    }
    __syncthreads();
    if (!s_last)
        return;
    // Last workgroup of this column tile: acquire the other splits' partials,
    // then a fixed-order reduction + epilogue.
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

    // Thread -> row rm = tid / 16, 16 columns starting at (tid % 16) * 16.
    const int rm = tid >> 4;
    const int cn = (tid & 15) * 16;
    float sum[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        sum[i] = 0.f;
    for (int s = 0; s < splits; ++s) {
        const float *src = ws + ((int64_t)s * 16 + rm) * ws_ld + n0 + cn;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(src + q * 4);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sum[q * 4 + r] += v[r];
        }
    }
    if (rm < M) {
        unsigned short *cp = p.C[0] + (int64_t)rm * p.ldc + n0 + cn;
        const int nbase = n0 + cn;
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float x = sum[i];
            if (p.bias != nullptr && nbase + i < N)
                x += from_bits<DT>(p.bias[nbase + i]);
            v[i] = activate<ACT>(x);
        }
        if (p.R != nullptr)
            add_residual<DT, 16>(p.R, p.ldr, rm, nbase, N, v);
        if (nbase + 16 <= N) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                u32x4 o = {pack2<DT>(v[8 * q + 0], v[8 * q + 1]), pack2<DT>(v[8 * q + 2], v[8 * q + 3]),
                           pack2<DT>(v[8 * q + 4], v[8 * q + 5]), pack2<DT>(v[8 * q + 6], v[8 * q + 7])};
                *reinterpret_cast<u32x4 *>(cp + 8 * q) = o;
            }
        } else {
            for (int i = 0; i < 16; ++i)
                if (nbase + i < N)
                    cp[i] = to_bits<DT>(v[i]);
        }
    }
    if (tid == 0)
        __hip_atomic_store(&counters[tile_n], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Streaming variant for the common case: W and X go from memory straight
// into LDS with 16-byte direct-to-LDS copies, STAGES-1 64-deep slabs ahead of
// use; no staging registers and no VALU transposition.  The W fragments (8
// consecutive k of one column per lane) come from the LDS transposing read,
// exactly as for B in the asynchronous square kernel.
//
// Two column widths.  BN = 256 (N a multiple of 256, K of 256): four stages
// of 36 KiB.  BN = 128 (N a multiple of 128, K of 512): eight stages of
// 20 KiB, so more bytes are in flight (seven 16 KiB slabs against three 32
// KiB ones) and a column tile needs half as many K splits for the same
// number of workgroups; the workgroup that combines a column tile's split
// partials then reads a quarter of the data, and that read, issued by one
// CU after every split has finished, is the part of the launch that no other
// work overlaps.
//
// LDS stage: W slab [64 k][BN n] (rows of 2 BN bytes, 16-byte granule c of
// row r stored at c ^ swz_w(r), which makes the transposing reads of two
// 16-lane groups at once conflict-free), then X slab [16 rows][64 k]
// (granule c of row r at c ^ (r & 7)), then 2 KiB that waves 2 and 3 fill
// with a second copy of X so every wave issues the same number of copies per
// slab.
namespace {

constexpr int SA_BK = 64, SA_NT = 256;
constexpr int SA_X_BYTES = 16 * SA_BK * 2; // 2 KiB

template <int BN>
struct SaCfg {
    static_assert(BN == 128 || BN == 256, "streaming column widths");
    static constexpr int STAGES = BN == 256 ? 4 : 8;
    static constexpr int W_BYTES = SA_BK * BN * 2;
    static constexpr int STAGE_BYTES = W_BYTES + 2 * SA_X_BYTES;
    static constexpr int W_COPIES = W_BYTES / 1024 / 4;  // 1 KiB W copies per wave per slab
    static constexpr int COPIES = W_COPIES + 1;          // plus one X copy
    static constexpr int ROWS_PER_COPY = 1024 / (2 * BN);
    static constexpr int GRANULES = BN / 8;              // 16-byte granules per W row
    static constexpr int WAVE_COLS = BN / 4;             // columns per wave
    static constexpr int NJ = WAVE_COLS / 16;            // 16-column MFMA blocks per wave
};

// Granule swizzle of W row r.  BN = 256 (512-byte rows, two bank sweeps per
// row): {0,6,10,12}[r & 3] ^ 2 ((r >> 3) & 1).  BN = 128 (256-byte rows, one
// sweep of the 64 four-byte banks): a 16-lane transposing read touches rows
// r0..r0+3 of one granule pair and a second group rows r0+8..r0+11, so the
// pair index is moved by r & 3 and by bit 3 of r: eight distinct pairs, all
// 64 banks.
template <int BN>
__host__ __device__ constexpr int swz_w(int r)
{
    if constexpr (BN == 256)
        return ((r & 3) == 0 ? 0 : (r & 3) == 1 ? 6 : (r & 3) == 2 ? 10 : 12) ^ (2 * ((r >> 3) & 1));
    else
        return 2 * ((r & 3) | (((r >> 3) & 1) << 2));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Calls f(integral_constant<I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

} // namespace

// MB: 16-row blocks of X and Y (1: M <= 16, 2: M <= 32).
template <int DT, int ACT, int BN, int MB>
__global__ __launch_bounds__(SA_NT, 1) void gemm_skinny_async_kernel(GemmArgs p, int k_chunk,
                                                                     int splits, float *ws,
                                                                     int *counters)
{
    static_assert(MB == 1 || MB == 2, "up to 32 rows");
    using C = SaCfg<BN>;
    constexpr int STAGES = C::STAGES, NJ = C::NJ;
    __shared__ __attribute__((aligned(1024))) unsigned char st[STAGES][C::STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile_n = blockIdx.x / splits;
    const int split = blockIdx.x - tile_n * splits;
    const int n0 = tile_n * BN;
    const int M = p.M;
    const int kbeg = split * k_chunk;
    const int slabs = (min(p.K, kbeg + k_chunk) - kbeg) / SA_BK; // a multiple of STAGES
    const unsigned short *W = p.B[0];

    // W copy c of this wave is copy q = wave W_COPIES + c of the slab: rows
    // ROWS_PER_COPY q .. +ROWS_PER_COPY-1; lane -> row ROWS_PER_COPY q +
    // lane / GRANULES, LDS granule lane % GRANULES, which holds W granule
    // (lane % GRANULES) ^ swz_w(row).
    const unsigned short *gw[C::W_COPIES];
#pragma unroll
    for (int c = 0; c < C::W_COPIES; ++c) {
        const int q = wave * C::W_COPIES + c;
        const int r = C::ROWS_PER_COPY * q + lane / C::GRANULES;
        gw[c] = W + (int64_t)(kbeg + r) * p.ldb + n0 + ((lane % C::GRANULES) ^ swz_w<BN>(r)) * 8;
    }
    // X copy: rows 8 w + lane/8 for MB = 2, rows 8 (w & 1) + lane/8 for
    // MB = 1 (waves 2 and 3 write the duplicate), clamped to M-1 (rows >= M
    // only feed output rows that are never stored), granule (lane%8) ^ (row & 7).
    const int xr = 8 * (MB == 2 ? wave : (wave & 1)) + (lane >> 3);
    const unsigned short *gx =
        p.A + (int64_t)min(xr, M - 1) * p.lda + kbeg + (((lane & 7) ^ (xr & 7)) * 8);
    const int64_t w_step = (int64_t)SA_BK * p.ldb;

    auto copy = [&](int s, unsigned char *stage, int c) {
        const unsigned lds = (unsigned)(uintptr_t)(lds_void *)stage;
        if (c < C::W_COPIES) {
            const unsigned dst = lds + (wave * C::W_COPIES + c) * 1024;
            asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gw[c] + s * w_step), "{m0}"(dst)
                         : "memory");
        } else {
            const unsigned dst = lds + C::W_BYTES + wave * 1024;
            asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gx + s * SA_BK), "{m0}"(dst)
                         : "memory");
        }
    };

    // fragments: wave w owns columns WAVE_COLS w .. +WAVE_COLS-1 (NJ blocks
    // of 16).  W fragment of block j, 32-deep half kk, read half h: 16-lane
    // group g, jj = lane % 16: row 32 kk + 8 g + 4 h + jj/4, column
    // WAVE_COLS w + 16 j + 4 (jj%4).
    int w_off[NJ][2][2];
    {
        const int g = lane >> 4, jj = lane & 15;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = 32 * kk + 8 * g + 4 * h + (jj >> 2);
                    const int col = wave * C::WAVE_COLS + 16 * j + 4 * (jj & 3);
                    w_off[j][kk][h] =
                        r * (2 * BN) + (((col >> 3) ^ swz_w<BN>(r)) * 16) + (col & 7) * 2;
                }
    }
    // X fragment of row block mb, half kk: row 16 mb + lane % 16, granule
    // 4 kk + lane / 16.
    int x_off[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int r = 16 * mb + (lane & 15);
            x_off[mb][kk] = C::W_BYTES + r * 128 + (((4 * kk + (lane >> 4)) ^ (r & 7)) * 16);
        }

    f32x4 acc[MB][NJ];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            acc[mb][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // each W fragment serves every 16-row block of X
    auto compute = [&](const unsigned char *stage) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            u32x4 xf[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                xf[mb] = *reinterpret_cast<const u32x4 *>(stage + x_off[mb][kk]);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const u32x2 lo = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                               (lds_s16x4 *)(stage + w_off[j][kk][0])));
                const u32x2 hi = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                               (lds_s16x4 *)(stage + w_off[j][kk][1])));
                const u32x4 wf = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb][j] = mfma16x16x32<DT>(wf, xf[mb], acc[mb][j]);
            }
        }
    };

    // slab s: wait for its copies (those of the next STAGES-2 slabs may stay
    // in flight), barrier, copy slab s+STAGES-1 into the stage slab s-1 used
    // (clamped past the end: repeats the last slab into a stage nobody
    // reads), compute.
    auto step = [&](int s, auto sidx) {
        constexpr int S = decltype(sidx)::value;
        wait_vmcnt<(STAGES - 2) * C::COPIES>();
        __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0)
        stage_barrier();
        const int sc = min(s + STAGES - 1, slabs - 1);
#pragma unroll
        for (int c = 0; c < C::COPIES; ++c)
            copy(sc, st[(S + STAGES - 1) % STAGES], c);
        compute(st[S]);
    };
    auto prologue = [&](auto sidx) {
        constexpr int S = decltype(sidx)::value;
#pragma unroll
        for (int c = 0; c < C::COPIES; ++c)
            copy(min(S, slabs - 1), st[S], c);
    };
    static_for<0, STAGES - 1>([&](auto i) { prologue(i); });
    for (int s = 0; s < slabs; s += STAGES)
        static_for<0, STAGES>([&](auto i) { step(s + decltype(i)::value, i); });
    wait_vmcnt<0>();

    // Lane l holds Y[m = 16 mb + l % 16][n = WAVE_COLS w + 16 j + 4 (l / 16) + r]
    // in acc[mb][j][r].
    auto store_rows = [&](const f32x4 (&val)[MB][NJ]) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int m = 16 * mb + (lane & 15);
            if (m < M) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int n = n0 + wave * C::WAVE_COLS + 16 * j + 4 * (lane >> 4);
                    float v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float x = val[mb][j][r];
                        if (p.bias != nullptr)
                            x += from_bits<DT>(p.bias[n + r]);
                        v[r] = activate<ACT>(x);
                    }
                    if (p.R != nullptr)
                        add_residual<DT, 4>(p.R, p.ldr, m, n, p.N, v);
                    u32x2 o = {pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3])};
                    *reinterpret_cast<u32x2 *>(p.C[0] + (int64_t)m * p.ldc + n) = o;
                }
            }
        }
    };
    if (splits == 1) {
        store_rows(acc);
        return;
    }

    // Split-K.  Each workgroup stores its FP32 partial in accumulator order
    // (workgroup block [4 waves][MB][NJ][64 lanes] of 16-byte vectors, the blocks
    // of one column tile's splits side by side), so every store and every
    // load below moves one contiguous KiB per wave.  The stores are
    // device-coherent (sc1: written through to the device coherence point,
    // since the XCDs' L2 caches are not coherent with each other) and waited
    // for, then one atomic per workgroup counts the split in.  The workgroup
    // that sees the count reach splits-1 reads the partials back with
    // device-coherent loads (sc1), adds them in split order 0..splits-1
    // (independent of arrival order), applies the epilogue, stores Y and
    // resets the counter.  Both sides use device-scope coherent
    // accesses, so no cache-wide writeback or invalidate is needed.
    constexpr int BLOCK = 16 * MB * BN; // floats per workgroup partial
    float *ws_tile = ws + (int64_t)tile_n * splits * BLOCK;
    const int lane_off = (wave * MB * NJ) * 256 + lane * 4;
    {
        f32x4 v[MB * NJ];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                v[mb * NJ + j] = acc[mb][j];
        store_partial<MB * NJ>(ws_tile + split * BLOCK + lane_off, v); // stores and waits
    }
    // Every wave has waited for its own copies, so the stages are idle and
    // the first word of stage 0 carries the arrival flag.
    int *s_last = reinterpret_cast<int *>(&st[0][0]);
    __syncthreads();
    if (tid == 0) {
        const int old = __hip_atomic_fetch_add(&counters[tile_n], 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        *s_last = (old == splits - 1);
    }
    __syncthreads();
    if (!*s_last)
        return;

    // The partials are read back in rounds of RS splits (one round for the
    // planner's split counts: 4 at BN = 128, 8 at BN = 256 with MB = 1), all
    // RS MB NJ loads of a round in flight together, then added in split order
    // (indices past the last split repeat it and are not added).  The own
    // split is read back too, so no branch sits between a load and its wait.
    constexpr int PV = MB * NJ;                       // vectors per lane per split
    constexpr int RS = (BN == 128 || MB == 2) ? 4 : 8;
    constexpr int L = RS * PV;                         // loads per round: 8, 16 or 32
    f32x4 sum[MB][NJ];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            sum[mb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp0 = 0; sp0 < splits; sp0 += RS) {
        f32x4 v[L];
#pragma unroll
        for (int u = 0; u < RS; ++u) {
            const float *src = ws_tile + min(sp0 + u, splits - 1) * BLOCK + lane_off;
#pragma unroll
            for (int t = 0; t < PV; ++t)
                asm volatile("global_load_dwordx4 %0, %1, off sc1"
                             : "=v"(v[u * PV + t])
                             : "v"(src + t * 256)
                             : "memory");
        }
        // the loads above are invisible to the compiler's wait tracking: wait
        // here and pass every value through, so nothing reads (or moves) one
        // earlier (loads return in order)
        if constexpr (L == 32) {
            asm volatile("s_waitcnt vmcnt(16)"
                         : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                           "+v"(v[6]), "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]),
                           "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15])
                         :
                         : "memory");
            asm volatile("s_waitcnt vmcnt(0)"
                         : "+v"(v[16]), "+v"(v[17]), "+v"(v[18]), "+v"(v[19]), "+v"(v[20]),
                           "+v"(v[21]), "+v"(v[22]), "+v"(v[23]), "+v"(v[24]), "+v"(v[25]),
                           "+v"(v[26]), "+v"(v[27]), "+v"(v[28]), "+v"(v[29]), "+v"(v[30]),
                           "+v"(v[31])
                         :
                         : "memory");
        } else if constexpr (L == 16) {
            asm volatile("s_waitcnt vmcnt(0)"
                         : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                           "+v"(v[6]), "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]),
                           "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15])
                         :
                         : "memory");
        } else {
            static_assert(L == 8, "combine operand count");
            asm volatile("s_waitcnt vmcnt(0)"
                         : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                           "+v"(v[6]), "+v"(v[7])
                         :
                         : "memory");
        }
#pragma unroll
        for (int u = 0; u < RS; ++u)
            if (sp0 + u < splits)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
                        sum[mb][j] += v[u * PV + mb * NJ + j];
    }
    store_rows(sum);
    if (tid == 0)
        __hip_atomic_store(&counters[tile_n], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Column-tile variant (N a multiple of 32 with at least 128 tiles, K a
// multiple of 256): no cross-workgroup communication at all.  Workgroup t
// owns 32 columns of W over the whole of K; its 4 waves each stream one
// quarter of K through a private LDS ring with direct-to-LDS copies (five
// 64-deep slabs ahead of use, no barriers in the loop since every wave only
// reads what it copied itself), multiply on v_mfma_f32_16x16x32, and the
// four partial sums are added in LDS in wave order (deterministic).  Tiles
// are placed XCD-contiguously so neighbouring 64-byte column pieces, which
// share 128-byte cache lines, are fetched by one L2.
//
// Ring slot (6 KiB): W [64 k][32 n] (64-byte rows, 16-byte granule c of row
// r at c ^ 2 (((r >> 1) ^ (r >> 3)) & 1), conflict-free for the transposing
// reads), then X [16 rows][64 k] (granule c of row r at c ^ (r & 7)).
namespace {

constexpr int SC_BN = 32, SC_BK = 64, SC_NT = 256, SC_SLOTS = 6;
constexpr int SC_W_BYTES = SC_BK * SC_BN * 2; // 4 KiB
constexpr int SC_X_BYTES = 16 * SC_BK * 2;    // 2 KiB
constexpr int SC_SLOT_BYTES = SC_W_BYTES + SC_X_BYTES;
constexpr int SC_COPIES = SC_SLOT_BYTES / 1024; // 6 per slab
constexpr int SC_AHEAD = SC_SLOTS - 1;          // slabs in flight beyond the current one

__host__ __device__ constexpr int swz_c(int r) { return 2 * (((r >> 1) ^ (r >> 3)) & 1); }

} // namespace

template <int DT, int ACT>
__global__ __launch_bounds__(SC_NT, 1) void gemm_skinny_cols_kernel(GemmArgs p, int n_tiles)
{
    __shared__ __attribute__((aligned(1024))) unsigned char ring[4 * SC_SLOTS * SC_SLOT_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const TileCoord tc = schedule_tile(1, n_tiles, 1, 1, blockIdx.x);
    const int n0 = tc.tn * SC_BN;
    const int M = p.M;
    const int kq = p.K / 4;           // this wave's quarter of K
    const int kbase = wave * kq;
    const int slabs = kq / SC_BK;     // >= 1
    const unsigned short *W = p.B[0];
    unsigned char *my = ring + wave * SC_SLOTS * SC_SLOT_BYTES;
    const unsigned my_lds = (unsigned)(uintptr_t)(lds_void *)my;

    // copy c < 4: W rows 16c + lane/4 of the slab, granule (lane%4) ^ swz_c(row);
    // copy 4, 5: X rows 8 (c-4) + lane/8 (clamped to M-1), granule (lane%8) ^ (row&7)
    const int wr = lane >> 2;
    const unsigned short *gw = W + (int64_t)(kbase + wr) * p.ldb + n0;
    int wg[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
        wg[c] = ((lane & 3) ^ swz_c(16 * c + wr)) * 8;
    const unsigned short *gx[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int r = 8 * c + (lane >> 3);
        gx[c] = p.A + (int64_t)min(r, M - 1) * p.lda + kbase + (((lane & 7) ^ (r & 7)) * 8);
    }
    const int64_t ldb16 = (int64_t)16 * p.ldb;

    auto issue = [&](int s) {
        const unsigned slot = my_lds + (s % SC_SLOTS) * SC_SLOT_BYTES;
        const unsigned short *w0 = gw + (int64_t)s * SC_BK * p.ldb;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(w0 + c * ldb16 + wg[c]),
                         "{m0}"(slot + c * 1024)
                         : "memory");
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gx[c] + s * SC_BK),
                         "{m0}"(slot + SC_W_BYTES + c * 1024)
                         : "memory");
        }
    };

    // fragment offsets within a slot
    int w_off[2][2][2]; // [nb][kk][h]
    {
        const int g = lane >> 4, jj = lane & 15;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = 32 * kk + 8 * g + 4 * h + (jj >> 2);
                    const int col = 16 * nb + 4 * (jj & 3);
                    w_off[nb][kk][h] = r * 64 + (((col >> 3) ^ swz_c(r)) * 16) + (col & 7) * 2;
                }
    }
    int x_off[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int r = lane & 15;
        x_off[kk] = SC_W_BYTES + r * 128 + (((4 * kk + (lane >> 4)) ^ (r & 7)) * 16);
    }

    f32x4 acc[2];
    acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};

    // prologue: SC_AHEAD slabs in flight (clamped repeats past the end land
    // in slots that are never read)
#pragma unroll
    for (int a = 0; a < SC_AHEAD; ++a)
        issue(min(a, slabs - 1));
    for (int s = 0; s < slabs; ++s) {
        // the copies of slabs s+1 .. s+SC_AHEAD-1 may stay in flight
        wait_vmcnt<(SC_AHEAD - 1) * SC_COPIES>();
        asm volatile("" ::: "memory");
        const unsigned char *st = my + (s % SC_SLOTS) * SC_SLOT_BYTES;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const u32x4 xf = *reinterpret_cast<const u32x4 *>(st + x_off[kk]);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const u32x2 lo = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                               (lds_s16x4 *)(st + w_off[nb][kk][0])));
                const u32x2 hi = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                               (lds_s16x4 *)(st + w_off[nb][kk][1])));
                acc[nb] = mfma16x16x32<DT>(u32x4{lo[0], lo[1], hi[0], hi[1]}, xf, acc[nb]);
            }
        }
        // this slab's reads are done before its slot is refilled
        __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0)
        asm volatile("" ::: "memory");
        issue(min(s + SC_AHEAD, slabs - 1));
    }
    wait_vmcnt<0>(); // no copy still writing LDS
    __syncthreads();

    // sum the four K-quarters in wave order; lane l holds
    // Y[m = l % 16][n = 16 nb + 4 (l / 16) + r] in acc[nb][r]
    f32x4 *part = reinterpret_cast<f32x4 *>(ring);
    if (wave != 0) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
            part[((wave - 1) * 2 + nb) * 64 + lane] = acc[nb];
    }
    __syncthreads();
    if (wave == 0) {
        const int m = lane & 15;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            f32x4 v = acc[nb];
#pragma unroll
            for (int w = 0; w < 3; ++w) {
                const f32x4 q = part[(w * 2 + nb) * 64 + lane];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    v[r] += q[r];
            }
            const int n = n0 + 16 * nb + 4 * (lane >> 4);
            float o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float x = v[r];
                if (p.bias != nullptr)
                    x += from_bits<DT>(p.bias[n + r]);
                o[r] = activate<ACT>(x);
            }
            if (m < M) {
                if (p.R != nullptr)
                    add_residual<DT, 4>(p.R, p.ldr, m, n, p.N, o);
                u32x2 ov = {pack2<DT>(o[0], o[1]), pack2<DT>(o[2], o[3])};
                *reinterpret_cast<u32x2 *>(p.C[0] + (int64_t)m * p.ldc + n) = ov;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Realigning variant: W off the 16-byte grid (a row pitch that is not a
// multiple of 8 elements, or a base address that is only 2-byte aligned),
// the shape of a decode step against an odd-sized vocabulary.  Row k of W
// then starts at element offset (w0 + k ldb) mod 8 inside a 16-byte piece (w0:
// the base's offset from the aligned address below it), different on each
// of 8 consecutive rows, so neither the direct-to-LDS copies nor the
// transposing LDS reads can take a row as it stands.
//
// Workgroup (tile, split) keeps 120 columns (fewer, down to 64, when that
// brings a grid of 257 to 511 tiles near two per CU) and one K-chunk.  For each row
// of a 64-deep slab it copies the 16 aligned pieces (128 elements) that begin
// with the piece holding the tile's first column: the 120 columns sit at the
// row's offset o (0 <= o <= 7) inside them.  A slab advances the address by
// 64 ldb elements, a multiple of 8, so the offset of slab row r is the same in
// every slab and every tile, o(r) = (w0 + r ldb) mod 8, and since the 8 k
// values of a fragment come from rows r = 0..7 mod 8, each fragment read has
// one offset shared by every lane: the W fragments are read element by
// element from LDS at that offset.  The MFMA covers 128 columns; the 8 past
// the tile's 120 (and those past N) are computed from whatever the pieces
// hold and never stored.  Pieces are clamped to the last one of the row that
// holds a column below N, so every piece read holds an element of W.
//
// LDS stage (20 KiB, 4 stages, two workgroups per CU): W [64 rows][16
// pieces], piece j of row r's run at position (j + 4 ((r >> 3) & 3)) mod 16,
// which places the four rows a 64-lane element read touches (one per 16-lane
// group, 8 rows apart) on disjoint banks; then X [16 rows][64 k] twice for
// M <= 16 (once per 16 rows for M <= 32), granule c of row r at c ^ (r & 7).
// X must be 16-byte aligned with a pitch of 8 elements and hold zeros (or
// readable values) up to K rounded up to 64; rows of W at or past K read as
// zero.  Split-K partials are combined as in the streaming kernel: in split
// order by the last workgroup of each tile.
//
// BT: B stored [N,K] (a linear layer's weight W[n][k], 16-byte aligned with
// a pitch of 8 elements).  Each row of W is then K-contiguous, the MFMA
// operand layout itself, and the tile keeps 128 columns: a slab is W [128
// rows n][64 k], copied 8 rows of 128 bytes (whole cache lines) per copy,
// granule c of row r at c ^ (r & 7) as for X, and each fragment is one
// 16-byte LDS read.  (Loading the fragments straight into registers reads
// 64 bytes of 16 different rows per load, half of each line, and measured
// 40 % slower.)  Rows at or past N read row N-1 (never stored); pieces at
// or past K read the last piece holding k = K-1 and are zeroed element by
// element.
namespace {

constexpr int SR_BN = 120; // columns stored per workgroup
constexpr int SR_BK = 64, SR_NT = 256, SR_STAGES = 4, SR_NJ = 2;
constexpr int SR_ROW_BYTES = 256;                         // 16 pieces per slab row
constexpr int SR_W_BYTES = SR_BK * SR_ROW_BYTES;          // 16 KiB
constexpr int SR_STAGE_BYTES = SR_W_BYTES + 2 * SA_X_BYTES;
constexpr int SR_COPIES = 5;                              // per wave per slab: 4 of W, 1 of X

// Zero the elements at or past `valid` of 8 packed 16-bit values.
__device__ __forceinline__ u32x4 keep_first(u32x4 v, int valid)
{
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        o[q] = 2 * q + 1 < valid ? v[q] : (2 * q < valid ? (v[q] & 0xFFFFu) : 0u);
    return o;
}

// Byte offset of element e (0 <= e < 136) of slab row r's run in a stage.
__host__ __device__ constexpr int sr_off(int r, int e)
{
    return r * SR_ROW_BYTES + ((((e >> 3) + 4 * ((r >> 3) & 3)) & 15) << 4) + ((e & 7) << 1);
}

} // namespace

// bn: columns stored per workgroup ([K,N]: a multiple of 8, at most 120;
// [N,K]: 128)
template <int DT, int ACT, int MB, bool BT>
__global__ __launch_bounds__(SR_NT, 2) void gemm_skinny_pieces_kernel(GemmArgs p, int n_tiles,
                                                                      int bn, int k_chunk,
                                                                      int splits, float *ws,
                                                                      int *counters)
{
    static_assert(MB == 1 || MB == 2, "up to 32 rows");
    const int TBN = BT ? 128 : bn;
    __shared__ __attribute__((aligned(1024))) unsigned char st[SR_STAGES][SR_STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // unit u = split n_tiles + tile, placed XCD-contiguously: neighbouring
    // tiles share the 128-byte line at their boundary, fetched through one L2
    const int units = n_tiles * splits;
    const int xcd = blockIdx.x % kNumXcd, slot = blockIdx.x / kNumXcd;
    const int uq = units / kNumXcd, ur = units % kNumXcd;
    const int u = xcd * uq + (xcd < ur ? xcd : ur) + slot;
    const int split = u / n_tiles;
    const int tile_n = u - split * n_tiles;
    const int n0 = tile_n * TBN;
    const int M = p.M, N = p.N, K = p.K;
    const int kbeg = split * k_chunk;
    const int slabs = (min(K, kbeg + k_chunk) - kbeg + SR_BK - 1) / SR_BK;
    const int64_t ldb = p.ldb;
    const int klast = ((K - 1) >> 3) << 3; // first k of the last piece holding k = K-1

    // W in 16-byte pieces counted from the aligned address at or below its base
    const uintptr_t wb = (uintptr_t)p.B[0];
    const unsigned char *wal = (const unsigned char *)(wb & ~(uintptr_t)15);
    const int64_t w0 = (int64_t)((wb & 15) >> 1);

    // [K,N]: W copy c of this wave is slab row r = 4 (4 wave + c) + lane / 16,
    // stage position lane % 16, which holds piece (lane % 16 - 4 ((r >> 3) &
    // 3)) mod 16 of the row's run, clamped to the row's last piece with a
    // column < N.  [N,K]: slab row (column n0 + r) r = 8 (4 wave + c) + lane /
    // 8, stage position lane % 8, which holds granule (lane % 8) ^ (r & 7);
    // wr[c] is then that granule's first k in slab 0.
    const unsigned char *gw[4];
    int wr[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if constexpr (BT) {
            const int r = 8 * (wave * 4 + c) + (lane >> 3);
            const int k = kbeg + 8 * ((lane & 7) ^ (r & 7));
            gw[c] = reinterpret_cast<const unsigned char *>(p.B[0] +
                                                            (int64_t)min(n0 + r, N - 1) * ldb + k);
            wr[c] = k;
        } else {
            const int r = 4 * (wave * 4 + c) + (lane >> 4);
            const int64_t e = w0 + (int64_t)(kbeg + r) * ldb; // row start, in elements
            const int64_t first = (e + n0) >> 3, last = (e + N - 1) >> 3;
            const int64_t j = ((lane & 15) - 4 * ((r >> 3) & 3)) & 15;
            gw[c] = wal + 16 * (first + j < last ? first + j : last);
            wr[c] = r;
        }
    }
    const int64_t w_step = BT ? 2 * SR_BK : 2 * (int64_t)SR_BK * ldb; // bytes per slab
    // X copy: rows 8 w + lane/8 for MB = 2, rows 8 (w & 1) + lane/8 for MB = 1
    // (waves 2 and 3 write the duplicate), clamped to M-1, granule (lane%8) ^ (row & 7)
    const int xr = 8 * (MB == 2 ? wave : (wave & 1)) + (lane >> 3);
    const unsigned short *gx =
        p.A + (int64_t)min(xr, M - 1) * p.lda + kbeg + (((lane & 7) ^ (xr & 7)) * 8);

    auto copy = [&](int s, unsigned char *stage, int c) {
        const unsigned lds = (unsigned)(uintptr_t)(lds_void *)stage;
        if (c < 4) {
            const unsigned char *src = gw[c] + s * w_step;
            if (kbeg + (s + 1) * SR_BK > K) {
                if constexpr (BT) {
                    // a granule at or past K reads the last one (masked at the read)
                    const int k = wr[c] + s * SR_BK;
                    if (k > klast)
                        src -= 2 * (k - klast);
                } else {
                    // a row k at or past K copies row k - 8d (d = ceil((k - K + 1)
                    // / 8)), whose run has the same offset; masked at the read
                    const int k = kbeg + s * SR_BK + wr[c];
                    if (k >= K)
                        src -= (int64_t)16 * ldb * ((k - K + 8) >> 3);
                }
            }
            asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src),
                         "{m0}"(lds + (wave * 4 + c) * 1024)
                         : "memory");
        } else {
            asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gx + s * SR_BK),
                         "{m0}"(lds + SR_W_BYTES + wave * 1024)
                         : "memory");
        }
    };

    // W fragment of block j, 32-deep half kk: lane l supplies column
    // 32 wave + 16 j + l % 16 at k = 32 kk + 8 (l / 16) + t, t = 0..7; row
    // 8 (l / 16) + t has offset o(t) = (w0 + t ldb) mod 8 (the same for every
    // lane), and half kk = 1 lies 32 rows (8 KiB) further on.
    // [N,K]: the fragment of block j, half kk is the 16 bytes of slab row
    // 32 wave + 16 j + l % 16 at granule 4 kk + l / 16 (w_off[j][kk]).
    int w_off[SR_NJ][8];
    {
        const int g = lane >> 4;
        if constexpr (BT) {
#pragma unroll
            for (int j = 0; j < SR_NJ; ++j)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int r = 32 * wave + 16 * j + (lane & 15);
                    w_off[j][kk] = r * 128 + (((4 * kk + g) ^ (r & 7)) * 16);
                }
        } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int o = (int)((w0 + t * (ldb & 7)) & 7);
#pragma unroll
                for (int j = 0; j < SR_NJ; ++j)
                    w_off[j][t] = sr_off(8 * g + t, o + 32 * wave + 16 * j + (lane & 15));
            }
        }
    }
    int x_off[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int r = 16 * mb + (lane & 15);
            x_off[mb][kk] = SR_W_BYTES + r * 128 + (((4 * kk + (lane >> 4)) ^ (r & 7)) * 16);
        }

    f32x4 acc[MB][SR_NJ];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < SR_NJ; ++j)
            acc[mb][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // kmax: rows of the slab below K (64 except in a last slab that K cuts)
    auto compute = [&](const unsigned char *stage, int kmax) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            u32x4 xf[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                xf[mb] = *reinterpret_cast<const u32x4 *>(stage + x_off[mb][kk]);
#pragma unroll
            for (int j = 0; j < SR_NJ; ++j) {
                u32x4 wf;
                if constexpr (BT) {
                    wf = *reinterpret_cast<const u32x4 *>(stage + w_off[j][kk]);
                    if (kmax < SR_BK)
                        wf = keep_first(wf, kmax - 32 * kk - 8 * (lane >> 4));
                } else {
                    unsigned v[8];
#pragma unroll
                    for (int t = 0; t < 8; ++t)
                        v[t] = *reinterpret_cast<const unsigned short *>(
                            stage + kk * 32 * SR_ROW_BYTES + w_off[j][t]);
                    if (kmax < SR_BK) {
                        const int r0 = 32 * kk + 8 * (lane >> 4);
#pragma unroll
                        for (int t = 0; t < 8; ++t)
                            v[t] = r0 + t < kmax ? v[t] : 0u;
                    }
                    wf = u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16),
                               v[6] | (v[7] << 16)};
                }
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb][j] = mfma16x16x32<DT>(wf, xf[mb], acc[mb][j]);
            }
        }
    };

    // slab s: wait for its copies (those of the next STAGES-2 slabs may stay
    // in flight), barrier, copy slab s+STAGES-1 into the stage slab s-1 used
    // (clamped past the end: repeats the last slab into a stage nobody
    // reads), compute (steps past the last slab only keep the counts even)
    auto step = [&](int s, auto sidx) {
        constexpr int S = decltype(sidx)::value;
        wait_vmcnt<(SR_STAGES - 2) * SR_COPIES>();
        __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0)
        stage_barrier();
        const int sc = min(s + SR_STAGES - 1, slabs - 1);
#pragma unroll
        for (int c = 0; c < SR_COPIES; ++c)
            copy(sc, st[(S + SR_STAGES - 1) % SR_STAGES], c);
        if (s < slabs)
            compute(st[S], min(SR_BK, K - (kbeg + s * SR_BK)));
    };
    auto prologue = [&](auto sidx) {
        constexpr int S = decltype(sidx)::value;
#pragma unroll
        for (int c = 0; c < SR_COPIES; ++c)
            copy(min(S, slabs - 1), st[S], c);
    };
    static_for<0, SR_STAGES - 1>([&](auto i) { prologue(i); });
    for (int s = 0; s < slabs; s += SR_STAGES)
        static_for<0, SR_STAGES>([&](auto i) { step(s + decltype(i)::value, i); });
    wait_vmcnt<0>();

    // Lane l holds Y[m = 16 mb + l % 16][n = n0 + 32 w + 16 j + 4 (l / 16) + r]
    // in acc[mb][j][r]; element-wise stores (Y, bias and R may sit anywhere).
    auto store_rows = [&](const f32x4 (&val)[MB][SR_NJ]) {
        const int nmax = min(N - n0, TBN);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int m = 16 * mb + (lane & 15);
            if (m >= M)
                continue;
#pragma unroll
            for (int j = 0; j < SR_NJ; ++j) {
                const int nl = wave * 32 + 16 * j + 4 * (lane >> 4);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (nl + r >= nmax)
                        continue;
                    const int n = n0 + nl + r;
                    float x = val[mb][j][r];
                    if (p.bias != nullptr)
                        x += from_bits<DT>(p.bias[n]);
                    x = activate<ACT>(x);
                    if (p.R != nullptr)
                        x += from_bits<DT>(p.R[(int64_t)m * p.ldr + n]);
                    p.C[0][(int64_t)m * p.ldc + n] = to_bits<DT>(x);
                }
            }
        }
    };
    if (splits == 1) {
        store_rows(acc);
        return;
    }

    // Split-K: partials in accumulator order, device-coherent stores and
    // loads, one arrival counter per tile, the last workgroup adds the
    // splits in order 0..splits-1 (as in the streaming kernel above).
    constexpr int PV = MB * SR_NJ;         // vectors per lane per split
    constexpr int BLOCK = 16 * MB * 128;   // floats per workgroup partial
    float *ws_tile = ws + (int64_t)tile_n * splits * BLOCK;
    const int lane_off = (wave * PV) * 256 + lane * 4;
    {
        f32x4 v[PV];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < SR_NJ; ++j)
                v[mb * SR_NJ + j] = acc[mb][j];
        store_partial<PV>(ws_tile + split * BLOCK + lane_off, v); // stores and waits
    }
    int *s_last = reinterpret_cast<int *>(&st[0][0]);
    __syncthreads();
    if (tid == 0) {
        const int old = __hip_atomic_fetch_add(&counters[tile_n], 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        *s_last = (old == splits - 1);
    }
    __syncthreads();
    if (!*s_last)
        return;

    constexpr int RS = 4;       // splits read back per round
    constexpr int L = RS * PV;  // loads per round: 8 or 16
    f32x4 sum[MB][SR_NJ];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < SR_NJ; ++j)
            sum[mb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp0 = 0; sp0 < splits; sp0 += RS) {
        f32x4 v[L];
#pragma unroll
        for (int q = 0; q < RS; ++q) {
            const float *src = ws_tile + min(sp0 + q, splits - 1) * BLOCK + lane_off;
#pragma unroll
            for (int t = 0; t < PV; ++t)
                asm volatile("global_load_dwordx4 %0, %1, off sc1"
                             : "=v"(v[q * PV + t])
                             : "v"(src + t * 256)
                             : "memory");
        }
        // the loads above are invisible to the compiler's wait tracking: wait
        // here and pass every value through, so nothing reads (or moves) one
        // earlier
        if constexpr (L == 16) {
            asm volatile("s_waitcnt vmcnt(0)"
                         : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                           "+v"(v[6]), "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]),
                           "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15])
                         :
                         : "memory");
        } else {
            static_assert(L == 8, "combine operand count");
            asm volatile("s_waitcnt vmcnt(0)"
                         : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                           "+v"(v[6]), "+v"(v[7])
                         :
                         : "memory");
        }
#pragma unroll
        for (int q = 0; q < RS; ++q)
            if (sp0 + q < splits)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int j = 0; j < SR_NJ; ++j)
                        sum[mb][j] += v[q * PV + mb * SR_NJ + j];
    }
    store_rows(sum);
    if (tid == 0)
        __hip_atomic_store(&counters[tile_n], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

namespace {

// Both layouts of the pieces kernel: up to two workgroups per CU (512 on 256
// CUs) resident at once, K split so the units fill them, in chunks of whole
// pipeline rounds; want_splits > 0 (or TG_SKINNY_SPLITS, for sweeps) asks for
// a count, clamped to the chunks.
SkinnyPlan plan_pieces(int M, int N, int K, int want_splits, bool bt)
{
    SkinnyPlan pl;
    pl.streaming = bt ? 4 : 3;
    pl.mb = M > 16 ? 2 : 1;
    pl.bn = bt ? 128 : SR_BN;
    pl.n_tiles = (N + pl.bn - 1) / pl.bn;
    if (!bt && pl.n_tiles > 256 && pl.n_tiles < 512) {
        // Between one and two workgroups per CU most CUs would hold one, with
        // half the copies in flight (16 x 32000 x 4096 with an odd pitch: 4.3
        // TB/s on 267 tiles): narrower tiles (at least 64 columns; each still
        // copies its 128-element runs) bring the count near 512.
        int bn = ((N + 511) / 512 + 7) / 8 * 8;
        bn = bn < 64 ? 64 : (bn > SR_BN ? SR_BN : bn);
        pl.bn = bn;
        pl.n_tiles = (N + bn - 1) / bn;
    }
    constexpr int round = SR_STAGES * SR_BK;
    const int quanta = (K + round - 1) / round;
    int splits = 512 / pl.n_tiles;
    const char *force = getenv("TG_SKINNY_SPLITS");
    if (force && atoi(force) > 0)
        splits = atoi(force);
    if (want_splits > 0)
        splits = want_splits;
    splits = splits < 1 ? 1 : (splits > quanta ? quanta : splits);
    const int per = (quanta + splits - 1) / splits;
    pl.k_chunk = per * round;
    pl.splits = (K + pl.k_chunk - 1) / pl.k_chunk;
    return pl;
}

} // namespace

SkinnyPlan plan_skinny_realign(int M, int N, int K, int want_splits)
{
    return plan_pieces(M, N, K, want_splits, false);
}

SkinnyPlan plan_skinny_nk(int M, int N, int K, int want_splits)
{
    return plan_pieces(M, N, K, want_splits, true);
}

SkinnyPlan plan_skinny(int M, int N, int K)
{
    SkinnyPlan pl;
    pl.mb = M > 16 ? 2 : 1;
    // The column-tile kernel needs no cross-workgroup reduction and is the
    // fastest when W is cache-resident, but its 64-byte row pieces stream
    // from HBM less efficiently than the split-K kernel's 512-byte pieces;
    // TG_SKINNY_COLS=1 selects it.
    const char *cols = getenv("TG_SKINNY_COLS");
    if (M <= 16 && N % SC_BN == 0 && N / SC_BN >= 128 && K % (4 * SC_BK) == 0 && cols &&
        cols[0] == '1') {
        pl.streaming = 2;
        pl.bn = SC_BN;
        pl.n_tiles = N / SC_BN;
        pl.splits = 1;
        pl.k_chunk = K;
        return pl;
    }
    // Streaming kernel, about one workgroup per CU.  128-column tiles when
    // 256-column ones would need four or more K splits to fill the chip (N <=
    // 16384): the combine then reads half as many splits of half as many
    // columns.  Wider N keeps the 256-column tiles, whose 512-byte row pieces
    // stream from HBM slightly faster (measured at N = 32768 and 65536).
    const bool ok256 = N % 256 == 0 && K % (SaCfg<256>::STAGES * SA_BK) == 0;
    const bool ok128 = N % 128 == 0 && K % (SaCfg<128>::STAGES * SA_BK) == 0;
    const char *bn_env = getenv("TG_SKINNY_BN"); // for sweeps
    const int want = bn_env && *bn_env ? atoi(bn_env) : 0;
    int bn = 0;
    if (want == 128 && ok128)
        bn = 128;
    else if (want == 256 && ok256)
        bn = 256;
    else if (ok128 && (N / 256 <= 64 || !ok256))
        bn = 128;
    else if (ok256)
        bn = 256;
    if (bn) {
        const int stages = bn == 256 ? SaCfg<256>::STAGES : SaCfg<128>::STAGES;
        pl.streaming = 1;
        pl.bn = bn;
        pl.n_tiles = N / bn;
        const int quanta = K / (stages * SA_BK);
        int splits = (256 + pl.n_tiles / 2) / pl.n_tiles;
        const char *force = getenv("TG_SKINNY_SPLITS"); // for sweeps
        if (force && atoi(force) > 0)
            splits = atoi(force);
        splits = splits < 1 ? 1 : (splits > quanta ? quanta : splits);
        const int per = (quanta + splits - 1) / splits;
        pl.k_chunk = per * stages * SA_BK;
        pl.splits = (K + pl.k_chunk - 1) / pl.k_chunk;
        return pl;
    }
    if (M > 16) {
        pl.streaming = -1; // the register-staged kernel holds 16 rows
        pl.bn = 0;
        pl.n_tiles = 0;
        pl.splits = 0;
        pl.k_chunk = 0;
        return pl;
    }
    pl.streaming = 0;
    pl.bn = SK_BN;
    pl.n_tiles = (N + SK_BN - 1) / SK_BN;
    const int kslabs = (K + SK_BK - 1) / SK_BK;
    // about two workgroups per CU (256 CUs), each with at least 4 slabs
    int splits = (512 + pl.n_tiles - 1) / pl.n_tiles;
    const int max_splits = (kslabs + 3) / 4;
    if (splits > max_splits)
        splits = max_splits;
    if (splits < 1)
        splits = 1;
    int slabs_per = (kslabs + splits - 1) / splits;
    slabs_per = (slabs_per + SK_DEPTH - 1) / SK_DEPTH * SK_DEPTH; // whole pipeline rounds
    pl.k_chunk = slabs_per * SK_BK;
    pl.splits = (K + pl.k_chunk - 1) / pl.k_chunk;
    if (pl.splits < 1)
        pl.splits = 1;
    return pl;
}

size_t skinny_ws_floats(const SkinnyPlan &pl, int M, int N)
{
    (void)M;
    if (pl.splits <= 1)
        return 0;
    if (pl.streaming >= 3) // 128 columns computed per workgroup
        return (size_t)pl.splits * 16 * (size_t)pl.mb * 128 * (size_t)pl.n_tiles;
    return pl.streaming ? (size_t)pl.splits * 16 * (size_t)pl.mb * (size_t)N
                        : (size_t)pl.splits * 16 * (size_t)pl.n_tiles * SK_BN;
}

hipError_t launch_skinny(int dt, int act, const GemmArgs &a, const SkinnyPlan &pl, float *ws,
                         int *counters, hipStream_t s)
{
    constexpr int D = SK_DEPTH;
    dim3 grid(pl.n_tiles * pl.splits), block(SK_NT);
    if (pl.streaming == 2) {
#define TG_SC(DT_, ACT_)                                                                         \
    hipLaunchKernelGGL((gemm_skinny_cols_kernel<DT_, ACT_>), grid, dim3(SC_NT), 0, s, a, pl.n_tiles)
        if (dt == DT_F16) {
            if (act == ACT_GELU)
                TG_SC(DT_F16, ACT_GELU);
            else
                TG_SC(DT_F16, ACT_NONE);
        } else {
            if (act == ACT_GELU)
                TG_SC(DT_BF16, ACT_GELU);
            else
                TG_SC(DT_BF16, ACT_NONE);
        }
#undef TG_SC
        return hipGetLastError();
    }
    if (pl.streaming >= 3) {
#define TG_SR(DT_, ACT_, MB_, BT_)                                                               \
    hipLaunchKernelGGL((gemm_skinny_pieces_kernel<DT_, ACT_, MB_, BT_>), grid, dim3(SR_NT), 0, s, \
                       a, pl.n_tiles, pl.bn, pl.k_chunk, pl.splits, ws, counters)
#define TG_SR_MB(DT_, ACT_)                                                                      \
    do {                                                                                         \
        if (pl.streaming == 4 && pl.mb == 2)                                                     \
            TG_SR(DT_, ACT_, 2, true);                                                           \
        else if (pl.streaming == 4)                                                              \
            TG_SR(DT_, ACT_, 1, true);                                                           \
        else if (pl.mb == 2)                                                                     \
            TG_SR(DT_, ACT_, 2, false);                                                          \
        else                                                                                     \
            TG_SR(DT_, ACT_, 1, false);                                                          \
    } while (0)
        if (dt == DT_F16) {
            if (act == ACT_GELU)
                TG_SR_MB(DT_F16, ACT_GELU);
            else
                TG_SR_MB(DT_F16, ACT_NONE);
        } else {
            if (act == ACT_GELU)
                TG_SR_MB(DT_BF16, ACT_GELU);
            else
                TG_SR_MB(DT_BF16, ACT_NONE);
        }
#undef TG_SR_MB
#undef TG_SR
        return hipGetLastError();
    }
    if (pl.streaming == 1) {
#define TG_SA(DT_, ACT_, BN_, MB_)                                                               \
    hipLaunchKernelGGL((gemm_skinny_async_kernel<DT_, ACT_, BN_, MB_>), grid, dim3(SA_NT), 0, s, \
                       a, pl.k_chunk, pl.splits, ws, counters)
#define TG_SA_BN(DT_, ACT_)                                                                      \
    do {                                                                                         \
        if (pl.bn == 128 && pl.mb == 2)                                                          \
            TG_SA(DT_, ACT_, 128, 2);                                                            \
        else if (pl.bn == 128)                                                                   \
            TG_SA(DT_, ACT_, 128, 1);                                                            \
        else if (pl.mb == 2)                                                                     \
            TG_SA(DT_, ACT_, 256, 2);                                                            \
        else                                                                                     \
            TG_SA(DT_, ACT_, 256, 1);                                                            \
    } while (0)
        if (dt == DT_F16) {
            if (act == ACT_GELU)
                TG_SA_BN(DT_F16, ACT_GELU);
            else
                TG_SA_BN(DT_F16, ACT_NONE);
        } else {
            if (act == ACT_GELU)
                TG_SA_BN(DT_BF16, ACT_GELU);
            else
                TG_SA_BN(DT_BF16, ACT_NONE);
        }
#undef TG_SA_BN
#undef TG_SA
        return hipGetLastError();
    }
    const bool fast = a.N % SK_BN == 0 && a.K % (D * SK_BK) == 0 && pl.k_chunk % (D * SK_BK) == 0 &&
                      (int64_t)a.ldb * SK_BK * 2 < (1ll << 30) && (int64_t)a.lda * 16 * 2 < (1ll << 30);
#define TG_SK(DT_, ACT_, EDGE_)                                                                  \
    hipLaunchKernelGGL((gemm_skinny_kernel<DT_, ACT_, (EDGE_ ? 2 : D), EDGE_>), grid, block, 0, s, \
                       a, pl.k_chunk, \
                       pl.splits, ws, counters)
#define TG_SK_E(DT_, ACT_)                                                                       \
    do {                                                                                         \
        if (fast)                                                                                \
            TG_SK(DT_, ACT_, false);                                                             \
        else                                                                                     \
            TG_SK(DT_, ACT_, true);                                                              \
    } while (0)
    if (dt == DT_F16) {
        if (act == ACT_GELU)
            TG_SK_E(DT_F16, ACT_GELU);
        else
            TG_SK_E(DT_F16, ACT_NONE);
    } else {
        if (act == ACT_GELU)
            TG_SK_E(DT_BF16, ACT_GELU);
        else
            TG_SK_E(DT_BF16, ACT_NONE);
    }
#undef TG_SK_E
#undef TG_SK
    return hipGetLastError();
}

} // namespace tg
