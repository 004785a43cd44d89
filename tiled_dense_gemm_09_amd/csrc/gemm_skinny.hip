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

SkinnyPlan plan_skinny(int M, int N, int K)
{
    (void)M;
    SkinnyPlan pl;
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
    (void)N;
    return pl.splits > 1 ? (size_t)pl.splits * 16 * (size_t)pl.n_tiles * SK_BN : 0;
}

hipError_t launch_skinny(int dt, int act, const GemmArgs &a, const SkinnyPlan &pl, float *ws,
                         int *counters, hipStream_t s)
{
    constexpr int D = SK_DEPTH;
    dim3 grid(pl.n_tiles * pl.splits), block(SK_NT);
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
