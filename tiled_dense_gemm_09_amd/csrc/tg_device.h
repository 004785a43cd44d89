// tg_device.h -- shared device/host helpers of the HIP library: vector types,
// the tile scheduler, LDS addressing, bounds predicate, the FP32 epilogue and
// the f16/bf16 output conversion.  Host-callable parts are __host__ __device__
// so the CPU tests exercise the same code the kernels run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

enum { DT_F16 = 1, DT_BF16 = 2 };
enum { ACT_NONE = 0, ACT_GELU = 1 };

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Number of XCDs on MI355X; the hardware hands workgroup b to XCD b % 8.
constexpr int kNumXcd = 8;

// Synchronising build (compiled with -DTG_DEBUG_SYNC into
// libtg_debugsync.so beside the library): every partial wait of a copy
// pipeline waits for all outstanding memory operations instead, and every
// pipeline barrier is preceded by such a wait, so no LDS stage is read
// before every copy into it has landed, nor refilled while a wave may still
// read it.  The arithmetic and its order are unchanged, so the outputs must
// equal the normal build's bit for bit; a difference exposes a wait or a
// barrier that the normal build gets wrong.
#ifdef TG_DEBUG_SYNC
constexpr bool kDebugSync = true;
#else
constexpr bool kDebugSync = false;
#endif

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at maximum);
// in the synchronising build, every counter at zero.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    if constexpr (kDebugSync)
        __builtin_amdgcn_s_waitcnt(0);
    else
        __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier for the copy pipelines.  The usual __syncthreads() adds
// a workgroup release fence, which waits for every outstanding direct-to-LDS
// copy (they count as LDS writes) and would drain all stages each step.  Here
// each wave waits for exactly the copies it needs with wait_vmcnt first; the
// empty asm statements keep the compiler from moving LDS accesses across the
// barrier.  The synchronising build waits for everything first.
__device__ __forceinline__ void stage_barrier()
{
    if constexpr (kDebugSync)
        __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

struct TileCoord {
    int mat, tm, tn;
};

// Tile scheduler ("Beyond Hand-Written CUDA", section 2: the tile
// scheduler stage; "TileIR": data movement is the main cost).
//
// 1. XCD-aware remap.  Consecutive workgroup ids land on different XCDs, each
//    with its own L2.  Workgroup b runs on XCD b % 8 as that XCD's
//    (b / 8)-th block; give it logical id prefix(xcd) + b / 8, so every XCD
//    works through one contiguous run of logical tiles.
// 2. Grouped order.  Logical ids walk group_m tile-rows at a time, column by
//    column, over a virtual grid of tiles_m x (n_mat * tiles_n) tiles, so the
//    tiles an XCD runs together share A row-panels and B column-panels.  For
//    the fused QKV projection the n_mat = 3 matrices sit side by side in the
//    virtual grid and reuse the same row-panels of X.
// Both steps are bijections, so every tile is computed exactly once.
// Step 2 alone: logical id -> tile in grouped order (a bijection of
// [0, tiles_m * tiles_n * n_mat) onto the tiles).
__host__ __device__ inline TileCoord grouped_tile(int tiles_m, int tiles_n, int n_mat, int group_m,
                                                  int logical)
{
    const int width = tiles_n * n_mat;
    const int group_size = group_m * width;
    const int g = logical / group_size;
    const int first_m = g * group_m;
    const int rows_left = tiles_m - first_m;
    const int gm = rows_left < group_m ? rows_left : group_m;
    const int in_group = logical - g * group_size;
    TileCoord t;
    t.tm = first_m + in_group % gm;
    const int tv = in_group / gm;
    t.mat = tv / tiles_n;
    t.tn = tv - t.mat * tiles_n;
    return t;
}

// Both steps: workgroup id -> tile.
__host__ __device__ inline TileCoord schedule_tile(int tiles_m, int tiles_n, int n_mat,
                                                   int group_m, int bid)
{
    const int total = tiles_m * tiles_n * n_mat;
    const int xcd = bid % kNumXcd;
    const int slot = bid / kNumXcd;
    const int q = total / kNumXcd, r = total % kNumXcd;
    return grouped_tile(tiles_m, tiles_n, n_mat, group_m, xcd * q + (xcd < r ? xcd : r) + slot);
}

// LDS tiles store rows of `cols` 16-bit elements with the row pitch padded by
// 8 elements (16 bytes).  With pitch (cols + 8) * 2 bytes, 16 consecutive
// rows read at the same column start on 16 distinct 16-byte bank groups, so
// the 128-bit fragment reads of one 16-lane phase are conflict-free.  For a
// 128-wide tile this is pitch 136 (the padded strided layout example of
// "TIRx", section 3.1).
__host__ __device__ constexpr int lds_pitch(int cols) { return cols + 8; }
__host__ __device__ inline int64_t lds_offset_bytes(int64_t cols, int64_t row, int64_t col)
{
    return (row * (cols + 8) + col) * 2;
}

// Logical bounds: (row, col) is inside a rows x cols matrix iff both
// coordinates are in range, whatever the linear offset ("TIRx", section 5.2:
// the out-of-bounds rule of the asynchronous copy).
__host__ __device__ inline bool in_bounds(int64_t rows, int64_t cols, int64_t row, int64_t col)
{
    return row >= 0 && col >= 0 && row < rows && col < cols;
}

// tanh form of GELU in FP32, evaluated through the identity
//     0.5 x (1 + tanh(u)) = x / (1 + e^{-2u}),   u = sqrt(2/pi) (x + 0.044715 x^3),
// so one exponential and one reciprocal per value: e^{-2u} = 2^{x (k1 + k2 x^2)}
// with k1 = -2 sqrt(2/pi) log2(e) and k2 = 0.044715 k1, both on the hardware
// base-2 exponential and reciprocal (about 1 ulp each; the result is rounded
// to f16/bf16 afterwards).  For large |x| the exponential saturates to 0 or
// +inf and the result to x or -0.
__device__ __forceinline__ float gelu_tanh_f32(float x)
{
    const float k1 = -2.302208198144325f;   // -2 sqrt(2/pi) / ln 2
    const float k2 = -0.1029432395800235f;  // 0.044715 k1
    const float t = __builtin_fmaf(x * x, k2, k1);
    const float e = __builtin_amdgcn_exp2f(x * t);
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}

template <int ACT>
__device__ __forceinline__ float activate(float v)
{
    if constexpr (ACT == ACT_GELU)
        return gelu_tanh_f32(v);
    else
        return v;
}

// f32 -> 16-bit pattern, round to nearest even.
template <int DT>
__device__ __forceinline__ unsigned short to_bits(float v)
{
    if constexpr (DT == DT_F16) {
        _Float16 h = (_Float16)v;
        return __builtin_bit_cast(unsigned short, h);
    } else {
        __bf16 h = (__bf16)v;
        return __builtin_bit_cast(unsigned short, h);
    }
}

template <int DT>
__device__ __forceinline__ float from_bits(unsigned short b)
{
    if constexpr (DT == DT_F16)
        return (float)__builtin_bit_cast(_Float16, b);
    else
        return __builtin_bit_cast(float, (unsigned int)b << 16);
}

// Two f32 values -> two 16-bit values packed low/high, round to nearest even
// (one v_cvt_pk_{f16,bf16}_f32 on gfx950).
template <int DT>
__device__ __forceinline__ unsigned int pack2(float lo, float hi)
{
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 v = {lo, hi};
    if constexpr (DT == DT_F16) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(unsigned int, __builtin_convertvector(v, h2));
    } else {
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(unsigned int, __builtin_convertvector(v, b2));
    }
}

// One 16x16x32 MFMA step: acc += src0 (16 rows x 32 k) * src1 (32 k x 16 cols).
// Lane l holds 8 k-values of row (l % 16) of src0 and of column (l % 16) of
// src1; both operands use the same k order, so any k permutation is harmless.
template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c)
{
    if constexpr (DT == DT_F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// v[r] += R[m][n + r] for r < CNT (the residual of the extended epilogue,
// added after the activation and before the rounding).  Columns at or past N
// are skipped; when all CNT columns are in range and CNT is a multiple of 4
// the row segment is read with 8-byte loads (n a multiple of 4, R 16-byte
// aligned and ldr a multiple of 8 on every path that passes CNT >= 4).
// VEC = false: element-wise loads only (R or its pitch not 8-byte aligned)
template <int DT, int CNT, bool VEC = true>
__device__ __forceinline__ void add_residual(const unsigned short *R, int64_t ldr, int64_t m,
                                             int n, int N, float *v)
{
    const unsigned short *rp = R + m * ldr + n;
    if (VEC && CNT % 4 == 0 && n + CNT <= N) {
#pragma unroll
        for (int q = 0; q < CNT / 4; ++q) {
            const u32x2 w = *reinterpret_cast<const u32x2 *>(rp + 4 * q);
            v[4 * q + 0] += from_bits<DT>((unsigned short)(w[0] & 0xFFFFu));
            v[4 * q + 1] += from_bits<DT>((unsigned short)(w[0] >> 16));
            v[4 * q + 2] += from_bits<DT>((unsigned short)(w[1] & 0xFFFFu));
            v[4 * q + 3] += from_bits<DT>((unsigned short)(w[1] >> 16));
        }
    } else {
#pragma unroll
        for (int r = 0; r < CNT; ++r)
            if (n + r < N)
                v[r] += from_bits<DT>(rp[r]);
    }
}

// One 32x32x16 MFMA step: acc += src0 (32 rows x 16 k) * src1 (16 k x 32 cols).
// Lane l holds 8 k-values of row (l % 32) of src0 and of column (l % 32) of
// src1 (the same k order on both sides).  Accumulator register r of lane l is
// element (row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32).
template <int DT>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c)
{
    if constexpr (DT == DT_F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Split-K partials: stores PV 16-byte vectors at dst + 1 KiB v (v = 0 ..
// PV-1) with device-coherent stores (sc1, written through to the device
// coherence point since the XCDs' L2 caches are not coherent with each
// other) and waits for them, all in one asm statement.
// The compiler treats the data registers of an asm store as free once the
// statement ends and may write them at once, while the store can still be
// reading them; with the wait inside the statement they stay untouched until
// every store has completed.  Four vectors share a base address (immediate
// offsets 0, 1, 2, 3 KiB).
#define TG_ST4(B, V0, V1, V2, V3)                                                                   \
    "global_store_dwordx4 %" #B ", %" #V0 ", off sc1\n\t"                                         \
    "global_store_dwordx4 %" #B ", %" #V1 ", off offset:1024 sc1\n\t"                             \
    "global_store_dwordx4 %" #B ", %" #V2 ", off offset:2048 sc1\n\t"                             \
    "global_store_dwordx4 %" #B ", %" #V3 ", off offset:3072 sc1\n\t"
template <int PV>
__device__ __forceinline__ void store_partial(float *dst, const f32x4 (&v)[PV])
{
    if constexpr (PV == 32) {
        asm volatile(TG_ST4(0, 8, 9, 10, 11) TG_ST4(1, 12, 13, 14, 15) TG_ST4(2, 16, 17, 18, 19)
                         TG_ST4(3, 20, 21, 22, 23) TG_ST4(4, 24, 25, 26, 27)
                             TG_ST4(5, 28, 29, 30, 31) TG_ST4(6, 32, 33, 34, 35)
                                 TG_ST4(7, 36, 37, 38, 39) "s_waitcnt vmcnt(0)" ::"v"(dst),
                     "v"(dst + 1024), "v"(dst + 2048), "v"(dst + 3072), "v"(dst + 4096),
                     "v"(dst + 5120), "v"(dst + 6144), "v"(dst + 7168), "v"(v[0]), "v"(v[1]),
                     "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]), "v"(v[8]),
                     "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]),
                     "v"(v[15]), "v"(v[16]), "v"(v[17]), "v"(v[18]), "v"(v[19]), "v"(v[20]),
                     "v"(v[21]), "v"(v[22]), "v"(v[23]), "v"(v[24]), "v"(v[25]), "v"(v[26]),
                     "v"(v[27]), "v"(v[28]), "v"(v[29]), "v"(v[30]), "v"(v[31])
                     : "memory");
    } else if constexpr (PV == 16) {
        asm volatile(TG_ST4(0, 4, 5, 6, 7) TG_ST4(1, 8, 9, 10, 11) TG_ST4(2, 12, 13, 14, 15)
                         TG_ST4(3, 16, 17, 18, 19) "s_waitcnt vmcnt(0)" ::"v"(dst),
                     "v"(dst + 1024), "v"(dst + 2048), "v"(dst + 3072), "v"(v[0]), "v"(v[1]),
                     "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]), "v"(v[8]),
                     "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]),
                     "v"(v[15])
                     : "memory");
    } else if constexpr (PV == 8) {
        asm volatile(TG_ST4(0, 2, 3, 4, 5) TG_ST4(1, 6, 7, 8, 9) "s_waitcnt vmcnt(0)" ::"v"(dst),
                     "v"(dst + 1024), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]),
                     "v"(v[5]), "v"(v[6]), "v"(v[7])
                     : "memory");
    } else if constexpr (PV == 4) {
        asm volatile(TG_ST4(0, 1, 2, 3, 4) "s_waitcnt vmcnt(0)" ::"v"(dst), "v"(v[0]), "v"(v[1]),
                     "v"(v[2]), "v"(v[3])
                     : "memory");
    } else {
        static_assert(PV == 2, "partial vector count");
        asm volatile("global_store_dwordx4 %0, %1, off sc1\n\t"
                     "global_store_dwordx4 %0, %2, off offset:1024 sc1\n\t"
                     "s_waitcnt vmcnt(0)" ::"v"(dst),
                     "v"(v[0]), "v"(v[1])
                     : "memory");
    }
}
#undef TG_ST4

// The counterpart of store_partial<32>: loads 32 16-byte vectors at src +
// 1 KiB v with device-coherent loads (sc1) and waits for them, all in one asm
// statement, so no result register is read (or copied) before its data has
// landed.
#define TG_LD4(B, V0, V1, V2, V3)                                                                   \
    "global_load_dwordx4 %" #V0 ", %" #B ", off sc1\n\t"                                        \
    "global_load_dwordx4 %" #V1 ", %" #B ", off offset:1024 sc1\n\t"                            \
    "global_load_dwordx4 %" #V2 ", %" #B ", off offset:2048 sc1\n\t"                            \
    "global_load_dwordx4 %" #V3 ", %" #B ", off offset:3072 sc1\n\t"
__device__ __forceinline__ void load_partial32(const float *src, f32x4 (&v)[32])
{
    asm volatile(TG_LD4(32, 0, 1, 2, 3) TG_LD4(33, 4, 5, 6, 7) TG_LD4(34, 8, 9, 10, 11)
                     TG_LD4(35, 12, 13, 14, 15) TG_LD4(36, 16, 17, 18, 19)
                         TG_LD4(37, 20, 21, 22, 23) TG_LD4(38, 24, 25, 26, 27)
                             TG_LD4(39, 28, 29, 30, 31) "s_waitcnt vmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
                   "=&v"(v[6]), "=&v"(v[7]), "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]),
                   "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]), "=&v"(v[14]), "=&v"(v[15]),
                   "=&v"(v[16]), "=&v"(v[17]), "=&v"(v[18]), "=&v"(v[19]), "=&v"(v[20]),
                   "=&v"(v[21]), "=&v"(v[22]), "=&v"(v[23]), "=&v"(v[24]), "=&v"(v[25]),
                   "=&v"(v[26]), "=&v"(v[27]), "=&v"(v[28]), "=&v"(v[29]), "=&v"(v[30]),
                   "=&v"(v[31])
                 : "v"(src), "v"(src + 1024), "v"(src + 2048), "v"(src + 3072), "v"(src + 4096),
                   "v"(src + 5120), "v"(src + 6144), "v"(src + 7168)
                 : "memory");
}
#undef TG_LD4

} // namespace tg
