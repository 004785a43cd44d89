// gemm_kpad.hip -- staging copies around the asynchronous kernels.
//
// K padding: for problems whose K is not a multiple of the asynchronous
// kernels' 128-deep loop, A (and B, in either layout) is copied into a
// workspace with K rounded up and the added entries zero, so the extra k
// terms of every dot product are exactly 0 and the result is the one the
// unpadded definition gives ("TileIR", the tile loop over K; the padding is
// the out-of-bounds-reads-as-zero rule of "TIRx", section 5.2, applied once
// up front instead of per tile).
//
// Operands off the 16-byte grid (pitches not a multiple of 8 elements,
// pointers only 2-byte aligned): the same zero-padded copies give the
// kernels aligned rows, and when the output itself is off the grid (or N is
// not a multiple of 8) the kernel writes an aligned, padded copy of C that
// unpad_copy_kernel moves into place ("TIRx", section 5.4: a legal
// dispatch for an operand layout the fast path cannot take directly).
#include "tg_device.h"
#include "tg_launch.h"

namespace tg {

namespace {

// Elements o .. o + 7 of the 16 elements held by two 16-byte pieces (o in
// 0 .. 7, the same in every lane of a row): a funnel shift by o halfwords.
__device__ __forceinline__ u32x4 funnel8(const u32x4 &lo, const u32x4 &hi, int o)
{
    const unsigned w[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    const int q = o >> 1;
    u32x4 out;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        unsigned x = w[k], y = w[k + 1];
#pragma unroll
        for (int t = 1; t < 4; ++t)
            if (q == t) {
                x = w[k + t];
                y = w[k + t + 1];
            }
        out[k] = (o & 1) ? ((x >> 16) | (y << 16)) : x;
    }
    return out;
}

// dst[r][c] = src[r][c] for r < src_rows and c < src_cols, else 0, for a
// dst_rows x dst_cols destination of pitch dst_cols (a multiple of 8).  One
// thread per 16-byte chunk of the destination.  The source (any 2-byte
// aligned pointer and pitch) is read in aligned 16-byte pieces: the piece
// that holds element c, and the next one only when it holds an element of
// the row (c + 8 - o < src_cols), so every piece read holds at least one
// element of the source; the thread's 8 elements are funnelled out of the
// two and those at or past src_cols are zeroed.
__global__ __launch_bounds__(256) void pad_copy_kernel(const unsigned short *src, int64_t lds,
                                                       int src_rows, int src_cols,
                                                       unsigned short *dst, int dst_rows,
                                                       int dst_cols)
{
    const int64_t chunks = dst_cols / 8;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)dst_rows * chunks)
        return;
    const int r = (int)(idx / chunks);
    const int c = (int)(idx % chunks) * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < src_rows && c < src_cols) {
        const unsigned short *p = src + (int64_t)r * lds + c;
        const int o = (int)(((uintptr_t)p >> 1) & 7);
        const unsigned short *b = p - o;
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(b);
        u32x4 hi = {0u, 0u, 0u, 0u};
        if (o != 0 && c + 8 - o < src_cols)
            hi = *reinterpret_cast<const u32x4 *>(b + 8);
        v = funnel8(lo, hi, o);
        if (c + 8 > src_cols) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (c + i >= src_cols)
                    v[i / 2] &= (i & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        }
    }
    *reinterpret_cast<u32x4 *>(dst + (int64_t)r * dst_cols + c) = v;
}

// dst[r][c] = src[r][c] for r < rows, c < cols.  src: rows of src_pitch
// elements (a multiple of 8), 16-byte aligned, readable for 8 elements past
// the end of its last row; dst: any 2-byte aligned pointer and pitch.
// Thread (r, j) writes the j-th 16-byte-aligned piece of destination row r,
// elements e0 .. e0 + 7 with e0 = 8 j - s (the row starts s elements past a
// 16-byte boundary): with one aligned 16-byte store when the piece lies
// inside the row, element by element at the row's ends.
__global__ __launch_bounds__(256) void unpad_copy_kernel(const unsigned short *src, int src_pitch,
                                                         unsigned short *dst, int64_t ldd,
                                                         int rows, int cols, int pieces)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)rows * pieces)
        return;
    const int r = (int)(idx / pieces);
    const int j = (int)(idx % pieces);
    unsigned short *drow = dst + (int64_t)r * ldd;
    const unsigned short *srow = src + (int64_t)r * src_pitch;
    const int s = (int)(((uintptr_t)drow >> 1) & 7);
    const int e0 = 8 * j - s;
    if (e0 >= 0 && e0 + 8 <= cols) {
        // elements e0 .. e0 + 7 of the source row out of the two aligned
        // 16-byte pieces that hold them (b + 16 <= e0 + 16 <= cols + 8)
        const int b = e0 & ~7, o = e0 & 7;
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(srow + b);
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(srow + b + 8);
        const u32x4 out = funnel8(lo, hi, o);
        *reinterpret_cast<u32x4 *>(drow + e0) = out;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = e0 + i;
            if (e >= 0 && e < cols)
                drow[e] = srow[e];
        }
    }
}

} // namespace

hipError_t launch_unpad_copy(const unsigned short *src, int src_pitch, unsigned short *dst,
                             int64_t ldd, int rows, int cols, hipStream_t s)
{
    if (src_pitch % 8 != 0 || cols > src_pitch || ldd < cols || ((uintptr_t)src & 15u) ||
        ((uintptr_t)dst & 1u))
        return hipErrorInvalidValue;
    const int pieces = (cols + 14) / 8; // a row starting 7 elements past a boundary needs one more
    const int64_t n = (int64_t)rows * pieces;
    if (n == 0)
        return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(unpad_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, src_pitch,
                       dst, ldd, rows, cols, pieces);
    return hipGetLastError();
}

hipError_t launch_pad_copy(const unsigned short *src, int64_t lds, int src_rows, int src_cols,
                           unsigned short *dst, int dst_rows, int dst_cols, hipStream_t s)
{
    if (dst_cols % 8 != 0 || src_rows > dst_rows || src_cols > dst_cols || ((uintptr_t)dst & 15u) ||
        ((uintptr_t)src & 1u))
        return hipErrorInvalidValue;
    const int64_t n = (int64_t)dst_rows * (dst_cols / 8);
    if (n == 0)
        return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(pad_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, lds,
                       src_rows, src_cols, dst, dst_rows, dst_cols);
    return hipGetLastError();
}

} // namespace tg
