// gemm_kpad.hip -- zero-padded operand copies for problems whose K is not a
// multiple of the asynchronous kernels' 128-deep loop.  A (and B, in either
// layout) is copied into a workspace with K rounded up and the added entries
// zero, so the extra k terms of every dot product are exactly 0 and the
// result is the one the unpadded definition gives ("TileIR", the tile
// loop over K; the padding is the out-of-bounds-reads-as-zero rule of
// "TIRx", section 5.2, applied once up front instead of per tile).
#include "tg_device.h"
#include "tg_launch.h"

namespace tg {

namespace {

// dst[r][c] = src[r][c] for r < src_rows and c < src_cols, else 0, for a
// dst_rows x dst_cols destination of pitch dst_cols (a multiple of 8).  One
// thread per 16-byte chunk of the destination; vec: the source rows are
// 16-byte aligned, so whole chunks inside the source load at once.
__global__ __launch_bounds__(256) void pad_copy_kernel(const unsigned short *src, int64_t lds,
                                                       int src_rows, int src_cols,
                                                       unsigned short *dst, int dst_rows,
                                                       int dst_cols, int vec)
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
        if (vec && c + 8 <= src_cols) {
            v = *reinterpret_cast<const u32x4 *>(p);
        } else {
            unsigned short e[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                e[i] = c + i < src_cols ? p[i] : (unsigned short)0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[i] = (unsigned int)e[2 * i] | ((unsigned int)e[2 * i + 1] << 16);
        }
    }
    *reinterpret_cast<u32x4 *>(dst + (int64_t)r * dst_cols + c) = v;
}

} // namespace

hipError_t launch_pad_copy(const unsigned short *src, int64_t lds, int src_rows, int src_cols,
                           unsigned short *dst, int dst_rows, int dst_cols, hipStream_t s)
{
    if (dst_cols % 8 != 0 || src_rows > dst_rows || src_cols > dst_cols || ((uintptr_t)dst & 15u))
        return hipErrorInvalidValue;
    const int vec = ((uintptr_t)src & 15u) == 0 && lds % 8 == 0;
    const int64_t n = (int64_t)dst_rows * (dst_cols / 8);
    if (n == 0)
        return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(pad_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, lds,
                       src_rows, src_cols, dst, dst_rows, dst_cols, vec);
    return hipGetLastError();
}

} // namespace tg
