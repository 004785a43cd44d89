// gemm_generic.hip -- the correct-but-slow fallback for operands the 128-bit
// MFMA path cannot take (pointers not 16-byte aligned, pitches that are not a
// multiple of 8 elements, a B stored [N,K] outside the shapes of the
// asynchronous-copy kernel).  One thread per output element, FP32 FMA over k,
// then the same FP32 epilogue and round-to-nearest-even store as the fast
// path.  It is chosen only by explicit dispatch and reported through
// tg_last_kernel(), never silently ("TIRx", section 5.4: a fallback comes
// with a diagnostic).
#include "tg_device.h"
#include "tg_launch.h"

namespace tg {

template <int DT, int ACT>
__global__ __launch_bounds__(256) void gemm_generic_kernel(GemmArgs p)
{
    const int64_t n = (int64_t)blockIdx.x * 16 + (threadIdx.x & 15);
    const int t = blockIdx.z;
    if (n >= p.N)
        return;
    const unsigned short *B = t == 0 ? p.B[0] : (t == 1 ? p.B[1] : p.B[2]);
    unsigned short *C = t == 0 ? p.C[0] : (t == 1 ? p.C[1] : p.C[2]);
    // rows in a grid-stride loop (grid.y is capped by the host)
    for (int64_t m = (int64_t)blockIdx.y * 16 + (threadIdx.x >> 4); m < p.M;
         m += (int64_t)gridDim.y * 16) {
        const unsigned short *a = p.A + m * p.lda;
        float acc = 0.f;
        // element (k, n) of op(B): B[k][n], or B[n][k] when B is stored [N,K]
        const int64_t bk = p.b_trans ? 1 : p.ldb, bn = p.b_trans ? p.ldb : 1;
        for (int k = 0; k < p.K; ++k)
            acc = __builtin_fmaf(from_bits<DT>(a[k]), from_bits<DT>(B[(int64_t)k * bk + n * bn]),
                                 acc);
        if (p.bias != nullptr)
            acc += from_bits<DT>(p.bias[n]);
        float v = activate<ACT>(acc);
        if (p.R != nullptr)
            add_residual<DT, 1>(p.R, p.ldr, m, (int)n, p.N, &v);
        C[m * p.ldc + n] = to_bits<DT>(v);
    }
}

hipError_t launch_generic(int dt, int act, const GemmArgs &a, hipStream_t s)
{
    const int64_t gy = ((int64_t)a.M + 15) / 16;
    dim3 grid((a.N + 15) / 16, (unsigned)(gy < 65535 ? gy : 65535), a.n_mat), block(256);
    if (dt == DT_F16) {
        if (act == ACT_GELU)
            hipLaunchKernelGGL((gemm_generic_kernel<DT_F16, ACT_GELU>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((gemm_generic_kernel<DT_F16, ACT_NONE>), grid, block, 0, s, a);
    } else {
        if (act == ACT_GELU)
            hipLaunchKernelGGL((gemm_generic_kernel<DT_BF16, ACT_GELU>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((gemm_generic_kernel<DT_BF16, ACT_NONE>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

} // namespace tg
