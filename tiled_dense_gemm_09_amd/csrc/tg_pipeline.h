// tg_pipeline.h -- pieces shared by the asynchronous-copy kernels: the
// 64-byte-row LDS swizzle, the copy-pipeline barrier and wait, and the
// epilogue that restages a wave's rounded output tile through LDS.
#pragma once

#include "tg_device.h"

namespace tg {

// Granule c (16 bytes) of row r of a 64-byte-row tile sits at c ^ swz_a(r).
// A 128-bit LDS read is served 16 lanes at a time from 64 four-byte banks
// (256 bytes, measured with the bank-conflict counter on gfx950); the 16
// consecutive rows that one such group reads then land on 16 different
// 16-byte bank groups: row r covers groups 4 (r % 4) + (c ^ swz_a(r)).
__host__ __device__ constexpr int swz_a(int r) { return (r >> 2) & 3; }

// The same for 128-byte rows (64 k, 8 granules): rows r and r + 2 start on
// the same bank, so the 16 rows of one read pass need 8 distinct XOR values
// for each row parity: granule c of row r sits at c ^ ((r >> 1) & 7), and
// the pass covers groups 8 (r % 2) + (c ^ ((r >> 1) & 7)), all 16 of them.
__host__ __device__ constexpr int swz_a8(int r) { return (r >> 1) & 7; }

// B swizzle for rows of 16 or more granules: {0, 6, 10, 12}[r & 3] as a
// nibble table (a shift, not a branch chain).  For 8-granule (128-byte) rows
// the rows r and r + 2 share banks; flipping granule bit 2 on rows with bit
// 1 set moves the four 64-byte row pieces one transposing read pass covers
// (rows 4q .. 4q+3, 64 bytes each) onto four disjoint quarters of the
// 256-byte bank window.
template <int BN>
__host__ __device__ constexpr int swz_b(int r)
{
    return BN >= 128 ? (0xCA60 >> (4 * (r & 3))) & 15 : 4 * ((r >> 1) & 1);
}

// B swizzle of the 16x16x32 kernel (512-byte rows): one transposing read
// pass covers rows 4q .. 4q+3 and 4q+8 .. 4q+11 (two 16-lane groups), 32
// bytes each; the row-bit-3 term puts the second group's rows on the other
// eight granule pairs, so the pass hits all 64 banks once.
__host__ __device__ constexpr int swz_b16(int r) { return swz_b<256>(r) ^ (2 * ((r >> 3) & 1)); }

// B swizzle of the 192 x 192 16x16x32 kernel (384-byte rows, 24 granules;
// rows of one parity start on the same bank, the other parity 128 bytes
// over).  A transposing read pass covers two granules of rows a, a + 1, a +
// 2, a + 3, a + 8, ..., a + 11 (a a multiple of 4): the four rows of each
// parity must take four different granule pairs, which (r & 2) | ((r >> 1)
// & 4) gives (bits 1 and 3 of the row); the XOR moves a granule only inside
// its aligned group of eight, so it stays inside the 24-granule row.
__host__ __device__ constexpr int swz_b192(int r) { return (r & 2) | ((r >> 1) & 4); }

// B swizzle of the 128 x 128 16x16x32 kernel (256-byte rows: every row spans
// the whole bank window from bank 0).  A transposing read pass covers one
// granule pair of rows a .. a + 3 and a + 8 .. a + 11; giving those eight
// rows the eight distinct even XOR values 2 (r % 4) + 8 (bit 3 of r) puts
// the eight pairs on disjoint banks, and an even XOR keeps each pair whole.
__host__ __device__ constexpr int swz_b128(int r) { return ((r & 3) << 1) | (r & 8); }

// Epilogue of one wave holding TI x TJ 32x32 FP32 accumulator blocks (the
// bias already inside).  Lane l of block (i, j) holds row 32 i + l % 32 and
// columns 32 j + 8 g + 4 (l / 32) + {0..3} in registers 4g..4g+3.  The
// activation, the residual (HR: R[m][n] added after it) and the rounding
// happen there; the rounded (32 TI) x (32 TJ) tile is then restaged through
// the wave's own LDS region `ep` (rows of 4 TJ 16-byte granules, granule c
// of row r at c ^ (r % 4TJ)) so that each global store writes whole
// 64 TJ-byte row segments instead of 16-byte pieces of 32 rows.  C points
// at the wave tile's first element; R likewise (row pitch ldr).
// Rows at or past `rows` and columns at or past `cols` (a multiple of 8;
// partial last row or column tiles) are neither read from R nor stored.
template <int DT, int ACT, int TI, int TJ, bool HR>
__device__ __forceinline__ void restaged_epilogue(const f32x16 (&acc)[TI][TJ], unsigned char *ep,
                                                  int lane, unsigned short *C, int64_t ldc,
                                                  const unsigned short *R, int64_t ldr,
                                                  int rows = 1 << 30, int cols = 1 << 30)
{
    constexpr int EG = 4 * TJ; // granules per row of the wave tile
#pragma unroll
    for (int i = 0; i < TI; ++i) {
        const int r = i * 32 + (lane & 31);
        u32x2 rr[TJ][4];
        if constexpr (HR) {
#pragma unroll
            for (int j = 0; j < TJ; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    rr[j][g] = r < rows && j * 32 + g * 8 + (lane >> 5) * 4 < cols
                                   ? *reinterpret_cast<const u32x2 *>(
                                         R + (int64_t)r * ldr + j * 32 + g * 8 + (lane >> 5) * 4)
                                   : u32x2{0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = activate<ACT>(acc[i][j][4 * g + e]);
                    if constexpr (HR)
                        v[e] += from_bits<DT>((unsigned short)(rr[j][g][e >> 1] >> (16 * (e & 1))));
                }
                const u32x2 o = {pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3])};
                const int c = (4 * j + g) ^ (r & (EG - 1));
                *reinterpret_cast<u32x2 *>(ep + r * (16 * EG) + c * 16 + (lane >> 5) * 8) = o;
            }
        }
    }
    // each lane reads back granule lane % EG of rows (64 / EG) t + lane / EG
    // (its own wave's writes, so no barrier) and stores it
    unsigned short *crow = C + (lane % EG) * 8;
#pragma unroll
    for (int t = 0; t < 2 * TI * TJ; ++t) {
        const int r = (64 / EG) * t + lane / EG;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(ep + r * (16 * EG) +
                                                         (((lane % EG) ^ (r & (EG - 1))) * 16));
        if (r < rows && (lane % EG) * 8 < cols)
            *reinterpret_cast<u32x4 *>(crow + (int64_t)r * ldc) = v;
    }
}

} // namespace tg
