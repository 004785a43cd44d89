// gemm_async.hip -- the tiled MFMA GEMM with asynchronous global->LDS copies
// for interior problems (M, N multiples of 256, K a multiple of 128).
//
// Same method as gemm_tiled (tile loop with an FP32 register accumulator and
// a register-resident epilogue; "TileIR", the matmul inner loop;
// "Beyond Hand-Written CUDA", section 4), mapped differently onto gfx950:
//
//  - Both operand tiles go from HBM straight into LDS with 16-byte
//    direct-to-LDS loads: no staging registers, no VALU work.  Lane l of a
//    wave-wide copy writes the 16 bytes at LDS base + 16 l, so each copy
//    instruction fills 1 KiB of LDS; which global chunk a lane fetches is
//    chosen so that the LDS image comes out swizzled.
//  - Four LDS stages of BK = 32 ("Beyond Hand-Written CUDA", section 5:
//    footprint = stages x (A tile + B tile) = 4 x 32 KiB = 128 KiB of the
//    160 KiB per CU).  The copies of step k+3 are issued while step k
//    computes, so every load has three K-steps of MFMA work to land.
//  - A is stored K-contiguous ([256 rows][32 k], 64-byte rows) and read with
//    128-bit LDS reads.  B stays as it is in memory, N-contiguous
//    ([32 k][256 n], 512-byte rows); its MFMA fragments (8 consecutive k of
//    one column per lane) come from the LDS transposing read, which hands
//    lane i of a 16-lane group element q = R[4q + i/4][i%4] of the 16 x 4
//    block R the group addressed.  With lane j addressing row (j/4), columns
//    4 (j%4)..4 (j%4)+3, lane i receives column i at 4 consecutive k; two
//    such reads give the 8 k of a 32x32x16 MFMA operand.
//  - XOR swizzles (16-byte granules) make both the 128-bit A reads and the
//    transposing B reads bank-conflict-free.  A 128-bit LDS read is served
//    16 lanes at a time from 64 four-byte banks (256 bytes), so the 16 rows
//    of 64 bytes that lanes 16q..16q+15 read must land on 16 different
//    16-byte bank groups: row r sits on groups 4 (r % 4) + (c ^ s(r)), and
//    s(r) = (r >> 2) & 3 covers the four values for each r % 4 (measured
//    with the bank-conflict counter on gfx950, as was the B pattern):
//        A: granule c of row r at c ^ ((r >> 2) & 3)
//        B: granule c of row r at c ^ {0, 6, 10, 12}[r & 3]
//           (64-column tiles: c ^ 4 ((r >> 1) & 1))
//    (power-of-two extents throughout; "TIRx", section 7 on XOR layouts).
#include <type_traits>

#include "tg_device.h"
#include "tg_launch.h"
#include "tg_pipeline.h"

namespace tg {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int AS_BK = 32, AS_STAGES = 4, AS_NT = 256;

// Tile geometry for TI x TJ 32x32 accumulator blocks per wave and 2 x 2
// waves: the workgroup tile is (64 TI) x (64 TJ).
template <int TI, int TJ>
struct AsGeom {
    static constexpr int BM = 64 * TI, BN = 64 * TJ;
    static constexpr int A_BYTES = BM * AS_BK * 2;      // [BM][32] K-contiguous
    static constexpr int B_BYTES = AS_BK * BN * 2;      // [32][BN] N-contiguous
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int COPIES = TI + TJ;              // 1 KiB copies per wave per step
    static constexpr int C1 = COPIES / 2;               // copies issued in the second half-step
    static constexpr int B_ROWS_PER_COPY = 512 / BN;    // 1 KiB of [32][BN]
    static constexpr int B_GRANULES = BN / 8;           // 16-byte granules per B row
    static_assert(BN >= 64, "B rows of at least 8 granules");
};

} // namespace

// K not a multiple of the 128-deep loop (KM kernels): the last, partial
// quad's copies whose 8 k (A, B stored [N,K]) or whose k row (B stored
// [K,N]) lie at or past K read this zero granule instead,
// so the added k terms multiply exact zeros on both sides ("TIRx", section
// 5.2: out-of-bounds reads give zeros, judged by the logical coordinate).
// K must be a multiple of 8, so a granule is never cut by K.
__device__ __align__(16) unsigned int kZeroGranule[4];

// Split-K partial exchange of one workgroup (see the kernel below).  The
// partial of a tile's split is [4 waves][4 TI TJ vectors][64 lanes] of
// 16-byte vectors, vector 4 (TJ i + j) + g holding registers 4g..4g+3 of
// accumulator block (i, j), so each store or load instruction moves one
// contiguous KiB per wave.  Returns true in the workgroup that completed
// the count, with acc replaced by the ordered sum of all the splits.
template <int TI, int TJ>
__device__ __forceinline__ bool combine_splits(f32x16 (&acc)[TI][TJ], float *ws, int *counters,
                                               int tile, int split, int splits, int wave, int lane)
{
    constexpr int PV = 4 * TI * TJ;                  // vectors per lane per split: 4, 8 or 16
    constexpr int BLOCK = AS_NT / 64 * PV * 256;     // floats per split partial
    constexpr int RS = 32 / PV;                      // splits read back per round
    __shared__ int s_last;
    float *ws_tile = ws + (int64_t)tile * splits * BLOCK;
    const int lane_off = wave * PV * 256 + lane * 4;
    {
        f32x4 v[PV];
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    v[(i * TJ + j) * 4 + g] = f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1],
                                                    acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        store_partial<PV>(ws_tile + (int64_t)split * BLOCK + lane_off, v);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int old = __hip_atomic_fetch_add(&counters[tile], 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old == splits - 1);
    }
    __syncthreads();
    if (!s_last)
        return false;

    // Rounds of RS splits, all 32 loads of a round in flight together, added
    // in split order; indices past the last split repeat it and are not
    // added.  The own split is read back too, so no branch sits between a
    // load and its wait.
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.f;
    for (int sp0 = 0; sp0 < splits; sp0 += RS) {
        f32x4 v[32];
#pragma unroll
        for (int u = 0; u < RS; ++u) {
            const float *src = ws_tile + (int64_t)min(sp0 + u, splits - 1) * BLOCK + lane_off;
#pragma unroll
            for (int t = 0; t < PV; ++t)
                asm volatile("global_load_dwordx4 %0, %1, off sc1"
                             : "=v"(v[u * PV + t])
                             : "v"(src + t * 256)
                             : "memory");
        }
        // the loads are invisible to the compiler's wait tracking: wait here
        // with every value passed through, so nothing reads one earlier
        // (loads return in order)
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
#pragma unroll
        for (int u = 0; u < RS; ++u)
            if (sp0 + u < splits)
#pragma unroll
                for (int i = 0; i < TI; ++i)
#pragma unroll
                    for (int j = 0; j < TJ; ++j)
#pragma unroll
                        for (int g = 0; g < 4; ++g)
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                acc[i][j][4 * g + e] += v[u * PV + (i * TJ + j) * 4 + g][e];
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&counters[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

// Split-K (splits > 1, grid = tiles x splits, block b = split * tiles + tile):
// split s covers k in [s K / splits, (s + 1) K / splits), a multiple of the
// four-step loop.  Each split's FP32 partial goes to ws with device-coherent
// stores (the XCDs' L2 caches are not coherent with each other); one atomic
// per workgroup counts it in, and the workgroup that completes the count
// reads every partial back (device-coherent loads), adds them in split order
// 0 .. splits-1 whatever the arrival order, runs the epilogue and resets the
// tile's counter to zero.  The bias enters through split 0's accumulators.
// ws holds splits x BM x BN floats per tile; counters one int per tile, zero
// before the launch and zero after it.
template <int DT, int ACT, int TI, int TJ, bool BT>
__global__ __launch_bounds__(AS_NT, TI * TJ >= 16 ? 1 : 2) void gemm_async_kernel(
    GemmArgs p, int tiles_m, int tiles_n, int group_m, int splits, float *ws, int *counters)
{
    using G = AsGeom<TI, TJ>;
    // one array per stage: with the K loop unrolled by the stage count every
    // copy and every read names its stage statically, so the compiler can
    // tell the stages apart and only waits for the copies of the stage it reads
    __shared__ __attribute__((aligned(1024))) unsigned char st0[G::STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) unsigned char st1[G::STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) unsigned char st2[G::STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) unsigned char st3[G::STAGE_BYTES];
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
    const int wave_m = wave >> 1, wave_n = wave & 1; // 2 x 2 waves of (32 TI) x (32 TJ)

    const int total = tiles_m * tiles_n * p.n_mat;
    const int split = (int)blockIdx.x / total;
    const int tile = (int)blockIdx.x - split * total;
    const TileCoord tc = schedule_tile(tiles_m, tiles_n, p.n_mat, group_m, tile);
    const int m0 = tc.tm * G::BM, n0 = tc.tn * G::BN;
    const unsigned short *Bm = tc.mat == 0 ? p.B[0] : (tc.mat == 1 ? p.B[1] : p.B[2]);
    unsigned short *Cm = tc.mat == 0 ? p.C[0] : (tc.mat == 1 ? p.C[1] : p.C[2]);
    const int KT = p.K / (AS_BK * splits);
    const int k0 = split * KT * AS_BK; // first k of this split

    // ---- copy plan: wave w issues copies q = TI w .. TI w + TI - 1 of A and
    // q = TJ w .. TJ w + TJ - 1 of B.
    // A copy q fills rows 16q..16q+15; lane -> (row 16q + lane/4, granule lane%4).
    // B copy q fills rows RPC q .. RPC q + RPC - 1 (RPC = 512 / BN rows of
    // BN / 8 granules); lane -> (row RPC q + lane / (BN/8), granule lane % (BN/8)).
    // B stored [N,K] (BT) is staged exactly like A: [BN][32] K-contiguous,
    // copy q fills n-rows 16q..16q+15 with the A swizzle.
    const unsigned short *ga[TI];
    const unsigned short *gb[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
        const int q = wave * TI + i;
        const int ra = 16 * q + (lane >> 2);
        const int ca = (lane & 3) ^ swz_a(ra);
        // rows past M (partial last row tile) read row M-1; their outputs
        // are never stored
        ga[i] = p.A + (int64_t)min(m0 + ra, p.M - 1) * p.lda + k0 + ca * 8;
    }
#pragma unroll
    for (int i = 0; i < TJ; ++i) {
        const int q = wave * TJ + i;
        if constexpr (BT) {
            const int rb = 16 * q + (lane >> 2);
            const int cb = (lane & 3) ^ swz_a(rb);
            gb[i] = Bm + (int64_t)min(n0 + rb, p.N - 1) * p.ldb + k0 + cb * 8;
        } else {
            const int rb = G::B_ROWS_PER_COPY * q + lane / G::B_GRANULES;
            const int cb = (lane % G::B_GRANULES) ^ swz_b<G::BN>(rb);
            // columns past N (partial last column tile) read the last 8;
            // their outputs are never stored
            gb[i] = Bm + (int64_t)(k0 + rb) * p.ldb + min(n0 + cb * 8, p.N - 8);
        }
    }
    const int64_t b_step = BT ? (int64_t)AS_BK : (int64_t)AS_BK * p.ldb; // per K-step

    // The copies are issued with inline assembly so that the compiler's own
    // wait insertion (which cannot tell the stages apart and would drain every
    // copy before each LDS read) stays out of the pipeline; the waits below
    // (wait_vmcnt) cover them explicitly.  m0 holds the copy's LDS address.
    // Copy c (0 .. COPIES-1) of step kt: c < TI is A copy TI wave + c, else
    // B copy TJ wave + c - TI.
    auto copy = [&](int kt, unsigned char *st, int c) {
        const unsigned lds = (unsigned)(uintptr_t)(lds_void *)st;
        if (c < TI) {
            const unsigned dst = lds + (wave * TI + c) * 1024;
            asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(ga[c] + kt * AS_BK), "{m0}"(dst)
                         : "memory");
        } else {
            const unsigned dst = lds + G::A_BYTES + (wave * TJ + c - TI) * 1024;
            asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gb[c - TI] + kt * b_step),
                         "{m0}"(dst)
                         : "memory");
        }
    };
    auto issue = [&](int kt, unsigned char *st) {
#pragma unroll
        for (int c = 0; c < G::COPIES; ++c)
            copy(kt, st, c);
    };

    // The accumulators start at bias[n] (or 0): the bias is added once per
    // output, before the sum over k instead of after it, and its loads and
    // conversions overlap the first copies instead of lengthening the
    // epilogue.  Lane l of 32x32 block (i, j) holds columns
    // n = 32 j + 8 g + 4 (l / 32) + {0..3} in registers 4g..4g+3 (any row).
    f32x16 acc[TI][TJ];
    if (p.bias != nullptr && split == 0) {
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int bc = n0 + wave_n * 32 * TJ + j * 32 + g * 8 + (lane >> 5) * 4;
                const u32x2 braw = bc < p.N ? *reinterpret_cast<const u32x2 *>(p.bias + bc)
                                            : u32x2{0u, 0u};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float b = from_bits<DT>((unsigned short)(braw[e >> 1] >> (16 * (e & 1))));
#pragma unroll
                    for (int i = 0; i < TI; ++i)
                        acc[i][j][4 * g + e] = b;
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[i][j][r] = 0.f;
    }

    // ---- fragment addressing (byte offsets within a stage)
    // A fragment i: row wave_m*32TI + i*32 + lane%32, k granule 2kk + lane/32.
    int a_off[TI][2];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
        const int r = wave_m * 32 * TI + i * 32 + (lane & 31);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            a_off[i][kk] = r * 64 + (((2 * kk + (lane >> 5)) ^ swz_a(r)) * 16);
    }
    // B fragment j, half h: 16-lane group g = lane/16, jj = lane%16:
    // row 16kk + 8(g/2) + 4h + jj/4, column wave_n*32TJ + 32j + 16(g%2) + 4(jj%4).
    // (BT: like A, n-row wave_n*32TJ + 32j + lane%32, k granule 2kk + lane/32.)
    int b_off[TJ][2][2];
    if constexpr (BT) {
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int r = wave_n * 32 * TJ + j * 32 + (lane & 31);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                b_off[j][kk][0] = b_off[j][kk][1] =
                    G::A_BYTES + r * 64 + (((2 * kk + (lane >> 5)) ^ swz_a(r)) * 16);
        }
    } else {
        const int g = lane >> 4, jj = lane & 15;
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = 16 * kk + 8 * (g >> 1) + 4 * h + (jj >> 2);
                    const int col = wave_n * 32 * TJ + 32 * j + 16 * (g & 1) + 4 * (jj & 3);
                    const int gran = (col >> 3) ^ swz_b<G::BN>(r);
                    b_off[j][kk][h] = G::A_BYTES + r * (2 * G::BN) + gran * 16 + (col & 7) * 2;
                }
    }

    struct Frag {
        u32x4 a[TI], b[TJ];
    };
    // fragment piece q of half kk: q < TI is A fragment q, then the two
    // transposing reads (q - TI even: low half, odd: high half) of B fragment
    // (q - TI) / 2 (BT: one 128-bit read of B fragment q - TI)
    constexpr int NREAD = TI + (BT ? TJ : 2 * TJ), NMMA = TI * TJ;
    auto read_piece = [&](Frag &f, const unsigned char *st, int kk, int q) {
        if (q < TI) {
            f.a[q] = *reinterpret_cast<const u32x4 *>(st + a_off[q][kk]);
        } else if constexpr (BT) {
            f.b[q - TI] = *reinterpret_cast<const u32x4 *>(st + b_off[q - TI][kk][0]);
        } else {
            const int j = (q - TI) >> 1, h = (q - TI) & 1;
            const s16x4 v =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(st + b_off[j][kk][h]));
            const u32x2 w = __builtin_bit_cast(u32x2, v);
            f.b[j][2 * h] = w[0];
            f.b[j][2 * h + 1] = w[1];
        }
    };
    auto read = [&](Frag &f, const unsigned char *st, int kk) {
#pragma unroll
        for (int q = 0; q < NREAD; ++q)
            read_piece(f, st, kk, q);
    };
    auto mma_one = [&](const Frag &f, int q) {
        const int i = q / TJ, j = q % TJ;
        acc[i][j] = mfma32x32x16<DT>(f.b[j], f.a[i], acc[i][j]);
    };

    // ---- pipeline.  Each step k (32 deep = two 16-deep halves h0, h1):
    //     MFMAs of h0, interleaved with the reads of h1 of stage k and the
    //     copies C1 .. COPIES-1 of step k+3 (into stage k-1, free since the
    //     barrier of step k-1)
    //     wait for this wave's copies of step k+1, barrier
    //     MFMAs of h1, interleaved with the reads of h0 of stage k+1 and the
    //     copies 0 .. C1-1 of step k+4 (into stage k, free after the barrier:
    //     both of its halves were read before it)
    // Every copy has three steps of MFMA work to land, and every LDS read
    // overlaps MFMAs.  K is a multiple of 4 steps, so the loop body is the 4
    // stages with their arrays named statically.  The MFMA / read / copy
    // order of each half is pinned: one MFMA and two fragment reads per slot
    // (the reads finish early in the half, leaving the last MFMAs as slack
    // before the wait), the copies spread over the middle slots.
    constexpr int SLOTS = (NMMA > NREAD ? NMMA : NREAD) > TI + G::COPIES - G::C1
                              ? (NMMA > NREAD ? NMMA : NREAD)
                              : TI + G::COPIES - G::C1;
    Frag f0, f1;
    auto step = [&](int kt, auto sidx) {
        constexpr int S = decltype(sidx)::value;
        unsigned char *cur = stage(sidx);
        unsigned char *nxt = stage(std::integral_constant<int, (S + 1) % 4>{});
        unsigned char *prv = stage(std::integral_constant<int, (S + 3) % 4>{});
        const int kp = min(kt + 3, KT - 1); // second part of the copies of step k+3
#pragma unroll
        for (int q = 0; q < SLOTS; ++q) {
            if (q < NMMA)
                mma_one(f0, q);
            if (2 * q < NREAD)
                read_piece(f1, cur, 1, 2 * q);
            if (2 * q + 1 < NREAD)
                read_piece(f1, cur, 1, 2 * q + 1);
            if (q >= TI && q < TI + G::COPIES - G::C1)
                copy(kp, prv, G::C1 + q - TI);
            __builtin_amdgcn_sched_barrier(0); // keep the MFMA / read / copy order
        }
        // The copies of steps k+2 and k+3 may stay in flight.  The loop body
        // is branch-free: past the last step the copies repeat the last tile
        // (into stages nobody reads any more), so this count always holds.
        wait_vmcnt<2 * G::COPIES>();
        __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0): this wave's reads of stage k are done
        stage_barrier();
        const int kc = min(kt + 4, KT - 1);
#pragma unroll
        for (int q = 0; q < SLOTS; ++q) {
            if (q < NMMA)
                mma_one(f1, q);
            if (2 * q < NREAD)
                read_piece(f0, nxt, 0, 2 * q);
            if (2 * q + 1 < NREAD)
                read_piece(f0, nxt, 0, 2 * q + 1);
            if (q < G::C1)
                copy(kc, cur, q);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    issue(0, st0);
    issue(1, st1);
    issue(2, st2);
    // step 3: copies 0 .. C1-1 now, the rest in the first half of step 0
#pragma unroll
    for (int c = 0; c < G::C1; ++c)
        copy(3, st3, c);
    wait_vmcnt<2 * G::COPIES + G::C1>();
    stage_barrier();
    read(f0, st0, 0);
    for (int kt = 0; kt < KT; kt += 4) {
        step(kt, std::integral_constant<int, 0>{});
        step(kt + 1, std::integral_constant<int, 1>{});
        step(kt + 2, std::integral_constant<int, 2>{});
        step(kt + 3, std::integral_constant<int, 3>{});
    }
    // Every copy has landed (this wave's, then everybody's after the
    // barrier) and every wave has finished reading the stages, so the LDS is
    // free for the epilogue.
    wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    stage_barrier();

    if constexpr (TI * TJ <= 4) {
        if (splits > 1) {
            if (!combine_splits<TI, TJ>(acc, ws, counters, tile, split, splits, wave, lane))
                return;
        }
    }

    // ---- epilogue: activation, residual and rounding in registers, the
    // rounded wave tile restaged through the wave's own stage for whole-row
    // stores.
    static_assert(2048 * TI * TJ <= G::STAGE_BYTES, "wave tile must fit its stage");
    unsigned char *ep = wave == 0 ? st0 : wave == 1 ? st1 : wave == 2 ? st2 : st3;
    const int64_t cm = m0 + wave_m * 32 * TI, cn = n0 + wave_n * 32 * TJ;
    unsigned short *cw = Cm + cm * p.ldc + cn;
    const int rows = (int)min((int64_t)(32 * TI), (int64_t)p.M - cm);
    const int cols = (int)min((int64_t)(32 * TJ), (int64_t)p.N - cn);
    if (p.R != nullptr)
        restaged_epilogue<DT, ACT, TI, TJ, true>(acc, ep, lane, cw, p.ldc, p.R + cm * p.ldr + cn,
                                                 p.ldr, rows, cols);
    else
        restaged_epilogue<DT, ACT, TI, TJ, false>(acc, ep, lane, cw, p.ldc, nullptr, 0, rows,
                                                  cols);
}

// ---------------------------------------------------------------------------
// 256 x 256 tiles on the 16x16x32 MFMA (B stored [K,N], or [N,K] staged
// like A).
//
// The same copy pipeline as above (four 32 KiB stages, direct-to-LDS copies
// of step k+4 issued three steps before they are read), with the product
// taken on v_mfma_f32_16x16x32 instead of 32x32x16.  For the same flops the
// smaller instruction moves half as many accumulator bytes through the
// register file (4 FP32 per lane per 16K flop against 16 per 32K flop);
// measured alone on random f16 operands it holds a 1.9 GHz clock where the
// larger one sags to 1.5 GHz, and this kernel is power-bound.  The tile is
// split over WN = 2 waves along N (4 waves of 128 x 128, one per SIMD, the
// default) or WN = 4 (8 waves of 128 x 64, two per SIMD).  One wave per SIMD
// issues this MFMA at only about 55 % of the matrix core's rate and two
// waves reach 85 % in a loop of MFMAs alone, but in the GEMM the 8-wave
// split reads a third more fragments from LDS and the power limit takes the
// difference back: it measures level with the 4-wave kernel (f16 4096^3
// within 1 %, QKV +0.5 %, bf16 8192^3 -1 %).
//
// Wave (wm, wn) keeps 8 x NJ accumulator blocks of 16 x 16 (NJ = 16 / WN):
// lane l of block (i, j) holds row 16 i + l % 16 and columns
// 16 j + 4 (l / 16) + {0..3} (B's fragment is src0, A's src1).
//  - A fragment i: row 16 i + l % 16, k granule l / 16 (one 128-bit read;
//    the A swizzle c ^ ((r >> 2) & 3) keeps the 16 rows a read pass covers
//    on 16 distinct 16-byte bank groups).
//  - B fragment j: two transposing reads, 16-lane group g at k-rows
//    8 g + 4 h + (l % 16) / 4 (h = 0, 1), columns 16 j + 4 (l % 4); lane i
//    of the group receives column 16 j + i at those k.  Groups g and g + 1
//    read rows 8 apart at the same columns, so the B swizzle gains a term in
//    bit 3 of the row: granule c of row r at c ^ {0,6,10,12}[r & 3] ^
//    2 ((r >> 3) & 1) (without it the bank-conflict counter doubles).
//  - Step k (32 deep): the step's MFMAs, with the fragment reads of stage
//    k+1 and the copies of step k+4 into stage k spread over the first three
//    quarters of them (stage k was read into registers during step k-1,
//    before the barrier that ended it); then wait for this wave's copies of
//    step k+2 and its reads, and barrier.  The MFMA order inside a step is
//    left to the compiler: pinning every MFMA with a scheduling barrier made
//    it rotate the accumulator blocks through spare registers (about 500
//    register moves per four steps at WN = 2).  A barrier in the middle of
//    the step, with the reads and copies packed into its second half,
//    measured 1.6 % slower at f16 4096^3 + GELU and 2.5 % at bf16 8192^3
//    (sustained, alternating order in one process).
namespace {

// Tiles of the 16x16x32 kernels: TM x TM outputs (256; 192 or 128 for sizes
// whose 256 x 256 tiles would leave most of a wave idle), K steps of KB = 32
// (or 64 on the 128 x 128 tiles: twice the MFMAs per step and per barrier,
// and every copy moves whole 128-byte row pieces).  A stage holds A [TM][KB]
// K-contiguous, then B [KB][TM] N-contiguous (or, stored [N,K], [TM][KB]
// like A).
template <int TM, int KB = 32>
struct A16Tile {
    static_assert(TM == 256 || TM == 192 || TM == 128, "16x16x32 tile sizes");
    static_assert(KB == 32 || (KB == 64 && TM == 128), "K step");
    static constexpr int A_BYTES = TM * KB * 2;
    static constexpr int STAGE = 2 * A_BYTES;
};
constexpr int A16_BM = 256, A16_BN = 256; // the stream-K kernel's tiles
constexpr int A16_STAGE = A16Tile<256>::STAGE;

// WN x 2 waves; each wave owns (TM / 2) x (TM / WN) outputs: MI x NJ blocks
// of 16 x 16.
template <int WN, bool BT, int TM = 256, int KB = 32>
struct A16Geom {
    static_assert(WN == 2 || (WN == 4 && TM == 256), "waves along N");
    static constexpr int NW = 2 * WN;               // waves
    static constexpr int NT = 64 * NW;              // lanes
    static constexpr int KH = KB / 32;              // 32-deep MFMA k slices per step
    static constexpr int MI = TM / 32;              // 16-row blocks per wave
    static constexpr int NJ = TM / 16 / WN;         // 16-column blocks per wave
    static constexpr int WROWS = 16 * MI;           // rows per wave
    static constexpr int WCOLS = 16 * NJ;           // columns per wave
    static constexpr int CA = TM * KB / 512 / NW;   // A copies of 1 KiB per wave per step
    static constexpr int COPIES = 2 * CA;           // + as many B copies
    // A reads + B reads (2 transposing each) per k slice
    static constexpr int R1 = MI + (BT ? NJ : 2 * NJ);
    static constexpr int READS = KH * R1;
    static constexpr int G = 2 * NJ;                // epilogue granules per wave-tile row
    static constexpr int EP_BYTES = WROWS * 16 * G; // wave tile restaged in LDS
};

// epilogue row swizzle: 16 rows of a read pass on 16 distinct bank groups
// (256-byte rows: r % 16; 128-byte rows: rows r, r + 1 share a bank sweep;
// 192-byte rows: rows r and r + 4 start on the same bank, so (r / 4) % 4
// moves the granule inside its aligned group of four)
template <int G>
__device__ __forceinline__ int ep_swz(int r)
{
    static_assert(G == 16 || G == 8 || G == 12, "epilogue row widths");
    return G == 16 ? (r & 15) : G == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}

} // namespace

template <int DT, int ACT, bool HR, int MI, int NJ>
__device__ __forceinline__ void restaged_epilogue16(const f32x4 (&acc)[MI][NJ], unsigned char *ep,
                                                    int lane, unsigned short *C, int64_t ldc,
                                                    const unsigned short *R, int64_t ldr,
                                                    int rows, int cols)
{
    // rows, cols: output rows and columns of this wave tile inside the
    // matrix (a multiple of 8 columns); the rest are neither read from R nor
    // stored
    // the rounded (16 MI) x (16 NJ) wave tile goes to the wave's own LDS
    // region (rows of G = 2 NJ granules, granule c of row r at c ^
    // ep_swz(r)), then each store writes 16 bytes per lane, whole row
    // segments
    constexpr int G = 2 * NJ;
    const int q = lane >> 4;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const int r = 16 * i + (lane & 15);
        u32x2 rr[NJ];
        if constexpr (HR) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                rr[j] = r < rows && 16 * j + 4 * q < cols
                            ? *reinterpret_cast<const u32x2 *>(R + (int64_t)r * ldr + 16 * j + 4 * q)
                            : u32x2{0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = activate<ACT>(acc[i][j][e]);
                if constexpr (HR)
                    v[e] += from_bits<DT>((unsigned short)(rr[j][e >> 1] >> (16 * (e & 1))));
            }
            const u32x2 o = {pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3])};
            const int c = (2 * j + (q >> 1)) ^ ep_swz<G>(r);
            *reinterpret_cast<u32x2 *>(ep + r * (16 * G) + c * 16 + (q & 1) * 8) = o;
        }
    }
    if constexpr (64 % G == 0) {
        // lane -> granule lane % G of rows (64 / G) t + lane / G
        unsigned short *crow = C + (lane % G) * 8;
#pragma unroll
        for (int t = 0; t < MI * G / 4; ++t) {
            const int r = (64 / G) * t + lane / G;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(ep + r * (16 * G) +
                                                             (((lane % G) ^ ep_swz<G>(r)) * 16));
            if (r < rows && (lane % G) * 8 < cols)
                *reinterpret_cast<u32x4 *>(crow + (int64_t)r * ldc) = v;
        }
    } else {
        // lane -> granule (64 t + lane) % G of row (64 t + lane) / G
#pragma unroll
        for (int t = 0; t < MI * G / 4; ++t) {
            const int r = (64 * t + lane) / G, g = (64 * t + lane) % G;
            const u32x4 v =
                *reinterpret_cast<const u32x4 *>(ep + r * (16 * G) + ((g ^ ep_swz<G>(r)) * 16));
            if (r < rows && g * 8 < cols)
                *reinterpret_cast<u32x4 *>(C + (int64_t)r * ldc + g * 8) = v;
        }
    }
}

// A pointer every lane holds the same value of, in scalar registers
__device__ __forceinline__ const unsigned short *uniform_ptr(const unsigned short *ptr)
{
    const uint64_t v = (uint64_t)(uintptr_t)ptr;
    const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)v);
    const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(v >> 32));
    return reinterpret_cast<const unsigned short *>(((uint64_t)hi << 32) | lo);
}

// The K loop of one TM x TM tile on the 16x16x32 MFMA: K-steps kt0 ..
// kt0 + KT - 1 (KT a multiple of the four stages) of the tile at (m0, n0)
// of the product with the weight Bm, accumulated into acc (which the caller
// has initialised).  On return every copy has landed and every wave has
// finished reading the stages, so the LDS is free.
template <int DT, int WN, bool BT, bool KM, int TM = 256, int KB = 32, bool SC = true>
__device__ __forceinline__ void a16_mainloop(
    const GemmArgs &p, int m0, int n0, const unsigned short *Bm, int kt0, int KT, int wave,
    int lane, unsigned char *st0, unsigned char *st1, unsigned char *st2, unsigned char *st3,
    f32x4 (&acc)[A16Geom<WN, BT, TM, KB>::MI][A16Geom<WN, BT, TM, KB>::NJ])
{
    // SC: copies from scalar tile-corner addresses (below); the tile and its
    // K range are the workgroup's, uniform
    if constexpr (SC) {
        m0 = __builtin_amdgcn_readfirstlane(m0);
        n0 = __builtin_amdgcn_readfirstlane(n0);
        kt0 = __builtin_amdgcn_readfirstlane(kt0);
        KT = __builtin_amdgcn_readfirstlane(KT);
        Bm = uniform_ptr(Bm);
    }
    using Gm = A16Geom<WN, BT, TM, KB>;
    constexpr int MI = Gm::MI, NJ = Gm::NJ, CA = Gm::CA, KH = Gm::KH;
    constexpr int A_BYTES = A16Tile<TM, KB>::A_BYTES;
    // A (and B stored [N,K]) rows of KB k: 64 bytes (4 granules, swizzle
    // swz_a) or 128 bytes (8 granules, swz_a8); one 1 KiB copy fills 16 or
    // 8 rows
    constexpr int RG = KB / 8;                 // granules per row
    constexpr int RPC = 64 / RG;               // rows per copy
    auto swz_row = [](int r) { return KB == 32 ? swz_a(r) : swz_a8(r); };
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
    const int wave_n = wave % WN;
    const int wave_m = wave / WN;

    // copy c < CA: A copy q = CA w + c, rows RPC q .. RPC q + RPC - 1 (lane
    // -> row RPC q + lane / RG, granule lane % RG); c >= CA: B copy q = CA w
    // + c - CA, bytes 1024 q .. 1024 q + 1023 of [KB][TM] (lane -> byte 1024
    // q + 16 lane: row rb of 2 TM bytes, granule gb; at TM = 256 rows 2 q +
    // lane / 32, granule lane % 32).  B stored [N,K] (BT) is staged like A:
    // [TM n][KB k] K-contiguous, B copy q filling n-rows RPC q .. RPC q +
    // RPC - 1 with the A swizzle.
    const int64_t b_step = BT ? (int64_t)KB : (int64_t)KB * p.ldb;
    // KM: copy c of step kt is inside K iff kt * 32 < a_kl[c] (b_kl[c]).
    // SC without KM: a copy is a uniform (scalar) tile-corner address plus
    // the lane's 32-bit byte offset oa[c] (ob[c]); the host keeps TM rows of
    // A (and of B stored [N,K]) within 4 GiB.  Otherwise each lane's 64-bit
    // address ga[c] (gb[c]).
    const unsigned short *ga[CA], *gb[CA];
    int a_kl[CA], b_kl[CA];
    unsigned oa[CA], ob[CA];
    const unsigned short *a_corner = p.A + (int64_t)m0 * p.lda + (int64_t)kt0 * KB;
    const unsigned short *b_corner =
        (BT ? Bm + (int64_t)n0 * p.ldb : Bm + n0) + (int64_t)kt0 * b_step;
    const unsigned short *zero = reinterpret_cast<const unsigned short *>(kZeroGranule);
#pragma unroll
    for (int c = 0; c < CA; ++c) {
        const int q = wave * CA + c;
        const int ra = RPC * q + lane / RG;
        const int ka = ((lane % RG) ^ swz_row(ra)) * 8;
        // rows past M (a last row tile that M does not fill) read row M-1:
        // every copy stays inside A, and those rows only reach outputs that
        // are never stored
        const int ra_in = min(m0 + ra, p.M - 1) - m0;
        ga[c] = a_corner + (int64_t)ra_in * p.lda + ka;
        oa[c] = 2u * ((unsigned)ra_in * (unsigned)p.lda + (unsigned)ka);
        a_kl[c] = p.K - kt0 * KB - ka;
        if constexpr (BT) {
            const int rn = min(n0 + ra, p.N - 1) - n0;
            gb[c] = b_corner + (int64_t)rn * p.ldb + ka;
            ob[c] = 2u * ((unsigned)rn * (unsigned)p.ldb + (unsigned)ka);
            b_kl[c] = a_kl[c];
        } else {
            int rb, cn;
            if constexpr (TM == 256) {
                rb = 2 * q + (lane >> 5);
                cn = min(n0 + ((lane & 31) ^ swz_b16(rb)) * 8, p.N - 8) - n0;
            } else {
                const unsigned byte = 1024u * q + 16u * lane;
                rb = (int)(byte / (2 * TM));
                const int gb0 = (int)(byte % (2 * TM) / 16) ^ (TM == 192 ? swz_b192(rb) : swz_b128(rb));
                cn = min(n0 + gb0 * 8, p.N - 8) - n0;
            }
            gb[c] = b_corner + (int64_t)rb * p.ldb + cn;
            ob[c] = 2u * ((unsigned)rb * (unsigned)p.ldb + (unsigned)cn);
            b_kl[c] = p.K - kt0 * KB - rb;
        }
    }
    auto copy = [&](int kt, unsigned char *st, int c) {
        const unsigned lds = (unsigned)(uintptr_t)(lds_void *)st;
        if (c < CA) {
            const unsigned dst = lds + (wave * CA + c) * 1024;
            if constexpr (KM || !SC) {
                const unsigned short *src = ga[c] + kt * KB;
                if constexpr (KM)
                    src = kt * KB < a_kl[c] ? src : zero;
                asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(dst) : "memory");
            } else {
                asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(oa[c]),
                             "s"(a_corner + (int64_t)kt * KB), "{m0}"(dst)
                             : "memory");
            }
        } else {
            const unsigned dst = lds + A_BYTES + (wave * CA + c - CA) * 1024;
            if constexpr (KM || !SC) {
                const unsigned short *src = gb[c - CA] + kt * b_step;
                if constexpr (KM)
                    src = kt * KB < b_kl[c - CA] ? src : zero;
                asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(dst) : "memory");
            } else {
                asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(ob[c - CA]),
                             "s"(b_corner + kt * b_step), "{m0}"(dst)
                             : "memory");
            }
        }
    };
    auto issue = [&](int kt, unsigned char *st) {
#pragma unroll
        for (int c = 0; c < Gm::COPIES; ++c)
            copy(kt, st, c);
    };

    // fragment offsets within a stage, per 32-deep k slice s: A row r, k
    // granule 4 s + l / 16
    const int q16 = lane >> 4;
    int a_off[KH][MI];
#pragma unroll
    for (int s = 0; s < KH; ++s)
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int r = wave_m * Gm::WROWS + 16 * i + (lane & 15);
            a_off[s][i] = r * (2 * KB) + (((4 * s + q16) ^ swz_row(r)) * 16);
        }
    // B fragment j: transposing reads of [KB k][TM n] (two per fragment; k
    // rows 32 s .. 32 s + 31 for slice s), or for BT one 128-bit read of
    // n-row wave_n WCOLS + 16 j + l % 16, k granule 4 s + l / 16 of [TM n][KB
    // k] (b_off[s][j][0])
    int b_off[KH][NJ][2];
    {
        const int jj = lane & 15;
#pragma unroll
        for (int s = 0; s < KH; ++s)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if constexpr (BT) {
                        const int r = wave_n * Gm::WCOLS + 16 * j + jj;
                        b_off[s][j][h] =
                            A_BYTES + r * (2 * KB) + (((4 * s + q16) ^ swz_row(r)) * 16);
                    } else {
                        const int r = 32 * s + 8 * q16 + 4 * h + (jj >> 2);
                        const int col = wave_n * Gm::WCOLS + 16 * j + 4 * (jj & 3);
                        const int sw =
                            TM == 256 ? swz_b16(r) : TM == 192 ? swz_b192(r) : swz_b128(r);
                        b_off[s][j][h] =
                            A_BYTES + r * (2 * TM) + (((col >> 3) ^ sw) * 16) + (col & 7) * 2;
                    }
                }
    }

    struct Frag {
        u32x4 a[KH][MI], b[KH][NJ];
    };
    // read piece q of slice s = q / R1, u = q % R1: u < MI is A fragment u,
    // then B fragment (u - MI) / 2, half (u - MI) % 2 (BT: B fragment u - MI)
    auto read_piece = [&](Frag &f, const unsigned char *st, int q) {
        const int s = q / Gm::R1, u = q % Gm::R1;
        if (u < MI) {
            f.a[s][u] = *reinterpret_cast<const u32x4 *>(st + a_off[s][u]);
        } else if constexpr (BT) {
            f.b[s][u - MI] = *reinterpret_cast<const u32x4 *>(st + b_off[s][u - MI][0]);
        } else {
            const int j = (u - MI) >> 1, h = (u - MI) & 1;
            const s16x4 v =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(st + b_off[s][j][h]));
            const u32x2 w = __builtin_bit_cast(u32x2, v);
            f.b[s][j][2 * h] = w[0];
            f.b[s][j][2 * h + 1] = w[1];
        }
    };

    constexpr int MT = KH * MI * NJ;  // MFMAs per step
    constexpr int OPS = Gm::READS + Gm::COPIES;
    constexpr int SPAN = MT * 3 / 4;  // MFMAs the reads and copies are spread over
    Frag f0, f1;
    auto step = [&](int kt, auto sidx, Frag &fc, Frag &fn) {
        constexpr int S = decltype(sidx)::value;
        unsigned char *cur = stage(sidx);
        unsigned char *nxt = stage(std::integral_constant<int, (S + 1) % 4>{});
        // past the last step the copies repeat the last tile into stages
        // nobody reads, so the wait counts below always hold
        const int kc = min(kt + 4, KT - 1);
#pragma unroll
        for (int q = 0; q < MT; ++q) {
            const int s = q / (MI * NJ), i = q % MI, j = q / MI % NJ;
            acc[i][j] = mfma16x16x32<DT>(fc.b[s][j], fc.a[s][i], acc[i][j]);
            if (q < SPAN) {
                // ops o0 .. o1-1 after this MFMA; op o is a copy where the
                // running count of copies (evenly spread) steps up, else a read
                const int o0 = q * OPS / SPAN, o1 = (q + 1) * OPS / SPAN;
                for (int o = o0; o < o1; ++o) {
                    const int upto = (o + 1) * Gm::COPIES / OPS, before = o * Gm::COPIES / OPS;
                    if (upto > before)
                        copy(kc, cur, upto - 1);
                    else
                        read_piece(fn, nxt, o - before);
                }
            }
            // B stored [N,K]: each MFMA kept with its reads and copies in
            // this order (bf16 1024 x 8192 x 8192 on 128 x 128 x 64 tiles
            // 1227-1229 against 1159-1191 TFLOP/s left to the scheduler)
            if constexpr (BT)
                __builtin_amdgcn_sched_barrier(0);
        }
        // Keep the next step's MFMAs below the wait and barrier: the compiler
        // otherwise moves them up behind the reads of their fragments and
        // reuses the fragment registers, so every 8 MFMAs wait on an LDS read
        // issued a few instructions before (bf16 4096^3: 1.09-1.15 PFLOP/s
        // with the hoist, 1.24-1.29 without).
        __builtin_amdgcn_sched_barrier(0);
        // copies of step k+2 landed (those of k+3 and k+4 may stay in
        // flight) and this wave's reads of stage k+1 done; then everybody's
        wait_vmcnt<2 * Gm::COPIES>();
        __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0)
        stage_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    issue(0, st0);
    issue(min(1, KT - 1), st1);
    issue(min(2, KT - 1), st2);
    issue(min(3, KT - 1), st3);
    wait_vmcnt<2 * Gm::COPIES>(); // steps 0 and 1 landed
    stage_barrier();
#pragma unroll
    for (int q = 0; q < Gm::READS; ++q)
        read_piece(f0, st0, q);
    // every wave's reads of stage 0 are done before step 0 copies into it
    __builtin_amdgcn_s_waitcnt(0xC07F);
    stage_barrier();
    for (int kt = 0; kt < KT; kt += 4) {
        step(kt, std::integral_constant<int, 0>{}, f0, f1);
        step(kt + 1, std::integral_constant<int, 1>{}, f1, f0);
        step(kt + 2, std::integral_constant<int, 2>{}, f0, f1);
        step(kt + 3, std::integral_constant<int, 3>{}, f1, f0);
    }
    wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    stage_barrier();
}

// Accumulators of a 16x16x32 wave tile set to bias[n] (or 0): lane l of
// block (i, j) holds columns 16 j + 4 (l / 16) + {0..3} of the wave's
// columns.
template <int DT, int WN, int TM = 256>
__device__ __forceinline__ void a16_init_acc(
    const GemmArgs &p, int n0, int wave, int lane, bool with_bias,
    f32x4 (&acc)[A16Geom<WN, false, TM>::MI][A16Geom<WN, false, TM>::NJ])
{
    constexpr int MI = A16Geom<WN, false, TM>::MI, NJ = A16Geom<WN, false, TM>::NJ;
    constexpr int WCOLS = 16 * NJ;
    const bool use = with_bias && p.bias != nullptr;
    const int wave_n = wave % WN;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        f32x4 b = {0.f, 0.f, 0.f, 0.f};
        if (use) {
            const int bc = n0 + wave_n * WCOLS + 16 * j + 4 * (lane >> 4);
            const u32x2 braw = bc < p.N ? *reinterpret_cast<const u32x2 *>(p.bias + bc)
                                        : u32x2{0u, 0u};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                b[e] = from_bits<DT>((unsigned short)(braw[e >> 1] >> (16 * (e & 1))));
        }
#pragma unroll
        for (int i = 0; i < MI; ++i)
            acc[i][j] = b;
    }
}

// Epilogue of a 16x16x32 wave tile: each wave restages its tile in its own
// EP_BYTES of the (idle) stages and stores whole row segments.
template <int DT, int ACT, int WN, bool BT, int TM = 256, int KB = 32>
__device__ __forceinline__ void a16_epilogue(
    const GemmArgs &p, unsigned short *Cm, int m0, int n0, int wave, int lane,
    unsigned char *st0, unsigned char *st1, unsigned char *st2, unsigned char *st3,
    const f32x4 (&acc)[A16Geom<WN, BT, TM>::MI][A16Geom<WN, BT, TM>::NJ])
{
    using Gm = A16Geom<WN, BT, TM>;
    constexpr int MI = Gm::MI, NJ = Gm::NJ;
    constexpr int PER_STAGE = A16Tile<TM, KB>::STAGE / Gm::EP_BYTES; // wave tiles per stage
    static_assert(PER_STAGE >= 1 && Gm::NW <= 4 * PER_STAGE, "epilogue fits the stages");
    const int es = wave / PER_STAGE;
    unsigned char *ep = (es == 0 ? st0 : es == 1 ? st1 : es == 2 ? st2 : st3) +
                        (wave % PER_STAGE) * Gm::EP_BYTES;
    const int64_t cm = m0 + (wave / WN) * Gm::WROWS, cn = n0 + (wave % WN) * Gm::WCOLS;
    unsigned short *cw = Cm + cm * p.ldc + cn;
    const int rows = (int)min((int64_t)Gm::WROWS, (int64_t)p.M - cm);
    const int cols = (int)min((int64_t)Gm::WCOLS, (int64_t)p.N - cn);
    if (p.R != nullptr)
        restaged_epilogue16<DT, ACT, true, MI, NJ>(acc, ep, lane, cw, p.ldc,
                                                   p.R + cm * p.ldr + cn, p.ldr, rows, cols);
    else
        restaged_epilogue16<DT, ACT, false, MI, NJ>(acc, ep, lane, cw, p.ldc, nullptr, 0, rows,
                                                    cols);
}

// Pair-staged K loop of the 256 x 256 tiles: two steps of 32 k share one
// region per operand (A in st0 / st2 as [256 rows][64 k] in 128-byte rows;
// B in st1 / st3 likewise when stored [N,K], else as [64 k][256 n] in
// 512-byte rows), so each 1 KiB copy moves whole lines (8 rows of 128
// bytes, or 2 of 512), and one pair is copied while the other is read.
// Steps 4t .. 4t+3 read pairs X = 2t (st0, st1) and Y = 2t + 1 (st2, st3):
//  4t:   MFMAs; read step 4t+1 (X, second half); wait for Y, barrier
//  4t+1: MFMAs; read step 4t+2 (Y, first half); copy pair 2t + 2 into X
//  4t+2: MFMAs; read step 4t+3 (Y, second half); wait for X, barrier
//  4t+3: MFMAs; read step 4t+4 (X, first half); copy pair 2t + 3 into Y
// Two barriers per four steps; a copy has 1.5 steps to land.  Steps kt0 ..
// kt0 + KT - 1, KT and kt0 multiples of 4; past the last pair the copies
// repeat it into the region nobody reads again.
template <int DT, int WN, bool BT>
__device__ __forceinline__ void a16_mainloop_pairs(
    const GemmArgs &p, int m0, int n0, const unsigned short *Bm, int kt0, int KT, int wave,
    int lane, unsigned char *st0, unsigned char *st1, unsigned char *st2, unsigned char *st3,
    f32x4 (&acc)[A16Geom<WN, BT, 256>::MI][A16Geom<WN, BT, 256>::NJ])
{
    using Gm = A16Geom<WN, BT, 256>;
    // the tile and its K range are the workgroup's: uniform, which the
    // copies' scalar addresses need (the stream-K work loop hides it from
    // the compiler)
    m0 = __builtin_amdgcn_readfirstlane(m0);
    n0 = __builtin_amdgcn_readfirstlane(n0);
    kt0 = __builtin_amdgcn_readfirstlane(kt0);
    KT = __builtin_amdgcn_readfirstlane(KT);
    Bm = uniform_ptr(Bm);
    constexpr int MI = Gm::MI, NJ = Gm::NJ;
    constexpr int PC = 256 * 128 / 1024 / Gm::NW; // copies per operand per wave per pair
    constexpr int COPIES = 2 * PC;
    constexpr int READS = MI + NJ; // fragment reads per step
    const int wave_n = wave % WN, wave_m = wave / WN;
    const int NP = KT / 2; // pairs
    // copy c: rows 8 q .. 8 q + 7 of a [256][64] region, q = PC wave + c
    // (lane -> row 8 q + lane / 8, granule lane % 8 with the 128-byte-row
    // swizzle); rows past M or N read the last one.  B stored [K,N]: k rows
    // 2 q, 2 q + 1 of the [64][256] region (lane -> row 2 q + lane / 32,
    // granule lane % 32 with the 512-byte-row swizzle), columns past N read
    // the last 8.  Each lane keeps a 32-bit byte offset from the tile's
    // corner, the corner of pair pc being a uniform (scalar) address; the
    // host keeps 256 rows of A (and of B stored [N,K]) within 4 GiB.
    unsigned oa[PC], ob[PC];
#pragma unroll
    for (int c = 0; c < PC; ++c) {
        const int r = 8 * (wave * PC + c) + (lane >> 3);
        const int kg = ((lane & 7) ^ swz_a8(r)) * 8;
        oa[c] = 2u * ((unsigned)(min(m0 + r, p.M - 1) - m0) * (unsigned)p.lda + kg);
        if constexpr (BT) {
            ob[c] = 2u * ((unsigned)(min(n0 + r, p.N - 1) - n0) * (unsigned)p.ldb + kg);
        } else {
            const int rb = 2 * (wave * PC + c) + (lane >> 5);
            ob[c] = 2u * ((unsigned)rb * (unsigned)p.ldb +
                          (unsigned)(min(n0 + ((lane & 31) ^ swz_b16(rb)) * 8, p.N - 8) - n0));
        }
    }
    const int64_t b_pair = BT ? 64 : (int64_t)64 * p.ldb; // B elements per pair
    const unsigned short *a_corner = p.A + (int64_t)m0 * p.lda + (int64_t)kt0 * 32;
    const unsigned short *b_corner =
        (BT ? Bm + (int64_t)n0 * p.ldb : Bm + n0) + (int64_t)(kt0 / 2) * b_pair;
    auto copy = [&](int pr, unsigned char *sa, unsigned char *sb, int c) {
        const int64_t pc = min(pr, NP - 1), k0 = pc * 64;
        if (c < PC) {
            const unsigned dst = (unsigned)(uintptr_t)(lds_void *)sa + (wave * PC + c) * 1024;
            asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(oa[c]), "s"(a_corner + k0),
                         "{m0}"(dst)
                         : "memory");
        } else {
            const unsigned dst =
                (unsigned)(uintptr_t)(lds_void *)sb + (wave * PC + c - PC) * 1024;
            asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(ob[c - PC]),
                         "s"(b_corner + pc * b_pair), "{m0}"(dst)
                         : "memory");
        }
    };
    // fragment offsets of step half h: row r, k granule 4 h + l / 16 of a
    // 128-byte row, so half 1 flips byte-offset bit 6.  B stored [K,N]: two
    // transposing reads per fragment from k rows 32 h + 8 (l / 16) + 4 hh +
    // (l % 16) / 4 (half 1: 32 rows, 16 KiB, further; the swizzle ignores
    // row bit 5); fragment column j sets granule bits 1..3 (2 j), which
    // neither the wave's column base (a multiple of 16 granules) nor the row
    // term touches, so fragment j's offset is fragment 0's XOR 32 j.
    static_assert(BT || (NJ <= 8 && Gm::WCOLS % 128 == 0), "B [K,N] offsets by XOR");
    const int q16 = lane >> 4, jj = lane & 15;
    int a_off[MI], b_off[NJ], bk_off[2];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const int r = wave_m * Gm::WROWS + 16 * i + (lane & 15);
        a_off[i] = r * 128 + ((q16 ^ swz_a8(r)) * 16);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int r = wave_n * Gm::WCOLS + 16 * j + jj;
        b_off[j] = r * 128 + ((q16 ^ swz_a8(r)) * 16);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int r = 8 * q16 + 4 * hh + (jj >> 2);
        const int col = wave_n * Gm::WCOLS + 4 * (jj & 3);
        bk_off[hh] = r * 512 + (((col >> 3) ^ swz_b16(r)) * 16) + (col & 7) * 2;
    }
    struct Frag {
        u32x4 a[MI], b[NJ];
    };
    // read piece q: B fragment q < NJ, then A fragment q - NJ.  (With the
    // A fragments first, the B [K,N] loop compiled to 380-500 moves of
    // accumulators between the register files per four steps; in this order
    // both layouts have none.)  A B [K,N] fragment's two transposing reads
    // are assigned as one vector.
    auto read_piece = [&](Frag &f, const unsigned char *sa, const unsigned char *sb, int h,
                          int q) {
        if (q >= NJ) {
            f.a[q - NJ] = *reinterpret_cast<const u32x4 *>(sa + (a_off[q - NJ] ^ (64 * h)));
        } else if constexpr (BT) {
            f.b[q] = *reinterpret_cast<const u32x4 *>(sb + (b_off[q] ^ (64 * h)));
        } else {
            const u32x2 w0 = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                           (lds_s16x4 *)(sb + h * 16384 + (bk_off[0] ^ (32 * q)))));
            const u32x2 w1 = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                           (lds_s16x4 *)(sb + h * 16384 + (bk_off[1] ^ (32 * q)))));
            f.b[q] = u32x4{w0[0], w0[1], w1[0], w1[1]};
        }
    };
    constexpr int MT = MI * NJ;
    constexpr int SPAN = MT * 3 / 4;
    // one step: the MFMAs of fc, with the reads of fn (half h of sa / sb)
    // and, when pr >= 0, the copies of pair pr into ca / cb spread over the
    // first three quarters; then the waits (and barrier) the schedule needs
    auto step = [&](Frag &fc, Frag &fn, const unsigned char *sa, const unsigned char *sb, int h,
                    int pr, unsigned char *ca, unsigned char *cb, bool bar) {
        const int ops = READS + (pr >= 0 ? COPIES : 0);
#pragma unroll
        for (int q = 0; q < MT; ++q) {
            const int i = q % MI, j = q / MI;
            acc[i][j] = mfma16x16x32<DT>(fc.b[j], fc.a[i], acc[i][j]);
            if (q < SPAN) {
                const int o0 = q * ops / SPAN, o1 = (q + 1) * ops / SPAN;
                for (int o = o0; o < o1; ++o) {
                    if (pr >= 0) {
                        const int upto = (o + 1) * COPIES / ops, before = o * COPIES / ops;
                        if (upto > before)
                            copy(pr, ca, cb, upto - 1);
                        else
                            read_piece(fn, sa, sb, h, o - before);
                    } else {
                        read_piece(fn, sa, sb, h, o);
                    }
                }
            }
            // B stored [N,K]: each MFMA with its reads and copies kept in
            // this order (bf16 8192^3 1479-1483 against 1417-1419 TFLOP/s
            // left to the scheduler); with B [K,N] the fence costs half the
            // rate (accumulator moves)
            if constexpr (BT)
                __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0)
        if (bar) {
            wait_vmcnt<0>();
            stage_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    Frag f0, f1;
    // prologue: pairs 0 and 1 in flight, pair 0 landed, fragments of step 0
#pragma unroll
    for (int c = 0; c < COPIES; ++c)
        copy(0, st0, st1, c);
#pragma unroll
    for (int c = 0; c < COPIES; ++c)
        copy(1, st2, st3, c);
    wait_vmcnt<COPIES>();
    stage_barrier();
#pragma unroll
    for (int q = 0; q < READS; ++q)
        read_piece(f0, st0, st1, 0, q);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    for (int t = 0; 4 * t < KT; ++t) {
        step(f0, f1, st0, st1, 1, -1, nullptr, nullptr, true);
        step(f1, f0, st2, st3, 0, 2 * t + 2, st0, st1, false);
        step(f0, f1, st2, st3, 1, -1, nullptr, nullptr, true);
        step(f1, f0, st0, st1, 0, 2 * t + 3, st2, st3, false);
    }
    wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    stage_barrier();
}

// Data-parallel kernel on the pair-staged loop (256 x 256 tiles, K a
// multiple of 128).
template <int DT, int ACT, int WN, bool BT>
__global__ __launch_bounds__(128 * WN, 1) void gemm_async16p_kernel(GemmArgs p, int tiles_m,
                                                                     int tiles_n, int group_m)
{
    constexpr int STAGE = A16Tile<256>::STAGE;
    __shared__ __attribute__((aligned(1024))) unsigned char st0[STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char st1[STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char st2[STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char st3[STAGE];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const TileCoord tc = schedule_tile(tiles_m, tiles_n, p.n_mat, group_m, blockIdx.x);
    const int m0 = tc.tm * 256, n0 = tc.tn * 256;
    const unsigned short *Bm = tc.mat == 0 ? p.B[0] : (tc.mat == 1 ? p.B[1] : p.B[2]);
    unsigned short *Cm = tc.mat == 0 ? p.C[0] : (tc.mat == 1 ? p.C[1] : p.C[2]);
    f32x4 acc[A16Geom<WN, BT, 256>::MI][A16Geom<WN, BT, 256>::NJ];
    a16_init_acc<DT, WN, 256>(p, n0, wave, lane, true, acc);
    a16_mainloop_pairs<DT, WN, BT>(p, m0, n0, Bm, 0, p.K / AS_BK, wave, lane, st0, st1, st2,
                                   st3, acc);
    a16_epilogue<DT, ACT, WN, BT, 256, 32>(p, Cm, m0, n0, wave, lane, st0, st1, st2, st3, acc);
}

// Split-K exchange of a 16x16x32 workgroup: the protocol of combine_splits
// (device-coherent partial stores, one atomic count per workgroup, the last
// workgroup reads every partial back and adds them in split order 0 ..
// splits-1), with a split's partial stored as [NW waves][MI NJ vectors][64
// lanes] of 16-byte vectors, vector NJ i + j holding accumulator block (i,
// j).  Returns true in the workgroup that completed the count, with acc
// replaced by the ordered sum of all the splits.
template <int NW, int MI, int NJ>
__device__ __forceinline__ bool combine_splits16(f32x4 (&acc)[MI][NJ], float *ws, int *counters,
                                                 int tile, int split, int splits, int wave,
                                                 int lane)
{
    constexpr int PV = MI * NJ;                      // vectors per lane per split
    static_assert(PV == 16, "the 128 x 128 tiles' partials");
    constexpr int BLOCK = NW * PV * 256;             // floats per split partial
    constexpr int RS = 32 / PV;                      // splits read back per round
    __shared__ int s_last16;
    float *ws_tile = ws + (int64_t)tile * splits * BLOCK;
    const int lane_off = wave * PV * 256 + lane * 4;
    {
        f32x4 v[PV];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                v[NJ * i + j] = acc[i][j];
        store_partial<PV>(ws_tile + (int64_t)split * BLOCK + lane_off, v);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int old = __hip_atomic_fetch_add(&counters[tile], 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        s_last16 = (old == splits - 1);
    }
    __syncthreads();
    if (!s_last16)
        return false;
    // rounds of RS splits, all 32 loads of a round in flight together, added
    // in split order; indices past the last split repeat it and are not added
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp0 = 0; sp0 < splits; sp0 += RS) {
        f32x4 v[32];
#pragma unroll
        for (int u = 0; u < RS; ++u) {
            const float *src = ws_tile + (int64_t)min(sp0 + u, splits - 1) * BLOCK + lane_off;
#pragma unroll
            for (int t = 0; t < PV; ++t)
                asm volatile("global_load_dwordx4 %0, %1, off sc1"
                             : "=v"(v[u * PV + t])
                             : "v"(src + t * 256)
                             : "memory");
        }
        // the loads are invisible to the compiler's wait tracking: wait here
        // with every value passed through, so nothing reads one earlier
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
#pragma unroll
        for (int u = 0; u < RS; ++u)
            if (sp0 + u < splits)
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
                        acc[i][j] += v[u * PV + NJ * i + j];
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&counters[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

// splits > 1 (128 x 128 tiles only; grid = tiles x splits, block b = split
// tiles + tile): split s runs steps [s KT / splits, (s + 1) KT / splits) of
// the K loop (K a multiple of the four steps times splits), the bias enters
// through split 0, and the partials meet in combine_splits16.
template <int DT, int ACT, int WN, bool BT, bool KM, int TM = 256, int KB = 32>
__global__ __launch_bounds__(128 * WN, 1) void gemm_async16_kernel(GemmArgs p, int tiles_m,
                                                                    int tiles_n, int group_m,
                                                                    int splits, float *ws,
                                                                    int *counters)
{
    constexpr int STAGE = A16Tile<TM, KB>::STAGE;
    __shared__ __attribute__((aligned(1024))) unsigned char st0[STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char st1[STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char st2[STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char st3[STAGE];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    constexpr bool SPLITS = TM == 128;
    const int total = tiles_m * tiles_n * p.n_mat;
    const int split = SPLITS ? (int)blockIdx.x / total : 0;
    const int tile = SPLITS ? (int)blockIdx.x - split * total : (int)blockIdx.x;
    const TileCoord tc = schedule_tile(tiles_m, tiles_n, p.n_mat, group_m, tile);
    const int m0 = tc.tm * TM, n0 = tc.tn * TM;
    const unsigned short *Bm = tc.mat == 0 ? p.B[0] : (tc.mat == 1 ? p.B[1] : p.B[2]);
    unsigned short *Cm = tc.mat == 0 ? p.C[0] : (tc.mat == 1 ? p.C[1] : p.C[2]);
    f32x4 acc[A16Geom<WN, BT, TM>::MI][A16Geom<WN, BT, TM>::NJ];
    a16_init_acc<DT, WN, TM>(p, n0, wave, lane, split == 0, acc);
    // KM (K off the 128 grid): the whole quads on the unmasked loop, then
    // the last, partial quad on its own with the k past K masked (a second
    // pipeline fill, but the masking's registers stay out of the main loop,
    // where they made the compiler move the accumulators in and out of the
    // register file)
    // split s (K a multiple of four steps times splits, never KM) runs steps
    // [s KT, (s + 1) KT) of KT = K / (KB splits)
    const int KT = p.K / (AS_STAGES * KB * (SPLITS ? splits : 1)) * AS_STAGES;
    if (!KM || KT > 0)
        a16_mainloop<DT, WN, BT, false, TM, KB>(p, m0, n0, Bm, split * KT, KT, wave, lane, st0,
                                                st1, st2, st3, acc);
    if constexpr (KM)
        a16_mainloop<DT, WN, BT, true, TM, KB>(p, m0, n0, Bm, KT, AS_STAGES, wave, lane, st0, st1,
                                               st2, st3, acc);
    if constexpr (SPLITS && !KM) {
        using Gm = A16Geom<WN, BT, TM>;
        if (splits > 1 && !combine_splits16<Gm::NW, Gm::MI, Gm::NJ>(acc, ws, counters, tile, split,
                                                                    splits, wave, lane))
            return;
    }
    a16_epilogue<DT, ACT, WN, BT, TM, KB>(p, Cm, m0, n0, wave, lane, st0, st1, st2, st3, acc);
}

// ---------------------------------------------------------------------------
// Stream-K over the 256 x 256 16x16x32 tiles ("TIRx", section 4.3: work
// partitioning decided at run time rather than by a static one-tile-per-
// workgroup dispatch; "Beyond Hand-Written CUDA", section 2: the tile
// scheduler stage).  A grid whose tile count is not a multiple of the
// workgroups that run at once leaves a last, partly filled wave; here the
// launch is persistent (plan.grid workgroups, one per compute unit) and
//  - tiles 0 .. dp_tiles - 1 (whole waves) run data-parallel, each
//    workgroup taking dp_tiles / grid consecutive ones;
//  - the last sk_tiles tiles are cut into 128-deep K quads, units (tile,
//    quad) in tile-major order, and workgroup w takes the contiguous units
//    [w per, (w + 1) per): whole tiles it covers are finished directly, a
//    tile it covers only in part gets its FP32 partial stored
//    (device-coherent) in the workgroup's slot (2 w for its first piece,
//    2 w + 1 for its last), counted in with one atomic, and the workgroup
//    that completes the count adds every piece of the tile in K order (the
//    piece starting at k = 0 carries the bias), runs the epilogue and
//    resets the counter; a workgroup that finds the other piece of a
//    two-piece tile already counted adds it to its own in registers
//    instead of storing.  No workgroup ever waits for another.
// Slot layout: [4 waves][64 vectors][64 lanes] of 16 bytes (vector 8 j + i
// holds accumulator block (i, j)), 256 KiB per slot.
namespace {
constexpr int SK_SLOT_FLOATS = 256 * 256;
} // namespace

template <int DT, int ACT, int WN, bool BT>
__global__ __launch_bounds__(128 * WN, 1) void gemm_async16_sk_kernel(GemmArgs p, int tiles_m,
                                                                       int tiles_n, int group_m,
                                                                       SkPlan sk, float *ws,
                                                                       int *counters)
{
    static_assert(WN == 2, "stream-K on the 4-wave 16x16x32 kernel");
    constexpr int NJ = 16 / WN, PV = 8 * NJ; // 64 accumulator vectors per lane
    __shared__ __attribute__((aligned(1024))) unsigned char st0[A16_STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char st1[A16_STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char st2[A16_STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char st3[A16_STAGE];
    __shared__ int s_last;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // XCD-aware placement: workgroup b runs on XCD b % 8, so it takes the
    // place v = (b % 8) (grid / 8) + b / 8 (grid a multiple of 8): each XCD
    // works through one contiguous run of data-parallel tiles and one of
    // split units, in grouped tile order, and its L2 keeps their panels.
    const int per_xcd = sk.grid / kNumXcd;
    const int w = ((int)blockIdx.x % kNumXcd) * per_xcd + (int)blockIdx.x / kNumXcd;
    const int Q = sk.q;
    f32x4 acc[8][NJ];

    // Each pass of the loops below takes lane and wave through an empty asm
    // statement, so the compiler cannot hoist the lane-dependent address
    // arithmetic of the K loop and the epilogue out of the persistent loop
    // (kept live across it, that arithmetic spills hundreds of registers).
    auto opaque = [&](int &ln, int &wv) {
        ln = lane;
        wv = wave;
        asm volatile("" : "+v"(ln), "+s"(wv));
    };
    auto coords = [&](int logical, int &m0, int &n0, const unsigned short *&Bm,
                      unsigned short *&Cm) {
        const TileCoord tc = grouped_tile(tiles_m, tiles_n, p.n_mat, group_m, logical);
        m0 = tc.tm * A16_BM;
        n0 = tc.tn * A16_BN;
        Bm = tc.mat == 0 ? p.B[0] : (tc.mat == 1 ? p.B[1] : p.B[2]);
        Cm = tc.mat == 0 ? p.C[0] : (tc.mat == 1 ? p.C[1] : p.C[2]);
    };
    // Work of this workgroup: its whole tiles of the data-parallel waves,
    // then its units [u0, u1) of the split tiles, taken
    // last piece first: the head of a tile (its K start) is then published
    // early by the workgroup before, and the tail, computed last, usually
    // finishes the tile.  One loop with one K loop and one epilogue (two
    // inlined copies of each grow the function past what the compiler
    // unrolls, and the accumulators end up on the stack).
    // data-parallel tiles (dp_tiles is a whole number of waves): the XCD's
    // run of per_xcd per_dp tiles, one contiguous slice of per_xcd tiles per
    // round
    const int per_dp = sk.dp_tiles / sk.grid;
    const int n_dp = per_dp;
    const int units = sk.sk_tiles * Q;
    const int u0 = w * sk.per, u1 = min(units, u0 + sk.per);
    int i_dp = 0, u = u1; // split units still to do: [u0, u)
    while (i_dp < n_dp || u > u0) {
        int logical, q0, q1, ts = -1;
        bool first_piece = false;
        if (i_dp < n_dp) {
            logical = (w / per_xcd) * per_xcd * per_dp + i_dp * per_xcd + w % per_xcd;
            q0 = 0;
            q1 = Q;
            ++i_dp;
        } else {
            ts = (u - 1) / Q; // stream-K tile of the last unit left
            q1 = u - ts * Q;
            q0 = max(0, q1 - (u - u0));
            logical = sk.dp_tiles + ts;
            first_piece = ts * Q + q0 == u0;
            u -= q1 - q0;
        }
        int m0, n0;
        const unsigned short *Bm;
        unsigned short *Cm;
        coords(logical, m0, n0, Bm, Cm);
        int ln, wv;
        opaque(ln, wv);
        a16_init_acc<DT, WN>(p, n0, wv, ln, q0 == 0, acc);
        // B stored [N,K]: the pair-staged loop.  B [K,N]: the 32-deep loop
        // with 64-bit lane addresses (in this kernel the pair-staged one
        // compiles to accumulator moves between the register files, and
        // the scalar-corner form measured level, 4352 x 4096 x 4096)
        if constexpr (BT)
            a16_mainloop_pairs<DT, WN, BT>(p, m0, n0, Bm, 4 * q0, 4 * (q1 - q0), wv, ln, st0,
                                           st1, st2, st3, acc);
        else
            a16_mainloop<DT, WN, BT, false, 256, 32, false>(p, m0, n0, Bm, 4 * q0, 4 * (q1 - q0),
                                                            wv, ln, st0, st1, st2, st3, acc);
        bool finish = q0 == 0 && q1 == Q;
        if (!finish) {
            // pieces of tile ts: workgroups w_first .. w_last, piece s stored
            // in slot 2 (w_first + s) (+ 1 for the first piece when the tile
            // does not start that workgroup's range: it is then that
            // workgroup's last piece)
            const int w_first = (ts * Q) / sk.per;
            const int w_last = ((ts + 1) * Q - 1) / sk.per;
            const int n_pieces = w_last - w_first + 1;
            const int lane_off = wv * PV * 256 + ln * 4;
            auto slot_of = [&](int wp) {
                return ws + (int64_t)(2 * wp + (wp == w_first && ts * Q != wp * sk.per ? 1 : 0)) *
                                SK_SLOT_FLOATS +
                       lane_off;
            };
            // half hh: vectors 32 hh .. 32 hh + 31 = blocks (i, j), j in 4 hh .. 4 hh + 3
            auto add_half = [&](auto hc, const float *src) {
                constexpr int hh = decltype(hc)::value;
                f32x4 v[32];
                load_partial32(src + hh * 32 * 256, v);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        acc[i][4 * hh + jj] += v[8 * jj + i];
            };
            // Every other piece of a two-piece tile already in: keep this one
            // in registers and add the other (a + b == b + a, so the bits do
            // not depend on which piece finishes; no piece is -0, since each
            // starts from +0 or from the bias, so 0 + a + b on the stored
            // path below gives the same bits).  Tiles of three pieces always
            // take the stored path, which adds in K order.
            if (threadIdx.x == 0)
                s_last = n_pieces == 2 && __hip_atomic_load(&counters[ts], __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT) == 1;
            __syncthreads();
            const bool in_registers = s_last;
            if (!in_registers) {
                float *dst =
                    ws + (int64_t)(2 * w + (first_piece ? 0 : 1)) * SK_SLOT_FLOATS + lane_off;
                auto store_half = [&](auto hc) {
                    constexpr int hh = decltype(hc)::value;
                    f32x4 v[32];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            v[8 * jj + i] = acc[i][4 * hh + jj];
                    store_partial<32>(dst + hh * 32 * 256, v);
                };
                static_assert(PV == 64, "two halves of 32 vectors");
                store_half(std::integral_constant<int, 0>{});
                store_half(std::integral_constant<int, 1>{});
                __syncthreads();
                if (threadIdx.x == 0) {
                    const int old = __hip_atomic_fetch_add(&counters[ts], 1, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
                    s_last = (old == n_pieces - 1);
                }
                __syncthreads();
                if (s_last) {
                    // the last piece in: every piece comes from memory
#pragma unroll
                    for (int i = 0; i < 8; ++i)
#pragma unroll
                        for (int j = 0; j < NJ; ++j)
                            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
            finish = s_last;
            if (finish) {
                // add the pieces in K order (the own one is already in the
                // registers when it stayed there)
                for (int wp = w_first; wp <= w_last; ++wp) {
                    if (in_registers && wp == w)
                        continue;
                    add_half(std::integral_constant<int, 0>{}, slot_of(wp));
                    add_half(std::integral_constant<int, 1>{}, slot_of(wp));
                }
            }
            if (finish && threadIdx.x == 0)
                __hip_atomic_store(&counters[ts], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (finish) {
            // the epilogue restages through the stages: every wave is done
            // with them before the next tile's copies land there
            a16_epilogue<DT, ACT, WN, BT>(p, Cm, m0, n0, wv, ln, st0, st1, st2, st3, acc);
            __builtin_amdgcn_s_waitcnt(0xC07F);
            stage_barrier();
        }
    }
}

namespace {
struct AsyncConfig {
    int ti, tj;
    int mfma16; // tiles on the 16x16x32 MFMA with this many waves; 0: 32x32x16
    bool forced_only; // taken only when TG_FORCE_CONFIG names it
    const char *name;
    int kb = 32;      // k per step of the K loop
    bool pairs = false; // the pair-staged K loop (256 x 256, K a multiple of 128)
};

// in order of preference: the first eligible configuration with a full wave
// of workgroups is taken
const AsyncConfig kAsyncConfigs[] = {
    // full waves of tiles: the pair-staged K loop (B stored [N,K]: bf16
    // 4096^3 to 8192^3 7 to 10 % ahead of the 32-deep loop; B [K,N]: f16
    // 4096^3 with GELU 3 % ahead, bf16 8192^3 and QKV level)
    {4, 4, 4, false, "async_256x256x32p_s4_mfma16", 32, true},
    {4, 4, 4, false, "async_256x256x32_s4_mfma16"},
    {4, 4, 8, true, "async_256x256x32_s4_mfma16_w8"}, // never ahead of the 4-wave kernel
    // 192 x 192 tiles fill a wave where 256 x 256 ones leave much of it idle
    // (3072^2 outputs: 256 tiles against 144)
    {3, 3, 4, false, "async_192x192x32_s4_mfma16"},
    // as fast as the 32x32x16 128 x 128 tiles (within 3 % over 264 shapes:
    // at this size the K loop is bound by the latency of its steps), and
    // unlike them it masks K off the 128 grid in the kernel
    {2, 2, 4, false, "async_128x128x32_s4_mfma16"},

    // 64-deep steps: half the barriers and waits per k, whole 128-byte row
    // pieces per copy (B [N,K] 1024 x 8192 x 8192: 117 against 156 us for the
    // 32-deep tiles)
    {2, 2, 4, false, "async_128x128x64_s4_mfma16", 64},
    {4, 4, 0, false, "async_256x256x32_s4"},
    {2, 2, 0, false, "async_128x128x32_s4"},
    {1, 2, 0, false, "async_64x128x32_s4"},
    {1, 1, 0, false, "async_64x64x32_s4"},
};
} // namespace

int num_async_configs() { return (int)(sizeof kAsyncConfigs / sizeof kAsyncConfigs[0]); }
const char *async_config_name(int cfg) { return kAsyncConfigs[cfg].name; }
bool async_forced_only(int cfg) { return kAsyncConfigs[cfg].forced_only; }
bool async_mfma16(int cfg) { return kAsyncConfigs[cfg].mfma16 != 0; }
bool async_pairs(int cfg) { return kAsyncConfigs[cfg].pairs; }
int async_tile_m(int cfg) { return 64 * kAsyncConfigs[cfg].ti; }
int async_tile_n(int cfg) { return 64 * kAsyncConfigs[cfg].tj; }
int async_k_step(int cfg) { return kAsyncConfigs[cfg].kb; }

int async_tiles_m(const GemmArgs &a, int cfg)
{
    return (a.M + async_tile_m(cfg) - 1) / async_tile_m(cfg);
}

int async_tiles_n(const GemmArgs &a, int cfg)
{
    return (a.N + async_tile_n(cfg) - 1) / async_tile_n(cfg);
}

// K a multiple of the loop's four steps (Q = 128 k, or 256 with 64-deep
// steps); on the 16x16x32 configurations also a multiple of 8 with at most
// as many padded k as real ones (the masked last quad multiplies zeros for
// the rest)
static bool async_k_ok(int K, bool masked_ok, int Q)
{
    return K > 0 && (K % Q == 0 || (masked_ok && K % 8 == 0 && (K + Q - 1) / Q * Q - K <= K));
}

bool async_eligible(const GemmArgs &a, int cfg, bool any_pad)
{
    // An M (or an N that is a multiple of 8) that is not a multiple of the
    // tile is taken when the partial last row (column) tile wastes at most
    // M / 8 rows (N / 8 columns), and always by the 64-row (64-column)
    // tiles: the copies of a partial tile read the last row (the last 8
    // columns) again and the stores stop at M (N), so any partial tile is
    // exact, and for such shapes the kernels left (element-wise loads, or
    // none for B stored [N,K]) are several times slower than the idle rows
    // of one tile cost.
    // any_pad drops the M / 8 bound (the tiles stay exact; the caller weighs
    // the idle rows and columns itself).
    const int tm = async_tile_m(cfg), tn = async_tile_n(cfg);
    const int pad = async_tiles_m(a, cfg) * tm - a.M;
    const bool m_ok = any_pad || a.M % tm == 0 || tm == 64 || (a.M > tm && 8 * pad <= a.M);
    const int padn = async_tiles_n(a, cfg) * tn - a.N;
    const bool n_ok = a.N % tn == 0 ||
                      (a.N % 8 == 0 && (any_pad || tn == 64 || (a.N > tn && 8 * padn <= a.N)));
    // the 16x16x32 kernels' copies: 256 rows of A (and of B stored [N,K])
    // within the 32-bit byte offsets of a lane
    const bool ld32 = a.lda < (1 << 23) && (!a.b_trans || a.ldb < (1 << 23));
    return m_ok && n_ok && (!kAsyncConfigs[cfg].mfma16 || ld32) &&
           async_k_ok(a.K, kAsyncConfigs[cfg].mfma16 != 0 && !kAsyncConfigs[cfg].pairs,
                      AS_STAGES * kAsyncConfigs[cfg].kb) &&
           ((uintptr_t)a.bias & 7u) == 0 &&
           ((uintptr_t)a.R & 15u) == 0 && a.ldr % 8 == 0;
}

int plan_async_splits(const GemmArgs &a, int cfg, int want)
{
    const AsyncConfig &c = kAsyncConfigs[cfg];
    // the 32x32x16 tiles up to 128 x 128, and the 16x16x32 128 x 128 ones
    if ((c.mfma16 && c.ti != 2) || c.ti * c.tj > 4 || want == 1)
        return 1;
    const int64_t tiles = (int64_t)async_tiles_m(a, cfg) * async_tiles_n(a, cfg) * a.n_mat;
    if (tiles > kMaxSplitTiles || (want <= 0 && tiles >= 240))
        return 1;
    // enough workgroups for one wave of the 256 CUs, at most 8 splits, each
    // a multiple of the four-step loop
    int s = want > 0 ? want : (int)(256 / tiles);
    s = s > 8 ? 8 : s;
    for (; s >= 2; --s)
        if (a.K % (s * AS_STAGES * c.kb) == 0)
            return s;
    return 1;
}

size_t async_ws_floats(const GemmArgs &a, int cfg, int splits)
{
    return (size_t)splits * (size_t)async_tiles_m(a, cfg) * async_tiles_n(a, cfg) * a.n_mat *
           async_tile_m(cfg) * async_tile_n(cfg);
}

SkPlan plan_stream_k(const GemmArgs &a, int cfg, int cus, bool any_size)
{
    SkPlan pl{0, 0, 0, 0, 0};
    if (kAsyncConfigs[cfg].mfma16 != 4 || kAsyncConfigs[cfg].ti != 4 || kAsyncConfigs[cfg].pairs ||
        !async_eligible(a, cfg) || cus <= 0 || cus % kNumXcd != 0)
        return pl;
    const int64_t tiles = (int64_t)async_tiles_m(a, cfg) * async_tiles_n(a, cfg) * a.n_mat;
    const int q = a.K / (AS_STAGES * AS_BK);
    if (a.K % (AS_STAGES * AS_BK) != 0)
        return pl;
    // whole waves need no split; below half a wave each tile would be cut
    // into more than two pieces, and the one workgroup that adds them reads
    // every 256 KiB partial back on its own (measured with pieces of
    // ceil(q / (CUs / tiles)) quads: 256 x 4096 x 4096, 16 tiles, 63.6 us
    // against 21.1 on 64 x 64 tiles; 512 x 14336 x 4096 80.8 against 63.2)
    if (tiles % cus == 0 || 2 * tiles < cus || q < 2 || tiles >= (int64_t)1 << 24)
        return pl;
    const int64_t full = tiles / cus, rest = tiles % cus;
    // Short of one wave the partly filled grid of whole tiles (or of 192 x
    // 192 ones) does better unless any_size: measured, bf16 3584^3 (196
    // tiles) 1141 TFLOP/s data-parallel against 890 split, 2049 x 4096 x
    // 4096 (144) 748 against 692.
    if (full == 0 && !any_size)
        return pl;
    // After whole waves, a last wave of at least half the compute units stays
    // data-parallel: the kernel is power-bound, and such a wave runs at a
    // higher clock than a full one, which recovers most of what the idle
    // units cost (measured: 5120^3, 400 tiles, 1222 TFLOP/s data-parallel
    // against 1149 with the last 144 tiles split).
    if (full >= 1 && 2 * rest >= cus)
        return pl;
    // Split tiles: all of them when there is no whole wave, else the short
    // last wave plus one whole wave, so that no tile is cut into more than
    // about two pieces.  The waves before run whole, in lockstep over K,
    // which keeps their panels in L2.
    const int64_t sk_tiles = full == 0 ? tiles : rest + cus;
    const int64_t units = sk_tiles * q;
    const int64_t per = (units + cus - 1) / cus;
    // each workgroup's share of the split tiles must be long enough to pay
    // for the partial exchange and for running out of lockstep: at least 16
    // quads (K = 2048) unless any_size (measured: 3072^3, 144 tiles of 14
    // quads each, is faster on 128 x 128 tiles)
    if (per < 16 && !any_size)
        return pl;
    pl.dp_tiles = (int)(tiles - sk_tiles);
    pl.sk_tiles = (int)sk_tiles;
    pl.q = q;
    pl.per = (int)per;
    pl.grid = cus; // places past the last unit get data-parallel tiles only
    return pl;
}

size_t stream_k_ws_floats(const SkPlan &sk) { return (size_t)2 * sk.grid * SK_SLOT_FLOATS; }

hipError_t launch_async_sk(int cfg, int dt, int act, const GemmArgs &a, int group_m,
                           const SkPlan &sk, float *ws, int *counters, hipStream_t s)
{
    if (kAsyncConfigs[cfg].mfma16 != 4 || kAsyncConfigs[cfg].ti != 4 || sk.sk_tiles <= 0 ||
        sk.grid <= 0 || sk.q <= 0 || sk.per <= 0 || ws == nullptr || counters == nullptr ||
        sk.grid % kNumXcd != 0 || (int64_t)sk.per * sk.grid < (int64_t)sk.sk_tiles * sk.q ||
        sk.dp_tiles % sk.grid != 0)
        return hipErrorInvalidValue;
    const int tiles_m = async_tiles_m(a, cfg), tiles_n = async_tiles_n(a, cfg);
    dim3 grid(sk.grid), block(A16Geom<2, false>::NT);
#define TG_SK(DT_, ACT_)                                                                         \
    do {                                                                                         \
        if (a.b_trans)                                                                           \
            hipLaunchKernelGGL((gemm_async16_sk_kernel<DT_, ACT_, 2, true>), grid, block, 0, s,  \
                               a, tiles_m, tiles_n, group_m, sk, ws, counters);                  \
        else                                                                                     \
            hipLaunchKernelGGL((gemm_async16_sk_kernel<DT_, ACT_, 2, false>), grid, block, 0, s, \
                               a, tiles_m, tiles_n, group_m, sk, ws, counters);                  \
    } while (0)
    if (dt == DT_F16) {
        if (act == ACT_GELU)
            TG_SK(DT_F16, ACT_GELU);
        else
            TG_SK(DT_F16, ACT_NONE);
    } else {
        if (act == ACT_GELU)
            TG_SK(DT_BF16, ACT_GELU);
        else
            TG_SK(DT_BF16, ACT_NONE);
    }
#undef TG_SK
    return hipGetLastError();
}

hipError_t launch_async(int cfg, int dt, int act, const GemmArgs &a, int group_m, int splits,
                        float *ws, int *counters, hipStream_t s)
{
    const int tiles_m = async_tiles_m(a, cfg), tiles_n = async_tiles_n(a, cfg);
    if (splits < 1 || (splits > 1 && (plan_async_splits(a, cfg, splits) != splits ||
                                      ws == nullptr || counters == nullptr)))
        return hipErrorInvalidValue;
    dim3 grid(tiles_m * tiles_n * a.n_mat * splits), block(AS_NT);
    const bool km = a.K % (AS_STAGES * kAsyncConfigs[cfg].kb) != 0;
    if (km && splits != 1)
        return hipErrorInvalidValue;
    if (kAsyncConfigs[cfg].mfma16) {
        static_assert(A16Geom<4, false>::NT == 512 && A16Geom<2, false>::NT == 256 &&
                          A16Geom<4, true>::NT == 512 && A16Geom<2, true>::NT == 256,
                      "block sizes below");
        const int wn = kAsyncConfigs[cfg].mfma16 / 2;
        if (kAsyncConfigs[cfg].pairs) {
            if (km || splits != 1 || kAsyncConfigs[cfg].ti != 4)
                return hipErrorInvalidValue;
#define TG_A16P(DT_, ACT_)                                                                       \
    do {                                                                                         \
        if (a.b_trans)                                                                           \
            hipLaunchKernelGGL((gemm_async16p_kernel<DT_, ACT_, 2, true>), grid, dim3(256), 0, s, \
                               a, tiles_m, tiles_n, group_m);                                    \
        else                                                                                     \
            hipLaunchKernelGGL((gemm_async16p_kernel<DT_, ACT_, 2, false>), grid, dim3(256), 0,  \
                               s, a, tiles_m, tiles_n, group_m);                                 \
    } while (0)
            if (dt == DT_F16) {
                if (act == ACT_GELU)
                    TG_A16P(DT_F16, ACT_GELU);
                else
                    TG_A16P(DT_F16, ACT_NONE);
            } else {
                if (act == ACT_GELU)
                    TG_A16P(DT_BF16, ACT_GELU);
                else
                    TG_A16P(DT_BF16, ACT_NONE);
            }
#undef TG_A16P
            return hipGetLastError();
        }
        const bool t192 = kAsyncConfigs[cfg].ti == 3, t128 = kAsyncConfigs[cfg].ti == 2;
        const bool k64 = kAsyncConfigs[cfg].kb == 64;
#define TG_A16K(DT_, ACT_, KM_)                                                                  \
    do {                                                                                         \
        if (t128 && k64 && a.b_trans)                                                            \
            hipLaunchKernelGGL((gemm_async16_kernel<DT_, ACT_, 2, true, KM_, 128, 64>), grid,     \
                               dim3(256), 0, s, a, tiles_m, tiles_n, group_m, splits, ws, counters);                   \
        else if (t128 && k64)                                                                    \
            hipLaunchKernelGGL((gemm_async16_kernel<DT_, ACT_, 2, false, KM_, 128, 64>), grid,    \
                               dim3(256), 0, s, a, tiles_m, tiles_n, group_m, splits, ws, counters);                   \
        else if (t128 && a.b_trans)                                                              \
            hipLaunchKernelGGL((gemm_async16_kernel<DT_, ACT_, 2, true, KM_, 128>), grid,         \
                               dim3(256), 0, s, a, tiles_m, tiles_n, group_m, splits, ws, counters);                   \
        else if (t128)                                                                           \
            hipLaunchKernelGGL((gemm_async16_kernel<DT_, ACT_, 2, false, KM_, 128>), grid,        \
                               dim3(256), 0, s, a, tiles_m, tiles_n, group_m, splits, ws, counters);                   \
        else if (t192 && a.b_trans)                                                              \
            hipLaunchKernelGGL((gemm_async16_kernel<DT_, ACT_, 2, true, KM_, 192>), grid,         \
                               dim3(256), 0, s, a, tiles_m, tiles_n, group_m, splits, ws, counters);                   \
        else if (t192)                                                                           \
            hipLaunchKernelGGL((gemm_async16_kernel<DT_, ACT_, 2, false, KM_, 192>), grid,        \
                               dim3(256), 0, s, a, tiles_m, tiles_n, group_m, splits, ws, counters);                   \
        else if (wn == 4 && a.b_trans)                                                           \
            hipLaunchKernelGGL((gemm_async16_kernel<DT_, ACT_, 4, true, KM_>), grid, dim3(512), \
                               0, s, a, tiles_m, tiles_n, group_m, splits, ws, counters);                              \
        else if (wn == 4)                                                                        \
            hipLaunchKernelGGL((gemm_async16_kernel<DT_, ACT_, 4, false, KM_>), grid, dim3(512), \
                               0, s, a, tiles_m, tiles_n, group_m, splits, ws, counters);                              \
        else if (a.b_trans)                                                                      \
            hipLaunchKernelGGL((gemm_async16_kernel<DT_, ACT_, 2, true, KM_>), grid, dim3(256), \
                               0, s, a, tiles_m, tiles_n, group_m, splits, ws, counters);                              \
        else                                                                                     \
            hipLaunchKernelGGL((gemm_async16_kernel<DT_, ACT_, 2, false, KM_>), grid, dim3(256), \
                               0, s, a, tiles_m, tiles_n, group_m, splits, ws, counters);                              \
    } while (0)
#define TG_A16(DT_, ACT_)                                                                        \
    do {                                                                                         \
        if (km)                                                                                  \
            TG_A16K(DT_, ACT_, true);                                                            \
        else                                                                                     \
            TG_A16K(DT_, ACT_, false);                                                           \
    } while (0)
        if (dt == DT_F16) {
            if (act == ACT_GELU)
                TG_A16(DT_F16, ACT_GELU);
            else
                TG_A16(DT_F16, ACT_NONE);
        } else {
            if (act == ACT_GELU)
                TG_A16(DT_BF16, ACT_GELU);
            else
                TG_A16(DT_BF16, ACT_NONE);
        }
#undef TG_A16
#undef TG_A16K
        return hipGetLastError();
    }
#define TG_AS(DT_, ACT_, TI_, TJ_)                                                               \
    do {                                                                                         \
        if (a.b_trans)                                                                           \
            hipLaunchKernelGGL((gemm_async_kernel<DT_, ACT_, TI_, TJ_, true>), grid, block, 0, s, \
                               a, tiles_m, tiles_n, group_m, splits, ws, counters);              \
        else                                                                                     \
            hipLaunchKernelGGL((gemm_async_kernel<DT_, ACT_, TI_, TJ_, false>), grid, block, 0,   \
                               s, a, tiles_m, tiles_n, group_m, splits, ws, counters);           \
    } while (0)
#define TG_AS_CFG(DT_, ACT_)                                                                     \
    do {                                                                                         \
        const AsyncConfig &c_ = kAsyncConfigs[cfg];                                              \
        if (c_.ti == 4)                                                                          \
            TG_AS(DT_, ACT_, 4, 4);                                                              \
        else if (c_.ti == 2)                                                                     \
            TG_AS(DT_, ACT_, 2, 2);                                                              \
        else if (c_.tj == 2)                                                                     \
            TG_AS(DT_, ACT_, 1, 2);                                                              \
        else                                                                                     \
            TG_AS(DT_, ACT_, 1, 1);                                                              \
    } while (0)
    if (dt == DT_F16) {
        if (act == ACT_GELU)
            TG_AS_CFG(DT_F16, ACT_GELU);
        else
            TG_AS_CFG(DT_F16, ACT_NONE);
    } else {
        if (act == ACT_GELU)
            TG_AS_CFG(DT_BF16, ACT_GELU);
        else
            TG_AS_CFG(DT_BF16, ACT_NONE);
    }
#undef TG_AS_CFG
#undef TG_AS
    return hipGetLastError();
}

} // namespace tg
