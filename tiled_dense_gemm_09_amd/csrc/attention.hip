// attention.hip -- fused forward attention with an online softmax.
//
//   O[i] = sum_j softmax_j( scale * Q[i] . K[j] + mask[i][j] ) V[j]
//
// "TileIR" (the attention block Softmax(Q K^T / sqrt(d)) V fused into one
// kernel at the tile level with an online softmax, so the score matrix is
// never materialised); "TIRx", section 6 (forward multi-head attention, head
// dimension 128, causal and non-causal).  Q, K, V, O: [B][H][S][128], f16 or
// bf16; FP32 scores, softmax and accumulation; optional log-sum-exp per row.
//
// Mapping onto gfx950 (one workgroup = 32 WAVES queries of one head, WAVES
// waves of 32 queries; K and V stream through LDS in 64-key tiles):
//  - Workgroup size.  Every K/V tile a workgroup copies into LDS serves all
//    of its queries, so the bytes moved per flop halve from 128 queries (4
//    waves, two workgroups per CU) to 256 (8 waves, one workgroup per CU);
//    both keep two waves per SIMD.  The copies' energy is what holds the
//    clock down under this load, so the larger block is the default when S
//    is a multiple of 256.
//  - S = Q K^T on v_mfma_f32_32x32x16 with K as src0 (its rows are keys) and
//    Q as src1: lane l then holds query l % 32 and keys 8g + 4(l/32) + e of
//    each 32-key block in register 4g + e.  Q's fragments (8 of 16 d) stay
//    in registers for the whole loop; K tiles are staged K-contiguous
//    (256-byte rows, granule c of row r at c ^ (r % 16)) and read with
//    128-bit reads.
//  - Online softmax in the log2 domain: t = s * scale * log2(e); per row a
//    reference maximum m and a sum l.  A row's 64 scores of a tile sit in
//    lanes l and l ^ 32 (32 each), combined with v_permlane32_swap.  The
//    reference is raised (and O and l rescaled by 2^(m_old - m_new)) only
//    when some row of the wave sees a tile maximum more than 8 above its
//    reference; otherwise the exponentials may reach 2^8, which FP32 and the
//    16-bit P hold with the same relative precision as values below 1.  Every
//    exponent of a row is still taken against the one reference its O and l
//    share, so the result is the same softmax.
//  - O += P V on the same MFMA with V as src0 (rows = d) and P as src1.  The
//    16 keys of each P chunk are taken in the order the S accumulator holds
//    them (registers 8c .. 8c+7: keys 16c + 4(l/32) + {0..3} and
//    16c + 8 + 4(l/32) + {0..3}), and V's fragment is read in the same key
//    order with two transposing reads (V stays N-contiguous in LDS, granule
//    c of row r at c ^ {0, 6, 10, 12}[r % 4]).  The sum over k is order-free,
//    so P never leaves the registers.
//  - K and V tiles arrive by direct global->LDS copies one tile ahead (two
//    stages, 64 KiB: two 4-wave workgroups or one 8-wave workgroup per CU,
//    two waves per SIMD either way); the epilogue divides by l, rounds, and
//    restages each wave's 32 x 128 tile through LDS for whole-row stores
//    (tg_pipeline.h).
//  - Causal: a wave skips the work of key tiles wholly above its diagonal
//    (they would add exp2(-inf) = 0 and raise no reference).
#include "tg_device.h"
#include "tg_launch.h"
#include "tg_pipeline.h"

namespace tg {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int AT_D = 128, AT_BN = 64;
constexpr float AT_SLACK = 8.f;                  // log2 units a tile maximum may exceed the reference
constexpr int AT_TILE = AT_BN * AT_D * 2;        // 16 KiB: one K or V tile
constexpr int AT_STAGE = 2 * AT_TILE;            // K tile, then V tile

__host__ __device__ constexpr int swz_k(int r) { return r & 15; }
__host__ __device__ constexpr int swz_v(int r) { return (0xCA60 >> (4 * (r & 3))) & 15; }

// max and sum over the lane pair (l, l ^ 32)
__device__ __forceinline__ float pair_max(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

} // namespace

template <int DT, bool CAUSAL, int WAVES>
__global__ __launch_bounds__(64 * WAVES, WAVES == 4 ? 2 : 1) void attn_fwd_kernel(AttnArgs p)
{
    static_assert(WAVES == 4 || WAVES == 8, "128 or 256 queries per workgroup");
    constexpr int BM = 32 * WAVES; // queries per workgroup
    constexpr int CPW = 16 / WAVES; // 1 KiB copies of K (and of V) per wave per tile
    constexpr int STAGES = 2; // tile t+1 lands while tile t is used
    __shared__ __attribute__((aligned(1024))) unsigned char lds[STAGES * AT_STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;
    const int nqb = p.S / BM;
    // grid (heads, query blocks): workgroups are dispatched with x fastest,
    // so every head's block of a given length goes out together; causal
    // blocks are taken longest first so the short ones fill the tail
    const int qb = CAUSAL ? nqb - 1 - (int)blockIdx.y : (int)blockIdx.y;
    const int64_t head = (int64_t)blockIdx.x * p.S * AT_D;
    const unsigned short *Qh = p.Q + head, *Kh = p.K + head, *Vh = p.V + head;
    const int q0 = qb * BM + wave * 32;      // this wave's first query
    const int myq = q0 + (lane & 31);        // the query this lane's scores belong to
    const int ntiles = CAUSAL ? ((qb + 1) * BM) / AT_BN : p.S / AT_BN;

    // ---- Q fragments: d 16 dc + 8 h .. + 7 of query myq (src1 operand)
    u32x4 qf[8];
#pragma unroll
    for (int dc = 0; dc < 8; ++dc)
        qf[dc] = *reinterpret_cast<const u32x4 *>(Qh + (int64_t)myq * AT_D + 16 * dc + 8 * h);
    wait_vmcnt<0>();

    // ---- copy plan: tile copy q (0..15) of K or V fills rows 4q .. 4q+3
    // (256 bytes each); lane -> (row 4q + lane/16, granule lane%16).  Wave w
    // issues K copies CPW w .. CPW w + CPW-1 and the same V copies.
    const unsigned short *gk[CPW], *gv[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int r = 4 * (wave * CPW + i) + (lane >> 4);
        gk[i] = Kh + (int64_t)r * AT_D + ((lane & 15) ^ swz_k(r)) * 8;
        gv[i] = Vh + (int64_t)r * AT_D + ((lane & 15) ^ swz_v(r)) * 8;
    }
    const unsigned lds_base = (unsigned)(uintptr_t)(lds_void *)lds;
    auto issue = [&](int t, int stage) {
        const unsigned st = lds_base + stage * AT_STAGE;
        const int64_t off = (int64_t)t * AT_BN * AT_D;
#pragma unroll
        for (int i = 0; i < CPW; ++i)
            asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gk[i] + off),
                         "{m0}"(st + (wave * CPW + i) * 1024)
                         : "memory");
#pragma unroll
        for (int i = 0; i < CPW; ++i)
            asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gv[i] + off),
                         "{m0}"(st + AT_TILE + (wave * CPW + i) * 1024)
                         : "memory");
    };

    // ---- fragment offsets within a stage
    // K fragment (block jb, d chunk dc): row 32 jb + lane%32, granule 2dc + h
    int k_off[2][8];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
        const int r = 32 * jb + (lane & 31);
#pragma unroll
        for (int dc = 0; dc < 8; ++dc)
            k_off[jb][dc] = r * 256 + (((2 * dc + h) ^ swz_k(r)) * 16);
    }
    // V fragment (key chunk c, d block db), read g (0, 1): the 16-lane group
    // gl = lane/16 addresses rows 16c + 8g + 4(gl/2) + jj/4 and columns
    // 32 db + 16 (gl % 2) + 4 (jj % 4), jj = lane % 16; lane i of the group
    // receives column 32 db + 16 (gl % 2) + i at those 4 rows.  The row's
    // low two bits are jj/4 for every (c, g), so the swizzle is per lane.
    int v_row[4][2];
    const int gl = lane >> 4, jj = lane & 15;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int g = 0; g < 2; ++g)
            v_row[c][g] = AT_TILE + (16 * c + 8 * g + 4 * (gl >> 1) + (jj >> 2)) * 256;
    const int v_gran = 2 * (gl & 1) + ((jj & 3) >> 1); // granule of the column (db = 0)
    const int v_sub = (jj & 1) * 8;                      // byte within the granule
    const int v_swz = swz_v(jj >> 2);

    f32x16 acc_o[1][4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc_o[0][db][r] = 0.f;
    float m_run = -__builtin_inff(), l_run = 0.f;
    const float c2 = p.scale_log2;

    // ---- per-tile pieces: S = Q K^T of a 64-key tile (two 32-key blocks),
    // the causal mask, the online softmax (which turns S into P in place),
    // and O += P V.
    auto qk = [&](f32x16 (&s)[2], const unsigned char *st) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[jb][r] = 0.f;
#pragma unroll
        for (int dc = 0; dc < 8; ++dc)
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                const u32x4 kf = *reinterpret_cast<const u32x4 *>(st + k_off[jb][dc]);
                s[jb] = mfma32x32x16<DT>(kf, qf[dc], s[jb]);
            }
    };
    // causal mask on the tiles that reach past this wave's first query
    auto mask = [&](f32x16 (&s)[2], int k0) {
        if (CAUSAL && k0 + AT_BN - 1 > q0) {
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 32 * jb + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (key > myq)
                        s[jb][r] = -__builtin_inff();
                }
        }
    };
    auto softmax = [&](f32x16 (&s)[2]) {
        float mx = -__builtin_inff();
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                mx = __builtin_fmaxf(mx, s[jb][r]);
        mx = pair_max(mx);
        const float tm = mx * c2;
        const bool raise = __builtin_amdgcn_ballot_w64(tm > m_run + AT_SLACK) != 0;
        const float m_new = raise ? __builtin_fmaxf(m_run, tm) : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float rs = 0.f;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[jb][r], c2, -m_new));
                s[jb][r] = e;
                rs += e;
            }
        rs = pair_sum(rs);
        l_run = l_run * alpha + rs;
        m_run = m_new;
        if (raise) {
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc_o[0][db][r] *= alpha;
        }
    };
    // O += P V: four 16-key chunks, four 32-column d blocks
    auto pv = [&](const f32x16 (&s)[2], const unsigned char *st) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int jb = c >> 1, cc = c & 1;
            u32x4 pf;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                pf[w] = pack2<DT>(s[jb][8 * cc + 2 * w], s[jb][8 * cc + 2 * w + 1]);
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                u32x4 vf;
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    const int off = v_row[c][g] + (((v_gran + 4 * db) ^ v_swz) * 16) + v_sub;
                    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(st + off));
                    const u32x2 w2 = __builtin_bit_cast(u32x2, v);
                    vf[2 * g] = w2[0];
                    vf[2 * g + 1] = w2[1];
                }
                acc_o[0][db] = mfma32x32x16<DT>(vf, pf, acc_o[0][db]);
            }
        }
    };
    // tile t lands in stage t % STAGES; before a tile's copies are issued
    // into a stage, every wave has finished the tile that stage held
    // (STAGES - 1 tiles earlier) and passed a barrier.
    auto stage_ptr = [&](int t) { return lds + (t % STAGES) * AT_STAGE; };
    auto sync_and_issue = [&](int t) {
        wait_vmcnt<0>();                      // this wave's copies of tile t
        __builtin_amdgcn_s_waitcnt(0xC07F);   // and its outstanding LDS reads
        stage_barrier();
        if (t + 1 < ntiles)
            issue(t + 1, (t + 1) % STAGES);
    };
    // causal: a tile wholly above this wave's diagonal adds exp2(-inf) = 0
    // to every row and raises no reference, so the wave skips its work (the
    // copies and barriers stay shared by the workgroup)
    auto active = [&](int t) { return !CAUSAL || t * AT_BN <= q0 + 31; };

    issue(0, 0);
    for (int t = 0; t < ntiles; ++t) {
        sync_and_issue(t);
        if (!active(t))
            continue;
        f32x16 s[2];
        qk(s, stage_ptr(t));
        mask(s, t * AT_BN);
        softmax(s);
        pv(s, stage_ptr(t));
    }

    // ---- epilogue: O / l, log-sum-exp, restaged stores
    const float inv_l = 1.0f / l_run;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc_o[0][db][r] *= inv_l;
    if (p.lse != nullptr && lane < 32)
        p.lse[(int64_t)blockIdx.x * p.S + myq] =
            (m_run + __builtin_amdgcn_logf(l_run)) * 0.6931471805599453f;
    wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    stage_barrier();
    restaged_epilogue<DT, ACT_NONE, 1, 4, false>(acc_o, lds + wave * 8192, lane,
                                                 p.O + head + (int64_t)q0 * AT_D, AT_D, nullptr,
                                                 0);
}

// ---------------------------------------------------------------------------
// Fallback for other shapes (any S, head dimension up to 128): one thread
// per query row, the same online softmax in FP32 over one key at a time.
template <int DT>
__global__ __launch_bounds__(128) void attn_fwd_generic_kernel(AttnArgs p, int D, int causal)
{
    const int64_t row = (int64_t)blockIdx.x * 128 + threadIdx.x;
    if (row >= (int64_t)p.BH * p.S)
        return;
    const int64_t hd = row / p.S, i = row % p.S;
    const unsigned short *Qh = p.Q + hd * p.S * D, *Kh = p.K + hd * p.S * D,
                         *Vh = p.V + hd * p.S * D;
    float q[128], o[128];
    for (int d = 0; d < D; ++d) {
        q[d] = from_bits<DT>(Qh[i * D + d]);
        o[d] = 0.f;
    }
    float m = -__builtin_inff(), l = 0.f;
    const int64_t nk = causal ? i + 1 : p.S;
    for (int64_t j = 0; j < nk; ++j) {
        float dot = 0.f;
        for (int d = 0; d < D; ++d)
            dot = __builtin_fmaf(q[d], from_bits<DT>(Kh[j * D + d]), dot);
        const float tj = dot * p.scale_log2;
        const float m_new = __builtin_fmaxf(m, tj);
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        const float e = __builtin_amdgcn_exp2f(tj - m_new);
        l = l * alpha + e;
        for (int d = 0; d < D; ++d)
            o[d] = __builtin_fmaf(e, from_bits<DT>(Vh[j * D + d]), o[d] * alpha);
        m = m_new;
    }
    for (int d = 0; d < D; ++d)
        p.O[row * D + d] = to_bits<DT>(o[d] / l);
    if (p.lse != nullptr)
        p.lse[row] = (m + __builtin_amdgcn_logf(l)) * 0.6931471805599453f;
}

bool attn_fast_eligible(const AttnArgs &a, int D)
{
    auto al16 = [](const void *q) { return ((uintptr_t)q & 15u) == 0; };
    return D == AT_D && a.S % 128 == 0 && a.S > 0 && al16(a.Q) && al16(a.K) && al16(a.V) &&
           al16(a.O);
}

int attn_block_m(const AttnArgs &a, int want)
{
    if (want == 128)
        return 128;
    return a.S % 256 == 0 ? 256 : 128;
}

hipError_t launch_attn(int dt, bool causal, int bm, const AttnArgs &a, hipStream_t s)
{
    const dim3 grid(a.BH, a.S / bm), block(bm * 2);
#define TG_AT(DT_, C_)                                                                           \
    do {                                                                                         \
        if (bm == 256)                                                                           \
            hipLaunchKernelGGL((attn_fwd_kernel<DT_, C_, 8>), grid, block, 0, s, a);             \
        else                                                                                     \
            hipLaunchKernelGGL((attn_fwd_kernel<DT_, C_, 4>), grid, block, 0, s, a);             \
    } while (0)
    if (dt == DT_F16) {
        if (causal)
            TG_AT(DT_F16, true);
        else
            TG_AT(DT_F16, false);
    } else {
        if (causal)
            TG_AT(DT_BF16, true);
        else
            TG_AT(DT_BF16, false);
    }
#undef TG_AT
    return hipGetLastError();
}

hipError_t launch_attn_generic(int dt, bool causal, const AttnArgs &a, int D, hipStream_t s)
{
    const int64_t rows = (int64_t)a.BH * a.S;
    const dim3 grid((unsigned)((rows + 127) / 128)), block(128);
    if (dt == DT_F16)
        hipLaunchKernelGGL((attn_fwd_generic_kernel<DT_F16>), grid, block, 0, s, a, D, causal ? 1 : 0);
    else
        hipLaunchKernelGGL((attn_fwd_generic_kernel<DT_BF16>), grid, block, 0, s, a, D, causal ? 1 : 0);
    return hipGetLastError();
}

} // namespace tg
