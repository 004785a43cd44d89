// tg_launch.h -- host-side launch interface between the C ABI (tg_api.cpp)
// and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

// Operands of one (possibly horizontally fused) GEMM launch.  n_mat is 1 for
// a plain GEMM and 3 for the QKV projection; B[t] and C[t] are the t-th
// weight and output.  All pitches are in elements.  Every kernel computes
// C = act(A . op(B) + bias) + R with one rounding at the end.
struct GemmArgs {
    const unsigned short *A;
    int64_t lda;
    const unsigned short *B[3];
    int64_t ldb;
    unsigned short *C[3];
    int64_t ldc;
    const unsigned short *bias; // [N] or nullptr
    const unsigned short *R;    // [M,N] residual added after the activation, or nullptr
    int64_t ldr;
    int M, N, K;
    int n_mat;
    int b_trans; // 1: B[t] is stored [N,K] (pitch ldb) and the product uses its transpose
};

// Tile configurations of the MFMA kernel: BM x BN output tile, BK deep,
// WM x WN waves of 64 lanes.
struct TileConfig {
    int bm, bn, bk, wm, wn;
    const char *name;
};

int num_tile_configs();
const TileConfig &tile_config(int i);

// Launchers; each returns the hipError_t of the launch.
hipError_t launch_tiled(int cfg, int dt, int act, const GemmArgs &a, int group_m,
                        hipStream_t stream);
// True when the tiled kernel must load and store element by element: a
// pointer not 16-byte aligned or a pitch not a multiple of 8 elements.  It
// still needs 2-byte aligned pointers and B stored [K,N].
bool tiled_unaligned(const GemmArgs &a);
hipError_t launch_generic(int dt, int act, const GemmArgs &a, hipStream_t stream);

// Asynchronous-copy MFMA kernel: 256 x 256 tiles (16x16x32 or 32x32x16
// MFMA), 128 x 128, 64 x 128 and 64 x 64 tiles (32x32x16), all 32 deep, 4
// stages; a
// problem is eligible for a configuration when K is a multiple of 128, M is
// a multiple of the tile height or leaves a partial last row tile of at
// most M / 8 padding rows, and N likewise (N a multiple of 8).
int num_async_configs();
const char *async_config_name(int cfg);
// taken only when TG_FORCE_CONFIG names it
bool async_forced_only(int cfg);
// true for the configurations on the 16x16x32 MFMA (256 x 256, 192 x 192 and 128 x 128 tiles)
bool async_mfma16(int cfg);
// the pair-staged K loop: taken only for full waves of tiles, never modelled
bool async_pairs(int cfg);
int async_tile_m(int cfg);
int async_tile_n(int cfg);
// k per step of the configuration's K loop (32, or 64)
int async_k_step(int cfg);
bool async_eligible(const GemmArgs &a, int cfg, bool any_pad = false);
// Row and column tiles of a problem: the ceilings of M / tile height and
// N / tile width (a partial last tile counts as a tile).
int async_tiles_m(const GemmArgs &a, int cfg);
int async_tiles_n(const GemmArgs &a, int cfg);
// Split-K for under-filled grids (128 x 128 and 64 x 128 tiles only, at most
// kMaxSplitTiles tiles): the number of K splits for the configuration, 1 for
// none.  want > 1 asks for that many (fewer when K does not divide), want
// == 1 disables it; want <= 0 splits only grids of fewer than 240 tiles,
// up to one wave of 256 workgroups.  The C ABI takes want from TG_SPLITK
// (default 1).
constexpr int kMaxSplitTiles = 4096;
int plan_async_splits(const GemmArgs &a, int cfg, int want);
// FP32 workspace the split kernel needs: splits x M x N x n_mat floats.
size_t async_ws_floats(const GemmArgs &a, int cfg, int splits);
// splits > 1 needs `ws` (async_ws_floats floats) and `counters` (one int per
// tile, zero before the launch; the kernel leaves them zero), and must equal
// plan_async_splits(a, cfg, splits).
hipError_t launch_async(int cfg, int dt, int act, const GemmArgs &a, int group_m, int splits,
                        float *ws, int *counters, hipStream_t stream);

// Stream-K over the 256 x 256 tiles of the 4-wave 16x16x32 kernel: a
// persistent grid of `grid` workgroups; logical tiles 0 .. dp_tiles - 1
// run whole (data-parallel), the last sk_tiles are split into 128-deep K
// quads (q per tile), `per` consecutive (tile, quad) units per workgroup.
// sk_tiles == 0: stream-K does not apply (the tiles fill whole waves, leave
// a last wave of at least half the compute units after whole ones, are
// fewer than half a wave, K is shorter than two quads or each workgroup's
// share shorter than 16, another configuration).
struct SkPlan {
    int dp_tiles, sk_tiles, q, per, grid;
};
// cus: workgroups that run at once (one per compute unit); any_size also
// splits shapes whose per-workgroup share of K is short (tests)
SkPlan plan_stream_k(const GemmArgs &a, int cfg, int cus, bool any_size);
// FP32 workspace: two 256 x 256 partial slots per workgroup; the counters
// (one int per stream-K tile, zero before the launch and after it) are
// separate.
size_t stream_k_ws_floats(const SkPlan &sk);
hipError_t launch_async_sk(int cfg, int dt, int act, const GemmArgs &a, int group_m,
                           const SkPlan &sk, float *ws, int *counters, hipStream_t stream);

// Block-scaled 8-bit GEMM: C = act(sum_k a(A[m][k]) 2^(SA[k/32][m]-127)
// * b(B[n][k]) 2^(SB[k/32][n]-127) + bias[n]).  A [M,K] and B [N,K] bytes
// (pitches in bytes), SA [K/32][M] and SB [K/32][N] e8m0 bytes, bias and C
// in the 16-bit output dtype.  fmt: 0 = e4m3, 1 = e5m2.
struct MxArgs {
    const unsigned char *A;
    int64_t lda;
    const unsigned char *SA;
    int64_t ldsa;
    const unsigned char *B;
    int64_t ldb;
    const unsigned char *SB;
    int64_t ldsb;
    const unsigned short *bias; // [N] or nullptr
    unsigned short *C;
    int64_t ldc;
    int M, N, K;
    int fmt_a, fmt_b;
};
// 256 x 256 tiles, 64-deep steps, 4 stages: M, N multiples of 256, K of 256,
// 16-byte aligned operands, byte pitches multiples of 16, ldc of 8.
bool mx_fast_eligible(const MxArgs &a);
hipError_t launch_mx(int dt, int act, const MxArgs &a, int group_m, hipStream_t stream);
hipError_t launch_mx_generic(int dt, int act, const MxArgs &a, hipStream_t stream);

// Fused forward attention: Q, K, V, O [BH][S][D] (BH = batch * heads),
// lse [BH][S] FP32 or nullptr; scale_log2 = softmax scale * log2(e).
struct AttnArgs {
    const unsigned short *Q, *K, *V;
    unsigned short *O;
    float *lse;
    int BH, S;
    float scale_log2;
};
// D = 128, S a multiple of 128, 16-byte aligned tensors
bool attn_fast_eligible(const AttnArgs &a, int D);
// Queries per workgroup of the fast kernel: 256 when S is a multiple of 256
// (unless want == 128), else 128.
int attn_block_m(const AttnArgs &a, int want);
hipError_t launch_attn(int dt, bool causal, int bm, const AttnArgs &a, hipStream_t stream);
hipError_t launch_attn_generic(int dt, bool causal, const AttnArgs &a, int D, hipStream_t stream);

// Zero-padded copy: dst[r][c] = src[r][c] inside src_rows x src_cols, else
// 0, for a dst_rows x dst_cols destination of pitch dst_cols (a multiple of
// 8, 16-byte aligned).  Used to round K up to the asynchronous kernels' loop.
hipError_t launch_pad_copy(const unsigned short *src, int64_t lds, int src_rows, int src_cols,
                           unsigned short *dst, int dst_rows, int dst_cols, hipStream_t stream);
// The way back: dst[r][c] = src[r][c] for r < rows, c < cols, from rows of
// src_pitch elements (a multiple of 8, 16-byte aligned, with 8 readable
// elements past the last row) into any 2-byte aligned dst of pitch ldd.
hipError_t launch_unpad_copy(const unsigned short *src, int src_pitch, unsigned short *dst,
                             int64_t ldd, int rows, int cols, hipStream_t stream);

// Small-M path (M <= 32): W streamed once, split over K.  `ws` is an FP32
// workspace of ws_floats floats and `counters` an int array of n_tiles
// entries that must be zero before the first call; the kernel leaves them
// zero.  M <= 16 has every kernel below; 16 < M <= 32 only the split-K
// streaming kernel (streaming = -1 when the shape does not fit it).
struct SkinnyPlan {
    int streaming; // 4: B [N,K] kernel, 3: realigning kernel, 2: column-tile kernel, 1: split-K streaming kernel, 0: register-staged kernel, -1: none
    int mb;       // 16-row blocks (1: M <= 16, 2: M <= 32)
    int bn;       // columns per workgroup
    int splits;   // K splits
    int k_chunk;  // K per split (multiple of the slab depth)
    int n_tiles;  // ceil(N / bn)
};
SkinnyPlan plan_skinny(int M, int N, int K);
// The realigning small-M kernel (streaming = 3): W at any 2-byte alignment
// and pitch, X 16-byte aligned with a pitch of 8 elements and readable (zero
// past K) up to K rounded up to 64 columns; Y, bias and R anywhere.
// want_splits > 0 asks for that many K splits (clamped to the K chunks).
SkinnyPlan plan_skinny_realign(int M, int N, int K, int want_splits = 0);
// The same kernel for B stored [N,K] (streaming = 4): W 16-byte aligned with
// a pitch of 8 elements, X as above; Y, bias and R anywhere.
SkinnyPlan plan_skinny_nk(int M, int N, int K, int want_splits = 0);
size_t skinny_ws_floats(const SkinnyPlan &pl, int M, int N);
hipError_t launch_skinny(int dt, int act, const GemmArgs &a, const SkinnyPlan &pl, float *ws,
                         int *counters, hipStream_t stream);

} // namespace tg
