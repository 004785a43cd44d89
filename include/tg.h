/*
 * tg.h -- C ABI of the tiled dense GEMM library for AMD Instinct MI355X (gfx950).
 *
 *     C = epilogue(A . B),  f16 or bf16 inputs, FP32 accumulation.
 *
 * The operation is the tiled matrix product that the pages lower to a tile
 * loop: an A tile and a B tile are loaded, multiplied into an FP32 register
 * accumulator, and the loop marches over K ("TileIR", the matmul inner loop;
 * "Beyond Hand-Written CUDA: Inside TileLang's Multi-Backend Tile Compiler
 * Architecture", section 4, the FP16 GEMM kernel with A(M,K), B(K,N),
 * C(M,N) and a float32 fragment).  The epilogue (bias + activation) is
 * applied while the accumulator is still in registers ("TileIR", epilogue
 * fusion), and the QKV entry point is the horizontal fusion of three
 * projections that share one input ("TileIR", horizontal fusion).
 *
 * Conventions shared by every entry point:
 *
 *  - Layout: all matrices are row-major.  A is [M,K] with row pitch lda, B is
 *    [K,N] with pitch ldb, C is [M,N] with pitch ldc.  Pitches are counted in
 *    elements and must be >= the row length.  bias is a dense [N] vector.
 *  - dtype: one element type for A, B, C and bias (TG_DTYPE_F16 or
 *    TG_DTYPE_BF16).  Products accumulate in FP32; the epilogue runs in
 *    FP32; the result is rounded once, to nearest even, to the dtype.
 *  - Memory: every pointer is a device pointer owned by the caller.  The
 *    library keeps no pointer after the call returns.  C must not overlap A,
 *    B or bias.
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *    stream).  Work is enqueued asynchronously; the call does not
 *    synchronise.  Arguments are validated on the host before anything is
 *    enqueued: on an invalid argument nothing is launched and an error code
 *    is returned.
 *  - Shapes: M, N, K >= 0 and < 2^31.  M == 0 or N == 0 is a no-op that
 *    returns TG_SUCCESS.  K == 0 gives C = act(bias) (act(0) without bias).
 *    Bounds are logical: element (i, k) of A is read only if i < M and k < K,
 *    whatever lies in the padding between K and lda.
 *  - Fast path: 16-byte aligned pointers and pitches that are multiples of
 *    8 elements take the MFMA kernels.  Other 2-byte aligned operands (B
 *    stored [K,N]) take an MFMA kernel that loads and stores element by
 *    element; anything else runs a slower, correct scalar fallback.  The
 *    choice is never silent: tg_last_kernel()
 *    names the kernel and tile configuration the last call on this host
 *    thread launched (and TG_LOG=1 in the environment prints it; TG_LOG=2
 *    also prints the launch-time model's estimate for each candidate
 *    configuration of the asynchronous kernels).
 *  - Workspace: the split-K paths of tg_gemm, tg_gemm_bias_act, tg_gemm_ex
 *    and tg_gemm_qkv (small M, and square tiles that would leave most
 *    compute units idle; tg_last_kernel() then ends in "_split..." or
 *    "_splitk<n>") and the K-padding path (K not a multiple of 128 on large
 *    problems; "_kpad") use a per-device workspace that is allocated on
 *    first use and grown when a larger one is needed (the only allocation
 *    the library makes; tg_workspace_bytes() reports its size).  Growing it
 *    synchronizes the device, frees the old buffer and clears the new one's
 *    counters on the caller's stream, so:
 *      - a call that would grow it while its stream is being captured into
 *        a HIP graph does not grow it: a K split that the launch-time
 *        model chose for the square tiles, and the small-M kernel for
 *        operands off the grid or B stored [N,K], run unsplit instead; the
 *        K-padding path runs a kernel that needs no workspace (all
 *        reported by tg_last_kernel()); a split that TG_SPLITK asked for,
 *        and the small-M streaming kernel's, launch nothing and return
 *        TG_ERROR_NOT_SUPPORTED (tg_last_kernel() says why);
 *      - a graph that captured a call using the workspace must not be
 *        replayed after a later call grew it.
 *    Calls that use it are ordered by their streams; two such calls on
 *    different streams of one device must not overlap.
 *  - Thread safety: entry points may be called from several host threads
 *    (the workspace rule above still applies to calls that use it).
 */
#ifndef TG_H
#define TG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every enum below carries two reserved enumerators that give it the range
 * of a 32-bit int, so that any int value a C caller passes is a value of the
 * type (and an unknown one is rejected with TG_ERROR_INVALID_VALUE) instead
 * of a value outside the C++ type's range. */
typedef enum {
    TG_DTYPE_F16 = 1,
    TG_DTYPE_BF16 = 2,
    TG_DTYPE_RESERVED_MIN_ = -0x7fffffff - 1,
    TG_DTYPE_RESERVED_MAX_ = 0x7fffffff
} tg_dtype;

/* act(x): identity, or the tanh form of GELU
 *     0.5 x (1 + tanh(u)),  u = sqrt(2/pi) (x + 0.044715 x^3),
 * evaluated in FP32 as the same function x / (1 + exp(-2u)). */
typedef enum {
    TG_ACT_NONE = 0,
    TG_ACT_GELU_TANH = 1,
    TG_ACT_RESERVED_MIN_ = -0x7fffffff - 1,
    TG_ACT_RESERVED_MAX_ = 0x7fffffff
} tg_act;

typedef enum {
    TG_SUCCESS = 0,
    TG_ERROR_INVALID_VALUE = 1, /* NULL pointer, bad size, pitch, dtype or act, overlap */
    TG_ERROR_NOT_SUPPORTED = 2, /* no device / not gfx950 / workspace growth during capture */
    TG_ERROR_LAUNCH_FAILED = 3, /* the HIP runtime reported an error at launch */
    TG_ERROR_OUT_OF_MEMORY = 4, /* workspace allocation failed */
    TG_STATUS_RESERVED_MIN_ = -0x7fffffff - 1,
    TG_STATUS_RESERVED_MAX_ = 0x7fffffff
} tg_status;

/* C = A . B.
 * "TileLang" section 4 (the FP16 GEMM kernel); "TileIR" (the matmul loop). */
tg_status tg_gemm(tg_dtype dt, int64_t M, int64_t N, int64_t K,
                  const void *A, int64_t lda,
                  const void *B, int64_t ldb,
                  void *C, int64_t ldc,
                  void *stream);

/* C = act(A . B + bias), bias[n] added per output column (NULL = no bias),
 * then act, both in FP32 on the register accumulator.
 * "TileIR", epilogue fusion. */
tg_status tg_gemm_bias_act(tg_dtype dt, int64_t M, int64_t N, int64_t K,
                           const void *A, int64_t lda,
                           const void *B, int64_t ldb,
                           const void *bias, tg_act act,
                           void *C, int64_t ldc,
                           void *stream);

/* tg_gemm_bias_act for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, same kernels and bit-identical results; it
 * never allocates, frees or clears memory through the runtime:
 *  - the split-K paths (small M, and the square tiles' K splits, chosen by
 *    the launch-time model or by TG_SPLITK; the model takes only splits
 *    whose partials fit this scratch) keep their partials and
 *    counters in a fixed scratch array of the library, 16 MiB + 16 KiB per
 *    device, held until the process ends (set up by the first call on each
 *    device, which also launches one small kernel that zeroes the
 *    counters; every split kernel leaves them at zero again); the small-M
 *    kernel for operands off the 16-byte grid also keeps its zero-padded
 *    copy of A there when A is off the grid or K is not a multiple of 64;
 *  - a problem whose partials (and copy) need more than 16 MiB (4 Mi
 *    floats) returns TG_ERROR_NOT_SUPPORTED and launches nothing
 *    (tg_last_kernel() gives the size it needed);
 *  - K off the 128 grid is never padded into a workspace (the kernels that
 *    need none run instead).
 * Every call on a device shares that device's scratch and finds it as the
 * last call left it: two calls that overlap on one device (different
 * streams, or host threads without ordering) race on it. */
tg_status tg_gemm_bias_act_noalloc(tg_dtype dt, int64_t M, int64_t N, int64_t K,
                                   const void *A, int64_t lda,
                                   const void *B, int64_t ldb,
                                   const void *bias, tg_act act,
                                   void *C, int64_t ldc,
                                   void *stream);

/* Storage of the B operand of tg_gemm_ex. */
typedef enum {
    TG_OP_N = 0, /* B is [K,N] row-major, pitch ldb >= N (as in every other entry point) */
    TG_OP_T = 1, /* B is stored [N,K] row-major, pitch ldb >= K (one output feature per
                    row, the usual weight layout); the product uses its transpose */
    TG_OP_RESERVED_MIN_ = -0x7fffffff - 1,
    TG_OP_RESERVED_MAX_ = 0x7fffffff
} tg_op;

/* C = act(A . op(B) + bias) + R, one rounding at the end.
 *  - R: an [M,N] residual with row pitch ldr (NULL = none), added after the
 *    activation in FP32: "TileIR", vertical fusion (the next elementwise
 *    operation, here a residual add, chained onto the product instead of a
 *    second pass over C).  R may be C itself (same pointer and ldr == ldc),
 *    an in-place residual add; any other overlap of R with C is rejected.
 *    R must be 2-byte aligned; the MFMA kernels also need it 16-byte
 *    aligned with ldr a multiple of 8.
 *  - op(B): B, or the transpose of a B stored [N,K] -- one logical operand
 *    with its two axes permuted and its placement unchanged ("TIRx",
 *    section 5.1, permute).  TG_OP_T runs the MFMA kernel when M is a
 *    multiple of 64, N of 128 and K of 128 (with the fast-path alignment);
 *    any other TG_OP_T problem runs the fallback kernel, which
 *    tg_last_kernel() reports.
 *  - bias, act and the other arguments as in tg_gemm_bias_act; with
 *    op_b == TG_OP_N and R == NULL the result is bit-identical to it. */
tg_status tg_gemm_ex(tg_dtype dt, int64_t M, int64_t N, int64_t K,
                     const void *A, int64_t lda,
                     const void *B, int64_t ldb, tg_op op_b,
                     const void *bias, tg_act act,
                     const void *R, int64_t ldr,
                     void *C, int64_t ldc,
                     void *stream);

/* 8-bit float formats of tg_gemm_mx (OCP 8-bit floating point). */
typedef enum {
    TG_FP8_E4M3 = 0, /* 1 sign, 4 exponent (bias 7), 3 fraction bits; no infinities, max 448 */
    TG_FP8_E5M2 = 1, /* 1 sign, 5 exponent (bias 15), 2 fraction bits; IEEE-style specials */
    TG_FP8_RESERVED_MIN_ = -0x7fffffff - 1,
    TG_FP8_RESERVED_MAX_ = 0x7fffffff
} tg_fp8_format;

/* Block-scaled 8-bit GEMM:
 *   C[m][n] = act( sum_k a(A[m][k]) 2^(SA[k/32][m] - 127) * b(B[n][k]) 2^(SB[k/32][n] - 127)
 *                  + bias[n] ),
 * FP32 accumulation and epilogue, one rounding to out_dt.  "TIRx", section
 * 6: the FP8 GEMM with e8m0 block-wise scaling.  The pages fix neither the
 * block length nor the axes; here one e8m0 scale (an exponent byte, 2^(e-127),
 * 0xFF = NaN) covers 32 consecutive k of one row of A or one column of B,
 * the block of the OCP microscaling formats and of gfx950's scaled matrix
 * cores.  Coarser schemes (1x128, 128x128) are the same with repeated scales.
 *  - A: [M,K] bytes, row pitch lda >= K (bytes).  B: stored [N,K] (one output
 *    column per row, K-contiguous like A), pitch ldb >= K.
 *  - scale_a: [K/32][M] bytes, pitch ld_sa >= M: block-major, the M scales
 *    of one k-block contiguous (so that each k-step's scales are contiguous
 *    runs); scale_b: [K/32][N], pitch ld_sb >= N.
 *  - bias: [N] in out_dt or NULL; C: [M,N] in out_dt, pitch ldc >= N.
 *  - K must be a multiple of 32.  M, N multiples of 256 and K of 256 with
 *    16-byte aligned operands and scales, byte pitches multiples of 16 and
 *    ldc a multiple of 8 run the MFMA kernel; anything else runs a slower
 *    fallback kernel (reported by tg_last_kernel()).
 *  - Validation and asynchronous execution as for the other entry points; C
 *    must not overlap any input. */
tg_status tg_gemm_mx(tg_fp8_format fmt_a, tg_fp8_format fmt_b,
                     int64_t M, int64_t N, int64_t K,
                     const void *A, int64_t lda, const void *scale_a, int64_t ld_sa,
                     const void *B, int64_t ldb, const void *scale_b, int64_t ld_sb,
                     const void *bias, tg_act act, tg_dtype out_dt,
                     void *C, int64_t ldc,
                     void *stream);

/* Fused forward attention ("TileIR": Softmax(Q K^T / sqrt(d)) V in one
 * kernel with an online softmax, the score matrix never materialised;
 * "TIRx", section 6: forward multi-head attention, head dimension 128,
 * causal and non-causal):
 *     O[b][h][i] = sum_j softmax_j( scale * Q[b][h][i] . K[b][h][j] + mask ) V[b][h][j]
 * with mask = -inf for j > i when causal != 0.  Q, K, V, O are contiguous
 * [batch][heads][seq][head_dim] tensors of dtype dt; scores, softmax and
 * accumulation in FP32, one rounding of O.  scale <= 0 means 1/sqrt(head_dim).
 * lse, if not NULL, receives the FP32 [batch][heads][seq] natural-log
 * log-sum-exp of each row's scaled scores.  head_dim 128 with seq a
 * multiple of 128 and 16-byte aligned tensors runs the MFMA kernel;
 * head_dim <= 128 otherwise runs a slower fallback (reported by
 * tg_last_kernel()); head_dim > 128 is TG_ERROR_NOT_SUPPORTED.  O must not
 * overlap Q, K, V or lse. */
tg_status tg_attention_fwd(tg_dtype dt, int64_t batch, int64_t heads, int64_t seq,
                           int64_t head_dim, const void *Q, const void *K, const void *V,
                           void *O, float *lse, float scale, int causal, void *stream);

/* Horizontally fused projection, one launch:
 *     Q = X . Wq,  Kout = X . Wk,  V = X . Wv.
 * X is [M,K] (pitch ldx); Wq, Wk, Wv are each [K,N] (shared pitch ldw);
 * Q, Kout, V are each [M,N] (shared pitch ldo).  Each output is bit-identical
 * to tg_gemm on the same operands.  "TileIR", horizontal fusion (Q, K and V
 * projections share their input). */
tg_status tg_gemm_qkv(tg_dtype dt, int64_t M, int64_t N, int64_t K,
                      const void *X, int64_t ldx,
                      const void *Wq, const void *Wk, const void *Wv, int64_t ldw,
                      void *Q, void *Kout, void *V, int64_t ldo,
                      void *stream);

/* Human-readable name of a status code (static storage; an unknown value
 * gives "TG_UNKNOWN_STATUS").  The statuses are the diagnostic half of the
 * dispatch contract: an unsupported case is rejected with a reason or runs
 * a registered fallback, never silently ("TIRx", section 5.4). */
const char *tg_status_string(tg_status s);

/* Kernel and tile configuration chosen by the last entry-point call on the
 * calling host thread, e.g. "tiled_256x256x64_w2x2", with the reason
 * appended when the call fell back to a slower kernel or launched nothing;
 * "none" before any call or after a no-op.  Thread-local, static storage,
 * valid until the thread's next call.  It exists because a silent fallback
 * to a slow path is the failure mode that a user cannot see ("Beyond
 * Hand-Written CUDA: Inside TileLang's Multi-Backend Tile Compiler
 * Architecture", section 5). */
const char *tg_last_kernel(void);

/* Bytes of the library-managed workspace on the current device (0 before its
 * first use).  A caller that captures HIP graphs can make one eager call of
 * each shape first, so that the captured calls find the workspace large
 * enough. */
int64_t tg_workspace_bytes(void);

/* ---- host-side introspection (no GPU needed; for tests and tools) ---- */

/* The tile scheduler's map of a linear workgroup id to (matrix, tile_m,
 * tile_n) for a grid of tiles_m x tiles_n tiles per matrix and n_mat
 * matrices, as the kernels compute it.  Returns 0, or -1 if block_id is out
 * of range or the grid has 2^31 tiles or more.  The map is a bijection onto
 * the tile grid. */
int tg_schedule_tile(int64_t tiles_m, int64_t tiles_n, int64_t n_mat, int64_t group_m,
                     int64_t block_id, int64_t *mat, int64_t *tile_m, int64_t *tile_n);

/* Byte offset of element (row, col) in the kernels' LDS tile of `cols`
 * 16-bit elements per row (row pitch padded by 8 elements); -1 when an
 * argument is negative or >= 2^31. */
int64_t tg_lds_offset(int64_t cols, int64_t row, int64_t col);

/* Granule swizzle of the asynchronous kernels' LDS tiles: 16-byte granule c
 * of tile row `row` is stored at granule c ^ tg_lds_swizzle(layout, row).
 * layout 0: A (and B stored [N,K]), 64-byte rows of 32 k; 1: B stored
 * [K,N], rows of 128 or more columns (256 bytes or more); 2: B stored
 * [K,N], 64-column (128-byte) rows; 3: B stored [K,N] in the 256 x 256
 * kernel on the 16x16x32 MFMA (512-byte rows); 4: B stored [K,N] in the
 * 192 x 192 kernel on the 16x16x32 MFMA (384-byte rows); 5: B stored [K,N]
 * in the 128 x 128 kernel on the 16x16x32 MFMA (256-byte rows); 6: A (and
 * B stored [N,K]) in 64-deep K steps, 128-byte rows of 64 k.  Returns -1
 * for an unknown layout or a negative row. */
int tg_lds_swizzle(int layout, int64_t row);

/* Logical bounds predicate used for every global load and store: 1 if
 * (row, col) lies inside a rows x cols matrix, else 0 (never judged by the
 * linear offset). */
int tg_in_bounds(int64_t rows, int64_t cols, int64_t row, int64_t col);

#ifdef __cplusplus
}
#endif

#endif /* TG_H */
