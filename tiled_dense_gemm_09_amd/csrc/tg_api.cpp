// tg_api.cpp -- the C ABI (include/tg.h): argument validation, kernel and tile
// selection, launch on the caller's stream, diagnostics.
//
// Validation is synchronous and complete before anything is enqueued; an
// invalid call launches nothing ("TIRx", section 5.4: unsupported cases are
// rejected or take a registered fallback with a diagnostic; "Beyond
// Hand-Written CUDA", section 5: a silent fallback to a slow path is the
// failure mode to avoid -- here the chosen kernel is always reported).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <cmath>
#include <mutex>

#include "../../include/tg.h"
#include "tg_device.h"
#include "tg_launch.h"
#include "tg_pipeline.h"

namespace {

thread_local char g_last_kernel[96] = "none";

void set_last(const char *name, const char *detail = nullptr)
{
    if (detail)
        snprintf(g_last_kernel, sizeof g_last_kernel, "%s%s", name, detail);
    else
        snprintf(g_last_kernel, sizeof g_last_kernel, "%s", name);
    static const bool log = [] {
        const char *e = getenv("TG_LOG");
        return e && (e[0] == '1' || e[0] == '2');
    }();
    if (log)
        fprintf(stderr, "[tg] kernel: %s\n", g_last_kernel);
}

constexpr int64_t kMaxDim = (int64_t)1 << 31;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// x rounded up to a multiple of m (m > 0, x >= 0), or -1 when the result
// would not stay below 2^31 - 1024 (sizes padded for the kernels must fit
// their 32-bit index arithmetic)
int round_up_dim(int64_t x, int64_t m)
{
    const int64_t r = (x + m - 1) / m * m;
    return r < kMaxDim - 1024 ? (int)r : -1;
}

// Byte span [lo, hi) of a rows x cols matrix with pitch ld (16-bit elements).
struct Span {
    uintptr_t lo, hi;
};
Span span_of(const void *p, int64_t rows, int64_t cols, int64_t ld)
{
    Span s;
    s.lo = (uintptr_t)p;
    s.hi = rows > 0 && cols > 0 ? s.lo + (uintptr_t)(((rows - 1) * ld + cols) * 2) : s.lo;
    return s;
}
bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.lo < a.hi && b.lo < b.hi; }

// A rows x cols matrix with pitch ld (elements of `bytes` bytes) at p has an
// extent the span arithmetic can hold: non-negative sizes, ld >= cols, at
// most 2^56 elements from its first to its last one, and no wrap past the
// end of the address space.  Rejecting larger pitches keeps every later
// (rows - 1) * ld in range.
bool extent_ok(const void *p, int64_t rows, int64_t cols, int64_t ld, int64_t bytes)
{
    constexpr int64_t kMaxElems = (int64_t)1 << 56;
    if (rows < 0 || cols < 0 || ld < cols || cols > kMaxElems)
        return false;
    if (rows > 1 && ld > (kMaxElems - cols) / (rows - 1))
        return false;
    if (rows == 0 || cols == 0)
        return true;
    const uint64_t span = (uint64_t)((rows - 1) * ld + cols) * (uint64_t)bytes;
    return (uintptr_t)p <= UINTPTR_MAX - span;
}

// ---- per-device workspace of the split-K and K-padding paths -------------
struct Workspace {
    void *ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_ws_mutex;
Workspace g_ws[64];

// Layout of every workspace: [counters: 4096 ints][floats...]
constexpr size_t kCounterBytes = 4096 * sizeof(int);

// True when `stream` is being captured into a graph (or when the runtime
// cannot tell, which is treated the same way).
bool stream_capturing(hipStream_t stream)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return true;
    }
    return cs != hipStreamCaptureStatusNone;
}

// The library-managed workspace of at least float_count floats, or nullptr
// with *st set.  Growing it frees the old buffer after a device
// synchronisation and clears the new counters on `stream`; none of that may
// happen inside a stream capture, so a call that would grow it while
// `stream` is capturing gets TG_ERROR_NOT_SUPPORTED (and launches nothing).
void *get_workspace(size_t float_count, hipStream_t stream, tg_status *st)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        *st = TG_ERROR_NOT_SUPPORTED;
        return nullptr;
    }
    const size_t need = kCounterBytes + float_count * sizeof(float);
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace &w = g_ws[dev];
    if (w.bytes < need) {
        if (stream_capturing(stream)) {
            *st = TG_ERROR_NOT_SUPPORTED;
            return nullptr;
        }
        if (w.ptr) {
            // the old buffer may still be in use by queued work
            if (hipDeviceSynchronize() != hipSuccess || hipFree(w.ptr) != hipSuccess) {
                *st = TG_ERROR_LAUNCH_FAILED;
                return nullptr;
            }
            w.ptr = nullptr;
            w.bytes = 0;
        }
        size_t bytes = need < ((size_t)16 << 20) ? ((size_t)16 << 20) : need;
        void *p = nullptr;
        if (hipMalloc(&p, bytes) != hipSuccess) {
            (void)hipGetLastError();
            *st = TG_ERROR_OUT_OF_MEMORY;
            return nullptr;
        }
        if (hipMemsetAsync(p, 0, kCounterBytes, stream) != hipSuccess) {
            (void)hipFree(p);
            *st = TG_ERROR_LAUNCH_FAILED;
            return nullptr;
        }
        w.ptr = p;
        w.bytes = bytes;
    }
    return w.ptr;
}

// ---- fixed scratch of the allocation-free entry point -------------------
// One array per device that runs the library, held until the process ends:
// the split-K counters, then kScratchFloats FP32 partials.  Host code never
// uses the array's name as an address; it takes the device address that
// hipGetSymbolAddress reports for the current device, once per device.
constexpr size_t kScratchFloats = (size_t)4 << 20; // 16 MiB of partials
constexpr size_t kScratchBytes = kCounterBytes + kScratchFloats * sizeof(float);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void zero_words_kernel(unsigned int *p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = 0u;
}

std::mutex g_scratch_mutex;
void *g_scratch[64];

// Device address of this device's scratch, or nullptr with *st set.  The
// first call on a device looks the address up and clears the counters with
// a fill kernel on `stream` (the split kernels leave them at zero after
// every launch).
void *get_scratch(hipStream_t stream, tg_status *st)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        *st = TG_ERROR_NOT_SUPPORTED;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch[dev] == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            *st = TG_ERROR_NOT_SUPPORTED;
            return nullptr;
        }
        constexpr int words = (int)(kCounterBytes / sizeof(unsigned int));
        hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, stream,
                           static_cast<unsigned int *>(ptr), words);
        if (hipGetLastError() != hipSuccess) {
            *st = TG_ERROR_LAUNCH_FAILED;
            return nullptr;
        }
        g_scratch[dev] = ptr;
    }
    return g_scratch[dev];
}

// Compute units of the current device (workgroups of the persistent
// stream-K grid), looked up once per device; 256 if the runtime cannot say.
int device_cus()
{
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0) {
            (void)hipGetLastError();
            n = 256;
        }
        cached[dev] = n;
    }
    return cached[dev];
}

int env_int(const char *name, int dflt)
{
    const char *e = getenv(name);
    return e && *e ? atoi(e) : dflt;
}

// Tile configuration for a problem: the largest tile that still gives about
// one full wave of workgroups (256 CUs); otherwise the smallest tile.
int choose_config(int64_t M, int64_t N, int n_mat)
{
    const char *force = getenv("TG_FORCE_CONFIG");
    if (force && *force) {
        for (int i = 0; i < tg::num_tile_configs(); ++i)
            if (strcmp(force, tg::tile_config(i).name) == 0)
                return i;
    }
    const int n = tg::num_tile_configs();
    for (int i = 0; i < n; ++i) {
        const tg::TileConfig &c = tg::tile_config(i);
        const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn) * n_mat;
        if (tiles >= 240)
            return i;
    }
    return n - 1;
}

// Launch-time model of the asynchronous configurations, for grids short of a
// full wave of 256 x 256 tiles.  A configuration with s K splits runs
// n = ceil(tiles s / CUs) workgroups per CU, and keeps the fraction u =
// tiles s / (n CUs) of the CUs busy; it costs
//     a + b (K / s) (1 + r (n - 1)) (1 + g u)           [us, K in thousands]
// with a and b per B layout, plus, split, e + h (partial bytes s M N 8, in
// MB: written once, read once) + h2 (bytes s TM TN 4 of one tile's partials,
// in MB: the workgroup that completes a tile reads them all on its own), and
// never less than the compulsory HBM traffic (A, B and C once) at bw.  K
// counts the k a masked last quad pads.  Per workgroup the K loop is
// latency-bound: a 64 x 64 tile takes 3.0 us per thousand k against 5.5 for
// 128 x 128 (four times the work) and 4.7 for 128 x 128 in 64-deep steps,
// so the larger tile wins wherever it still fills the chip, and split-K buys
// back the waves that a small grid leaves idle; g, the cost of a full wave
// over an empty one, is the clock the board gives up under full load.  The
// coefficients are a least-squares fit (relative error) of 7361 launches
// timed back to back on MI355X: bf16, B in both layouts, 518 shapes (M
// 64..3072, also off the tile grid, over 20 (N, K) pairs from 1024 to
// 14336), every configuration with 1, 2, 4 and 8 splits; 7.4% rms error.
// Fitted on four fifths of the shapes, its choice lands within 0.5% of the
// fastest measured launch summed over those, 0.8% over the fifth held out.
struct WaveCost {
    int tm, tn;
    bool m16;
    int kb;
    double a_kn, b_kn, a_nk, b_nk, r, e;
};
constexpr WaveCost kWaveCost[] = {
    {64, 64, false, 32, 1.93, 3.00, 1.36, 3.19, 0.84, 1.92},
    {64, 128, false, 32, 2.16, 3.92, 1.18, 4.59, 0.96, 1.47},
    {128, 128, false, 32, 2.23, 5.54, 1.68, 6.09, 1.04, 1.00},
    {128, 128, true, 32, 3.86, 5.45, 3.50, 5.94, 1.11, 1.29},
    {128, 128, true, 64, 5.12, 4.66, 4.92, 4.42, 1.24, 0.86},
    {192, 192, true, 32, 6.96, 9.78, 6.62, 10.46, 1.08, 0.00},
    {256, 256, false, 32, 8.24, 14.35, 7.79, 14.52, 1.21, 0.00},
    {256, 256, true, 32, 8.69, 15.86, 7.78, 16.69, 1.00, 0.00},
};
constexpr double kSplitUsPerMB = 0.148;    // partial traffic of a split, all tiles
constexpr double kCombineUsPerMB = 11.29;  // one tile's partials, read by one workgroup
constexpr double kModelHbmBytesPerUs = 4.574e6;
constexpr double kFullWaveCost = 0.485;    // g: per-k cost of a full wave over an empty one

// Modelled microseconds of configuration cfg with s splits (plus a 1 %
// tie-break); < 0 when the configuration has no coefficients.
double wave_cost_us(const tg::GemmArgs &a, int cfg, int s, int cus)
{
    const int tm = tg::async_tile_m(cfg), tn = tg::async_tile_n(cfg);
    const bool m16 = tg::async_mfma16(cfg);
    const int kb = tg::async_k_step(cfg);
    for (const WaveCost &w : kWaveCost) {
        if (w.tm != tm || w.tn != tn || w.m16 != m16 || w.kb != kb)
            continue;
        const double tiles = (double)tg::async_tiles_m(a, cfg) * tg::async_tiles_n(a, cfg) * a.n_mat;
        const double n = std::ceil(tiles * s / cus);
        const double u = tiles * s / (n * cus);
        const int q = 4 * kb; // k of the loop's four steps: a masked last quad pads to it
        const double k = m16 ? (double)((a.K + q - 1) / q * q) : (double)a.K;
        const double wa = a.b_trans ? w.a_nk : w.a_kn, wb = a.b_trans ? w.b_nk : w.b_kn;
        double t = wa + wb * (k / s / 1000.0) * (1.0 + w.r * (n - 1.0)) * (1.0 + kFullWaveCost * u);
        if (s > 1)
            t += w.e + kSplitUsPerMB * s * (double)a.M * a.N * a.n_mat * 8.0 / 1e6 +
                 kCombineUsPerMB * s * (double)tm * tn * 4.0 / 1e6;
        const double bytes =
            2.0 * ((double)a.M * a.K + (double)a.n_mat * ((double)a.K * a.N + (double)a.M * a.N));
        // on the HBM floor the candidates tie: 1 % of the compute time
        // breaks the tie towards the least work (64 x 4096 x 14336, 119 MB:
        // four splits of 64 x 64 tiles, 25 us, not seven of half-empty
        // 128 x 128 tiles, 33 us)
        return std::max(t, bytes / kModelHbmBytesPerUs) + 0.01 * t;
    }
    return -1.0;
}

// Split count the model takes for configuration cfg (1 when no split is
// possible or none pays).  Only splits whose partials fit the fixed scratch
// are taken, so the allocation-free entry point makes the same choice.
int model_splits(const tg::GemmArgs &a, int cfg, int cus)
{
    int best_s = 1;
    double best_t = wave_cost_us(a, cfg, 1, cus);
    for (int s = 2; s <= 8 && best_t >= 0.0; ++s) {
        if (tg::plan_async_splits(a, cfg, s) != s || tg::async_ws_floats(a, cfg, s) > kScratchFloats)
            continue;
        const double t = wave_cost_us(a, cfg, s, cus);
        if (t >= 0.0 && t < best_t) {
            best_t = t;
            best_s = s;
        }
    }
    return best_s;
}

// Asynchronous-copy configuration for a problem, or -1: a forced name, else
// the 256 x 256 tiles on the 16x16x32 MFMA with about a full wave of
// workgroups (a whole one or more with a short last one is stream-K's,
// decided before); with fewer, the configuration and split count of least
// modelled time.  K off the 128 grid is masked on the 16x16x32 tiles only:
// there they need half a wave of tiles, else K padding or the tiled kernel
// does better.  splits (may be null: unsplit candidates only) receives the
// model's split count for the returned configuration (1 for a forced one:
// TG_SPLITK alone splits those).
int choose_async(const tg::GemmArgs &a, const char *force, int *splits = nullptr)
{
    const int n = tg::num_async_configs();
    const int cus = device_cus();
    if (splits)
        *splits = 1;
    if (force && strncmp(force, "async", 5) == 0) {
        // a forced configuration takes any padding of the last tiles (they
        // stay exact; the cost is the caller's choice)
        for (int i = 0; i < n; ++i)
            if (strcmp(force, tg::async_config_name(i)) == 0) {
                return tg::async_eligible(a, i, true) ? i : -1;
            }
        return -1;
    }
    auto tiles = [&](int i) {
        return (int64_t)tg::async_tiles_m(a, i) * tg::async_tiles_n(a, i) * a.n_mat;
    };
    for (int i = 0; i < n; ++i)
        if (!tg::async_forced_only(i) && tg::async_mfma16(i) && tg::async_tile_m(i) == 256 &&
            tg::async_eligible(a, i) && tiles(i) >= 240)
            return i;
    // Any padding of the last row or column tile is a candidate here: the
    // model counts the padded tiles (640 x 14336: 168 tiles of 256 x 256,
    // the last row half empty, against 560 of 128 x 128).
    // TG_LOG=2: every candidate's modelled time on stderr
    static const bool log_model = [] {
        const char *e = getenv("TG_LOG");
        return e && e[0] == '2';
    }();
    int best = -1, best_s = 1;
    double best_t = 0.0;
    for (int i = 0; i < n; ++i) {
        if (tg::async_forced_only(i) || tg::async_pairs(i) || !tg::async_eligible(a, i, true))
            continue;
        if (a.K % 128 != 0 && (!tg::async_mfma16(i) || 2 * tiles(i) < cus))
            continue;
        const int s = splits ? model_splits(a, i, cus) : 1;
        const double t = wave_cost_us(a, i, s, cus);
        if (log_model)
            fprintf(stderr, "[tg] model %lldx%lldx%lld: %s, %d split(s): %.1f us\n",
                    (long long)a.M, (long long)a.N, (long long)a.K, tg::async_config_name(i), s, t);
        if (t >= 0.0 && (best < 0 || t < best_t)) {
            best = i;
            best_s = s;
            best_t = t;
        }
    }
    if (splits)
        *splits = best_s;
    return best;
}

// A problem worth padding K to the asynchronous kernels' loop: one matrix,
// K not a multiple of 128, at least 2^30 multiply-adds, at most K / 8 added
// k (the padded multiply-adds are wasted work on top of the copies), no
// forced configuration, and the padded problem eligible for a configuration
// with a full wave of tiles.
bool kpad_eligible(const tg::GemmArgs &a, const char *force)
{
    const int K2 = round_up_dim(a.K, 128);
    if ((force && *force) || a.n_mat != 1 || a.K % 128 == 0 || a.K < 128 || K2 < 0 ||
        round_up_dim(a.N, 8) < 0 ||
        (double)a.M * a.N * a.K < (double)(1 << 30) || 8 * (K2 - a.K) > a.K)
        return false;
    tg::GemmArgs a2 = a;
    a2.K = K2;
    a2.lda = a2.K;
    a2.ldb = a.b_trans ? a2.K : round_up_dim(a.N, 8);
    if (choose_async(a2, nullptr) < 0)
        return false;
    for (int i = 0; i < tg::num_async_configs(); ++i)
        if (!tg::async_forced_only(i) && tg::async_eligible(a2, i) &&
            (int64_t)tg::async_tiles_m(a2, i) * tg::async_tiles_n(a2, i) >= 240)
            return true;
    return false;
}

// Operands off the 16-byte grid (a pitch that is not a multiple of 8
// elements, or a pointer that is only 2-byte aligned) on a problem of at
// least 2^30 multiply-adds: A and B are copied into aligned, zero-padded
// buffers (K rounded up to 8, or to 128 when no asynchronous configuration
// takes the former), the residual and the bias too when they are off the
// grid or N is not a multiple of 8, and the asynchronous kernel writes C
// itself when C is on the grid with N a multiple of 8, otherwise an aligned
// copy that is then moved into place.  The element counts are rounded up to
// 128 (256-byte aligned pieces); the staged output has 8 spare elements for
// the copy back, which reads whole 16-byte pieces.
struct StagePlan {
    int cfg = -1;                  // configuration on the staged problem; -1: not staged
    int K2 = 0, N8 = 0;            // staged K and N
    tg::SkPlan sk{0, 0, 0, 0, 0};  // stream-K plan on the staged problem (sk_tiles 0: none)
    bool c = false, r = false, bias = false; // output, residual, bias staged
    int64_t a_elems = 0, b_elems = 0, c_elems = 0, r_elems = 0, bias_elems = 0;
    int64_t total() const { return a_elems + b_elems + c_elems + r_elems + bias_elems; }
};

// cus > 0 and sk_mode != 0: stream-K is planned on the staged problem as on
// an aligned one (K then rounded up to 128, at most K / 8 added).
StagePlan plan_staging(const tg::GemmArgs &a, const char *force, int cus, int sk_mode)
{
    StagePlan sp;
    if ((force && *force) || a.n_mat != 1 || a.M <= 32 || a.K < 8 ||
        (double)a.M * a.N * a.K < (double)(1 << 30))
        return sp;
    const int N8 = round_up_dim(a.N, 8), K8 = round_up_dim(a.K, 8);
    const int K128 = round_up_dim(a.K, 128);
    if (N8 < 0 || K8 < 0 || K128 < 0)
        return sp;
    const bool c_ok = aligned16(a.C[0]) && a.ldc % 8 == 0 && N8 == a.N;
    const bool r_ok = a.R == nullptr || (aligned16(a.R) && a.ldr % 8 == 0 && c_ok);
    const bool bias_ok = a.bias == nullptr || (((uintptr_t)a.bias & 7u) == 0 && N8 == a.N);
    auto staged = [&](int K2) {
        tg::GemmArgs a2 = a;
        a2.K = K2;
        a2.lda = K2;
        a2.ldb = a.b_trans ? K2 : N8;
        a2.N = N8;
        // the staged residual and bias are aligned, the others passed the
        // checks above
        a2.bias = nullptr;
        a2.R = nullptr;
        a2.ldr = 0;
        return a2;
    };
    auto take = [&](int cfg, int K2) {
        auto round = [](int64_t e) { return (e + 127) / 128 * 128; };
        sp.cfg = cfg;
        sp.K2 = K2;
        sp.N8 = N8;
        sp.c = !c_ok;
        sp.r = !r_ok;
        sp.bias = !bias_ok;
        sp.a_elems = round((int64_t)a.M * K2);
        sp.b_elems = round((int64_t)N8 * K2);
        sp.c_elems = sp.c ? round((int64_t)a.M * N8 + 8) : 0;
        sp.r_elems = sp.r ? round((int64_t)a.M * N8) : 0;
        sp.bias_elems = sp.bias ? round(N8) : 0;
    };
    if (sk_mode != 0 && cus > 0 && 8 * (K128 - a.K) <= a.K) {
        const tg::GemmArgs a2 = staged(K128);
        for (int i = 0; i < tg::num_async_configs(); ++i) {
            if (tg::async_forced_only(i))
                continue;
            const tg::SkPlan sk = tg::plan_stream_k(a2, i, cus, sk_mode == 2);
            if (sk.sk_tiles > 0 && sk.sk_tiles <= tg::kMaxSplitTiles) {
                take(i, K128);
                sp.sk = sk;
                return sp;
            }
        }
    }
    for (const int K2 : {K8, K128}) {
        const int cfg = choose_async(staged(K2), nullptr);
        if (cfg >= 0) {
            take(cfg, K2);
            return sp;
        }
    }
    return sp;
}

// noalloc: the split paths take the fixed scratch (never the growable
// workspace) and nothing is padded or staged, so the call allocates nothing.
tg_status run(tg_dtype dt, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
              const void *const B[3], int64_t ldb, const void *bias, tg_act act, void *const C[3],
              int64_t ldc, int n_mat, void *stream, int b_trans = 0, const void *R = nullptr,
              int64_t ldr = 0, bool noalloc = false)
{
    if (dt != TG_DTYPE_F16 && dt != TG_DTYPE_BF16)
        return TG_ERROR_INVALID_VALUE;
    if (act != TG_ACT_NONE && act != TG_ACT_GELU_TANH)
        return TG_ERROR_INVALID_VALUE;
    if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
        return TG_ERROR_INVALID_VALUE;
    if (M == 0 || N == 0) {
        set_last("none");
        return TG_SUCCESS;
    }
    // B is [K,N] (pitch >= N), or stored [N,K] (pitch >= K) when b_trans
    const int64_t b_rows = b_trans ? N : K, b_cols = b_trans ? K : N;
    if (lda < K || ldb < b_cols || ldc < N)
        return TG_ERROR_INVALID_VALUE;
    if (R != nullptr && (ldr < N || ((uintptr_t)R & 1u) != 0))
        return TG_ERROR_INVALID_VALUE;
    if ((K > 0 && !extent_ok(A, M, K, lda, 2)) || !extent_ok(bias, 1, N, N, 2) ||
        (R != nullptr && !extent_ok(R, M, N, ldr, 2)))
        return TG_ERROR_INVALID_VALUE;
    for (int t = 0; t < n_mat; ++t)
        if ((K > 0 && !extent_ok(B[t], b_rows, b_cols, ldb, 2)) || !extent_ok(C[t], M, N, ldc, 2))
            return TG_ERROR_INVALID_VALUE;
    if (K > 0 && A == nullptr)
        return TG_ERROR_INVALID_VALUE;
    for (int t = 0; t < n_mat; ++t) {
        if (C[t] == nullptr || (K > 0 && B[t] == nullptr))
            return TG_ERROR_INVALID_VALUE;
    }
    // Outputs must not overlap any input or each other.
    for (int t = 0; t < n_mat; ++t) {
        const Span c = span_of(C[t], M, N, ldc);
        if (K > 0 && overlaps(c, span_of(A, M, K, lda)))
            return TG_ERROR_INVALID_VALUE;
        for (int u = 0; u < n_mat; ++u) {
            if (K > 0 && overlaps(c, span_of(B[u], b_rows, b_cols, ldb)))
                return TG_ERROR_INVALID_VALUE;
            if (u != t && overlaps(c, span_of(C[u], M, N, ldc)))
                return TG_ERROR_INVALID_VALUE;
        }
        if (bias && overlaps(c, span_of(bias, 1, N, N)))
            return TG_ERROR_INVALID_VALUE;
        // the residual may be C itself (each element is read before it is
        // overwritten, by the thread that overwrites it or after a wait on
        // that read), but not any other overlap
        if (R && !(R == C[t] && ldr == ldc) && overlaps(c, span_of(R, M, N, ldr)))
            return TG_ERROR_INVALID_VALUE;
    }
    if (((uintptr_t)bias & 1u) != 0)
        return TG_ERROR_INVALID_VALUE;

    tg::GemmArgs a;
    a.A = static_cast<const unsigned short *>(A);
    a.lda = lda;
    for (int t = 0; t < 3; ++t) {
        a.B[t] = static_cast<const unsigned short *>(B[t < n_mat ? t : 0]);
        a.C[t] = static_cast<unsigned short *>(C[t < n_mat ? t : 0]);
    }
    a.ldb = ldb;
    a.ldc = ldc;
    a.bias = static_cast<const unsigned short *>(bias);
    a.R = static_cast<const unsigned short *>(R);
    a.ldr = R ? ldr : 0;
    a.b_trans = b_trans;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.n_mat = n_mat;

    bool fast = (lda % 8 == 0) && (ldb % 8 == 0) && (ldc % 8 == 0) && (K == 0 || aligned16(A)) &&
                (R == nullptr || (aligned16(R) && ldr % 8 == 0));
    for (int t = 0; t < n_mat; ++t)
        fast = fast && aligned16(C[t]) && (K == 0 || aligned16(B[t]));

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int kdt = dt == TG_DTYPE_F16 ? tg::DT_F16 : tg::DT_BF16;
    const int kact = act == TG_ACT_GELU_TANH ? tg::ACT_GELU : tg::ACT_NONE;
    const char *force = getenv("TG_FORCE_CONFIG");
    const bool force_generic = force && strcmp(force, "generic") == 0;
    const bool force_tiled = force && strncmp(force, "tiled", 5) == 0;

    // An error left behind by an earlier, unrelated runtime call must not be
    // reported as this launch's failure.
    (void)hipGetLastError();
    hipError_t err;
    const bool trans_async = b_trans && fast && !force_generic && choose_async(a, force) >= 0;
    // Pitches or pointers off the 16-byte grid but every pointer 2-byte
    // aligned: the tiled MFMA kernel with element-wise loads and stores.
    bool even = ((uintptr_t)A & 1u) == 0;
    for (int t = 0; t < n_mat; ++t)
        even = even && ((uintptr_t)C[t] & 1u) == 0 && ((uintptr_t)B[t] & 1u) == 0;
    const bool unal_tiled = !fast && even && !b_trans && K > 0 && !force_generic;
    // Workspace of the split-K paths: the growable one, or the fixed scratch
    // for the allocation-free entry point.  On failure *st is set and
    // ws_note says why for tg_last_kernel().
    char ws_note[128] = "";
    auto split_workspace = [&](size_t float_count, tg_status *st) -> void * {
        if (noalloc) {
            if (float_count > kScratchFloats) {
                *st = TG_ERROR_NOT_SUPPORTED;
                snprintf(ws_note, sizeof ws_note,
                         " (not launched: needs %zu bytes of scratch, the fixed scratch holds %zu)",
                         kCounterBytes + float_count * sizeof(float), kScratchBytes);
                return nullptr;
            }
            void *p = get_scratch(s, st);
            if (!p)
                snprintf(ws_note, sizeof ws_note, " (not launched: no scratch on this device)");
            return p;
        }
        void *p = get_workspace(float_count, s, st);
        if (!p)
            snprintf(ws_note, sizeof ws_note, "%s",
                     *st == TG_ERROR_NOT_SUPPORTED
                         ? " (not launched: its workspace would grow during stream capture)"
                         : " (not launched: no workspace)");
        return p;
    };
    // K padding needs the workspace; when it cannot be had (a capture that
    // would grow it, no memory) the kernels that need none run instead
    bool kpad = !noalloc && fast && !force_generic && M > 32 && kpad_eligible(a, force);
    // (both sizes fit when kpad_eligible holds; -1 otherwise, then unused)
    const int kpad_k2 = round_up_dim(a.K, 128), kpad_n8 = round_up_dim(a.N, 8);
    const int64_t kpad_a_elems = (int64_t)a.M * kpad_k2;
    const int64_t kpad_b_elems = b_trans ? (int64_t)a.N * kpad_k2 : (int64_t)kpad_k2 * kpad_n8;
    void *kpad_base = nullptr;
    const char *kpad_note = nullptr;
    if (kpad) {
        tg_status st = TG_SUCCESS;
        kpad_base = get_workspace((size_t)((kpad_a_elems + kpad_b_elems) / 2 + 64), s, &st);
        if (!kpad_base) {
            kpad = false;
            kpad_note = st == TG_ERROR_NOT_SUPPORTED ? " (no K padding: stream capture)"
                                                     : " (no K padding: no workspace)";
        }
    }
    // Operands off the 16-byte grid: staged through aligned copies (above)
    // when the problem pays for the copies and the workspace can be had,
    // else the element-wise kernels below.
    StagePlan stg;
    void *stg_base = nullptr;
    const char *stg_note = nullptr;
    const int sk_mode = env_int("TG_STREAMK", 1);
    size_t stg_sk_floats = 0;
    if (!fast && even && !force_generic && !noalloc) {
        stg = plan_staging(a, force, device_cus(), sk_mode);
        if (stg.cfg >= 0) {
            // stream-K partial slots (after the counters), then the staged copies
            stg_sk_floats = stg.sk.sk_tiles > 0 ? tg::stream_k_ws_floats(stg.sk) : 0;
            tg_status st = TG_SUCCESS;
            stg_base = get_workspace(stg_sk_floats + (size_t)(stg.total() / 2 + 64), s, &st);
            if (!stg_base) {
                stg.cfg = -1;
                stg_note = st == TG_ERROR_NOT_SUPPORTED ? " (not staged: stream capture)"
                                                        : " (not staged: no workspace)";
            }
        }
    }
    // Stream-K: the 4-wave 256 x 256 configuration when its tiles leave a
    // partial last wave (unforced, or forced by name); TG_STREAMK=0 turns it
    // off, TG_STREAMK=2 also takes shapes whose K share per workgroup is
    // short.  It needs the workspace for its partial tiles; without one (a
    // capture that would grow it, no memory) the tiles run data-parallel.
    tg::SkPlan sk{0, 0, 0, 0, 0};
    int sk_cfg = -1;
    void *sk_base = nullptr;
    const char *sk_note = nullptr;
    if (fast && !noalloc && !force_generic && !force_tiled && sk_mode != 0 &&
        !(n_mat == 1 && M <= 32)) {
        for (int i = 0; i < tg::num_async_configs() && sk_cfg < 0; ++i) {
            if (tg::async_forced_only(i) ||
                (force && *force && strcmp(force, tg::async_config_name(i)) != 0))
                continue;
            sk = tg::plan_stream_k(a, i, device_cus(), sk_mode == 2);
            if (sk.sk_tiles > 0)
                sk_cfg = i;
        }
        if (sk_cfg >= 0) {
            tg_status st = TG_SUCCESS;
            static_assert(tg::kMaxSplitTiles * sizeof(int) <= kCounterBytes, "counter room");
            sk_base = sk.sk_tiles <= tg::kMaxSplitTiles
                          ? get_workspace(tg::stream_k_ws_floats(sk), s, &st)
                          : nullptr;
            if (!sk_base) {
                sk_note = st == TG_ERROR_NOT_SUPPORTED ? " (no stream-K: stream capture)"
                                                       : " (no stream-K: no workspace)";
                sk_cfg = -1;
            }
        }
    }
    // Small M (n_mat 1, M <= 32, N and K of at least 256; the bounds keep K
    // and its roundings inside int):
    //  - B [K,N] with W (or Y) off the 16-byte grid: the realigning streaming
    //    kernel, which reads W through aligned 16-byte pieces.  Aligned shapes
    //    that the split-K streaming kernel cannot take (N or K off its
    //    multiples) run on it as well: it measured faster than the
    //    register-staged kernel, which TG_SKINNY_REGS=1 selects (M <= 16).
    //  - B stored [N,K], 16-byte aligned with a pitch of 8 elements: the
    //    same kernel with whole K-contiguous rows of W copied to LDS.
    // X is copied into the workspace, zero-padded to a multiple of 64
    // columns, when it is off the grid or K is not a multiple of 64; the
    // split-K partials need the workspace too, and
    // without one the call runs unsplit (or, when X must be copied, on the
    // kernels below).
    const bool unforced = !(force && *force);
    const bool small_m = n_mat == 1 && M <= 32 && K >= 256 && K < kMaxDim - 1024 && N >= 256 &&
                         even;
    const bool force_realign = force && strcmp(force, "skinny_realign") == 0;
    const bool force_nk = force && strcmp(force, "skinny_nk") == 0;
    const bool nk = small_m && b_trans && aligned16(B[0]) && ldb % 8 == 0 &&
                    (force_nk || unforced);
    const bool realign = small_m && !b_trans &&
                         (force_realign || (unforced && !fast) ||
                          (unforced && fast && env_int("TG_SKINNY_REGS", 0) != 1 &&
                           tg::plan_skinny(a.M, a.N, a.K).streaming <= 0));
    bool small_run = nk || realign;
    tg::SkinnyPlan rpl{};
    float *r_ws = nullptr;
    int *r_counters = nullptr;
    unsigned short *r_x = nullptr;
    const int64_t r_kx = (K + 63) / 64 * 64; // columns of a copied X
    if (small_run) {
        rpl = nk ? tg::plan_skinny_nk(a.M, a.N, a.K) : tg::plan_skinny_realign(a.M, a.N, a.K);
        if (rpl.n_tiles > (int)(kCounterBytes / sizeof(int)))
            rpl.splits = 1;
        const bool x_ok = aligned16(A) && lda % 8 == 0 && K % 64 == 0;
        // floats: the partials (a multiple of 4, so X stays 16-byte aligned), then X
        const size_t p_floats =
            rpl.splits > 1 ? (tg::skinny_ws_floats(rpl, a.M, a.N) + 3) / 4 * 4 : 0;
        const size_t x_floats = x_ok ? 0 : (size_t)((M * r_kx + 1) / 2 + 4);
        void *base = nullptr;
        if (p_floats + x_floats > 0) {
            tg_status st = TG_SUCCESS;
            base = split_workspace(p_floats + x_floats, &st);
            if (!base && noalloc) {
                // the allocation-free call runs the same kernels as the
                // allocating one or nothing
                set_last(nk ? "skinny_nk" : "skinny_realign", ws_note);
                return st;
            }
            if (!base && x_ok && p_floats > 0) // unsplit: no workspace at all
                rpl.splits = 1;
        }
        if (rpl.splits == 1) // one K chunk in the kernel's granule
            rpl = nk ? tg::plan_skinny_nk(a.M, a.N, a.K, 1)
                     : tg::plan_skinny_realign(a.M, a.N, a.K, 1);
        if (!x_ok && !base) {
            small_run = false;
            if (!stg_note)
                stg_note = " (X not copied: no workspace)";
        } else if (base) {
            r_counters = static_cast<int *>(base);
            r_ws = reinterpret_cast<float *>(static_cast<char *>(base) + kCounterBytes);
            if (!x_ok)
                r_x = reinterpret_cast<unsigned short *>(r_ws + p_floats);
            if (rpl.splits == 1)
                r_ws = nullptr;
        }
    }
    if (small_run) {
        tg::GemmArgs a2 = a;
        err = hipSuccess;
        if (r_x) {
            err = tg::launch_pad_copy(a.A, a.lda, a.M, a.K, r_x, a.M, (int)r_kx, s);
            a2.A = r_x;
            a2.lda = r_kx;
        }
        if (err == hipSuccess)
            err = tg::launch_skinny(kdt, kact, a2, rpl, r_ws, r_counters, s);
        char detail[64];
        snprintf(detail, sizeof detail, "_%s_bn%d_split%dx%d%s%s", nk ? "nk" : "realign", rpl.bn,
                 rpl.splits, rpl.k_chunk, rpl.mb == 2 ? "_m32" : "", r_x ? "_xstaged" : "");
        set_last("skinny", detail);
    } else if (sk_cfg >= 0) {
        const int group_m = env_int("TG_GROUP_M", 4);
        err = tg::launch_async_sk(sk_cfg, kdt, kact, a, group_m > 0 ? group_m : 4, sk,
                                  reinterpret_cast<float *>(static_cast<char *>(sk_base) +
                                                            kCounterBytes),
                                  static_cast<int *>(sk_base), s);
        set_last(tg::async_config_name(sk_cfg), "_streamk");
    } else if (stg.cfg >= 0) {
        // staged copies in, the asynchronous kernel, the output copied out
        float *sk_slots = reinterpret_cast<float *>(static_cast<char *>(stg_base) + kCounterBytes);
        unsigned short *p = reinterpret_cast<unsigned short *>(sk_slots + stg_sk_floats);
        unsigned short *Ap = p, *Bp = p + stg.a_elems;
        p = Bp + stg.b_elems;
        unsigned short *Cp = stg.c ? p : nullptr;
        p += stg.c_elems;
        unsigned short *Rp = stg.r ? p : nullptr;
        p += stg.r_elems;
        unsigned short *biasp = stg.bias ? p : nullptr;
        const int K2 = stg.K2, N8 = stg.N8;
        err = tg::launch_pad_copy(a.A, a.lda, a.M, a.K, Ap, a.M, K2, s);
        if (err == hipSuccess)
            err = b_trans ? tg::launch_pad_copy(a.B[0], a.ldb, a.N, a.K, Bp, N8, K2, s)
                          : tg::launch_pad_copy(a.B[0], a.ldb, a.K, a.N, Bp, K2, N8, s);
        if (err == hipSuccess && Rp)
            err = tg::launch_pad_copy(a.R, a.ldr, a.M, a.N, Rp, a.M, N8, s);
        if (err == hipSuccess && biasp)
            err = tg::launch_pad_copy(a.bias, a.N, 1, a.N, biasp, 1, N8, s);
        tg::GemmArgs a2 = a;
        a2.A = Ap;
        a2.lda = K2;
        a2.B[0] = a2.B[1] = a2.B[2] = Bp;
        a2.ldb = b_trans ? K2 : N8;
        a2.K = K2;
        a2.N = N8;
        if (Cp) {
            a2.C[0] = a2.C[1] = a2.C[2] = Cp;
            a2.ldc = N8;
        }
        if (Rp) {
            a2.R = Rp;
            a2.ldr = N8;
        }
        if (biasp)
            a2.bias = biasp;
        if (err == hipSuccess) {
            const int group_m = env_int("TG_GROUP_M", 4);
            err = stg.sk.sk_tiles > 0
                      ? tg::launch_async_sk(stg.cfg, kdt, kact, a2, group_m > 0 ? group_m : 4,
                                            stg.sk, sk_slots, static_cast<int *>(stg_base), s)
                      : tg::launch_async(stg.cfg, kdt, kact, a2, group_m > 0 ? group_m : 4, 1,
                                         nullptr, nullptr, s);
        }
        if (err == hipSuccess && Cp)
            err = tg::launch_unpad_copy(Cp, N8, a.C[0], a.ldc, a.M, a.N, s);
        set_last(tg::async_config_name(stg.cfg), stg.sk.sk_tiles > 0 ? "_streamk_staged" : "_staged");
    } else if (unal_tiled) {
        const int cfg = choose_config(M, N, n_mat);
        const tg::TileConfig &c = tg::tile_config(cfg);
        const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn) * n_mat;
        if (tiles >= kMaxDim)
            return TG_ERROR_NOT_SUPPORTED;
        const int group_m = env_int("TG_GROUP_M", 4);
        err = tg::launch_tiled(cfg, kdt, kact, a, group_m > 0 ? group_m : 4, s);
        char detail[64];
        snprintf(detail, sizeof detail, "_unaligned%s", stg_note ? stg_note : "");
        set_last(c.name, detail);
    } else if (!fast || force_generic || (b_trans && !trans_async && !kpad)) {
        err = tg::launch_generic(kdt, kact, a, s);
        set_last(!fast            ? "generic_fma (unaligned operands)"
                 : force_generic ? "generic_fma (forced)"
                                 : "generic_fma (B stored [N,K] outside the async tile shapes)",
                 !fast ? stg_note : kpad_note);
    } else if (n_mat == 1 && M <= 32 && K >= 256 && N >= 256 && !force_tiled && !b_trans &&
               tg::plan_skinny(a.M, a.N, a.K).streaming >= 0) {
        // M <= 16 always; 16 < M <= 32 when the streaming kernel fits the shape
        const tg::SkinnyPlan pl = tg::plan_skinny(a.M, a.N, a.K);
        float *ws = nullptr;
        int *counters = nullptr;
        if (pl.splits > 1) {
            if (pl.n_tiles > (int)(kCounterBytes / sizeof(int)))
                return TG_ERROR_NOT_SUPPORTED;
            tg_status st = TG_SUCCESS;
            void *base = split_workspace(tg::skinny_ws_floats(pl, a.M, a.N), &st);
            if (!base) {
                set_last("skinny", ws_note);
                return st;
            }
            counters = static_cast<int *>(base);
            ws = reinterpret_cast<float *>(static_cast<char *>(base) + kCounterBytes);
        }
        err = tg::launch_skinny(kdt, kact, a, pl, ws, counters, s);
        char detail[48];
        snprintf(detail, sizeof detail, "%s_bn%d_split%dx%d%s",
                 pl.streaming == 2 ? "_cols" : (pl.streaming ? "_stream" : ""), pl.bn, pl.splits,
                 pl.k_chunk, pl.mb == 2 ? "_m32" : "");
        set_last("skinny", detail);
    } else if ((!force_tiled || b_trans) && choose_async(a, force) >= 0) {
        int auto_splits = 1;
        const int cfg = choose_async(a, force, &auto_splits);
        const int group_m = env_int("TG_GROUP_M", 4);
        // Split-K (the 32x32x16 tiles up to 128 x 128 and the 16x16x32 128 x
        // 128 ones): the count the launch-time model took with the
        // configuration (64 x 4096 x 4096: four splits of 64 x 64 tiles, 12.2
        // us against 20.0 unsplit).  TG_SPLITK=n asks
        // for n splits, 0 for enough to fill one wave, 1 for none.  A
        // modelled split whose workspace cannot be had (a capture that would
        // grow it, no memory) runs unsplit; a requested one, or one on the
        // allocation-free entry point, launches nothing and says why.
        const bool split_asked = getenv("TG_SPLITK") && *getenv("TG_SPLITK");
        const int want = split_asked ? env_int("TG_SPLITK", 1) : auto_splits;
        int splits = tg::plan_async_splits(a, cfg, want);
        float *ws = nullptr;
        int *counters = nullptr;
        const char *split_note = nullptr;
        if (splits > 1) {
            static_assert(tg::kMaxSplitTiles * sizeof(int) <= kCounterBytes, "counter room");
            tg_status st = TG_SUCCESS;
            void *base = split_workspace(tg::async_ws_floats(a, cfg, splits), &st);
            if (!base && (split_asked || noalloc)) {
                char name[64];
                snprintf(name, sizeof name, "%s_splitk%d", tg::async_config_name(cfg), splits);
                set_last(name, ws_note);
                return st;
            }
            if (base) {
                counters = static_cast<int *>(base);
                ws = reinterpret_cast<float *>(static_cast<char *>(base) + kCounterBytes);
            } else {
                splits = 1;
                split_note = st == TG_ERROR_NOT_SUPPORTED ? " (unsplit: stream capture)"
                                                          : " (unsplit: no workspace)";
            }
        }
        err = tg::launch_async(cfg, kdt, kact, a, group_m > 0 ? group_m : 4, splits, ws, counters,
                               s);
        char detail[64] = "";
        if (splits > 1)
            snprintf(detail, sizeof detail, "_splitk%d", splits);
        else if (split_note)
            snprintf(detail, sizeof detail, "%s", split_note);
        else if (sk_note)
            snprintf(detail, sizeof detail, "%s", sk_note);
        set_last(tg::async_config_name(cfg), detail);
    } else if (kpad) {
        // K off the 128 grid on a large problem: A and B copied with K
        // rounded up to 128 and zeros in the added entries, then the
        // asynchronous kernel (partial last tiles for M and N) writes C.
        tg::GemmArgs a2 = a;
        const int K2 = kpad_k2, N8 = kpad_n8;
        unsigned short *Ap = reinterpret_cast<unsigned short *>(static_cast<char *>(kpad_base) +
                                                                kCounterBytes);
        unsigned short *Bp = Ap + (kpad_a_elems + 127) / 128 * 128;
        err = tg::launch_pad_copy(a.A, a.lda, a.M, a.K, Ap, a.M, K2, s);
        if (err == hipSuccess)
            err = b_trans ? tg::launch_pad_copy(a.B[0], a.ldb, a.N, a.K, Bp, a.N, K2, s)
                          : tg::launch_pad_copy(a.B[0], a.ldb, a.K, a.N, Bp, K2, N8, s);
        a2.A = Ap;
        a2.lda = K2;
        a2.B[0] = a2.B[1] = a2.B[2] = Bp;
        a2.ldb = b_trans ? K2 : N8;
        a2.K = K2;
        const int cfg = choose_async(a2, nullptr);
        if (err == hipSuccess) {
            const int group_m = env_int("TG_GROUP_M", 4);
            err = tg::launch_async(cfg, kdt, kact, a2, group_m > 0 ? group_m : 4, 1, nullptr,
                                   nullptr, s);
        }
        set_last(tg::async_config_name(cfg), "_kpad");
    } else {
        const int cfg = choose_config(M, N, n_mat);
        const tg::TileConfig &c = tg::tile_config(cfg);
        const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn) * n_mat;
        if (tiles >= kMaxDim)
            return TG_ERROR_NOT_SUPPORTED;
        const int group_m = env_int("TG_GROUP_M", 4);
        err = tg::launch_tiled(cfg, kdt, kact, a, group_m > 0 ? group_m : 4, s);
        set_last(c.name, kpad_note);
    }
    if (err != hipSuccess) {
        char detail[64];
        snprintf(detail, sizeof detail, " (launch failed: %s)", hipGetErrorName(err));
        char name[96];
        snprintf(name, sizeof name, "%s", g_last_kernel);
        set_last(name, detail);
        return TG_ERROR_LAUNCH_FAILED;
    }
    return TG_SUCCESS;
}

} // namespace

extern "C" {

tg_status tg_gemm(tg_dtype dt, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                  const void *B, int64_t ldb, void *C, int64_t ldc, void *stream)
{
    const void *Bs[3] = {B, nullptr, nullptr};
    void *Cs[3] = {C, nullptr, nullptr};
    return run(dt, M, N, K, A, lda, Bs, ldb, nullptr, TG_ACT_NONE, Cs, ldc, 1, stream);
}

tg_status tg_gemm_bias_act(tg_dtype dt, int64_t M, int64_t N, int64_t K, const void *A,
                           int64_t lda, const void *B, int64_t ldb, const void *bias, tg_act act,
                           void *C, int64_t ldc, void *stream)
{
    const void *Bs[3] = {B, nullptr, nullptr};
    void *Cs[3] = {C, nullptr, nullptr};
    return run(dt, M, N, K, A, lda, Bs, ldb, bias, act, Cs, ldc, 1, stream);
}

tg_status tg_gemm_bias_act_noalloc(tg_dtype dt, int64_t M, int64_t N, int64_t K, const void *A,
                                   int64_t lda, const void *B, int64_t ldb, const void *bias,
                                   tg_act act, void *C, int64_t ldc, void *stream)
{
    const void *Bs[3] = {B, nullptr, nullptr};
    void *Cs[3] = {C, nullptr, nullptr};
    return run(dt, M, N, K, A, lda, Bs, ldb, bias, act, Cs, ldc, 1, stream, 0, nullptr, 0, true);
}

tg_status tg_gemm_ex(tg_dtype dt, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                     const void *B, int64_t ldb, tg_op op_b, const void *bias, tg_act act,
                     const void *R, int64_t ldr, void *C, int64_t ldc, void *stream)
{
    if (op_b != TG_OP_N && op_b != TG_OP_T)
        return TG_ERROR_INVALID_VALUE;
    const void *Bs[3] = {B, B, B};
    void *Cs[3] = {C, C, C};
    return run(dt, M, N, K, A, lda, Bs, ldb, bias, act, Cs, ldc, 1, stream, op_b == TG_OP_T ? 1 : 0,
               R, ldr);
}

tg_status tg_gemm_qkv(tg_dtype dt, int64_t M, int64_t N, int64_t K, const void *X, int64_t ldx,
                      const void *Wq, const void *Wk, const void *Wv, int64_t ldw, void *Q,
                      void *Kout, void *V, int64_t ldo, void *stream)
{
    const void *Bs[3] = {Wq, Wk, Wv};
    void *Cs[3] = {Q, Kout, V};
    return run(dt, M, N, K, X, ldx, Bs, ldw, nullptr, TG_ACT_NONE, Cs, ldo, 3, stream);
}

tg_status tg_gemm_mx(tg_fp8_format fmt_a, tg_fp8_format fmt_b, int64_t M, int64_t N, int64_t K,
                     const void *A, int64_t lda, const void *scale_a, int64_t ld_sa,
                     const void *B, int64_t ldb, const void *scale_b, int64_t ld_sb,
                     const void *bias, tg_act act, tg_dtype out_dt, void *C, int64_t ldc,
                     void *stream)
{
    if ((fmt_a != TG_FP8_E4M3 && fmt_a != TG_FP8_E5M2) ||
        (fmt_b != TG_FP8_E4M3 && fmt_b != TG_FP8_E5M2))
        return TG_ERROR_INVALID_VALUE;
    if (out_dt != TG_DTYPE_F16 && out_dt != TG_DTYPE_BF16)
        return TG_ERROR_INVALID_VALUE;
    if (act != TG_ACT_NONE && act != TG_ACT_GELU_TANH)
        return TG_ERROR_INVALID_VALUE;
    if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim || K % 32 != 0)
        return TG_ERROR_INVALID_VALUE;
    if (M == 0 || N == 0) {
        set_last("none");
        return TG_SUCCESS;
    }
    const int64_t KB = K / 32;
    if (ldc < N || (K > 0 && (lda < K || ldb < K || ld_sa < M || ld_sb < N)))
        return TG_ERROR_INVALID_VALUE;
    if (!extent_ok(C, M, N, ldc, 2) || !extent_ok(bias, 1, N, N, 2) ||
        (K > 0 && (!extent_ok(A, M, K, lda, 1) || !extent_ok(B, N, K, ldb, 1) ||
                   !extent_ok(scale_a, KB, M, ld_sa, 1) || !extent_ok(scale_b, KB, N, ld_sb, 1))))
        return TG_ERROR_INVALID_VALUE;
    if (C == nullptr || (K > 0 && (A == nullptr || B == nullptr || scale_a == nullptr ||
                                   scale_b == nullptr)))
        return TG_ERROR_INVALID_VALUE;
    if (((uintptr_t)bias & 1u) != 0 || ((uintptr_t)C & 1u) != 0)
        return TG_ERROR_INVALID_VALUE;
    // C must not overlap any input (byte spans; the 8-bit operands and the
    // scales are byte matrices, C and bias 16-bit)
    auto bytes = [](const void *p, int64_t rows, int64_t cols, int64_t ld) {
        Span sp;
        sp.lo = (uintptr_t)p;
        sp.hi = rows > 0 && cols > 0 ? sp.lo + (uintptr_t)((rows - 1) * ld + cols) : sp.lo;
        return sp;
    };
    const Span c = span_of(C, M, N, ldc);
    if (K > 0 && (overlaps(c, bytes(A, M, K, lda)) || overlaps(c, bytes(B, N, K, ldb)) ||
                  overlaps(c, bytes(scale_a, KB, M, ld_sa)) ||
                  overlaps(c, bytes(scale_b, KB, N, ld_sb))))
        return TG_ERROR_INVALID_VALUE;
    if (bias && overlaps(c, span_of(bias, 1, N, N)))
        return TG_ERROR_INVALID_VALUE;

    tg::MxArgs a;
    a.A = static_cast<const unsigned char *>(A);
    a.lda = lda;
    a.SA = static_cast<const unsigned char *>(scale_a);
    a.ldsa = ld_sa;
    a.B = static_cast<const unsigned char *>(B);
    a.ldb = ldb;
    a.SB = static_cast<const unsigned char *>(scale_b);
    a.ldsb = ld_sb;
    a.bias = static_cast<const unsigned short *>(bias);
    a.C = static_cast<unsigned short *>(C);
    a.ldc = ldc;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.fmt_a = fmt_a == TG_FP8_E5M2 ? 1 : 0;
    a.fmt_b = fmt_b == TG_FP8_E5M2 ? 1 : 0;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int kdt = out_dt == TG_DTYPE_F16 ? tg::DT_F16 : tg::DT_BF16;
    const int kact = act == TG_ACT_GELU_TANH ? tg::ACT_GELU : tg::ACT_NONE;
    const char *force = getenv("TG_FORCE_CONFIG");
    const bool force_generic = force && strcmp(force, "generic") == 0;
    (void)hipGetLastError();
    hipError_t err;
    if (tg::mx_fast_eligible(a) && !force_generic) {
        const int group_m = env_int("TG_GROUP_M", 4);
        err = tg::launch_mx(kdt, kact, a, group_m > 0 ? group_m : 4, s);
        set_last("mx_256x256x64_s4");
    } else {
        err = tg::launch_mx_generic(kdt, kact, a, s);
        set_last(force_generic ? "mx_generic (forced)" : "mx_generic (shape or alignment)");
    }
    if (err != hipSuccess) {
        char detail[64];
        snprintf(detail, sizeof detail, " (launch failed: %s)", hipGetErrorName(err));
        char name[96];
        snprintf(name, sizeof name, "%s", g_last_kernel);
        set_last(name, detail);
        return TG_ERROR_LAUNCH_FAILED;
    }
    return TG_SUCCESS;
}

tg_status tg_attention_fwd(tg_dtype dt, int64_t batch, int64_t heads, int64_t seq,
                           int64_t head_dim, const void *Q, const void *K, const void *V,
                           void *O, float *lse, float scale, int causal, void *stream)
{
    if (dt != TG_DTYPE_F16 && dt != TG_DTYPE_BF16)
        return TG_ERROR_INVALID_VALUE;
    if (batch < 0 || heads < 0 || seq < 0 || head_dim <= 0)
        return TG_ERROR_INVALID_VALUE;
    if (head_dim > 128)
        return TG_ERROR_NOT_SUPPORTED;
    if (batch >= kMaxDim || heads >= kMaxDim || seq >= kMaxDim)
        return TG_ERROR_INVALID_VALUE;
    const int64_t bh = batch * heads; // < 2^62
    if (bh >= kMaxDim || (seq > 0 && bh > (((int64_t)1 << 40) / head_dim) / seq))
        return TG_ERROR_INVALID_VALUE;
    if (bh == 0 || seq == 0) {
        set_last("none");
        return TG_SUCCESS;
    }
    if (!Q || !K || !V || !O)
        return TG_ERROR_INVALID_VALUE;
    if (((uintptr_t)lse & 3u) != 0 || ((uintptr_t)Q & 1u) || ((uintptr_t)K & 1u) ||
        ((uintptr_t)V & 1u) || ((uintptr_t)O & 1u))
        return TG_ERROR_INVALID_VALUE;
    const Span o = span_of(O, bh * seq, head_dim, head_dim);
    if (overlaps(o, span_of(Q, bh * seq, head_dim, head_dim)) ||
        overlaps(o, span_of(K, bh * seq, head_dim, head_dim)) ||
        overlaps(o, span_of(V, bh * seq, head_dim, head_dim)))
        return TG_ERROR_INVALID_VALUE;
    if (lse) {
        Span l;
        l.lo = (uintptr_t)lse;
        l.hi = l.lo + (uintptr_t)(bh * seq) * sizeof(float);
        if (overlaps(o, l))
            return TG_ERROR_INVALID_VALUE;
    }
    if (!(scale > 0.f))
        scale = 1.0f / sqrtf((float)head_dim);

    tg::AttnArgs a;
    a.Q = static_cast<const unsigned short *>(Q);
    a.K = static_cast<const unsigned short *>(K);
    a.V = static_cast<const unsigned short *>(V);
    a.O = static_cast<unsigned short *>(O);
    a.lse = lse;
    a.BH = (int)bh;
    a.S = (int)seq;
    a.scale_log2 = scale * 1.4426950408889634f;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int kdt = dt == TG_DTYPE_F16 ? tg::DT_F16 : tg::DT_BF16;
    const char *force = getenv("TG_FORCE_CONFIG");
    const bool force_generic = force && strcmp(force, "generic") == 0;
    (void)hipGetLastError();
    hipError_t err;
    if (!force_generic && tg::attn_fast_eligible(a, (int)head_dim) && a.S / 128 < 65536) {
        const int bm = tg::attn_block_m(a, env_int("TG_ATTN_BM", 0)); // override for sweeps
        err = tg::launch_attn(kdt, causal != 0, bm, a, s);
        set_last(bm == 256 ? (causal ? "attn_fwd_256x64_causal" : "attn_fwd_256x64")
                           : (causal ? "attn_fwd_128x64_causal" : "attn_fwd_128x64"));
    } else {
        err = tg::launch_attn_generic(kdt, causal != 0, a, (int)head_dim, s);
        set_last(force_generic ? "attn_generic (forced)" : "attn_generic (shape or alignment)");
    }
    if (err != hipSuccess) {
        char detail[64];
        snprintf(detail, sizeof detail, " (launch failed: %s)", hipGetErrorName(err));
        char name[96];
        snprintf(name, sizeof name, "%s", g_last_kernel);
        set_last(name, detail);
        return TG_ERROR_LAUNCH_FAILED;
    }
    return TG_SUCCESS;
}

const char *tg_status_string(tg_status s)
{
    switch (s) {
    case TG_SUCCESS: return "TG_SUCCESS";
    case TG_ERROR_INVALID_VALUE: return "TG_ERROR_INVALID_VALUE";
    case TG_ERROR_NOT_SUPPORTED: return "TG_ERROR_NOT_SUPPORTED";
    case TG_ERROR_LAUNCH_FAILED: return "TG_ERROR_LAUNCH_FAILED";
    case TG_ERROR_OUT_OF_MEMORY: return "TG_ERROR_OUT_OF_MEMORY";
    default: break;
    }
    return "TG_UNKNOWN_STATUS";
}

const char *tg_last_kernel(void) { return g_last_kernel; }

int64_t tg_workspace_bytes(void)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 0;
    }
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    return (int64_t)g_ws[dev].bytes;
}

int tg_schedule_tile(int64_t tiles_m, int64_t tiles_n, int64_t n_mat, int64_t group_m,
                     int64_t block_id, int64_t *mat, int64_t *tile_m, int64_t *tile_n)
{
    if (tiles_m <= 0 || tiles_n <= 0 || n_mat <= 0 || group_m <= 0 || tiles_m >= kMaxDim ||
        tiles_n >= kMaxDim || n_mat >= kMaxDim || group_m >= kMaxDim)
        return -1;
    const int64_t plane = tiles_m * tiles_n; // < 2^62
    if (plane > (kMaxDim - 1) / n_mat)
        return -1;
    const int64_t total = plane * n_mat;
    if (block_id < 0 || block_id >= total)
        return -1;
    const tg::TileCoord t = tg::schedule_tile((int)tiles_m, (int)tiles_n, (int)n_mat,
                                              (int)group_m, (int)block_id);
    *mat = t.mat;
    *tile_m = t.tm;
    *tile_n = t.tn;
    return 0;
}

int64_t tg_lds_offset(int64_t cols, int64_t row, int64_t col)
{
    if (cols < 0 || row < 0 || col < 0 || cols >= kMaxDim || row >= kMaxDim || col >= kMaxDim)
        return -1;
    return tg::lds_offset_bytes(cols, row, col);
}

int tg_lds_swizzle(int layout, int64_t row)
{
    if (row < 0)
        return -1;
    const int r = (int)(row & 0x7fffffff);
    switch (layout) {
    case 0:
        return tg::swz_a(r);
    case 1:
        return tg::swz_b<128>(r);
    case 2:
        return tg::swz_b<64>(r);
    case 3:
        return tg::swz_b16(r);
    case 4:
        return tg::swz_b192(r);
    case 5:
        return tg::swz_b128(r);
    case 6:
        return tg::swz_a8(r);
    default:
        return -1;
    }
}

int tg_in_bounds(int64_t rows, int64_t cols, int64_t row, int64_t col)
{
    return tg::in_bounds(rows, cols, row, col) ? 1 : 0;
}

} // extern "C"
