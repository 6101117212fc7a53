// C-ABI entry points: argument validation, quick returns, kernel choice, launch.
// Validation and planning touch no HIP API, so every error below the device
// check is reported identically with or without a GPU.
#include "sgemm_f32.h"
#include "sgemm_internal.h"
#include "transpose_internal.h"
#include "probe_internal.h"

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <mutex>

namespace sgemm {
namespace {

// Row and column indices are formed in int32 inside the kernels, a tile past
// the last one included: dimensions stay 1024 below 2^31.
constexpr int64_t kMaxDim = ((int64_t)1 << 31) - 1025;
// A launch covers fewer than 2^32 work-items.
constexpr int64_t kMaxWorkItems = ((int64_t)1 << 32) - 1;
constexpr int kMaxDevices = 64;

struct Plan {
    int status = SGEMM_OK;
    int kid = KID_NONE;
    bool transB = false;
    bool vec = false;
    int64_t tiles_m = 0, tiles_n = 0;
};

// Bytes spanned by a rows x cols row-major matrix with leading dimension ld,
// or -1 if that does not fit comfortably in int64.
int64_t span_bytes(int64_t rows, int64_t cols, int64_t ld)
{
    if (rows <= 0 || cols <= 0)
        return 0;
    const int64_t lim = std::numeric_limits<int64_t>::max() / 8;
    if (ld > lim / rows)
        return -1;
    return ((rows - 1) * ld + cols) * (int64_t)sizeof(float);
}

bool overlaps(const void *p, int64_t pb, const void *q, int64_t qb)
{
    if (pb <= 0 || qb <= 0)
        return false;
    const uintptr_t p0 = reinterpret_cast<uintptr_t>(p), q0 = reinterpret_cast<uintptr_t>(q);
    return p0 < q0 + (uintptr_t)qb && q0 < p0 + (uintptr_t)pb;
}

bool aligned16(const void *p, int64_t ld) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0 && (ld & 3) == 0; }

// A float pointer must hold a float boundary: the MFMA kernels read 16 bytes
// at a time from any such address.
bool float_aligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

// MFMA tile from a wave-quantisation model.  Every tile has the 256 CUs as
// workgroup slots (the 256 x 256 and 128 x 128 tiles hold a CU each; 64 x 64
// workgroups share one up to 4 at a time and are dealt round-robin), so the
// busiest CU runs c = ceil(tiles / 256) of them and the grid runs at
// rate x (tiles / 256) / c, times the share of the tiles' area inside M x N
// (edge tiles compute their whole area).  Rates in TFLOP/s, measured on
// MI355X over square and rectangular shapes from 768 to 8192: 256 x 256 143,
// 128 x 128 136, 64 x 64 121 (97 with one workgroup per CU).  On the 24
// shapes measured it picked the fastest of the three tiles every time.  Ties
// go to the larger tile.
double mfma_rate(int kid, int64_t M, int64_t N)
{
    const TileShape t = tile_shape(kid);
    const double tiles = (double)(ceil_div(M, t.bm) * ceil_div(N, t.bn));
    const double c = std::ceil(tiles / 256.0);
    double r = 0.0;
    switch (kid) {
    case KID_MFMA_L: r = 143.0; break;
    case KID_MFMA_M: r = 136.0; break;
    default: r = c > 1.0 ? 121.0 : 97.0; break;
    }
    return r * (tiles / 256.0) / c * ((double)M * (double)N / (tiles * t.bm * t.bn));
}

// The FP32 MFMA kernels of the plain call.
bool is_mfma_f32(int kid)
{
    return kid == KID_MFMA_L || kid == KID_MFMA_M || kid == KID_MFMA_S || kid == KID_MFMA_S2 || kid == KID_MFMA_T ||
           kid == KID_MFMA_R;
}

constexpr int64_t kSmallGrid = 144;

int choose_mfma(int64_t M, int64_t N, int64_t K)
{
    const int kids[3] = {KID_MFMA_L, KID_MFMA_M, KID_MFMA_S};
    int best = KID_MFMA_L;
    double best_rate = -1.0;
    for (int kid : kids) {
        const TileShape t = tile_shape(kid);
        const int64_t threads = kid == KID_MFMA_S ? 256 : 512;
        if (ceil_div(M, t.bm) * ceil_div(N, t.bn) * threads > kMaxWorkItems)
            continue;  // grid too large for one launch
        const double r = mfma_rate(kid, M, N);
        if (r > best_rate) {
            best_rate = r;
            best = kid;
        }
    }
    // Within the 64 x 64 tile, the 8-wavefront variant (k split two ways in
    // the workgroup) measured 1.5-5% faster on MI355X except when the grid is
    // 257 to 512 tiles: the 4-wavefront workgroups then all run at once, two
    // per CU, where the 8-wavefront ones take a second, partial round (1280^3:
    // 97 against 90 TFLOP/s; 3584^3: 115 against 121); and with K below 256,
    // where each half has too few k-steps to pay for adding the halves (128^3:
    // 4.4 against 4.7 us).
    if (best == KID_MFMA_S) {
        const int64_t tiles = ceil_div(M, 64) * ceil_div(N, 64);
        if ((tiles <= 256 || tiles > 512) && K >= 256 && tiles * 512 <= kMaxWorkItems)
            best = KID_MFMA_S2;
        // Grids of 257 to 512 such tiles: the 128 x 64 tile (8 wavefronts, k
        // split two ways) gives one workgroup per CU with a quarter fewer
        // operand bytes per FLOP than two 64 x 64 workgroups, where it stays
        // within 256 tiles and pads at most 1/16 more rows.  Measured on MI355X:
        // 512 x 4096 x 4096 130.0 -> 133.6 TFLOP/s, 1024 x 2048 x 2048 126.2 ->
        // 129.0, 768 x 2048 x 4096 98.4 -> 101.0, 1280^3 96.6 -> 97.0.
        const int64_t rows_r = ceil_div(M, 128) * 128, rows_s = ceil_div(M, 64) * 64;
        if (tiles > 256 && tiles <= 512 && K >= 256 && ceil_div(M, 128) * ceil_div(N, 64) <= 256 &&
            rows_r * 16 <= rows_s * 17)
            best = KID_MFMA_R;
        // With at most kSmallGrid tiles of 64 x 64 the grid leaves most CUs
        // idle (or, above 128 tiles, gives a few of them a second round): the
        // 32 x 32 tile with k split four ways inside the workgroup gives each
        // CU one or two workgroups of a quarter of the work.  Measured on
        // MI355X: 512^3 11.2 -> 5.6 us, 128^3 4.4 -> 4.1 us, 768^3 15.8 ->
        // 15.2 us, 512 x 512 x 8192 138 -> 46 us; at 169 tiles (832^3) it is
        // 13% slower.
        if (tiles <= kSmallGrid)
            best = KID_MFMA_T;
    }
    return best;
}

// k-split geometry: k per split, a whole number of 32-wide k-tiles, and the
// number of non-empty splits that gives.
constexpr int64_t kSplitKTile = 32;
constexpr int64_t kMaxSplits = 64;
void split_geometry(int64_t K, int64_t splits, int64_t &kc, int64_t &used)
{
    kc = ceil_div(ceil_div(K, splits), kSplitKTile) * kSplitKTile;
    used = ceil_div(K, kc);
}

// Splits AUTO uses with a workspace (measured on MI355X): none while the
// 64 x 64 tile grid keeps at least half of the 256 CUs busy (splitting such
// grids unbalances them more than it gains).  Otherwise two workgroups per CU
// when each split still gets at least kSplitLongK of k (the second workgroup
// hides the first one's memory waits: 6-8% faster at 512 x 512 x 8192 and
// 256 x 256 x 32768), else the most splits that give one workgroup per CU and
// at least kSplitMinK of k each.  The partial pass always runs the 64 x 64
// tile, the fastest per split measured.
constexpr int64_t kSplitMinK = 128;
constexpr int64_t kSplitLongK = 1024;
constexpr int64_t kSplitMinTiles = 128;
constexpr int64_t kPlainSmallWorkgroups = 4;  // 32 x 32 workgroups per 64 x 64 tile
int64_t auto_splits(int64_t M, int64_t N, int64_t K)
{
    const TileShape t = tile_shape(KID_MFMA_S);
    const int64_t tiles = ceil_div(M, t.bm) * ceil_div(N, t.bn);
    if (tiles >= kSplitMinTiles)
        return 1;
    const int64_t s2 = 512 / tiles;
    if (s2 <= kMaxSplits && K / s2 >= kSplitLongK)
        return s2;
    int64_t s = 256 / tiles;
    s = s < K / kSplitMinK ? s : K / kSplitMinK;
    s = s < kMaxSplits ? s : kMaxSplits;
    // Such grids run the plain call on the 32 x 32 tile: four workgroups per
    // 64 x 64 tile, each with all of k.  Four splits or fewer add a reduction
    // for no more workgroups (512^3: 5.6 us plain against 9.5 us in 4 splits).
    return s > kPlainSmallWorkgroups ? s : 1;
}

int threads_per_block(int kid)
{
    return (kid == KID_MFMA_L || kid == KID_MFMA_M || kid == KID_MFMA_S2 || kid == KID_MFMA_R) ? 512
                                                                                              : 256;  // KID_MFMA_T: 256
}

Plan make_plan(int algo, int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
               const float *B, int64_t ldb, int transB, float beta, const float *C, int64_t ldc)
{
    Plan p;
    auto fail = [&](int s) {
        p.status = s;
        p.kid = KID_NONE;
        return p;
    };
    if (algo < SGEMM_ALGO_AUTO || algo > SGEMM_ALGO_MFMA_128X64)
        return fail(SGEMM_ERR_INVALID_VALUE);
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return fail(SGEMM_ERR_INVALID_VALUE);
    if (transB != 0 && transB != 1)
        return fail(SGEMM_ERR_INVALID_VALUE);
    p.transB = transB == 1;
    const int64_t b_rows = p.transB ? N : K, b_cols = p.transB ? K : N;
    if (lda < (K > 1 ? K : 1) || ldb < (b_cols > 1 ? b_cols : 1) || ldc < (N > 1 ? N : 1))
        return fail(SGEMM_ERR_INVALID_VALUE);
    const int64_t a_bytes = span_bytes(M, K, lda);
    const int64_t b_bytes = span_bytes(b_rows, b_cols, ldb);
    const int64_t c_bytes = span_bytes(M, N, ldc);
    if (a_bytes < 0 || b_bytes < 0 || c_bytes < 0)
        return fail(SGEMM_ERR_INVALID_VALUE);
    if (M == 0 || N == 0)
        return p;  // nothing to do
    if (C == nullptr || !float_aligned(C))
        return fail(SGEMM_ERR_INVALID_VALUE);
    const bool product = alpha != 0.0f && K > 0;
    if (!product) {
        if (beta == 1.0f)
            return p;  // C is already the result
        p.kid = KID_SCALE;
        p.tiles_m = M;
        p.tiles_n = ceil_div(N, 256);
        if (p.tiles_m * p.tiles_n * 256 > kMaxWorkItems)
            return fail(SGEMM_ERR_INVALID_VALUE);
        return p;
    }
    if (A == nullptr || B == nullptr || !float_aligned(A) || !float_aligned(B))
        return fail(SGEMM_ERR_INVALID_VALUE);
    if (overlaps(C, c_bytes, A, a_bytes) || overlaps(C, c_bytes, B, b_bytes))
        return fail(SGEMM_ERR_ALIAS);
    p.vec = aligned16(A, lda) && aligned16(B, ldb);
    switch (algo) {
    case SGEMM_ALGO_NAIVE: p.kid = KID_NAIVE; break;
    case SGEMM_ALGO_NAIVE_WG: p.kid = KID_NAIVE_WG; break;
    case SGEMM_ALGO_LDS_TILED: p.kid = KID_TILED_PAD; break;
    case SGEMM_ALGO_LDS_TILED_NOPAD: p.kid = KID_TILED_NOPAD; break;
    case SGEMM_ALGO_REGBLOCK: p.kid = KID_REGBLOCK; break;
    case SGEMM_ALGO_MFMA:
    case SGEMM_ALGO_AUTO: p.kid = choose_mfma(M, N, K); break;
    case SGEMM_ALGO_MFMA_256: p.kid = KID_MFMA_L; break;
    case SGEMM_ALGO_MFMA_128: p.kid = KID_MFMA_M; break;
    case SGEMM_ALGO_MFMA_64: p.kid = KID_MFMA_S; break;
    case SGEMM_ALGO_MFMA_32: p.kid = KID_MFMA_T; break;
    case SGEMM_ALGO_MFMA_128X64: p.kid = KID_MFMA_R; break;
    }
    const TileShape t = tile_shape(p.kid);
    p.tiles_m = ceil_div(M, t.bm);
    p.tiles_n = ceil_div(N, t.bn);
    // (the wavefront-per-output kernel loops over outputs with a capped grid)
    if (p.kid != KID_NAIVE_WG && p.tiles_m * p.tiles_n * threads_per_block(p.kid) > kMaxWorkItems)
        return fail(SGEMM_ERR_INVALID_VALUE);
    return p;
}

// AUTO sends matrices with fewer source rows (columns) than this to the
// element-per-work-item kernels.
constexpr int64_t kTransposeNarrow = 32;

struct TransposePlan {
    int status = SGEMM_OK;
    int kid = KID_NONE;
    bool vec = false;
    int64_t blocks = 0;
    int64_t rows = 0, cols = 0;
};

TransposePlan make_transpose_plan(int algo, int64_t rows, int64_t cols, const float *src, int64_t ld_src,
                                  const float *dst, int64_t ld_dst)
{
    TransposePlan p;
    p.rows = rows;
    p.cols = cols;
    auto fail = [&](int s) {
        p.status = s;
        p.kid = KID_NONE;
        p.blocks = 0;
        return p;
    };
    if (algo < SGEMM_TRANSPOSE_AUTO || algo > SGEMM_TRANSPOSE_NARROW)
        return fail(SGEMM_ERR_INVALID_VALUE);
    if (rows < 0 || cols < 0 || rows > kMaxDim || cols > kMaxDim)
        return fail(SGEMM_ERR_INVALID_VALUE);
    if (ld_src < (cols > 1 ? cols : 1) || ld_dst < (rows > 1 ? rows : 1))
        return fail(SGEMM_ERR_INVALID_VALUE);
    const int64_t src_bytes = span_bytes(rows, cols, ld_src);
    const int64_t dst_bytes = span_bytes(cols, rows, ld_dst);
    if (src_bytes < 0 || dst_bytes < 0)
        return fail(SGEMM_ERR_INVALID_VALUE);
    if (rows == 0 || cols == 0)
        return p;  // nothing to do
    if (src == nullptr || dst == nullptr)
        return fail(SGEMM_ERR_INVALID_VALUE);
    if (overlaps(dst, dst_bytes, src, src_bytes))
        return fail(SGEMM_ERR_ALIAS);
    switch (algo) {
    case SGEMM_TRANSPOSE_NAIVE: p.kid = KID_TRANSPOSE_NAIVE; break;
    case SGEMM_TRANSPOSE_LDS: p.kid = KID_TRANSPOSE_LDS_PAD; break;
    case SGEMM_TRANSPOSE_LDS_NOPAD: p.kid = KID_TRANSPOSE_LDS_NOPAD; break;
    case SGEMM_TRANSPOSE_NARROW: p.kid = KID_TRANSPOSE_NARROW; break;
    default:  // AUTO: tiles unless a 128-wide tile would run mostly empty
        p.kid = rows < kTransposeNarrow ? KID_TRANSPOSE_NAIVE
                : cols < kTransposeNarrow ? KID_TRANSPOSE_NARROW : KID_TRANSPOSE_LDS_PAD;
        break;
    }
    p.vec = aligned16(src, ld_src);
    if (transpose_tiles(p.kid, rows, cols) > (int64_t)UINT32_MAX)
        return fail(SGEMM_ERR_INVALID_VALUE);
    p.blocks = transpose_blocks(p.kid, rows, cols);
    return p;
}

const char *kernel_label(int kid)
{
    switch (kid) {
    case KID_NONE: return "none";
    case KID_SCALE: return "scale";
    case KID_NAIVE: return "naive";
    case KID_NAIVE_WG: return "naive_wave_per_output";
    case KID_TILED_PAD: return "lds_tiled_16x16_pad1";
    case KID_TILED_NOPAD: return "lds_tiled_16x16_pad0";
    case KID_REGBLOCK: return "regblock_128x128x8_t8x8";
    case KID_MFMA_L: return "mfma_256x256x32_w4x2";
    case KID_MFMA_M: return "mfma_128x128x32_w2x2_ks2";
    case KID_MFMA_S: return "mfma_64x64x32_w2x2";
    case KID_MFMA_S2: return "mfma_64x64x32_w2x2_ks2";
    case KID_MFMA_R: return "mfma_128x64x32_w4x1_ks2";
    case KID_MFMA_T: return "mfma_32x32x32_w1x1_ks4";
    case KID_MFMA_L_SK: return "mfma_256x256x32_w4x2_streamk";
    case KID_MFMA_M_SK: return "mfma_128x128x32_w2x2_ks2_streamk";
    case KID_MFMA_LP_F16: return "mfma_lp_f16_256x256x32_w4x2";
    case KID_MFMA_LP_BF16: return "mfma_lp_bf16_256x256x32_w4x2";
    case KID_MFMA_LP_F16_S: return "mfma_lp_f16_64x64x32_w2x1";
    case KID_MFMA_LP_BF16_S: return "mfma_lp_bf16_64x64x32_w2x1";
    case KID_LP16_F16: return "lp16_f16_256x256x32_w4x4_s4 (+ rounding pass)";
    case KID_LP16_BF16: return "lp16_bf16_256x256x32_w4x4_s4 (+ rounding pass)";
    case KID_LP16_F16_S: return "lp16_f16_128x128x32_w2x4_s4 up to K = 3072, else w2x2 (+ rounding pass)";
    case KID_LP16_BF16_S: return "lp16_bf16_128x128x32_w2x4_s4 up to K = 3072, else w2x2 (+ rounding pass)";
    case KID_TRANSPOSE_NAIVE: return "transpose_naive_64x16";
    case KID_TRANSPOSE_LDS_PAD: return "transpose_lds_128x128_pad1";
    case KID_TRANSPOSE_LDS_NOPAD: return "transpose_lds_128x128_pad0";
    case KID_TRANSPOSE_NARROW: return "transpose_narrow_64x16";
    default: return "unknown";
    }
}

// The code objects hold gfx950 code only.  `arch` is a device's
// architecture name as HIP reports it: the processor, optionally followed by
// target features after a ':' ("gfx950:sramecc+:xnack-").
int arch_status(const char *arch)
{
    if (arch == nullptr)
        return SGEMM_ERR_UNSUPPORTED_ARCH;
    const size_t n = std::strcspn(arch, ":");
    return (n == 6 && std::strncmp(arch, "gfx950", 6) == 0) ? SGEMM_OK : SGEMM_ERR_UNSUPPORTED_ARCH;
}

// SGEMM_F32_ALGO, read once per process, replaces the shape-based choice of
// the public AUTO entry points (sgemm_f32, and sgemm_f32_algo / _plan with
// SGEMM_ALGO_AUTO) by a fixed algorithm: a name of the sgemm_algo list in
// lower case without the prefix ("naive", "lds_tiled", "mfma_64", ...) or its
// number.  Unset or empty: no override.  Anything else: those calls return
// SGEMM_ERR_INVALID_VALUE, so a mistyped override fails loudly.  The calls
// with a workspace and the mixed-precision calls keep their own choices.
constexpr int kNoOverride = -1, kBadOverride = -2;

int parse_algo_override(const char *v)
{
    if (v == nullptr || *v == '\0')
        return kNoOverride;
    static const char *const names[] = {"auto",     "naive",    "lds_tiled", "regblock", "mfma",   "lds_tiled_nopad",
                                        "naive_wg", "mfma_256", "mfma_128",  "mfma_64",  "mfma_32", "mfma_128x64"};
    const int n = (int)(sizeof(names) / sizeof(names[0]));
    for (int i = 0; i < n; ++i)
        if (std::strcmp(v, names[i]) == 0)
            return i == SGEMM_ALGO_AUTO ? kNoOverride : i;
    char *end = nullptr;
    const long x = std::strtol(v, &end, 10);
    if (end != v && *end == '\0' && x >= 0 && x < n)
        return x == SGEMM_ALGO_AUTO ? kNoOverride : (int)x;
    return kBadOverride;
}

int auto_algo(int algo)
{
    if (algo != SGEMM_ALGO_AUTO)
        return algo;
    static const int over = parse_algo_override(std::getenv("SGEMM_F32_ALGO"));
    return over == kNoOverride ? SGEMM_ALGO_AUTO : over;  // kBadOverride fails validation
}

// 0 = unknown, 1 = gfx950, 2 = other architecture.
std::atomic<int> g_arch[kMaxDevices];

int check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return SGEMM_ERR_NO_DEVICE;
    if (dev >= kMaxDevices)
        return SGEMM_ERR_UNSUPPORTED_ARCH;
    int st = g_arch[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return SGEMM_ERR_NO_DEVICE;
        st = arch_status(prop.gcnArchName) == SGEMM_OK ? 1 : 2;
        g_arch[dev].store(st, std::memory_order_release);
    }
    return st == 1 ? SGEMM_OK : SGEMM_ERR_UNSUPPORTED_ARCH;
}

int run(int algo, int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
        const float *B, int64_t ldb, int transB, float beta, float *C, int64_t ldc, void *stream)
{
    const Plan p = make_plan(algo, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc);
    if (p.status != SGEMM_OK || p.kid == KID_NONE)
        return p.status;
    const int dev_status = check_device();
    if (dev_status != SGEMM_OK)
        return dev_status;
    GemmArgs a;
    a.A = A;
    a.B = B;
    a.C = C;
    a.lda = lda;
    a.ldb = ldb;
    a.ldc = ldc;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.alpha = alpha;
    a.beta = beta;
    const int64_t off_limit = ((int64_t)1 << 31) / 256;
    a.flags = (lda < off_limit && ldb < off_limit) ? GEMM_FLAG_DIRECT : 0;
    a.k_split = 0;
    a.c_split_stride = 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();  // report this launch's status, not an older one
    hipError_t e;
    switch (p.kid) {
    case KID_SCALE: e = launch_scale(a, s); break;
    case KID_NAIVE: e = launch_naive(a, p.transB, s); break;
    case KID_NAIVE_WG: e = launch_naive_wg(a, p.transB, s); break;
    case KID_TILED_PAD: e = launch_tiled(a, p.transB, true, s); break;
    case KID_TILED_NOPAD: e = launch_tiled(a, p.transB, false, s); break;
    case KID_REGBLOCK: e = launch_regblock(a, p.transB, p.vec, s); break;
    default: e = launch_mfma(a, p.kid, p.transB, s); break;
    }
    return e == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

// A workspace can hold `need` bytes and starts on a 16-byte boundary (the
// stream-K fix-up and the two-pass GEMM read it with 128-bit accesses; the
// k-split keeps the same rule).
bool ws_fits(const void *ws, int64_t ws_bytes, int64_t need)
{
    return ws != nullptr && ws_bytes >= need && (reinterpret_cast<uintptr_t>(ws) & 15) == 0;
}

struct SplitPlan {
    Plan base;            // the plain call's validation and plan
    int64_t splits = 1;   // splits that will run (1: the plain path)
    int64_t kc = 0;       // k per split
    int kid = KID_NONE;   // MFMA tile of the partial pass
    int64_t bytes = 0;    // workspace bytes the partial pass needs
};

// splits_req: 0 = AUTO, otherwise the requested count (clipped to non-empty
// splits).  With too small a workspace AUTO runs the plain path and an
// explicit request fails.
SplitPlan make_split_plan(int64_t splits_req, int64_t M, int64_t N, int64_t K, float alpha, const float *A,
                          int64_t lda, const float *B, int64_t ldb, int transB, float beta, const float *C,
                          int64_t ldc, const void *ws, int64_t ws_bytes, bool check_ws)
{
    SplitPlan sp;
    sp.base = make_plan(SGEMM_ALGO_AUTO, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc);
    auto fail = [&](int s) {
        sp.base.status = s;
        sp.base.kid = KID_NONE;
        sp.splits = 1;
        sp.kid = KID_NONE;
        sp.bytes = 0;
        return sp;
    };
    if (splits_req < 0 || splits_req > kMaxSplits || ws_bytes < 0)
        return fail(SGEMM_ERR_INVALID_VALUE);
    sp.kid = sp.base.kid;
    const bool mfma = is_mfma_f32(sp.base.kid);
    if (sp.base.status != SGEMM_OK || !mfma)
        return sp;  // errors, quick returns and the product-free cases are the plain call's
    const int64_t want = splits_req == 0 ? auto_splits(M, N, K) : splits_req;
    int64_t kc, used;
    split_geometry(K, want, kc, used);
    if (used <= 1)
        return sp;
    const int64_t bytes = used * M * N * (int64_t)sizeof(float);
    if (!check_ws) {  // query: report what a large enough workspace would get
        sp.splits = used;
        sp.kc = kc;
        sp.kid = KID_MFMA_S;
        sp.bytes = bytes;
        return sp;
    }
    if (!ws_fits(ws, ws_bytes, bytes)) {
        if (splits_req == 0)
            return sp;  // AUTO without room for the partials: the plain path
        return fail(SGEMM_ERR_INVALID_VALUE);
    }
    const int64_t a_bytes = span_bytes(M, K, lda);
    const int64_t b_bytes = span_bytes(sp.base.transB ? N : K, sp.base.transB ? K : N, ldb);
    const int64_t c_bytes = span_bytes(M, N, ldc);
    if (overlaps(ws, bytes, A, a_bytes) || overlaps(ws, bytes, B, b_bytes) || overlaps(ws, bytes, C, c_bytes))
        return fail(SGEMM_ERR_ALIAS);
    sp.splits = used;
    sp.kc = kc;
    sp.kid = KID_MFMA_S;
    sp.bytes = bytes;
    const TileShape t = tile_shape(sp.kid);
    if (ceil_div(M, t.bm) * ceil_div(N, t.bn) * used * threads_per_block(sp.kid) > kMaxWorkItems)
        return fail(SGEMM_ERR_INVALID_VALUE);
    return sp;
}

int run_split(int64_t splits_req, int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
              const float *B, int64_t ldb, int transB, float beta, float *C, int64_t ldc, void *ws,
              int64_t ws_bytes, void *stream)
{
    const SplitPlan sp = make_split_plan(splits_req, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, ws,
                                         ws_bytes, true);
    if (sp.base.status != SGEMM_OK)
        return sp.base.status;
    if (sp.splits <= 1)
        return run(SGEMM_ALGO_AUTO, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, stream);
    const int dev_status = check_device();
    if (dev_status != SGEMM_OK)
        return dev_status;
    float *W = static_cast<float *>(ws);
    GemmArgs a;
    a.A = A;
    a.B = B;
    a.C = W;
    a.lda = lda;
    a.ldb = ldb;
    a.ldc = N;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.alpha = 1.0f;
    a.beta = 0.0f;
    const int64_t off_limit = ((int64_t)1 << 31) / 256;
    a.flags = (lda < off_limit && ldb < off_limit) ? GEMM_FLAG_DIRECT : 0;
    a.k_split = (int)sp.kc;
    a.c_split_stride = M * N;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    hipError_t e = launch_mfma(a, sp.kid, sp.base.transB, s, (int)sp.splits);
    if (e != hipSuccess)
        return SGEMM_ERR_LAUNCH;
    const bool rvec = (N % 4) == 0 && aligned16(W, N) && aligned16(C, ldc);
    e = launch_splitk_reduce(W, (int)sp.splits, M * N, (int)M, (int)N, alpha, beta, C, ldc, rvec, s);
    return e == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

// ---- k-split on the library's static scratch --------------------------------

// For callers that cannot allocate: the k-split partials go to this array
// instead of a caller workspace.  Every GPU the library runs on holds its own
// copy, at its own address, until the process ends.  In host code the name
// stands for no device address: the kernels get the address that
// hipGetSymbolAddress returns on the device, cached per device below.
constexpr int64_t kScratchBytes = SGEMM_F32_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

std::mutex g_scratch_mu;
float *g_scratch[kMaxDevices];  // per-device address of `scratch`, guarded by g_scratch_mu

// Device address of `scratch` on the current device, looked up on the first
// call on that device (which must be current and checked).
int scratch_address(float **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return SGEMM_ERR_NO_DEVICE;
    if (dev >= kMaxDevices)
        return SGEMM_ERR_UNSUPPORTED_ARCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return SGEMM_ERR_LAUNCH;
        g_scratch[dev] = static_cast<float *>(p);
    }
    *out = g_scratch[dev];
    return SGEMM_OK;
}

int run_split_noalloc(int64_t splits_req, int64_t M, int64_t N, int64_t K, float alpha, const float *A,
                      int64_t lda, const float *B, int64_t ldb, int transB, float beta, float *C, int64_t ldc,
                      void *stream)
{
    const SplitPlan sp = make_split_plan(splits_req, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, nullptr,
                                         0, false);
    if (sp.base.status != SGEMM_OK)
        return sp.base.status;
    if (sp.splits <= 1)  // the plain call, which uses no scratch
        return run(SGEMM_ALGO_AUTO, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, stream);
    if (sp.bytes > kScratchBytes)
        return SGEMM_ERR_SCRATCH_LIMIT;
    const int dev_status = check_device();
    if (dev_status != SGEMM_OK)
        return dev_status;
    float *ws = nullptr;
    const int st = scratch_address(&ws);
    if (st != SGEMM_OK)
        return st;
    return run_split(splits_req, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, ws, kScratchBytes, stream);
}

// ---- stream-K -------------------------------------------------------------

constexpr int64_t kSkWorkers = 256;  // one stream-K workgroup per CU (both tiles hold a CU)

struct SkPlan {
    Plan base;             // the plain call's validation and plan
    int kid = KID_NONE;    // KID_MFMA_L_SK or KID_MFMA_M_SK; KID_NONE: the plain path runs
    int tile_kid = KID_NONE;
    SkArgs sk = {};
    int64_t bytes = 0;     // workspace: two slots per worker
};

// Schedule of the tile `kid` (KID_MFMA_L or KID_MFMA_M): the whole waves of
// tiles run data-parallel, the remaining tiles (all of them when there are
// fewer than 256) are shared out by k-iteration over up to 256 workers.
SkPlan sk_schedule(const Plan &base, int kid, int64_t M, int64_t N, int64_t K)
{
    SkPlan sp;
    sp.base = base;
    sp.tile_kid = kid;
    sp.kid = kid == KID_MFMA_L ? KID_MFMA_L_SK : KID_MFMA_M_SK;
    const TileShape t = tile_shape(kid);
    const int64_t tiles = ceil_div(M, t.bm) * ceil_div(N, t.bn);
    const int64_t iters = ceil_div(K, (int64_t)mfma_stage_k(kid));
    const int64_t rem = tiles % kSkWorkers;
    const int64_t dp = tiles - rem;
    const int64_t workers = rem == 0 ? 0 : (rem * iters < kSkWorkers ? rem * iters : kSkWorkers);
    sp.sk.ws = nullptr;
    sp.sk.dp = (int)dp;
    sp.sk.sk_tiles = (int)rem;
    sp.sk.workers = (int)workers;
    sp.sk.iters = (int)iters;
    sp.bytes = 2 * workers * t.bm * t.bn * (int64_t)sizeof(float);
    sp.base.tiles_m = ceil_div(M, t.bm);
    sp.base.tiles_n = ceil_div(N, t.bn);
    return sp;
}

// Modelled times in microseconds.  The plain call runs at its tile model's
// rate; the stream-K schedule keeps every CU busy at the tile's own rate on
// the padded tile area (143 TFLOP/s for 256 x 256, 133 for 128 x 128, as
// measured under stream-K on MI355X), plus the fix-up: 6 us of launch and
// tail, and every piece written and read back once at ~5 TB/s.  On the 24
// shapes of the tile sweep the choice this makes between the plain call and
// the two stream-K tiles came within 1.5% of the fastest every time.
double plain_time_us(int64_t M, int64_t N, int64_t K)
{
    int kid = choose_mfma(M, N, K);
    if (kid == KID_MFMA_R)
        kid = KID_MFMA_S;  // modelled as the 64 x 64 grid it replaces (it runs ~2% faster)
    return 2.0 * (double)M * (double)N * (double)K / (mfma_rate(kid, M, N) * 1e6);
}

double sk_time_us(const SkPlan &sp, int64_t K)
{
    const TileShape t = tile_shape(sp.tile_kid);
    const double tiles = (double)(sp.base.tiles_m * sp.base.tiles_n);
    const double rate = sp.tile_kid == KID_MFMA_L ? 143.0 : 133.0;
    const double compute = tiles * t.bm * t.bn * 2.0 * (double)K / (rate * 1e6);
    const double pieces = sp.sk.sk_tiles > 0 ? (double)(sp.sk.workers + sp.sk.sk_tiles) : 0.0;
    const double fix = pieces > 0 ? 6.0 + pieces * t.bm * t.bn * 4.0 * 2.0 / 5e6 : 0.0;
    return compute + fix;
}

// tile_req: 0 = the faster modelled tile, 256 or 128 = that tile.
SkPlan make_sk_plan(int tile_req, int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
                    const float *B, int64_t ldb, int transB, float beta, const float *C, int64_t ldc)
{
    const Plan base = make_plan(SGEMM_ALGO_AUTO, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc);
    SkPlan sp;
    sp.base = base;
    if (tile_req != 0 && tile_req != 256 && tile_req != 128) {
        sp.base.status = SGEMM_ERR_INVALID_VALUE;
        sp.base.kid = KID_NONE;
        return sp;
    }
    const bool mfma = is_mfma_f32(base.kid);
    if (base.status != SGEMM_OK || !mfma)
        return sp;  // errors, quick returns and the product-free cases are the plain call's
    if (tile_req == 256)
        sp = sk_schedule(base, KID_MFMA_L, M, N, K);
    else if (tile_req == 128)
        sp = sk_schedule(base, KID_MFMA_M, M, N, K);
    else {
        const SkPlan l = sk_schedule(base, KID_MFMA_L, M, N, K), m = sk_schedule(base, KID_MFMA_M, M, N, K);
        sp = sk_time_us(l, K) <= sk_time_us(m, K) ? l : m;
    }
    const int64_t blocks = (int64_t)sp.sk.dp + sp.sk.workers;
    if (blocks * threads_per_block(sp.tile_kid) > kMaxWorkItems || blocks == 0) {
        sp.base.status = SGEMM_ERR_INVALID_VALUE;
        sp.kid = KID_NONE;
        sp.base.kid = KID_NONE;
    }
    return sp;
}

// Workspace checks shared by the stream-K, k-split and two-pass calls.
int check_workspace(const void *ws, int64_t ws_bytes, int64_t need, int64_t M, int64_t N, int64_t K,
                    const float *A, int64_t lda, const float *B, int64_t ldb, int transB, const float *C,
                    int64_t ldc)
{
    if (!ws_fits(ws, ws_bytes, need))
        return SGEMM_ERR_INVALID_VALUE;
    const int64_t a_bytes = span_bytes(M, K, lda);
    const int64_t b_bytes = span_bytes(transB ? N : K, transB ? K : N, ldb);
    const int64_t c_bytes = span_bytes(M, N, ldc);
    if (overlaps(ws, need, A, a_bytes) || overlaps(ws, need, B, b_bytes) || overlaps(ws, need, C, c_bytes))
        return SGEMM_ERR_ALIAS;
    return SGEMM_OK;
}

int launch_sk_plan(const SkPlan &sp, int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
                   const float *B, int64_t ldb, float beta, float *C, int64_t ldc, void *ws, void *stream)
{
    const int dev_status = check_device();
    if (dev_status != SGEMM_OK)
        return dev_status;
    GemmArgs a;
    a.A = A;
    a.B = B;
    a.C = C;
    a.lda = lda;
    a.ldb = ldb;
    a.ldc = ldc;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.alpha = alpha;
    a.beta = beta;
    const int64_t off_limit = ((int64_t)1 << 31) / 256;
    a.flags = (lda < off_limit && ldb < off_limit) ? GEMM_FLAG_DIRECT : 0;
    a.k_split = 0;
    a.c_split_stride = 0;
    SkArgs sk = sp.sk;
    sk.ws = static_cast<float *>(ws);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const hipError_t e = launch_mfma_sk(a, sk, sp.tile_kid, sp.base.transB, s);
    return e == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

int run_sk(int tile_req, int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
           const float *B, int64_t ldb, int transB, float beta, float *C, int64_t ldc, void *ws, int64_t ws_bytes,
           void *stream)
{
    if (ws_bytes < 0)
        return SGEMM_ERR_INVALID_VALUE;
    const SkPlan sp = make_sk_plan(tile_req, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc);
    if (sp.base.status != SGEMM_OK)
        return sp.base.status;
    if (sp.kid == KID_NONE)
        return run(SGEMM_ALGO_AUTO, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, stream);
    const int ws_status = check_workspace(ws, ws_bytes, sp.bytes, M, N, K, A, lda, B, ldb, transB, C, ldc);
    if (ws_status != SGEMM_OK && sp.bytes > 0)
        return ws_status;
    return launch_sk_plan(sp, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, ws, stream);
}

// What sgemm_f32_ws does: the k-split when its rule splits; otherwise stream-K
// when the model puts it at least 1% ahead of the plain call; otherwise the
// plain call.  `method`: 0 plain, 1 k-split, 2 stream-K.
struct WsChoice {
    int method = 0;
    SplitPlan split;
    SkPlan sk;
};

WsChoice ws_auto(int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda, const float *B,
                 int64_t ldb, int transB, float beta, const float *C, int64_t ldc)
{
    WsChoice c;
    c.split = make_split_plan(0, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, nullptr, 0, false);
    if (c.split.base.status != SGEMM_OK)
        return c;
    if (c.split.splits > 1) {
        c.method = 1;
        return c;
    }
    // Grids that the plain call runs on the 32 x 32 tile are too small for the
    // stream-K schedule to pay for its fix-up.
    if (c.split.base.kid == KID_MFMA_T)
        return c;
    c.sk = make_sk_plan(0, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc);
    if (c.sk.base.status == SGEMM_OK && c.sk.kid != KID_NONE && c.sk.sk.sk_tiles > 0 &&
        sk_time_us(c.sk, K) < 0.99 * plain_time_us(M, N, K))
        c.method = 2;
    return c;
}

int run_ws_auto(int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda, const float *B,
                int64_t ldb, int transB, float beta, float *C, int64_t ldc, void *ws, int64_t ws_bytes, void *stream)
{
    if (ws_bytes < 0)
        return SGEMM_ERR_INVALID_VALUE;
    const WsChoice c = ws_auto(M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc);
    if (c.method == 2) {
        const int st = check_workspace(ws, ws_bytes, c.sk.bytes, M, N, K, A, lda, B, ldb, transB, C, ldc);
        if (st == SGEMM_ERR_ALIAS)
            return st;
        if (st == SGEMM_OK)
            return launch_sk_plan(c.sk, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, ws, stream);
        return run(SGEMM_ALGO_AUTO, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, stream);
    }
    return run_split(0, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, ws, ws_bytes, stream);
}

// Mixed precision: the FP32 call's validation and quick returns; the product
// runs the 16-bit MFMA kernel.
Plan make_lowp_plan(int precision, int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
                    const float *B, int64_t ldb, int transB, float beta, const float *C, int64_t ldc)
{
    if (precision != SGEMM_PREC_FP16 && precision != SGEMM_PREC_BF16) {
        Plan p;
        p.status = SGEMM_ERR_INVALID_VALUE;
        return p;
    }
    Plan p = make_plan(SGEMM_ALGO_AUTO, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc);
    if (p.status != SGEMM_OK || !is_mfma_f32(p.kid))
        return p;
    // the 256 x 256 tile once it keeps at least half of the 256 CUs busy, else 64 x 64
    const TileShape tl = lp_tile_shape(true);
    const bool large = ceil_div(M, tl.bm) * ceil_div(N, tl.bn) >= 128;
    const bool bf16 = precision == SGEMM_PREC_BF16;
    p.kid = large ? (bf16 ? KID_MFMA_LP_BF16 : KID_MFMA_LP_F16) : (bf16 ? KID_MFMA_LP_BF16_S : KID_MFMA_LP_F16_S);
    const TileShape t = lp_tile_shape(large);
    p.tiles_m = ceil_div(M, t.bm);
    p.tiles_n = ceil_div(N, t.bn);
    if (p.tiles_m * p.tiles_n * (large ? 512 : 128) > kMaxWorkItems) {
        p.status = SGEMM_ERR_INVALID_VALUE;
        p.kid = KID_NONE;
    }
    return p;
}

int run_lowp(int precision, int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
             const float *B, int64_t ldb, int transB, float beta, float *C, int64_t ldc, void *stream)
{
    const Plan p = make_lowp_plan(precision, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc);
    if (p.status != SGEMM_OK || p.kid == KID_NONE)
        return p.status;
    if (p.kid == KID_SCALE)  // no product: C <- beta*C, the same as the FP32 call
        return run(SGEMM_ALGO_AUTO, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, stream);
    const int dev_status = check_device();
    if (dev_status != SGEMM_OK)
        return dev_status;
    GemmArgs a;
    a.A = A;
    a.B = B;
    a.C = C;
    a.lda = lda;
    a.ldb = ldb;
    a.ldc = ldc;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.alpha = alpha;
    a.beta = beta;
    a.flags = 0;
    a.k_split = 0;
    a.c_split_stride = 0;
    (void)hipGetLastError();
    const bool large = p.kid == KID_MFMA_LP_F16 || p.kid == KID_MFMA_LP_BF16;
    const bool bf16 = p.kid == KID_MFMA_LP_BF16 || p.kid == KID_MFMA_LP_BF16_S;
    const hipError_t e = launch_mfma_lp(a, large, bf16, p.transB, p.vec, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

// Two-pass mixed precision with a caller workspace: the one-pass call's
// validation and quick returns; the two passes only where they measured
// faster, with 256 x 256 tiles when there are more than 128 of them, else
// 128 x 128.  `bytes` is what the workspace must hold.
struct Lp16Plan {
    Plan base;
    int kid = KID_NONE;  // KID_LP16_*; KID_NONE: the one-pass call runs
    bool large = false;
    int64_t bytes = 0;
};

// forced: always the two passes (tile_req 0 = the tile rule below, 256 or 128
// = that tile); otherwise only where they measured faster.
Lp16Plan make_lp16_plan(bool forced, int tile_req, int precision, int64_t M, int64_t N, int64_t K, float alpha,
                        const float *A, int64_t lda, const float *B, int64_t ldb, int transB, float beta,
                        const float *C, int64_t ldc)
{
    Lp16Plan lp;
    lp.base = make_lowp_plan(precision, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc);
    if (lp.base.status == SGEMM_OK && tile_req != 0 && tile_req != 256 && tile_req != 128) {
        lp.base.status = SGEMM_ERR_INVALID_VALUE;
        lp.base.kid = KID_NONE;
        return lp;
    }
    const Plan &p = lp.base;
    const bool product = p.kid == KID_MFMA_LP_F16 || p.kid == KID_MFMA_LP_BF16 || p.kid == KID_MFMA_LP_F16_S ||
                         p.kid == KID_MFMA_LP_BF16_S;
    if (p.status != SGEMM_OK || !product)
        return lp;
    // Measured on MI355X (bf16): the two passes beat the one-pass kernel from
    // ~1e10 FLOPs (2048^3: 392 against 348 TFLOP/s, 8192^3: 933 against 687)
    // and on smaller products with edge tiles or a k tail, which the rounding
    // pass pads away (1000 x 1017 x 999: 65 against 46); below, the pass costs
    // more than it saves (1024^3: 77 against 117).
    // From 4e9 FLOPs they also win where K >= min(M, N): the one-pass kernel's
    // small tile then runs long k-loops (measured with the current kernels:
    // 1024 x 1024 x 4096 79.3 against 51.5 us, 2048 x 1024 x 2048 43.5 against
    // 35.8, 1280^3 29.4 against 27.8), while shallow products stay faster in
    // one pass (2048 x 2048 x 1024 27.8 against 29.2, x 512 17.9 against 20.9).
    const double flops = 2.0 * (double)M * (double)N * (double)K;
    const bool ragged = (M % 64) != 0 || (N % 64) != 0 || (K % 32) != 0;
    const bool deep = flops >= 4e9 && K >= (M < N ? M : N);
    if (!forced && !(flops >= 1e10 || deep || (flops >= 1e9 && ragged)))
        return lp;
    const bool bf16 = precision == SGEMM_PREC_BF16;
    // 256 x 256 tiles once they keep more than half the CUs busy, else 128 x 128
    // (2560^3: 483 against 346 TFLOP/s; 3000^3: 478 against 458; with the
    // 16-wavefront 256 x 256 GEMM, 144 tiles (3072^3) 93.4 against 105.5 us,
    // but exactly 128 (4096 x 2048 x 2048) 67.2 against 57.6 us)
    const TileShape tl = lp16_tile_shape(true);
    lp.large = tile_req == 0 ? ceil_div(M, tl.bm) * ceil_div(N, tl.bn) > 128 : tile_req == 256;
    const TileShape t = lp16_tile_shape(lp.large);
    const int64_t tiles = ceil_div(M, t.bm) * ceil_div(N, t.bn);
    // the rounding transpose of op(B) = B launches ceil(K / 64) workgroup rows
    // (a grid's y extent is at most 65535)
    // (no layout of the two-pass GEMM launches more than 1024 work-items a workgroup)
    if (tiles * 1024 > kMaxWorkItems || ceil_div(K, 32) * 32 > std::numeric_limits<int>::max() ||
        ceil_div(K, 64) > 65535) {
        if (forced) {
            lp.base.status = SGEMM_ERR_INVALID_VALUE;
            lp.base.kid = KID_NONE;
        }
        return lp;  // the one-pass call handles (or rejects) it
    }
    lp.kid = lp.large ? (bf16 ? KID_LP16_BF16 : KID_LP16_F16) : (bf16 ? KID_LP16_BF16_S : KID_LP16_F16_S);
    lp.bytes = lp16_workspace_bytes(M, N, K, lp.large);
    lp.base.tiles_m = ceil_div(M, t.bm);
    lp.base.tiles_n = ceil_div(N, t.bn);
    return lp;
}

int run_lowp_ws(bool forced, int tile_req, int precision, int64_t M, int64_t N, int64_t K, float alpha,
                const float *A, int64_t lda, const float *B, int64_t ldb, int transB, float beta, float *C,
                int64_t ldc, void *ws, int64_t ws_bytes, void *stream)
{
    if (ws_bytes < 0)
        return SGEMM_ERR_INVALID_VALUE;
    const Lp16Plan lp =
        make_lp16_plan(forced, tile_req, precision, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc);
    if (lp.base.status != SGEMM_OK)
        return lp.base.status;
    if (lp.kid == KID_NONE)  // quick returns, product-free cases, or the one-pass call is faster
        return run_lowp(precision, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, stream);
    if (!ws_fits(ws, ws_bytes, lp.bytes)) {
        if (forced)
            return SGEMM_ERR_INVALID_VALUE;
        return run_lowp(precision, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, stream);
    }
    const int ws_status = check_workspace(ws, ws_bytes, lp.bytes, M, N, K, A, lda, B, ldb, transB, C, ldc);
    if (ws_status != SGEMM_OK)
        return ws_status;
    const int dev_status = check_device();
    if (dev_status != SGEMM_OK)
        return dev_status;
    GemmArgs a;
    a.A = A;
    a.B = B;
    a.C = C;
    a.lda = lda;
    a.ldb = ldb;
    a.ldc = ldc;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.alpha = alpha;
    a.beta = beta;
    a.flags = 0;
    a.k_split = 0;
    a.c_split_stride = 0;
    (void)hipGetLastError();
    const bool bf16 = precision == SGEMM_PREC_BF16;
    const hipError_t e = launch_lp16(a, lp.large, bf16, lp.base.transB, ws, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

int run_transpose(int algo, int64_t rows, int64_t cols, const float *src, int64_t ld_src, float *dst,
                  int64_t ld_dst, void *stream)
{
    const TransposePlan p = make_transpose_plan(algo, rows, cols, src, ld_src, dst, ld_dst);
    if (p.status != SGEMM_OK || p.kid == KID_NONE)
        return p.status;
    const int dev_status = check_device();
    if (dev_status != SGEMM_OK)
        return dev_status;
    TransposeArgs a;
    a.src = src;
    a.dst = dst;
    a.ld_src = ld_src;
    a.ld_dst = ld_dst;
    a.rows = (int)rows;
    a.cols = (int)cols;
    (void)hipGetLastError();
    const hipError_t e = launch_transpose(a, p.kid, p.vec, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

}  // namespace
}  // namespace sgemm

extern "C" {

int sgemm_f32(int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda, const float *B,
              int64_t ldb, int transB, float beta, float *C, int64_t ldc, void *stream)
{
    return sgemm::run(sgemm::auto_algo(SGEMM_ALGO_AUTO), M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc,
                      stream);
}

int sgemm_f32_algo(int algo, int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
                   const float *B, int64_t ldb, int transB, float beta, float *C, int64_t ldc, void *stream)
{
    return sgemm::run(sgemm::auto_algo(algo), M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, stream);
}

int sgemm_f32_plan(int algo, int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
                   const float *B, int64_t ldb, int transB, float beta, const float *C, int64_t ldc,
                   int *kernel_id, int64_t *tiles_m, int64_t *tiles_n, char *name, int name_len)
{
    const sgemm::Plan p = sgemm::make_plan(sgemm::auto_algo(algo), M, N, K, alpha, A, lda, B, ldb, transB, beta, C,
                                           ldc);
    if (kernel_id)
        *kernel_id = p.kid;
    if (tiles_m)
        *tiles_m = p.kid == sgemm::KID_NONE ? 0 : p.tiles_m;
    if (tiles_n)
        *tiles_n = p.kid == sgemm::KID_NONE ? 0 : p.tiles_n;
    if (name && name_len > 0) {
        std::snprintf(name, (size_t)name_len, "%s transB=%d vec=%d", sgemm::kernel_label(p.kid),
                      p.transB ? 1 : 0, p.vec ? 1 : 0);
    }
    return p.status;
}

int sgemm_f32_splitk_plan(int64_t splits, int64_t M, int64_t N, int64_t K, int transB, int64_t *splits_used,
                          int *kernel_id, int64_t *workspace_bytes)
{
    // Shape-only query: fake, well-separated operands with minimal leading
    // dimensions stand in for the caller's.
    const float *A = reinterpret_cast<const float *>((uintptr_t)1 << 40);
    const float *B = reinterpret_cast<const float *>((uintptr_t)1 << 50);
    const float *C = reinterpret_cast<const float *>((uintptr_t)1 << 58);
    const int64_t lda = K > 1 ? K : 1, ldc = N > 1 ? N : 1;
    const int64_t ldb = transB == 1 ? lda : ldc;
    const sgemm::SplitPlan sp = sgemm::make_split_plan(splits, M, N, K, 1.0f, A, lda, B, ldb, transB, 0.0f, C, ldc,
                                                       nullptr, 0, false);
    if (splits_used)
        *splits_used = sp.base.status == SGEMM_OK ? sp.splits : 0;
    if (kernel_id)
        *kernel_id = sp.kid;
    if (workspace_bytes)
        *workspace_bytes = sp.bytes;
    return sp.base.status;
}

int sgemm_f32_splitk_noalloc(int64_t splits, int64_t M, int64_t N, int64_t K, float alpha, const float *A,
                             int64_t lda, const float *B, int64_t ldb, int transB, float beta, float *C,
                             int64_t ldc, void *stream)
{
    return sgemm::run_split_noalloc(splits, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, stream);
}

int sgemm_f32_ws(int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda, const float *B,
                 int64_t ldb, int transB, float beta, float *C, int64_t ldc, void *workspace,
                 int64_t workspace_bytes, void *stream)
{
    return sgemm::run_ws_auto(M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, workspace, workspace_bytes,
                              stream);
}

int sgemm_f32_ws_plan(int64_t M, int64_t N, int64_t K, int transB, int *method, int *kernel_id,
                      int64_t *workspace_bytes)
{
    const float *A = reinterpret_cast<const float *>((uintptr_t)1 << 40);
    const float *B = reinterpret_cast<const float *>((uintptr_t)1 << 50);
    const float *C = reinterpret_cast<const float *>((uintptr_t)1 << 58);
    const int64_t lda = K > 1 ? K : 1, ldc = N > 1 ? N : 1;
    const int64_t ldb = transB == 1 ? lda : ldc;
    const sgemm::WsChoice c = sgemm::ws_auto(M, N, K, 1.0f, A, lda, B, ldb, transB, 0.0f, C, ldc);
    const int st = c.split.base.status;
    if (method)
        *method = st == SGEMM_OK ? c.method : 0;
    if (kernel_id)
        *kernel_id = c.method == 2 ? c.sk.kid : c.split.kid;
    if (workspace_bytes)
        *workspace_bytes = c.method == 2 ? c.sk.bytes : (c.method == 1 ? c.split.bytes : 0);
    return st;
}

int sgemm_f32_lowp_ws(int precision, int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
                      const float *B, int64_t ldb, int transB, float beta, float *C, int64_t ldc, void *workspace,
                      int64_t workspace_bytes, void *stream)
{
    return sgemm::run_lowp_ws(false, 0, precision, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, workspace,
                              workspace_bytes, stream);
}

int sgemm_f32_lowp_2pass(int precision, int tile, int64_t M, int64_t N, int64_t K, float alpha, const float *A,
                         int64_t lda, const float *B, int64_t ldb, int transB, float beta, float *C, int64_t ldc,
                         void *workspace, int64_t workspace_bytes, void *stream)
{
    return sgemm::run_lowp_ws(true, tile, precision, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, workspace,
                              workspace_bytes, stream);
}

static int lowp_ws_plan(bool forced, int tile, int precision, int64_t M, int64_t N, int64_t K, int transB,
                        int *kernel_id, int64_t *tiles_m, int64_t *tiles_n, int64_t *workspace_bytes)
{
    const float *A = reinterpret_cast<const float *>((uintptr_t)1 << 40);
    const float *B = reinterpret_cast<const float *>((uintptr_t)1 << 50);
    const float *C = reinterpret_cast<const float *>((uintptr_t)1 << 58);
    const int64_t lda = K > 1 ? K : 1, ldc = N > 1 ? N : 1;
    const int64_t ldb = transB == 1 ? lda : ldc;
    const sgemm::Lp16Plan lp =
        sgemm::make_lp16_plan(forced, tile, precision, M, N, K, 1.0f, A, lda, B, ldb, transB, 0.0f, C, ldc);
    const bool two = lp.base.status == SGEMM_OK && lp.kid != sgemm::KID_NONE;
    if (kernel_id)
        *kernel_id = two ? lp.kid : lp.base.kid;
    if (tiles_m)
        *tiles_m = lp.base.kid == sgemm::KID_NONE ? 0 : lp.base.tiles_m;
    if (tiles_n)
        *tiles_n = lp.base.kid == sgemm::KID_NONE ? 0 : lp.base.tiles_n;
    if (workspace_bytes)
        *workspace_bytes = two ? lp.bytes : 0;
    return lp.base.status;
}

int sgemm_f32_lowp_ws_plan(int precision, int64_t M, int64_t N, int64_t K, int transB, int *kernel_id,
                           int64_t *tiles_m, int64_t *tiles_n, int64_t *workspace_bytes)
{
    return lowp_ws_plan(false, 0, precision, M, N, K, transB, kernel_id, tiles_m, tiles_n, workspace_bytes);
}

int sgemm_f32_lowp_2pass_plan(int precision, int tile, int64_t M, int64_t N, int64_t K, int transB, int *kernel_id,
                              int64_t *tiles_m, int64_t *tiles_n, int64_t *workspace_bytes)
{
    return lowp_ws_plan(true, tile, precision, M, N, K, transB, kernel_id, tiles_m, tiles_n, workspace_bytes);
}

int sgemm_f32_streamk_plan(int tile, int64_t M, int64_t N, int64_t K, int transB, int *kernel_id,
                           int64_t *dp_tiles, int64_t *sk_tiles, int64_t *workers, int64_t *workspace_bytes)
{
    const float *A = reinterpret_cast<const float *>((uintptr_t)1 << 40);
    const float *B = reinterpret_cast<const float *>((uintptr_t)1 << 50);
    const float *C = reinterpret_cast<const float *>((uintptr_t)1 << 58);
    const int64_t lda = K > 1 ? K : 1, ldc = N > 1 ? N : 1;
    const int64_t ldb = transB == 1 ? lda : ldc;
    const sgemm::SkPlan sp = sgemm::make_sk_plan(tile, M, N, K, 1.0f, A, lda, B, ldb, transB, 0.0f, C, ldc);
    const bool sk = sp.base.status == SGEMM_OK && sp.kid != sgemm::KID_NONE;
    if (kernel_id)
        *kernel_id = sk ? sp.kid : sp.base.kid;
    if (dp_tiles)
        *dp_tiles = sk ? sp.sk.dp : 0;
    if (sk_tiles)
        *sk_tiles = sk ? sp.sk.sk_tiles : 0;
    if (workers)
        *workers = sk ? sp.sk.workers : 0;
    if (workspace_bytes)
        *workspace_bytes = sk ? sp.bytes : 0;
    return sp.base.status;
}

int sgemm_f32_streamk(int tile, int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
                      const float *B, int64_t ldb, int transB, float beta, float *C, int64_t ldc, void *workspace,
                      int64_t workspace_bytes, void *stream)
{
    return sgemm::run_sk(tile, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, workspace, workspace_bytes,
                         stream);
}

int sgemm_f32_splitk(int64_t splits, int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
                     const float *B, int64_t ldb, int transB, float beta, float *C, int64_t ldc, void *workspace,
                     int64_t workspace_bytes, void *stream)
{
    if (splits < 1)
        return SGEMM_ERR_INVALID_VALUE;
    return sgemm::run_split(splits, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, workspace,
                            workspace_bytes, stream);
}

int sgemm_f32_lowp(int precision, int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
                   const float *B, int64_t ldb, int transB, float beta, float *C, int64_t ldc, void *stream)
{
    return sgemm::run_lowp(precision, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc, stream);
}

int sgemm_f32_lowp_plan(int precision, int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
                        const float *B, int64_t ldb, int transB, float beta, const float *C, int64_t ldc,
                        int *kernel_id, int64_t *tiles_m, int64_t *tiles_n, char *name, int name_len)
{
    const sgemm::Plan p = sgemm::make_lowp_plan(precision, M, N, K, alpha, A, lda, B, ldb, transB, beta, C, ldc);
    if (kernel_id)
        *kernel_id = p.kid;
    if (tiles_m)
        *tiles_m = p.kid == sgemm::KID_NONE ? 0 : p.tiles_m;
    if (tiles_n)
        *tiles_n = p.kid == sgemm::KID_NONE ? 0 : p.tiles_n;
    if (name && name_len > 0)
        std::snprintf(name, (size_t)name_len, "%s transB=%d vec=%d", sgemm::kernel_label(p.kid), p.transB ? 1 : 0,
                      p.vec ? 1 : 0);
    return p.status;
}

int sgemm_f32_transpose(int64_t rows, int64_t cols, const float *src, int64_t ld_src, float *dst, int64_t ld_dst,
                        void *stream)
{
    return sgemm::run_transpose(SGEMM_TRANSPOSE_AUTO, rows, cols, src, ld_src, dst, ld_dst, stream);
}

int sgemm_f32_transpose_algo(int algo, int64_t rows, int64_t cols, const float *src, int64_t ld_src, float *dst,
                             int64_t ld_dst, void *stream)
{
    return sgemm::run_transpose(algo, rows, cols, src, ld_src, dst, ld_dst, stream);
}

int sgemm_f32_transpose_plan(int algo, int64_t rows, int64_t cols, const float *src, int64_t ld_src,
                             const float *dst, int64_t ld_dst, int *kernel_id, int64_t *blocks, char *name,
                             int name_len)
{
    const sgemm::TransposePlan p = sgemm::make_transpose_plan(algo, rows, cols, src, ld_src, dst, ld_dst);
    if (kernel_id)
        *kernel_id = p.kid;
    if (blocks)
        *blocks = p.blocks;
    if (name && name_len > 0) {
        const bool tiles = p.kid == sgemm::KID_TRANSPOSE_LDS_PAD || p.kid == sgemm::KID_TRANSPOSE_LDS_NOPAD;
        const int shape = tiles ? sgemm::transpose_shape(p.rows, p.cols) : -1;
        const char *label = !tiles ? sgemm::kernel_label(p.kid)
                            : shape == sgemm::TSHAPE_SMALL
                                ? (p.kid == sgemm::KID_TRANSPOSE_LDS_PAD ? "transpose_lds_64x64_pad1"
                                                                          : "transpose_lds_64x64_pad0")
                                : sgemm::kernel_label(p.kid);
        const char *suffix = !tiles ? ""
                             : shape == sgemm::TSHAPE_SMALL ? ""
                             : shape == sgemm::TSHAPE_PIPE ? "_pipe"
                             : (p.vec && p.kid == sgemm::KID_TRANSPOSE_LDS_PAD) ? "_stream_v4" : "_stream";
        std::snprintf(name, (size_t)name_len, "%s%s", label, suffix);
    }
    return p.status;
}

const char *sgemm_f32_status_string(int status)
{
    switch (status) {
    case SGEMM_OK: return "SGEMM_OK";
    case SGEMM_ERR_INVALID_VALUE: return "SGEMM_ERR_INVALID_VALUE: invalid argument";
    case SGEMM_ERR_ALIAS: return "SGEMM_ERR_ALIAS: output overlaps an input";
    case SGEMM_ERR_NO_DEVICE: return "SGEMM_ERR_NO_DEVICE: no HIP device is current";
    case SGEMM_ERR_UNSUPPORTED_ARCH: return "SGEMM_ERR_UNSUPPORTED_ARCH: device is not gfx950";
    case SGEMM_ERR_LAUNCH: return "SGEMM_ERR_LAUNCH: kernel launch failed";
    case SGEMM_ERR_SCRATCH_LIMIT:
        return "SGEMM_ERR_SCRATCH_LIMIT: the k-split partials need more than the library's 16 MiB static scratch";
    default: return "SGEMM: unknown status";
    }
}

const char *sgemm_f32_version(void)
{
#if defined(SGEMM_DEBUG_POISON_LDS)
    return "sgemm_f32 0.1.0 (gfx950, debug: LDS poisoned before staging)";
#elif defined(SGEMM_DEBUG_SANITIZE)
    return "sgemm_f32 0.1.0 (gfx950, debug: host code under ASan and UBSan)";
#else
    return "sgemm_f32 0.1.0 (gfx950)";
#endif
}

int sgemm_f32_arch_status(const char *arch) { return sgemm::arch_status(arch); }

int sgemm_f32_device_status(void) { return sgemm::check_device(); }

int sgemm_f32_mfma_probe(int64_t workgroups, int64_t trips, float *sink, unsigned long long *clocks, void *stream)
{
    if (workgroups < 1 || workgroups > (int64_t{1} << 20) || trips < 1 || trips > (int64_t{1} << 24) ||
        sink == nullptr || clocks == nullptr)
        return SGEMM_ERR_INVALID_VALUE;
    if (sgemm::overlaps(sink, workgroups * 256 * (int64_t)sizeof(float), clocks,
                        workgroups * 2 * (int64_t)sizeof(unsigned long long)))
        return SGEMM_ERR_ALIAS;
    const int dev_status = sgemm::check_device();
    if (dev_status != SGEMM_OK)
        return dev_status;
    const hipError_t e = sgemm::launch_mfma_probe((int)workgroups, (int)trips, sink, clocks,
                                                  reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

int sgemm_f32_mfma_probe_lp(int precision, int zero_operands, int64_t workgroups, int64_t trips, float *sink,
                            unsigned long long *clocks, void *stream)
{
    if ((precision != SGEMM_PREC_FP16 && precision != SGEMM_PREC_BF16) || (zero_operands != 0 && zero_operands != 1))
        return SGEMM_ERR_INVALID_VALUE;
    if (workgroups < 1 || workgroups > (int64_t{1} << 20) || trips < 1 || trips > (int64_t{1} << 24) ||
        sink == nullptr || clocks == nullptr)
        return SGEMM_ERR_INVALID_VALUE;
    if (sgemm::overlaps(sink, workgroups * 256 * (int64_t)sizeof(float), clocks,
                        workgroups * 2 * (int64_t)sizeof(unsigned long long)))
        return SGEMM_ERR_ALIAS;
    const int dev_status = sgemm::check_device();
    if (dev_status != SGEMM_OK)
        return dev_status;
    const hipError_t e = sgemm::launch_mfma_lp_probe(precision == SGEMM_PREC_BF16, zero_operands == 1, (int)workgroups,
                                                     (int)trips, sink, clocks, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

int sgemm_f32_load_probe(int waves, int depth, int64_t workgroups, const void *src, int64_t src_bytes,
                         int64_t region_bytes, int64_t share, int64_t loads, unsigned long long *clocks, void *stream)
{
    if ((waves != 4 && waves != 8) || (depth != 1 && depth != 2 && depth != 4 && depth != 8))
        return SGEMM_ERR_INVALID_VALUE;
    if (workgroups < 1 || workgroups > (int64_t{1} << 16) || share < 1 || share > (int64_t{1} << 16) || loads < 1 ||
        loads > (int64_t{1} << 24) || region_bytes < 1024 || region_bytes % 1024 != 0 ||
        region_bytes > (int64_t{1} << 31) || src == nullptr || clocks == nullptr ||
        (reinterpret_cast<uintptr_t>(src) & 15) != 0)
        return SGEMM_ERR_INVALID_VALUE;
    // The last region read: 8 * (((workgroups - 1) / 8) / share) + 7 at most.
    const int64_t regions = 8 * (((workgroups - 1) / 8) / share) + 8;
    if (src_bytes < 0 || regions > src_bytes / region_bytes)
        return SGEMM_ERR_INVALID_VALUE;
    if (sgemm::overlaps(src, regions * region_bytes, clocks, workgroups * 2 * (int64_t)sizeof(unsigned long long)))
        return SGEMM_ERR_ALIAS;
    const int dev_status = sgemm::check_device();
    if (dev_status != SGEMM_OK)
        return dev_status;
    const hipError_t e = sgemm::launch_load_probe(waves, depth, (int)workgroups, src, region_bytes, (int)share,
                                                  (int)loads, clocks, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

}  // extern "C"
