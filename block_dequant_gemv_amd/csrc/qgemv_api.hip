// qgemv_api.hip -- the C ABI of libqgemv (declared in include/qgemv.h).
//
// Every entry point checks its arguments on the host first (no HIP call before
// the checks pass, so the checks run on a machine without a GPU), then picks a
// launch plan and enqueues kernels on the caller's stream. Nothing here
// allocates device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <mutex>
#include <cstdio>
#include <cstring>
#include <string>

#include "layout.h"
#include "qgemm_kernels.h"
#include "qgemv.h"
#include "qgemv_kernels.h"

using qgl::Geometry;

namespace {

thread_local std::string g_last_error;

qg_status fail(qg_status s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    qgk::set_launch_events(nullptr, nullptr);
    return s;
}

qg_status ok()
{
    g_last_error.clear();
    return QG_OK;
}

qg_status hip_fail(hipError_t e, const char *what)
{
    return fail(QG_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb)
{
    uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

bool valid_qtype(int qt) { return qt == QG_Q8_0 || qt == QG_Q4_0 || qt == QG_Q4_K || qt == QG_Q6_K; }

// The 256-weight super-block types: the plain single-row GEMV only.
bool super_block_qtype(int qt) { return qt == QG_Q4_K || qt == QG_Q6_K; }

// K granularity of a quantised type: 32 weights per block, 256 per Q4_K / Q6_K super-block.
int64_t k_unit(int qt) { return super_block_qtype(qt) ? 256 : 32; }

// Shape limits: rows and K must index 64-bit byte offsets safely and the grid
// must fit 2^31 workgroups.
constexpr int64_t kMaxDim = (int64_t)1 << 40;

qg_status check_qshape(int qt, int64_t N, int64_t K, const char *fn)
{
    if (!valid_qtype(qt)) return fail(QG_EUNSUPPORTED, "%s: unknown qtype %d", fn, qt);
    if (N <= 0 || K <= 0 || N > kMaxDim || K > kMaxDim)
        return fail(QG_EINVAL, "%s: N=%lld K=%lld must be positive", fn, (long long)N, (long long)K);
    if (K % k_unit(qt) != 0)
        return fail(QG_EINVAL, "%s: K=%lld is not a multiple of %lld", fn, (long long)K, (long long)k_unit(qt));
    if (N * (K / 32) > ((int64_t)1 << 42)) return fail(QG_EINVAL, "%s: matrix too large", fn);
    return QG_OK;
}

int64_t env_int(const char *name, int64_t dflt)
{
    const char *v = getenv(name);
    return (v && *v) ? atoll(v) : dflt;
}

// Launch-shape overrides for sweeps and tests (QG_SPLIT_K, QG_PERSIST,
// QG_X_GLOBAL, QG_TILES_PER_GROUP, QG_WAVES_PER_WG, QG_PREFETCH, QG_F16_ROWS,
// QG_F16_WAVES, QG_STRIDE_GROUPS, QG_GEMM_MT, QG_GEMM_WAVES, QG_GEMM_ROWGROUPS,
// QG_GEMM_KSPLIT, QG_F16_FORM, QG_F16_CPL). They are read from the environment once, on first use, and
// again on qg_reload_tuning(): a GEMV call itself reads no environment.
enum TuneKey {
    kSplitK, kPersist, kXGlobal, kTilesPerGroup, kWavesPerWg, kPrefetch, kF16Rows, kF16Waves, kStrideGroups,
    kGemmMT, kGemmWaves, kGemmRowGroups, kGemmKSplit, kF16Form, kF16Cpl, kVerifyRowGroups, kNumTune
};
const char *const kTuneNames[kNumTune] = {"QG_SPLIT_K",      "QG_PERSIST",  "QG_X_GLOBAL",  "QG_TILES_PER_GROUP",
                                          "QG_WAVES_PER_WG", "QG_PREFETCH", "QG_F16_ROWS",  "QG_F16_WAVES",
                                          "QG_STRIDE_GROUPS", "QG_GEMM_MT", "QG_GEMM_WAVES", "QG_GEMM_ROWGROUPS",
                                          "QG_GEMM_KSPLIT", "QG_F16_FORM", "QG_F16_CPL", "QG_VERIFY_ROW_GROUPS"};
const int64_t kTuneDefaults[kNumTune] = {0, -1, -1, 0, 0, 0, 0, 0, -1, 0, 0, 0, 0, -1, 0, 0};
std::atomic<int64_t> g_tune[kNumTune];
std::atomic<bool> g_tune_loaded{false};

void load_tuning()
{
    for (int i = 0; i < kNumTune; ++i) g_tune[i].store(env_int(kTuneNames[i], kTuneDefaults[i]), std::memory_order_relaxed);
    g_tune_loaded.store(true, std::memory_order_release);
}

int64_t tune(TuneKey k)
{
    if (!g_tune_loaded.load(std::memory_order_acquire)) load_tuning();
    return g_tune[k].load(std::memory_order_relaxed);
}

// Wavefronts that split one tile along K. Depends only on (rows, K): a matrix
// with few row tiles gets more wavefronts per tile so that the chip has enough
// loads in flight. The decode and the verify call of the same weight always
// get the same split, and so add in the same order. A tile of three segments
// gets three wavefronts, one segment each: with two, one of them computes two
// segments in a row, which made the 1024x3072 down projection about 1.1 us
// slower back to back (measured). (QG_SPLIT_K overrides the choice for
// launch-shape sweeps; it must then be the same for every call.)
int split_k_waves(int64_t rows, int64_t K)
{
    const int64_t n_tiles = (rows + qgl::kTileRows - 1) / qgl::kTileRows;
    const int64_t nseg = (K / 32 + qgl::kSegBlocks - 1) / qgl::kSegBlocks;
    const int64_t forced = tune(kSplitK);
    if (forced == 1 || forced == 2 || forced == 3 || forced == 4 || forced == 8)
        return forced <= nseg ? (int)forced : 1;
    int W = 1;
    while (W < 8 && 2 * W <= nseg && n_tiles * W < 2048) W *= 2;
    if (W == 2 && nseg == 3) W = 3;
    return W;
}

constexpr size_t kLdsLimit = 96 * 1024;                        // single-row calls: above this, x is read from L2
constexpr size_t kLdsLimitMulti = qgk::kLdsPerWorkgroup;       // verify calls: the whole LDS of a CU (gfx950)

// Launch shape of the one-wavefront-per-tile form (measured on MI355X with
// cold weights):
//  - one row tile per group of W wavefronts;
//  - 4 wavefronts per workgroup share one LDS copy of the activations, fewer
//    only when there are too few groups to cover the CUs;
//  - for M = 1, activations are staged in LDS when a workgroup streams at least
//    2x as many weight bytes as it stages, otherwise read from global memory
//    (L2); with several activation rows (verify) each staged value is reused
//    M times per weight, so LDS is used whenever it fits.
// The overrides QG_TILES_PER_GROUP, QG_WAVES_PER_WG (split 1 only),
// QG_X_GLOBAL (0/1) and QG_PREFETCH (1/2) change none of a row's operations.

// CUs of the current device (cached per device); 256, the MI355X count, when
// no device answers (host-only planning).
int cu_count()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Persistent form (see qgemv_persist): used for matrices with fewer than
// kPersistTiles row tiles but at least kPersistUnits (tile, segment) units.
// There one tile per wavefront leaves the CUs unevenly loaded (2 or 3 small
// workgroups per CU); smaller matrices are launch-bound and run faster in the
// other form, larger ones balance themselves (measured). The choice and the K
// split (ranges) depend only on (rows, K) and the device's CU count, never on
// M, so the decode and the verify call of a weight run the same per-row
// operations. QG_PERSIST=0/1 overrides the choice for launch-shape sweeps.
constexpr int64_t kPersistTiles = 4096;
constexpr int64_t kPersistUnits = 2048;   // below this many (tile, segment) units the other form is faster
constexpr size_t kPartialBudget = 64 * 1024;   // LDS for the range partials at M = 6

bool plan_persist(int qt, int64_t rows, int64_t K, int64_t *ranges, int64_t *grid, int64_t *max_tiles)
{
    const int64_t n_tiles = (rows + qgl::kTileRows - 1) / qgl::kTileRows;
    const int64_t nseg = (K / 32 + qgl::kSegBlocks - 1) / qgl::kSegBlocks;
    const int64_t forced = tune(kPersist);
    if (forced == 0 || (forced != 1 && (n_tiles >= kPersistTiles || n_tiles * nseg < kPersistUnits))) return false;
    *grid = std::min<int64_t>(cu_count(), n_tiles);
    // a workgroup owns up to ceil(2 n_tiles / grid) half-tiles, which touch at
    // most one tile more than half of them (a run may start at a tile's second half)
    const int64_t halves = (2 * n_tiles + *grid - 1) / *grid;
    *max_tiles = (halves + 2) / 2;
    // the kernel addresses a workgroup's tiles with 32-bit offsets below 2^31,
    // products of 24-bit tile indices and tile sizes
    const qgl::Geometry g = qgl::geometry(qt, rows, K);
    const int64_t tile_bytes = std::max(g.tile_q, std::max(g.tile_s, g.tile_u));
    if (tile_bytes >= ((int64_t)1 << 24) || *max_tiles * tile_bytes >= ((int64_t)1 << 31)) return false;
    // one segment per item when the partials fit, else the largest divisor of nseg that fits
    int64_t r = std::min<int64_t>(nseg, 32);
    while (r > 1 && (nseg % r != 0 || (size_t)(*max_tiles * r * 6 * qgl::kTileRows * 4) > kPartialBudget)) --r;
    *ranges = r;
    return true;
}

// The RMSNorm prologue needs the activations staged in LDS: whole 1024-weight
// segments of them next to the largest static array of the one-wavefront-per-tile
// form (8 split-K wavefronts), i.e. K <= 39 * 1024 = 39936.
constexpr int64_t kNormMaxK =
    (int64_t)((kLdsLimitMulti - qgk::static_lds_bytes(qgk::tile_red_floats(1, 8, true))) /
              (qgl::kSegWeights * sizeof(float))) * qgl::kSegWeights;

qgk::QPlan make_qplan(int qt, int64_t rows, int64_t K, int M, bool norm = false)
{
    qgk::QPlan p;
    p.norm = norm;
    const Geometry g = qgl::geometry(qt, rows, K);
    // the staged copy of the activations (with their block sums where
    // x_sums_staged)
    const size_t xbytes = (size_t)M * (size_t)g.nseg * qgk::staged_seg_bytes(qt, norm);
    const int64_t xg_env = tune(kXGlobal);
    int64_t ranges = 1, pgrid = 0, max_tiles = 0;
    p.persist = plan_persist(qt, rows, K, &ranges, &pgrid, &max_tiles);
    p.depth = 1;
    p.tpg = 1;
    p.tstride = 0;
    p.phases = 1;
    if (p.persist) {
        p.ranges = (int)ranges;
        p.max_tiles = max_tiles;
        p.W = (int)ranges;
        p.grid = pgrid;
        const size_t part = ranges > 1 ? (size_t)max_tiles * ranges * M * qgl::kTileRows * 4 : 0;
        // LDS left for the activations and the partials next to the static array
        const size_t budget = kLdsLimitMulti - qgk::static_lds_bytes(qgk::persist_red_floats(norm));
        bool lds = xbytes + part <= budget;
        // Several activation rows that do not fit (M K 4 bytes above the LDS):
        // walk the K ranges in the fewest phases whose largest activation window
        // (ceil(ranges / phases) ranges) fits, instead of reading every unit's
        // activations from L2 (5120 x 17408 at M = 3..6: 47-82 us from L2).
        // Phases change which wavefront adds an item and when, not any row's
        // operations.
        const size_t seg_bytes = (size_t)M * qgk::staged_seg_bytes(qt, norm);   // one segment, M rows
        const int64_t seg_per_range = g.nseg / ranges;
        auto window = [&](int64_t ph) { return (size_t)((ranges + ph - 1) / ph * seg_per_range) * seg_bytes; };
        if (!lds && M > 1 && !norm) {
            for (int64_t ph = 2; ph <= ranges; ++ph)
                if (window(ph) + part <= budget) {
                    p.phases = (int)ph;
                    lds = true;
                    break;
                }
        }
        if (!norm && (xg_env == 0 || xg_env == 1)) lds = lds && xg_env == 0;
        if (!lds) p.phases = 1;
        if (lds || !norm) {
            p.x_in_lds = lds;
            p.lds_bytes = (lds ? window(p.phases) : 0) + part;
            p.one_unit = ranges == g.nseg;
            p.block = qgk::persist_threads(qt, M, lds, p.one_unit, p.phases > 1);
            return p;
        }
        // The RMSNorm prologue needs the staged copy: when it does not fit next to
        // the partials, use the other form, which needs no partials in LDS.
        p.persist = false;
        p.phases = 1;
    }
    p.ranges = 1;
    p.max_tiles = 0;
    p.W = split_k_waves(rows, K);
    // One row tile per group: many short, independent wavefronts, which the
    // hardware dispatcher balances across the CUs better than longer chains
    // (measured on both LM-head shapes).
    const int64_t tpg_env = tune(kTilesPerGroup);
    if (tpg_env > 0) p.tpg = tpg_env;
    int64_t groups = (g.n_tiles + p.tpg - 1) / p.tpg;
    // Grid-stride tile order (QG_STRIDE_GROUPS = number of groups; off by
    // default: in interleaved measurements it gained on some shapes and lost on
    // others, the plain and the RMSNorm-prologue calls alike).
    p.tstride = 0;
    const int64_t sg = tune(kStrideGroups);
    if (sg > 0 && sg < g.n_tiles) {
        p.tstride = sg;
        groups = sg;
    }
    const size_t lds_limit = M > 1 ? kLdsLimitMulti : kLdsLimit;
    int G;   // groups per workgroup
    if (p.W > 1) {
        G = 1;
        p.block = 64 * p.W;
    } else {
        G = groups >= 512 ? 4 : (groups >= 256 ? 2 : 1);
        // a verify call whose activations take more than half the LDS runs one
        // workgroup per CU: give it 8 wavefronts
        if (M > 1 && xbytes > 80 * 1024 && xbytes <= lds_limit && groups >= 2048) G = 8;
        const int64_t g_env = tune(kWavesPerWg);
        if (g_env == 1 || g_env == 2 || g_env == 4 || g_env == 8) G = (int)g_env;
        G = std::min(G, qgk::qgemv_max_threads(qt, M, 1) / 64);   // the kernel's launch bound
        p.block = 64 * G;
    }
    if (p.tstride > 0) {
        // every group index below tstride must exist: round the groups up to whole workgroups
        p.tstride = (groups + G - 1) / G * G;
        if (p.tstride >= g.n_tiles) {
            p.tstride = 0;
            groups = (g.n_tiles + p.tpg - 1) / p.tpg;
        }
    }
    p.grid = (groups + G - 1) / G;
    const double tiles_per_group = p.tstride > 0 ? (double)g.n_tiles / (double)p.tstride : (double)p.tpg;
    const double wg_weight_bytes = (double)G * tiles_per_group * (double)(g.tile_q + g.tile_s);
    // The staged copy must fit next to the kernel's static array (the split-K
    // partials of W > 1 wavefronts take up to 1.5 KiB).
    const bool fits = xbytes + qgk::static_lds_bytes(qgk::tile_red_floats(M, p.W, norm)) <= kLdsLimitMulti;
    // A split tile's wavefronts (W > 1) take their activations from one staged copy
    // (measured faster than each reading its range from L2, e.g. Q4_0 640 x 17408
    // at W = 8: 8.1 against 8.6 us).
    bool lds = fits && xbytes <= lds_limit && (M > 1 || p.W > 1 || wg_weight_bytes >= 2.0 * (double)xbytes);
    if (xg_env == 0 || xg_env == 1) lds = fits && xbytes <= lds_limit && xg_env == 0;
    if (norm) lds = fits;   // the prologue normalises the staged copy
    p.x_in_lds = lds;
    p.lds_bytes = p.x_in_lds ? xbytes : 0;
    // Prefetch depth: one unit in flight ahead of the one being computed. A
    // depth of 2 (single-row kernels only) measured no faster on any of the
    // workload shapes and costs registers; it stays reachable for sweeps.
    const int64_t d_env = tune(kPrefetch);
    if (d_env == 1 || d_env == 2) p.depth = (int)d_env;
    return p;
}

hipStream_t as_stream(void *s) { return (hipStream_t)s; }

// Addends and output type of the affine epilogue (kEpiAffine only).
struct Affine {
    const float *bias = nullptr;
    const float *residual = nullptr;
    int out_type = QG_OUT_F32;
};

// The RMSNorm prologue (qgemv_rmsnorm*): gamma [K] and eps.
struct Norm {
    bool on = false;
    const float *gamma = nullptr;
    float eps = 0.0f;
};

// Row groups of a verify call (see run_qgemv): where the tile form launches at
// most half as many wavefronts as the chip has SIMDs, the fewest groups (a
// divisor of M) that give every SIMD a wavefront, else M groups of one row.
// Measured on MI355X, cold, interleaved (us, one group -> the chosen groups):
// Q8_0 4096 x 1024 (512 wavefronts) M = 2 / 3 / 4 / 6: 5.15 -> 4.47, 5.31 ->
// 4.81, 5.86 -> 5.36, 6.62 -> 5.27; Q8_0 1024 x 1024 (128) M = 3 / 6: 5.53 ->
// 4.61, 8.71 -> 4.65; Q4_K 4096 x 1024 M = 6: 6.98 -> 5.17. With 768 wavefronts
// (6144 x 1024) groups won at M = 2 and 6 and lost at M = 3 and 4, so they stay
// off there. QG_VERIFY_ROW_GROUPS = g forces g groups where g divides M and the
// tile form applies.
int verify_row_groups(int qt, int64_t rows, int64_t K, int M, const qgk::QPlan &p, int epi, bool norm)
{
    if (M < 2 || epi != qgk::kEpiPlain || norm || p.persist) return 1;
    auto usable = [&](int g) {
        if (g < 2 || M % g != 0) return false;
        const qgk::QPlan q = make_qplan(qt, rows, K, M / g, false);
        return !q.persist;
    };
    const int64_t forced = tune(kVerifyRowGroups);
    if (forced >= 1) return usable((int)forced) ? (int)forced : 1;
    const int64_t simds = cu_count() * 4;
    const int64_t waves = p.grid * (p.block / 64);
    if (2 * waves > simds) return 1;
    for (int g = 2; g <= M; ++g)
        if (M % g == 0 && waves * g >= simds && usable(g)) return g;
    return usable(M) ? M : 1;
}

qg_status run_qgemv(int qt, int epi, const void *w, const float *x, void *y, int64_t rows, int64_t n_out,
                    int64_t K, int M, void *stream, const char *fn, const Affine &af = Affine(),
                    const Norm &nm = Norm())
{
    qg_status st = check_qshape(qt, rows, K, fn);
    if (st) return st;
    if (!w || !x || !y) return fail(QG_EINVAL, "%s: null pointer", fn);
    if (af.out_type != QG_OUT_F32 && af.out_type != QG_OUT_F16)
        return fail(QG_EUNSUPPORTED, "%s: unknown output type %d", fn, af.out_type);
    const bool f16 = af.out_type == QG_OUT_F16;
    if (!aligned(w, 16)) return fail(QG_EALIGN, "%s: packed weights must be 16-byte aligned", fn);
    if (!aligned(x, 16)) return fail(QG_EALIGN, "%s: activations must be 16-byte aligned", fn);
    if (!aligned(y, f16 ? 2 : 4)) return fail(QG_EALIGN, "%s: output must be %d-byte aligned", fn, f16 ? 2 : 4);
    if (!aligned(af.bias, 4) || !aligned(af.residual, 4))
        return fail(QG_EALIGN, "%s: bias and residual must be 4-byte aligned", fn);
    if (nm.on) {
        if (!nm.gamma) return fail(QG_EINVAL, "%s: null gamma", fn);
        if (!aligned(nm.gamma, 16)) return fail(QG_EALIGN, "%s: gamma must be 16-byte aligned", fn);
        if (!(nm.eps >= 0.0f) || nm.eps == __builtin_inff())
            return fail(QG_EINVAL, "%s: eps must be finite and >= 0", fn);
        if (K > kNormMaxK)
            return fail(QG_EUNSUPPORTED, "%s: K=%lld above %lld (the normalised activations live in LDS)", fn,
                        (long long)K, (long long)kNormMaxK);
    }
    const Geometry g = qgl::geometry(qt, rows, K);
    const size_t ybytes = (size_t)M * (size_t)n_out * (f16 ? 2 : sizeof(float));
    const size_t xbytes = (size_t)M * (size_t)K * sizeof(float);
    const size_t abytes = (size_t)n_out * sizeof(float);
    if (overlap(y, ybytes, x, xbytes)) return fail(QG_EINVAL, "%s: y overlaps x", fn);
    if (overlap(y, ybytes, w, (size_t)g.total)) return fail(QG_EINVAL, "%s: y overlaps the weights", fn);
    if (af.bias && overlap(y, ybytes, af.bias, abytes)) return fail(QG_EINVAL, "%s: y overlaps bias", fn);
    if (nm.on && overlap(y, ybytes, nm.gamma, (size_t)K * sizeof(float)))
        return fail(QG_EINVAL, "%s: y overlaps gamma", fn);
    // residual == y (fp32) is the in-place update y += W x; any other overlap is refused
    if (af.residual && !(af.residual == y && !f16) && overlap(y, ybytes, af.residual, abytes))
        return fail(QG_EINVAL, "%s: y overlaps residual (only residual == y with fp32 output is allowed)", fn);

    qgk::QPlan p = make_qplan(qt, rows, K, M, nm.on);
    if (nm.on && !p.x_in_lds) return fail(QG_EUNSUPPORTED, "%s: activations do not fit in LDS", fn);
    // Verify on a matrix with few row tiles: split the activation rows into
    // groups (gridDim.y) of M / groups rows, each group a launch-wide copy of
    // the tile form over all tiles, so that more wavefronts share the work.
    // Every row keeps the M = 1 operations.
    const int groups = verify_row_groups(qt, rows, K, M, p, epi, nm.on);
    if (groups > 1) {
        p = make_qplan(qt, rows, K, M / groups, false);
        p.row_groups = groups;
        M /= groups;
    }
    qgk::QArgs a;
    a.geo = g;
    a.n_out = n_out;
    a.x_stride = K;
    a.y_stride = n_out;
    a.tpg = p.tpg;
    a.tstride = p.tstride;
    a.n_wg = p.grid;
    a.halves_base = p.persist ? 2 * g.n_tiles / p.grid : 0;
    a.halves_extra = p.persist ? 2 * g.n_tiles % p.grid : 0;
    a.ranges = p.ranges;
    a.range_segs = g.nseg / p.ranges;
    a.phases = p.phases;
    a.bias = af.bias;
    a.residual = af.residual;
    a.out_f16 = f16 ? 1 : 0;
    a.gamma = nm.gamma;
    a.eps = nm.eps;
    hipError_t e = qgk::launch_qgemv(qt, M, epi, p, (const uint8_t *)w, x, (float *)y, a, as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

qg_status check_pack(int qt, const void *canon, const void *packed, int64_t N, int64_t K, const char *fn)
{
    qg_status st = check_qshape(qt, N, K, fn);
    if (st) return st;
    if (!canon || !packed) return fail(QG_EINVAL, "%s: null pointer", fn);
    return QG_OK;
}

void host_pack_rows(const Geometry &g, const uint8_t *canon, uint8_t *packed, int64_t row0, int64_t nrows,
                    bool pad)
{
    const int64_t rb = qgl::canon_row_bytes(g.qt, g.K);
    for (int64_t r = 0; r < nrows; ++r)
        for (int64_t b = 0; b < g.KB; ++b) qgl::pack_block(g, canon + r * rb, packed, row0 + r, b);
    if (pad)
        for (int64_t r = g.N; r < g.n_tiles * qgl::kTileRows; ++r)
            for (int64_t b = 0; b < g.KB; ++b) qgl::pack_block(g, nullptr, packed, r, b);
}

// Small-M GEMM: activation rows are processed in tiles of 16, MT tiles per
// workgroup (the last group padded with zero rows). The workspace holds, each
// part 256-byte aligned: one unscale factor per padded row, the split
// activations (M_pad * K * 2 halves) and, when K is split across workgroups,
// the partial sums (ksplit * M * N floats).
constexpr int64_t kGemmMaxM = (int64_t)1 << 20;

struct GemmPlan {
    int MT, RG, G;
    int64_t n_mg, M_pad, row_blocks, ksplit;
    size_t off_xs, off_part, bytes;
};

// Launch plan of qgemm_prefill (depends on the shape and the device's CU count).
//
// K split (gridDim.y ranges added by the K-sum kernel): it changes a row's
// rounding, so it depends on the weight's shape alone, never on M or the
// tiling. None below 16 chunks (K < 2048: the K-sum launch and the partial
// sums cost more than the extra workgroups gain; measured on MI355X, Q8_0
// 4096 x 1024 at M = 16 / 128: 11.2 / 15.6 us unsplit against 12.0 / 21.1 us in
// four ranges). Otherwise ranges of at least two chunks until the row blocks of
// the default tiling (8 wavefronts, 2 row groups for Q4_0, 1 for Q8_0) times the
// ranges come near half the CUs, so two activation groups fill the chip in one
// round (Q4_0 5120 x 17408 at M = 128: 6 ranges, 240 workgroups, 78.6 us; 7
// ranges put 280 workgroups in two rounds, 118 us).
//
// Tiling (MT activation tiles, G wavefronts, RG row groups per workgroup): the
// candidate with the least estimated time, rounds x RG x MT / e, where rounds =
// workgroups / (CUs x workgroups per CU) rounded up (one workgroup of 8
// wavefronts per CU; two of 4 where their staging ring fits in half the LDS),
// RG x MT is each wavefront's work per block, and e the relative throughput of
// a full CU measured on MI355X on the LM heads (M = 128, many rounds: Q4_0
// 248320 x 5120 731.8 us at MT 4 / 8 wavefronts / 2 row groups = 1.00, Q8_0
// 151936 x 1024 199.0 us at MT 4 / 8 / 1 = 1.00). Four wavefronts alone on a CU
// (no more workgroups than CUs) get the whole SIMD each: e x 1.3. Over the
// prefill shapes of the configurations at M = 16 .. 256 the choice is within
// 1% in total of the fastest candidate per case (5089 against 5044 us).
//
// QG_GEMM_MT (1..4), QG_GEMM_WAVES (1, 2, 4, 8), QG_GEMM_ROWGROUPS (1, 2) and
// QG_GEMM_KSPLIT override the choices for launch-shape sweeps.
GemmPlan plan_gemm(int qt, int64_t N, int64_t K, int64_t M)
{
    GemmPlan p;
    const Geometry g = qgl::geometry(qt, N, K);
    const int64_t n_mt = (M + qgk::kGemmTileM - 1) / qgk::kGemmTileM;
    const int64_t cus = cu_count();
    auto rbs = [&](int G, int RG) { return (g.n_tiles + 2 * RG * G - 1) / (2 * RG * G); };
    constexpr int CPS = qgl::kSegBlocks / qgk::kGemmChunk;
    const int64_t n_chunks =
        (g.nseg - 1) * CPS + (qgl::seg_blocks(g, g.nseg - 1) + qgk::kGemmChunk - 1) / qgk::kGemmChunk;
    const int base_rg = qt == qgl::kQ8_0 ? 1 : 2;
    const int64_t base = rbs(8, base_rg);
    p.ksplit = 1;
    if (n_chunks >= 16 && 2 * base < cus)
        p.ksplit = std::min<int64_t>(std::max<int64_t>(n_chunks / 2, 1), std::max<int64_t>(1, (cus / 2 + base / 2) / base));
    const int64_t ks_env = tune(kGemmKSplit);
    if (ks_env >= 1) p.ksplit = std::min<int64_t>(n_chunks, ks_env);

    struct Cand {
        int MT, G, RG, eff;   // eff: relative throughput of a full CU, percent
    };
    static constexpr Cand q4c[] = {{4, 8, 2, 100}, {4, 8, 1, 79}, {2, 8, 2, 80}, {2, 8, 1, 80},
                                   {1, 8, 2, 67},  {1, 8, 1, 59}, {1, 4, 1, 54}, {2, 4, 1, 62}};
    static constexpr Cand q8c[] = {{4, 8, 1, 100}, {2, 8, 1, 79}, {1, 8, 1, 70}, {1, 4, 1, 69}, {2, 4, 1, 75}};
    const Cand *cand = qt == qgl::kQ8_0 ? q8c : q4c;
    const int ncand = qt == qgl::kQ8_0 ? (int)(sizeof(q8c) / sizeof(q8c[0])) : (int)(sizeof(q4c) / sizeof(q4c[0]));
    double best = -1.0;
    p.MT = 1;
    p.G = 4;
    p.RG = 1;
    for (int ci = 0; ci < ncand; ++ci) {
        const Cand &c = cand[ci];
        if (c.MT > 1 && c.MT > n_mt) continue;
        const size_t lds = qgk::gemm_lds_bytes(qt, c.MT, c.RG, c.G);
        if (lds > qgk::kLdsPerWorkgroup) continue;
        const int64_t per_cu = (c.G == 4 && lds <= qgk::kLdsPerWorkgroup / 2) ? 2 : 1;
        const int64_t wgs = rbs(c.G, c.RG) * ((n_mt + c.MT - 1) / c.MT) * p.ksplit;
        const int64_t rounds = (wgs + cus * per_cu - 1) / (cus * per_cu);
        double e = c.eff / 100.0;
        if (c.G == 4 && wgs <= cus) e *= 1.3;
        const double cost = (double)rounds * c.RG * c.MT / e;
        if (best < 0.0 || cost < best * (1.0 - 1e-9)) {
            best = cost;
            p.MT = c.MT;
            p.G = c.G;
            p.RG = c.RG;
        }
    }
    const int64_t mt_env = tune(kGemmMT);
    if (mt_env >= 1 && mt_env <= qgk::kGemmMaxMT) p.MT = (int)mt_env;
    const int64_t g_env = tune(kGemmWaves);
    if (g_env == 1 || g_env == 2 || g_env == 4 || g_env == 8) p.G = (int)g_env;
    const int64_t rg_env = tune(kGemmRowGroups);
    if (rg_env == 1 || rg_env == 2) p.RG = (int)rg_env;
    // the staging ring must fit in the LDS of one workgroup (Q8_0 weights take twice Q4_0's)
    while (p.G > 1 && qgk::gemm_lds_bytes(qt, p.MT, p.RG, p.G) > qgk::kLdsPerWorkgroup) p.G /= 2;
    p.n_mg = (n_mt + p.MT - 1) / p.MT;
    p.M_pad = p.n_mg * p.MT * qgk::kGemmTileM;
    p.row_blocks = rbs(p.G, p.RG);
    p.off_xs = (size_t)qgl::round_up(p.M_pad * (int64_t)sizeof(float), 256);
    p.off_part = p.off_xs + (size_t)qgl::round_up(p.M_pad * K * 2 * (int64_t)sizeof(_Float16), 256);
    p.bytes = p.off_part + (p.ksplit > 1 ? (size_t)p.ksplit * (size_t)M * (size_t)N * sizeof(float) : 0);
    return p;
}

// Launch plan of gemv_f16_splitk (depends on the shape and on whether w and x
// are 16-byte aligned). Three forms, all deterministic with a fixed order of
// additions:
//  - split-K row form (short matrices, fewer than 1024 rows): one row per
//    workgroup, K split into consecutive ranges over its wavefronts (4 16-byte
//    chunks per lane), partials added in wavefront order. Measured on MI355X,
//    cold, back to back against the row form: 640 x 5120 3.70 against 4.10 us;
//    48 and 256 rows x 5120 within 0.1-0.3 us (every form of these two reads
//    the ~3.9 us dispatch floor by kernel timestamps);
//  - row form (K = 512 L, L <= 16): one wavefront per row with the whole row's
//    loads in flight at once, x staged in LDS once per workgroup of 4 rows
//    (8 from 4096 rows on, which halves the activation copies: one 4 K-byte
//    copy per 8 rows instead of per 4; cold, kernel timestamps: 5120 x 5120
//    10.04 -> 9.84 us, 17408 x 5120 28.0 -> 27.7, 5120 x 8192 unchanged).
//    Measured on MI355X, cold, against the lane-split form: 5120 x 5120 9.96
//    against 10.78 us, 5120 x 8192 15.3 against 17.2, 17408 x 4096 22.4
//    against 27.0;
//  - lane-split form (any other K, or unaligned pointers): one row per
//    workgroup, K split over the lanes of one wavefront (four below 1024 rows)
//    in 8-element chunks.
// QG_F16_FORM = 0 / 1 / 2 forces the lane-split / row / split-K row form (where
// K and the alignment allow it), QG_F16_CPL = 1, 2, 4 the chunks per lane of
// the split-K row form, QG_F16_WAVES and QG_F16_ROWS the other forms' shapes.
// Checks shared by the two prefill entry points (no HIP call): sizes, types,
// null pointers, alignment.
qg_status check_prefill(int qtype, const void *w_packed, const float *X, const float *Y, int64_t N, int64_t K,
                        int64_t M, const char *fn)
{
    qg_status st = check_qshape(qtype, N, K, fn);
    if (st) return st;
    if (super_block_qtype(qtype)) return fail(QG_EUNSUPPORTED, "%s: Q4_K / Q6_K weights have the GEMV only", fn);
    if (M <= 0 || M > kGemmMaxM) return fail(QG_EINVAL, "%s: M=%lld outside 1..%lld", fn, (long long)M,
                                             (long long)kGemmMaxM);
    if (!w_packed || !X || !Y) return fail(QG_EINVAL, "%s: null pointer", fn);
    if (!aligned(w_packed, 16)) return fail(QG_EALIGN, "%s: packed weights must be 16-byte aligned", fn);
    if (!aligned(X, 4) || !aligned(Y, 4)) return fail(QG_EALIGN, "%s: X and Y must be 4-byte aligned", fn);
    return QG_OK;
}

// Y against X and the weights (after every alignment check).
qg_status check_prefill_overlap(int qtype, const void *w_packed, const float *X, const float *Y, int64_t N,
                                int64_t K, int64_t M, const char *fn)
{
    const Geometry g = qgl::geometry(qtype, N, K);
    const size_t xb = (size_t)M * (size_t)K * sizeof(float), yb = (size_t)M * (size_t)N * sizeof(float);
    if (overlap(Y, yb, X, xb) || overlap(Y, yb, w_packed, (size_t)g.total))
        return fail(QG_EINVAL, "%s: Y overlaps X, the weights or the workspace", fn);
    return QG_OK;
}

// Enqueue the split, the GEMM passes and (with a K split) the sum of the ranges
// on `workspace` (plan_gemm(...).bytes bytes, 256-byte aligned).
qg_status run_prefill(int qtype, const void *w_packed, const float *X, float *Y, int64_t N, int64_t K, int64_t M,
                      void *workspace, void *stream, const char *fn)
{
    const GemmPlan p = plan_gemm(qtype, N, K, M);
    const Geometry g = qgl::geometry(qtype, N, K);
    float *unscale = (float *)workspace;
    _Float16 *xs = (_Float16 *)((uint8_t *)workspace + p.off_xs);
    hipStream_t s = as_stream(stream);
    // the split pass is not timed: a bound event pair goes to the GEMM
    hipError_t e = qgk::launch_split_x(qtype, X, xs, unscale, M, p.M_pad, K, s);
    if (e != hipSuccess) return hip_fail(e, fn);
    qgk::GemmArgs a;
    a.geo = g;
    a.N = N;
    a.M = M;
    a.n_mg = p.n_mg;
    a.y_stride = N;
    a.ksplit = p.ksplit;
    a.part = p.ksplit > 1 ? (float *)((uint8_t *)workspace + p.off_part) : nullptr;
    e = qgk::launch_qgemm(qtype, p.MT, p.RG, p.G, p.row_blocks, (const uint8_t *)w_packed, xs, unscale, Y, a, s);
    if (e != hipSuccess) return hip_fail(e, fn);
    if (p.ksplit > 1) {
        e = qgk::launch_ksum(a.part, Y, p.ksplit, M, N, s);
        if (e != hipSuccess) return hip_fail(e, fn);
    }
    return ok();
}

// Scratch of qgemm_prefill_noalloc: a file-scope device array, one copy per GPU
// the library runs on, held until the process ends. In host code its name is a
// host-side stand-in, not a device address; the device address is taken once
// per device (with that device current) by hipGetSymbolAddress and used in its
// place wherever host code needs the array's memory.
constexpr size_t kNoAllocScratchBytes = QG_PREFILL_NOALLOC_MAX_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

qg_status scratch_address(void **out, const char *fn)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, fn);
    if (dev < 0 || dev >= kMaxDevices) return fail(QG_EUNSUPPORTED, "%s: device %d", fn, dev);
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_acquire);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return hip_fail(e, fn);
            if (p == nullptr) return fail(QG_EHIP, "%s: no device address for the scratch array", fn);
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return QG_OK;
}

qgk::F16Plan plan_f16(int64_t N, int64_t K, const void *w_f16, const float *x)
{
    qgk::F16Plan p;
    p.vec = (K % 8 == 0) && aligned(w_f16, 16) && aligned(x, 16);
    p.L = 0;
    p.cpl = 0;
    p.R = 1;
    const int64_t w_env = tune(kF16Waves);
    const int64_t form = tune(kF16Form);
    const int64_t nch = K / 8;
    const int64_t cpl_env = tune(kF16Cpl);
    const int64_t cpl = (cpl_env == 1 || cpl_env == 2 || cpl_env == 4) ? cpl_env : 4;
    const bool wsplit_ok = p.vec && nch <= 16 * 64 * cpl && N <= INT32_MAX;   // one workgroup per row
    if (wsplit_ok && (form == 2 || (form < 0 && N < 1024))) {
        p.cpl = (int)cpl;
        p.waves = (int)((nch + 64 * cpl - 1) / (64 * cpl));
        p.grid = N;
        return p;
    }
    const bool row_ok = p.vec && K % 512 == 0 && K / 512 <= qgk::kF16RowMaxL;
    if (row_ok && form != 0) {
        p.L = (int)(K / 512);
        p.waves = (w_env == 2 || w_env == 4 || w_env == 8) ? (int)w_env : (N < 1024 ? 2 : (N < 4096 ? 4 : 8));
        p.grid = (N + p.waves - 1) / p.waves;
        return p;
    }
    const int64_t r_env = tune(kF16Rows);
    if (r_env == 1 || r_env == 2 || r_env == 4) p.R = (int)r_env;
    int64_t waves = N >= 1024 ? 1 : 4;
    if (w_env > 0) waves = w_env;
    if (waves > 16) waves = 16;
    if (waves < 1) waves = 1;
    p.waves = (int)waves;
    p.grid = (N + p.R - 1) / p.R;
    return p;
}

}  // namespace

extern "C" {

size_t qg_packed_size(int qtype, int64_t N, int64_t K)
{
    if (!valid_qtype(qtype) || N <= 0 || K <= 0 || K % k_unit(qtype) || N > kMaxDim || K > kMaxDim) return 0;
    return (size_t)qgl::geometry(qtype, N, K).total;
}

qg_status qg_pack(int qtype, const void *canonical, void *packed, int64_t N, int64_t K, void *stream)
{
    return qg_pack_rows(qtype, canonical, packed, N, 0, N, K, stream);
}

qg_status qg_pack_rows(int qtype, const void *canonical, void *packed, int64_t N_total, int64_t row0, int64_t nrows,
                       int64_t K, void *stream)
{
    const char *fn = "qg_pack_rows";
    qg_status st = check_pack(qtype, canonical, packed, N_total, K, fn);
    if (st) return st;
    if (row0 < 0 || nrows <= 0 || row0 + nrows > N_total)
        return fail(QG_EINVAL, "%s: rows [%lld, %lld) outside [0, %lld)", fn, (long long)row0,
                    (long long)(row0 + nrows), (long long)N_total);
    if (!aligned(packed, 16)) return fail(QG_EALIGN, "%s: packed buffer must be 16-byte aligned", fn);
    const Geometry g = qgl::geometry(qtype, N_total, K);
    const size_t cbytes = (size_t)nrows * (size_t)qgl::canon_row_bytes(qtype, K);
    if (overlap(canonical, cbytes, packed, (size_t)g.total)) return fail(QG_EINVAL, "%s: buffers overlap", fn);
    const bool last = row0 + nrows == N_total;
    const int64_t rows_to_write = nrows + (last ? g.n_tiles * qgl::kTileRows - N_total : 0);
    hipError_t e = qgk::launch_pack(g, (const uint8_t *)canonical, nullptr, (uint8_t *)packed, qgk::kPackRows, row0,
                                    nrows, rows_to_write, last, as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

qg_status qg_pack_gateup(int qtype, const void *gate, const void *up, void *packed, int64_t N_ff, int64_t K,
                         void *stream)
{
    const char *fn = "qg_pack_gateup";
    qg_status st = check_pack(qtype, gate, packed, 2 * N_ff, K, fn);
    if (st) return st;
    if (!up) return fail(QG_EINVAL, "%s: null pointer", fn);
    if (!aligned(packed, 16)) return fail(QG_EALIGN, "%s: packed buffer must be 16-byte aligned", fn);
    const Geometry g = qgl::geometry(qtype, 2 * N_ff, K);
    const size_t cbytes = (size_t)N_ff * (size_t)qgl::canon_row_bytes(qtype, K);
    if (overlap(gate, cbytes, packed, (size_t)g.total) || overlap(up, cbytes, packed, (size_t)g.total))
        return fail(QG_EINVAL, "%s: buffers overlap", fn);
    hipError_t e = qgk::launch_pack(g, (const uint8_t *)gate, (const uint8_t *)up, (uint8_t *)packed,
                                    qgk::kPackGateUp, 0, 2 * N_ff, g.n_tiles * qgl::kTileRows, true,
                                    as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

qg_status qg_pack_host(int qtype, const void *canonical_host, void *packed_host, int64_t N, int64_t K)
{
    qg_status st = check_pack(qtype, canonical_host, packed_host, N, K, "qg_pack_host");
    if (st) return st;
    const Geometry g = qgl::geometry(qtype, N, K);
    memset(packed_host, 0, (size_t)g.total);
    host_pack_rows(g, (const uint8_t *)canonical_host, (uint8_t *)packed_host, 0, N, true);
    return ok();
}

qg_status qg_unpack_host(int qtype, const void *packed_host, void *canonical_host, int64_t N, int64_t K)
{
    qg_status st = check_pack(qtype, canonical_host, packed_host, N, K, "qg_unpack_host");
    if (st) return st;
    const Geometry g = qgl::geometry(qtype, N, K);
    const int64_t rb = qgl::canon_row_bytes(qtype, K);
    if (super_block_qtype(qtype))   // Q4_K / Q6_K blocks are OR-ed into their super-blocks
        memset(canonical_host, 0, (size_t)(N * rb));
    for (int64_t r = 0; r < N; ++r)
        for (int64_t b = 0; b < g.KB; ++b)
            qgl::unpack_block(g, (const uint8_t *)packed_host, (uint8_t *)canonical_host + r * rb, r, b);
    return ok();
}

qg_status qg_pack_gateup_host(int qtype, const void *gate_host, const void *up_host, void *packed_host, int64_t N_ff,
                              int64_t K)
{
    qg_status st = check_pack(qtype, gate_host, packed_host, 2 * N_ff, K, "qg_pack_gateup_host");
    if (st) return st;
    if (!up_host) return fail(QG_EINVAL, "qg_pack_gateup_host: null pointer");
    const Geometry g = qgl::geometry(qtype, 2 * N_ff, K);
    const int64_t rb = qgl::canon_row_bytes(qtype, K);
    memset(packed_host, 0, (size_t)g.total);
    for (int64_t v = 0; v < 2 * N_ff; ++v) {
        const uint8_t *base = (const uint8_t *)((v & 1) ? up_host : gate_host);
        for (int64_t b = 0; b < g.KB; ++b) qgl::pack_block(g, base + (v >> 1) * rb, (uint8_t *)packed_host, v, b);
    }
    for (int64_t v = 2 * N_ff; v < g.n_tiles * qgl::kTileRows; ++v)
        for (int64_t b = 0; b < g.KB; ++b) qgl::pack_block(g, nullptr, (uint8_t *)packed_host, v, b);
    return ok();
}

qg_status qgemv_q8_0(const void *w_packed, const float *x, float *y, int64_t N, int64_t K, void *stream)
{
    return run_qgemv(QG_Q8_0, qgk::kEpiPlain, w_packed, x, y, N, N, K, 1, stream, "qgemv_q8_0");
}

qg_status qgemv_q4_0(const void *w_packed, const float *x, float *y, int64_t N, int64_t K, void *stream)
{
    return run_qgemv(QG_Q4_0, qgk::kEpiPlain, w_packed, x, y, N, N, K, 1, stream, "qgemv_q4_0");
}

qg_status qgemv_epilogue(int qtype, const void *w_packed, const float *x, const float *bias, const float *residual,
                         void *y, int out_type, int64_t N, int64_t K, void *stream)
{
    Affine af;
    af.bias = bias;
    af.residual = residual;
    af.out_type = out_type;
    return run_qgemv(qtype, qgk::kEpiAffine, w_packed, x, y, N, N, K, 1, stream, "qgemv_epilogue", af);
}

qg_status qgemv_rmsnorm(int qtype, const void *w_packed, const float *x, const float *gamma, float eps, float *y,
                        int64_t N, int64_t K, void *stream)
{
    Norm nm;
    nm.on = true;
    nm.gamma = gamma;
    nm.eps = eps;
    return run_qgemv(qtype, qgk::kEpiPlain, w_packed, x, y, N, N, K, 1, stream, "qgemv_rmsnorm", Affine(), nm);
}

qg_status qgemv_rmsnorm_gateup_silu(int qtype, const void *w_gateup_packed, const float *x, const float *gamma,
                                    float eps, float *y, int64_t N_ff, int64_t K, void *stream)
{
    if (N_ff <= 0 || N_ff > kMaxDim)
        return fail(QG_EINVAL, "qgemv_rmsnorm_gateup_silu: N_ff=%lld", (long long)N_ff);
    Norm nm;
    nm.on = true;
    nm.gamma = gamma;
    nm.eps = eps;
    return run_qgemv(qtype, qgk::kEpiGateUp, w_gateup_packed, x, y, 2 * N_ff, N_ff, K, 1, stream,
                     "qgemv_rmsnorm_gateup_silu", Affine(), nm);
}

qg_status qg_rmsnorm(const float *x, const float *gamma, float eps, float *out, int64_t K, void *stream)
{
    const char *fn = "qg_rmsnorm";
    if (K <= 0 || K > kMaxDim) return fail(QG_EINVAL, "%s: K=%lld must be positive", fn, (long long)K);
    if (!x || !gamma || !out) return fail(QG_EINVAL, "%s: null pointer", fn);
    if (!aligned(x, 4) || !aligned(gamma, 4) || !aligned(out, 4))
        return fail(QG_EALIGN, "%s: x, gamma and out must be 4-byte aligned", fn);
    if (!(eps >= 0.0f) || eps == __builtin_inff()) return fail(QG_EINVAL, "%s: eps must be finite and >= 0", fn);
    const size_t nb = (size_t)K * sizeof(float);
    if (overlap(out, nb, x, nb) || overlap(out, nb, gamma, nb))
        return fail(QG_EINVAL, "%s: out overlaps x or gamma", fn);
    hipError_t e = qgk::launch_rmsnorm(x, gamma, eps, out, K, as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

// ---- small-M GEMM (prefill chunks) ------------------------------------------

size_t qg_prefill_workspace_size(int qtype, int64_t N, int64_t K, int64_t M)
{
    if (!valid_qtype(qtype) || super_block_qtype(qtype) || N <= 0 || N > kMaxDim || M <= 0 || M > kGemmMaxM || K <= 0 ||
        K % 32 ||
        K > kMaxDim)
        return 0;
    return plan_gemm(qtype, N, K, M).bytes;
}

qg_status qgemm_prefill(int qtype, const void *w_packed, const float *X, float *Y, int64_t N, int64_t K, int64_t M,
                        void *workspace, size_t workspace_bytes, void *stream)
{
    const char *fn = "qgemm_prefill";
    qg_status st = check_prefill(qtype, w_packed, X, Y, N, K, M, fn);
    if (st) return st;
    if (!workspace) return fail(QG_EINVAL, "%s: null pointer", fn);
    if (!aligned(workspace, 256)) return fail(QG_EALIGN, "%s: workspace must be 256-byte aligned", fn);
    const size_t need = plan_gemm(qtype, N, K, M).bytes;
    if (workspace_bytes < need)
        return fail(QG_EINVAL, "%s: workspace of %zu bytes, %zu needed (qg_prefill_workspace_size)", fn,
                    workspace_bytes, need);
    st = check_prefill_overlap(qtype, w_packed, X, Y, N, K, M, fn);
    if (st) return st;
    const Geometry g = qgl::geometry(qtype, N, K);
    const size_t xb = (size_t)M * (size_t)K * sizeof(float), yb = (size_t)M * (size_t)N * sizeof(float);
    if (overlap(Y, yb, workspace, need)) return fail(QG_EINVAL, "%s: Y overlaps X, the weights or the workspace", fn);
    if (overlap(workspace, need, X, xb) || overlap(workspace, need, w_packed, (size_t)g.total))
        return fail(QG_EINVAL, "%s: the workspace overlaps X or the weights", fn);
    return run_prefill(qtype, w_packed, X, Y, N, K, M, workspace, stream, fn);
}

qg_status qgemm_prefill_noalloc(int qtype, const void *w_packed, const float *X, float *Y, int64_t N, int64_t K,
                                int64_t M, void *stream)
{
    const char *fn = "qgemm_prefill_noalloc";
    qg_status st = check_prefill(qtype, w_packed, X, Y, N, K, M, fn);
    if (st) return st;
    st = check_prefill_overlap(qtype, w_packed, X, Y, N, K, M, fn);
    if (st) return st;
    const size_t need = plan_gemm(qtype, N, K, M).bytes;
    if (need > kNoAllocScratchBytes)
        return fail(QG_EUNSUPPORTED,
                    "%s: this shape needs %zu bytes of scratch, above the %zu bytes the library holds per GPU "
                    "(call qgemm_prefill with a workspace of qg_prefill_workspace_size bytes)",
                    fn, need, kNoAllocScratchBytes);
    void *ws = nullptr;
    st = scratch_address(&ws, fn);
    if (st) return st;
    return run_prefill(qtype, w_packed, X, Y, N, K, M, ws, stream, fn);
}

qg_status qgemv_q4_k(const void *w_packed, const float *x, float *y, int64_t N, int64_t K, void *stream)
{
    return run_qgemv(QG_Q4_K, qgk::kEpiPlain, w_packed, x, y, N, N, K, 1, stream, "qgemv_q4_k");
}

qg_status qgemv_q6_k(const void *w_packed, const float *x, float *y, int64_t N, int64_t K, void *stream)
{
    return run_qgemv(QG_Q6_K, qgk::kEpiPlain, w_packed, x, y, N, N, K, 1, stream, "qgemv_q6_k");
}

qg_status qgemv_fused_gateup_silu(int qtype, const void *w_gateup_packed, const float *x, float *y, int64_t N_ff,
                                  int64_t K, void *stream)
{
    if (N_ff <= 0 || N_ff > kMaxDim) return fail(QG_EINVAL, "qgemv_fused_gateup_silu: N_ff=%lld", (long long)N_ff);
    return run_qgemv(qtype, qgk::kEpiGateUp, w_gateup_packed, x, y, 2 * N_ff, N_ff, K, 1, stream,
                     "qgemv_fused_gateup_silu");
}

qg_status qgemv_verify(int qtype, const void *w_packed, const float *X, float *Y, int64_t N, int64_t K, int M,
                       void *stream)
{
    if (M < 2 || M > 6) return fail(QG_EUNSUPPORTED, "qgemv_verify: M=%d outside 2..6", M);
    return run_qgemv(qtype, qgk::kEpiPlain, w_packed, X, Y, N, N, K, M, stream, "qgemv_verify");
}

qg_status gemv_f16_splitk(const void *w_f16, const float *x, float *y, int64_t N, int64_t K, void *stream)
{
    const char *fn = "gemv_f16_splitk";
    if (N <= 0 || K <= 0 || N > kMaxDim || K > kMaxDim)
        return fail(QG_EINVAL, "%s: N=%lld K=%lld must be positive", fn, (long long)N, (long long)K);
    if (!w_f16 || !x || !y) return fail(QG_EINVAL, "%s: null pointer", fn);
    if (!aligned(w_f16, 2)) return fail(QG_EALIGN, "%s: weights must be 2-byte aligned", fn);
    if (!aligned(x, 4) || !aligned(y, 4)) return fail(QG_EALIGN, "%s: x and y must be 4-byte aligned", fn);
    if (overlap(y, (size_t)N * 4, x, (size_t)K * 4)) return fail(QG_EINVAL, "%s: y overlaps x", fn);
    if (overlap(y, (size_t)N * 4, w_f16, (size_t)N * (size_t)K * 2))
        return fail(QG_EINVAL, "%s: y overlaps the weights", fn);

    const qgk::F16Plan p = plan_f16(N, K, w_f16, x);
    hipError_t e = qgk::launch_f16(p, (const uint16_t *)w_f16, x, y, N, K, as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

const char *qg_status_str(int status)
{
    switch (status) {
    case QG_OK: return "QG_OK";
    case QG_EINVAL: return "QG_EINVAL: invalid argument";
    case QG_EALIGN: return "QG_EALIGN: misaligned pointer";
    case QG_EUNSUPPORTED: return "QG_EUNSUPPORTED: unsupported type or row count";
    case QG_EHIP: return "QG_EHIP: HIP runtime error";
    default: return "unknown qg_status";
    }
}

const char *qg_last_error(void) { return g_last_error.c_str(); }

qg_status qg_plan_info(int qtype, int64_t N, int64_t K, int M, int rmsnorm, int *split_k_ways, int64_t *workgroups,
                       int *x_in_lds, int *persistent, int64_t *lds_bytes)
{
    qg_status st = check_qshape(qtype, N, K, "qg_plan_info");
    if (st) return st;
    if (M < 1 || M > 6) return fail(QG_EUNSUPPORTED, "qg_plan_info: M=%d", M);
    const bool norm = rmsnorm != 0;
    if (norm && M != 1) return fail(QG_EUNSUPPORTED, "qg_plan_info: the RMSNorm prologue takes M = 1");
    if (norm && K > kNormMaxK)
        return fail(QG_EUNSUPPORTED, "qg_plan_info: K=%lld above %lld (the normalised activations live in LDS)",
                    (long long)K, (long long)kNormMaxK);
    qgk::QPlan p = make_qplan(qtype, N, K, M, norm);
    if (norm && !p.x_in_lds) return fail(QG_EUNSUPPORTED, "qg_plan_info: activations do not fit in LDS");
    // a verify call (M >= 2, plain store) as qgemv_verify launches it
    const int groups = verify_row_groups(qtype, N, K, M, p, qgk::kEpiPlain, norm);
    if (groups > 1) {
        p = make_qplan(qtype, N, K, M / groups, false);
        M /= groups;
    }
    if (split_k_ways) *split_k_ways = p.W;
    if (workgroups) *workgroups = p.grid * groups;
    if (x_in_lds) *x_in_lds = p.x_in_lds ? 1 : 0;
    if (persistent) *persistent = p.persist ? 1 : 0;
    if (lds_bytes) {
        const int floats = p.persist ? qgk::persist_red_floats(norm) : qgk::tile_red_floats(M, p.W, norm);
        *lds_bytes = (int64_t)(qgk::static_lds_bytes(floats) + p.lds_bytes);
    }
    return ok();
}

qg_status qg_f16_plan_info(int64_t N, int64_t K, const void *w_f16, const float *x, int *form, int *waves,
                           int64_t *workgroups)
{
    if (N <= 0 || K <= 0 || N > kMaxDim || K > kMaxDim)
        return fail(QG_EINVAL, "qg_f16_plan_info: N=%lld K=%lld must be positive", (long long)N, (long long)K);
    const qgk::F16Plan p = plan_f16(N, K, w_f16, x);
    if (form) *form = p.cpl > 0 ? 2 : (p.L > 0 ? 1 : 0);
    if (waves) *waves = p.waves;
    if (workgroups) *workgroups = p.grid;
    return ok();
}

qg_status qg_probe_stream(const void *buf, size_t bytes, uint32_t *sink, void *stream)
{
    const char *fn = "qg_probe_stream";
    if (!buf || !sink) return fail(QG_EINVAL, "%s: null pointer", fn);
    if (bytes == 0 || bytes % 1024 != 0 || bytes > ((size_t)1 << 40))
        return fail(QG_EINVAL, "%s: bytes=%zu must be a positive multiple of 1024", fn, bytes);
    if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(QG_EALIGN, "%s: buf 16-byte, sink 4-byte aligned", fn);
    if (overlap(sink, 4, buf, bytes)) return fail(QG_EINVAL, "%s: sink overlaps buf", fn);
    hipError_t e = qgk::launch_probe_stream(buf, bytes, sink, 0x9E3779B9u, as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

qg_status qg_probe_empty(void *stream)
{
    hipError_t e = qgk::launch_probe_empty(as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, "qg_probe_empty");
    return ok();
}

qg_status qg_reload_tuning(void)
{
    load_tuning();
    return ok();
}

qg_status qg_time_next_launch(void *start_event, void *stop_event)
{
    if ((start_event == nullptr) != (stop_event == nullptr))
        return fail(QG_EINVAL, "qg_time_next_launch: give both events or neither");
    qgk::set_launch_events((hipEvent_t)start_event, (hipEvent_t)stop_event);
    return ok();
}

}  // extern "C"
