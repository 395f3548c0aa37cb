// C ABI of the fused fp32 linear layer (include/lin_epi.h): argument
// validation, kernel selection, workspace management and optional per-kernel
// timing.  Kernels live in gemm_mfma.hpp and epilogue.hpp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <new>
#include <vector>

#include "gemm_mfma.hpp"
#include "lin_epi.h"

using namespace lin_epi;

namespace {

// Tile table.  All use v_mfma_f32_32x32x2_f32 and two LDS stages; they
// differ in workgroup tile and wavefront count, and the dispatcher picks one
// per call (choose_plan below).  All stage 32-deep K steps with
// direct-to-LDS buffer loads (LDS figures below; rows padded to 36 floats,
// 12 % more, on the register-staged path used when a tile's rows of X or W
// span 1 GiB or more):
//   LARGE  256x256, 8 wavefronts (4x2, 64x128 each), 128 KiB LDS, 1 WG/CU
//   MID    128x256, 8 wavefronts (2x4, 64x64 each),   96 KiB LDS, 1 WG/CU
//   SMALL  128x128, 4 wavefronts (2x2, 64x64 each),   64 KiB LDS, 2 WG/CU
//   TINY    64x64,  4 wavefronts (2x2, 32x32 each),   32 KiB LDS, 4 WG/CU
//   SKINNY  32x128, 4 wavefronts (1x4, 32x32 each),  40 KiB LDS, 4 WG/CU:
//           few rows of X against a long stream of W rows (the small-M,
//           weight-streaming regime, where HBM rather than MFMA bounds);
//           small workgroups so that two or more share a CU and keep enough
//           weight bytes in flight
using CfgLarge = TileCfg<256, 256, 32, 4, 2, 1>;
using CfgMid = TileCfg<128, 256, 32, 2, 4, 1>;
using CfgSmall = TileCfg<128, 128, 32, 2, 2, 2>;
using CfgTiny = TileCfg<64, 64, 32, 2, 2, 4>;
using CfgSkinny = TileCfg<32, 128, 32, 1, 4, 4>;

enum CfgId { CFG_LARGE = 0, CFG_MID = 1, CFG_SMALL = 2, CFG_TINY = 3, CFG_SKINNY = 4, CFG_COUNT = 5 };

struct CfgInfo {
    int bm, bn, bk, wgs_per_cu;
    double efficiency;  // fraction of the CU's 2.4 GHz fp32 MFMA peak, fitted to MI355X timings
};

constexpr CfgInfo kCfgs[CFG_COUNT] = {
    {CfgLarge::BM, CfgLarge::BN, CfgLarge::BK, CfgLarge::WG_PER_CU, 0.94},
    {CfgMid::BM, CfgMid::BN, CfgMid::BK, CfgMid::WG_PER_CU, 0.90},
    {CfgSmall::BM, CfgSmall::BN, CfgSmall::BK, CfgSmall::WG_PER_CU, 0.88},
    {CfgTiny::BM, CfgTiny::BN, CfgTiny::BK, CfgTiny::WG_PER_CU, 0.80},
    {CfgSkinny::BM, CfgSkinny::BN, CfgSkinny::BK, CfgSkinny::WG_PER_CU, 0.60},
};
static_assert(CfgLarge::LDS_BYTES * CfgLarge::WG_PER_CU <= 160 * 1024 &&
                  CfgMid::LDS_BYTES * CfgMid::WG_PER_CU <= 160 * 1024 &&
                  CfgSmall::LDS_BYTES * CfgSmall::WG_PER_CU <= 160 * 1024 &&
                  CfgTiny::LDS_BYTES * CfgTiny::WG_PER_CU <= 160 * 1024 &&
                  CfgSkinny::LDS_BYTES * CfgSkinny::WG_PER_CU <= 160 * 1024,
              "LDS budget");

// Time-model constants of the planner, fitted (with the efficiencies above)
// to 177 timed (shape, tail, configuration, split) combinations over 15
// problems on MI355X, each timed after 60 ms of warm-up so the engine clock
// has ramped up; the chosen plan is the measured best for 10 of them and
// within 6 % for the rest (all under 1 % but two problems under 0.1 ms).
constexpr double kCuPeakFlops = 256.0 * 2.4e9;  // fp32 MFMA FLOP/s of one CU at the 2.4 GHz peak clock
constexpr double kRoundFixedS = 5e-6;           // per round of workgroups: first loads, epilogue, drain
constexpr double kPassFixedS = 2e-6;            // one more kernel on the stream
constexpr double kPassBytesPerS = 4e12;         // sustained HBM rate of the second passes
constexpr double kGemmBytesPerS = 6.2e12;       // sustained HBM rate of a weight-streaming GEMM
constexpr double kSingleStreamRate = 0.7;       // fraction of it with fewer than 2 workgroups per CU

struct PendingTiming {
    int role;
    hipEvent_t start, stop;
};

}  // namespace

struct lin_epi_ctx {
    hipStream_t stream = nullptr;
    int device = -1;
    int num_cus = 0;
    void *ws = nullptr;
    size_t ws_bytes = 0;
    int64_t split_opt = 0;
    int64_t tile_opt = 0;
    bool profile = false;
    bool unfused = false;
    bool reg_staging = false;
    bool has_plan = false;
    lin_epi_plan plan{};
    std::vector<PendingTiming> pending;
    std::vector<hipEvent_t> spare_events;  // recycled by lin_epi_profile_read
    lin_epi_profile prof{};
};

namespace {

int ensure_device(lin_epi_ctx *h)
{
    if (h->device >= 0) return LIN_EPI_OK;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return LIN_EPI_EHIP;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return LIN_EPI_EHIP;
    h->device = dev;
    h->num_cus = cus > 0 ? cus : 256;
    return LIN_EPI_OK;
}

int ensure_workspace(lin_epi_ctx *h, size_t bytes)
{
    if (bytes <= h->ws_bytes) return LIN_EPI_OK;
    if (h->ws) {
        // A run still in flight on this stream may be using the old buffer.
        if (hipStreamSynchronize(h->stream) != hipSuccess) return LIN_EPI_EHIP;
        (void)hipFree(h->ws);
        h->ws = nullptr;
        h->ws_bytes = 0;
    }
    const size_t rounded = (bytes + (1u << 20) - 1) & ~(size_t)((1u << 20) - 1);
    if (hipMalloc(&h->ws, rounded) != hipSuccess) {
        (void)hipGetLastError();
        h->ws = nullptr;
        return LIN_EPI_ENOMEM;
    }
    h->ws_bytes = rounded;
    return LIN_EPI_OK;
}

// An event for profiling, reused from earlier reads when possible so that a
// timed launch costs two event records and no event creation.
int take_event(lin_epi_ctx *h, hipEvent_t *e)
{
    if (!h->spare_events.empty()) {
        *e = h->spare_events.back();
        h->spare_events.pop_back();
        return LIN_EPI_OK;
    }
    return hipEventCreate(e) == hipSuccess ? LIN_EPI_OK : LIN_EPI_EHIP;
}

template <typename Launch>
int timed_launch(lin_epi_ctx *h, int role, Launch &&launch)
{
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (h->profile) {
        if (take_event(h, &e0) != LIN_EPI_OK) return LIN_EPI_EHIP;
        if (take_event(h, &e1) != LIN_EPI_OK) {
            h->spare_events.push_back(e0);
            return LIN_EPI_EHIP;
        }
        if (hipEventRecord(e0, h->stream) != hipSuccess) {
            h->spare_events.push_back(e0);
            h->spare_events.push_back(e1);
            return LIN_EPI_EHIP;
        }
    }
    launch();
    const bool launched = hipGetLastError() == hipSuccess;
    if (h->profile) {
        if (!launched || hipEventRecord(e1, h->stream) != hipSuccess) {
            // e0 may already be recorded; drop both rather than reuse them
            (void)hipEventDestroy(e0);
            (void)hipEventDestroy(e1);
            return LIN_EPI_EHIP;
        }
        h->pending.push_back({role, e0, e1});
    }
    return launched ? LIN_EPI_OK : LIN_EPI_EHIP;
}

// reg_staging: stage operands through registers even where the buffer-load
// (direct-to-LDS) path is usable (LIN_EPI_OPT_REG_STAGING).
template <class Cfg, int EPI>
void launch_gemm_cfg(const GemmArgs &g, int64_t grid_x, int split, hipStream_t s, bool reg_staging)
{
    const dim3 grid((unsigned)grid_x, (unsigned)split), block(Cfg::THREADS);
    if constexpr (Cfg::BUFLOAD) {
        // buffer loads while a tile's rows of X and W span less than the window
        if (!reg_staging && (int64_t)std::max(Cfg::BM, Cfg::BN) * g.K * 4 < kBufferWindow) {
            hipLaunchKernelGGL((gemm_epi_kernel<Cfg, EPI, true>), grid, block, 0, s, g);
            return;
        }
    }
    hipLaunchKernelGGL((gemm_epi_kernel<Cfg, EPI, false>), grid, block, 0, s, g);
}

template <int EPI>
void launch_gemm(int cfg, const GemmArgs &g, int64_t grid_x, int split, hipStream_t s, bool reg_staging)
{
    switch (cfg) {
        case CFG_LARGE: launch_gemm_cfg<CfgLarge, EPI>(g, grid_x, split, s, reg_staging); break;
        case CFG_MID: launch_gemm_cfg<CfgMid, EPI>(g, grid_x, split, s, reg_staging); break;
        case CFG_SMALL: launch_gemm_cfg<CfgSmall, EPI>(g, grid_x, split, s, reg_staging); break;
        case CFG_TINY: launch_gemm_cfg<CfgTiny, EPI>(g, grid_x, split, s, reg_staging); break;
        default: launch_gemm_cfg<CfgSkinny, EPI>(g, grid_x, split, s, reg_staging); break;
    }
}

template <int EPI>
void launch_reduce(const float *P, const float *bias, float *Y, int64_t MN, int N, int S, TailParams t,
                   hipStream_t s)
{
    const int32_t vec4 = (N % 4 == 0) && (((uintptr_t)Y & 15u) == 0) && (((uintptr_t)P & 15u) == 0);
    int64_t blocks = ((vec4 ? MN / 4 : MN) + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL((splitk_reduce_kernel<EPI>), dim3((unsigned)blocks), dim3(256), 0, s, P, bias, Y, MN, N, S, t,
                       vec4);
}

struct Plan {
    int cfg;
    int split;
    int64_t k_slice;
    int tiles_m, tiles_n;
};

// Pick the tile configuration and the number of K slices by estimated time.
// For each configuration and slice count S (1..16, at most one per K step):
//   units = tiles * S workgroups, each computing a BM x BN tile over
//   ceil(steps / S) K steps; the busiest CU runs load = ceil(units / CUs) of
//   them, w = WG_PER_CU at a time, sharing its matrix pipes, so
//     t_gemm = ceil(load / w) * t_round + load * 2*BM*BN*k_slice / (peak * eff)
//   (but never less than the time to stream W and X from HBM once, 1/0.7
//   times longer when fewer than two workgroups per CU stream), and a
//   second pass (split-K or row-max finalize) costs
//     t_pass = t_launch + (S + 1) * M * N * 4 bytes / HBM rate   (S > 1)
//            = t_launch                                          (S = 1, row max)
// Padding waste is included (a tile's work counts in full).  The fastest
// estimate wins; LIN_EPI_OPT_SPLIT_K = 1 forbids a split and S >= 2 forces
// one (clamped to the K steps available, so every slice owns at least one).
// For the row-max tails a split moves pooling, GELU and the max into the
// second pass, which reads complete sums.
Plan choose_plan(const lin_epi_ctx *h, int64_t M, int64_t N, int64_t K, int kind, int num_cus)
{
    Plan best{CFG_SMALL, 1, 0, 0, 0};
    double best_t = 1e300;
    // (every configuration that is not excluded by the override scores at
    // least S = 1, so `best` is always set)
    const bool rowmax = kind == LIN_EPI_POOL_GELU_SCALE_ROWMAX || kind == LIN_EPI_GELU_SCALE_ROWMAX;
    for (int c = 0; c < CFG_COUNT; ++c) {
        const CfgInfo &ci = kCfgs[c];
        const int64_t tm = (M + ci.bm - 1) / ci.bm, tn = (N + ci.bn - 1) / ci.bn;
        const int64_t tiles = tm * tn;
        const int64_t steps = (K + ci.bk - 1) / ci.bk;
        if (h->tile_opt > 0 && c != h->tile_opt - 1) continue;
        int s_lo = 1, s_hi = (int)std::min<int64_t>(16, std::max<int64_t>(steps, 1));
        if (h->split_opt == 1) s_hi = 1;
        if (h->split_opt >= 2) s_lo = s_hi = (int)std::min<int64_t>(h->split_opt, std::max<int64_t>(steps, 1));
        for (int S = s_lo; S <= s_hi; ++S) {
            const int64_t units = tiles * S;
            const int64_t load = (units + num_cus - 1) / num_cus;
            const int64_t kslice = ((steps + S - 1) / S) * ci.bk;
            const double wg_flops = 2.0 * ci.bm * ci.bn * (double)kslice;
            double t = (double)((load + ci.wgs_per_cu - 1) / ci.wgs_per_cu) * kRoundFixedS +
                       (double)load * wg_flops / (kCuPeakFlops * ci.efficiency);
            // every byte of W (and of X) crosses HBM at least once, at the
            // full rate only with two or more workgroups per CU streaming
            double t_hbm = 4.0 * ((double)N * K + (double)M * K) / kGemmBytesPerS;
            if (units < 2 * (int64_t)num_cus) t_hbm /= kSingleStreamRate;
            t = std::max(t, t_hbm);
            if (S > 1)
                t += kPassFixedS + (S + 1) * (double)M * (double)N * 4.0 / kPassBytesPerS;
            else if (rowmax)
                t += kPassFixedS;
            if (t < best_t) {
                best_t = t;
                best = Plan{c, S, 0, (int)tm, (int)tn};
            }
        }
    }
    const CfgInfo &ci = kCfgs[best.cfg];
    const int64_t steps = (K + ci.bk - 1) / ci.bk;
    if (best.split > 1 && steps > 0) {
        best.k_slice = (steps + best.split - 1) / best.split * ci.bk;
        best.split = (int)((K + best.k_slice - 1) / best.k_slice);
    }
    if (best.split <= 1) {
        best.split = 1;
        best.k_slice = steps > 0 ? steps * ci.bk : ci.bk;
    }
    return best;
}

bool is_rowmax(int kind)
{
    return kind == LIN_EPI_POOL_GELU_SCALE_ROWMAX || kind == LIN_EPI_GELU_SCALE_ROWMAX;
}

// The launch plan of one lin_epi_run call: tile configuration and K slices
// from choose_plan, then the kernels the chosen path launches and the
// workspace it needs.
//   fused, no split:       GEMM+tail (1 kernel); row-max kinds add the
//                          finalize pass and M*tiles_n partial maxima
//   fused, split S:        GEMM partials [S,M,N] + second pass (2 kernels)
//   unfused ablation:      GEMM (+ reduce if split) to raw y, then a tail
//                          kernel (none for kind 0); raw y for the row-max
//                          kinds lives in the workspace after the partials
lin_epi_plan describe(const lin_epi_ctx *h, const Plan &pl, int64_t M, int64_t N, int kind)
{
    lin_epi_plan p{};
    p.tile_m = kCfgs[pl.cfg].bm;
    p.tile_n = kCfgs[pl.cfg].bn;
    p.tile_k = kCfgs[pl.cfg].bk;
    p.split_k = pl.split;
    p.grid_main = (int64_t)pl.tiles_m * pl.tiles_n * pl.split;
    const int64_t MN = M * N;
    const int64_t partials = pl.split > 1 ? (int64_t)pl.split * MN : 0;
    if (h->unfused) {
        p.kernels = (pl.split > 1 ? 2 : 1) + (kind != LIN_EPI_NONE ? 1 : 0);
        p.workspace_bytes = (partials + (is_rowmax(kind) ? MN : 0)) * (int64_t)sizeof(float);
    } else if (pl.split > 1) {
        p.kernels = 2;
        p.workspace_bytes = partials * (int64_t)sizeof(float);
    } else if (is_rowmax(kind)) {
        p.kernels = 2;
        p.workspace_bytes = M * pl.tiles_n * (int64_t)sizeof(float);
    } else {
        p.kernels = 1;
        p.workspace_bytes = 0;
    }
    return p;
}

// Host-side argument checks shared by lin_epi_run and lin_epi_query_plan.
int validate_desc(int64_t M, int64_t N, int64_t K, const lin_epi_desc *desc)
{
    if (!desc) return LIN_EPI_EINVAL;
    if (M < 0 || N < 0 || K < 0) return LIN_EPI_EINVAL;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return LIN_EPI_EINVAL;
    const int kind = desc->kind;
    if (kind < LIN_EPI_NONE || kind > LIN_EPI_GELU_SCALE_ROWMAX) return LIN_EPI_EINVAL;
    if (kind == LIN_EPI_SCALE_HARDTANH_GELU && !(desc->ht_min <= desc->ht_max)) return LIN_EPI_EINVAL;
    if (kind == LIN_EPI_POOL_GELU_SCALE_ROWMAX) {
        if (desc->pool_kernel != 16 || desc->pool_stride != desc->pool_kernel) return LIN_EPI_ENOTSUP;
        if (N > 0 && N < 16) return LIN_EPI_ENOTSUP;
    }
    if (K % 4 != 0) return LIN_EPI_EALIGN;
    return LIN_EPI_OK;
}

}  // namespace

extern "C" {

const char *lin_epi_status_string(int status)
{
    switch (status) {
        case LIN_EPI_OK: return "ok";
        case LIN_EPI_EINVAL: return "invalid argument";
        case LIN_EPI_EALIGN: return "misaligned pointer or K not a multiple of 4";
        case LIN_EPI_ENOTSUP: return "unsupported tail parameters";
        case LIN_EPI_ENOMEM: return "device workspace allocation failed";
        case LIN_EPI_EHIP: return "HIP call or kernel launch failed";
        default: return "unknown status";
    }
}

int lin_epi_create(lin_epi_handle *out, void *hip_stream)
{
    if (!out) return LIN_EPI_EINVAL;
    *out = nullptr;
    lin_epi_ctx *h = new (std::nothrow) lin_epi_ctx();
    if (!h) return LIN_EPI_ENOMEM;
    h->stream = reinterpret_cast<hipStream_t>(hip_stream);
    *out = h;
    return LIN_EPI_OK;
}

int lin_epi_destroy(lin_epi_handle h)
{
    if (!h) return LIN_EPI_OK;
    int rc = LIN_EPI_OK;
    if (h->ws || !h->pending.empty()) {
        if (hipStreamSynchronize(h->stream) != hipSuccess) rc = LIN_EPI_EHIP;
    }
    for (auto &p : h->pending) {
        (void)hipEventDestroy(p.start);
        (void)hipEventDestroy(p.stop);
    }
    for (hipEvent_t e : h->spare_events) (void)hipEventDestroy(e);
    if (h->ws) (void)hipFree(h->ws);
    delete h;
    return rc;
}

int lin_epi_set_option(lin_epi_handle h, int32_t option, int64_t value)
{
    if (!h) return LIN_EPI_EINVAL;
    switch (option) {
        case LIN_EPI_OPT_SPLIT_K:
            if (value < 0 || value > 64) return LIN_EPI_EINVAL;
            h->split_opt = value;
            return LIN_EPI_OK;
        case LIN_EPI_OPT_PROFILE:
            if (value != 0 && value != 1) return LIN_EPI_EINVAL;
            h->profile = value != 0;
            return LIN_EPI_OK;
        case LIN_EPI_OPT_TILE:
            if (value < 0 || value > CFG_COUNT) return LIN_EPI_EINVAL;
            h->tile_opt = value;
            return LIN_EPI_OK;
        case LIN_EPI_OPT_UNFUSED:
            if (value != 0 && value != 1) return LIN_EPI_EINVAL;
            h->unfused = value != 0;
            return LIN_EPI_OK;
        case LIN_EPI_OPT_REG_STAGING:
            if (value != 0 && value != 1) return LIN_EPI_EINVAL;
            h->reg_staging = value != 0;
            return LIN_EPI_OK;
        default: return LIN_EPI_EINVAL;
    }
}

int lin_epi_last_plan(lin_epi_handle h, lin_epi_plan *out)
{
    if (!h || !out) return LIN_EPI_EINVAL;
    if (!h->has_plan) return LIN_EPI_EINVAL;
    *out = h->plan;
    return LIN_EPI_OK;
}

int lin_epi_profile_read(lin_epi_handle h, lin_epi_profile *out)
{
    if (!h || !out) return LIN_EPI_EINVAL;
    int rc = LIN_EPI_OK;
    if (!h->pending.empty()) {
        if (hipStreamSynchronize(h->stream) != hipSuccess) rc = LIN_EPI_EHIP;
        for (auto &p : h->pending) {
            float ms = 0.f;
            if (rc == LIN_EPI_OK && hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
                h->prof.launches[p.role] += 1;
                h->prof.total_ms[p.role] += ms;
            } else {
                rc = LIN_EPI_EHIP;
            }
            h->spare_events.push_back(p.start);
            h->spare_events.push_back(p.stop);
        }
        h->pending.clear();
    }
    *out = h->prof;
    h->prof = lin_epi_profile{};
    return rc;
}

int lin_epi_run(lin_epi_handle h, int64_t M, int64_t N, int64_t K, const float *X, const float *W, const float *b,
                const lin_epi_desc *desc, float *Y)
{
    // ---- validation: host only, before any HIP call
    if (!h) return LIN_EPI_EINVAL;
    int rc = validate_desc(M, N, K, desc);
    if (rc != LIN_EPI_OK && rc != LIN_EPI_EALIGN) return rc;
    if (M == 0 || N == 0) return LIN_EPI_OK;
    if (!b || !Y) return LIN_EPI_EINVAL;
    if (K > 0 && (!X || !W)) return LIN_EPI_EINVAL;
    if (rc != LIN_EPI_OK) return rc;
    if (K > 0 && (((uintptr_t)X | (uintptr_t)W) & 15u)) return LIN_EPI_EALIGN;
    if (((uintptr_t)Y | (uintptr_t)b) & 3u) return LIN_EPI_EALIGN;
    const int kind = desc->kind;

    rc = ensure_device(h);
    if (rc != LIN_EPI_OK) return rc;

    const bool rowmax = is_rowmax(kind);
    const bool unfused = h->unfused;
    const Plan pl = choose_plan(h, M, N, K, kind, h->num_cus);
    const int tiles_m = pl.tiles_m, tiles_n = pl.tiles_n;
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    const int split = pl.split;
    const int64_t MN = M * N;
    lin_epi_plan plan = describe(h, pl, M, N, kind);

    GemmArgs g{};
    g.X = X;
    g.W = W;
    g.bias = b;
    g.M = (int32_t)M;
    g.N = (int32_t)N;
    g.K = (int32_t)K;
    g.k_slice = (int32_t)pl.k_slice;
    g.tiles_m = tiles_m;
    g.tiles_n = tiles_n;
    g.tail = TailParams{desc->scale, desc->ht_min, desc->ht_max};

    hipStream_t s = h->stream;
    if (!unfused && rowmax && split > 1) {
        // Split-K partial sums -> one pass that adds the slices in order,
        // adds the bias, pools, applies GELU and the scale and takes the max.
        const size_t bytes = (size_t)split * MN * sizeof(float);
        rc = ensure_workspace(h, bytes);
        if (rc != LIN_EPI_OK) return rc;
        g.out = static_cast<float *>(h->ws);
        rc = timed_launch(h, 0, [&] { launch_gemm<EPI_SPLITK_PARTIAL>(pl.cfg, g, tiles, split, s, h->reg_staging); });
        if (rc != LIN_EPI_OK) return rc;
        const float *P = static_cast<const float *>(h->ws);
        const int32_t pool = kind == LIN_EPI_POOL_GELU_SCALE_ROWMAX ? 16 : 1;
        const float scale = desc->scale;
        const int32_t Ni = (int32_t)N;
        rc = timed_launch(h, 1, [&] {
            hipLaunchKernelGGL(rowmax_pass_kernel, dim3((unsigned)M), dim3(256), 0, s, P, b, Y, MN, Ni, split, pool,
                               scale, (int32_t)(N % 4 == 0));
        });
        if (rc != LIN_EPI_OK) return rc;
    } else if (!unfused && rowmax) {
        // GEMM with the row-max epilogue -> per-(row, column tile) partials ->
        // deterministic max over column tiles.
        const size_t bytes = (size_t)M * tiles_n * sizeof(float);
        rc = ensure_workspace(h, bytes);
        if (rc != LIN_EPI_OK) return rc;
        g.out = static_cast<float *>(h->ws);
        rc = timed_launch(h, 0, [&] {
            if (kind == LIN_EPI_POOL_GELU_SCALE_ROWMAX)
                launch_gemm<EPI_POOL_GELU_SCALE_ROWMAX>(pl.cfg, g, tiles, 1, s, h->reg_staging);
            else
                launch_gemm<EPI_GELU_SCALE_ROWMAX>(pl.cfg, g, tiles, 1, s, h->reg_staging);
        });
        if (rc != LIN_EPI_OK) return rc;
        const float *part = static_cast<const float *>(h->ws);
        const int32_t Mi = (int32_t)M;
        rc = timed_launch(h, 1, [&] {
            hipLaunchKernelGGL(rowmax_finalize_kernel, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, part, Y, Mi,
                               (int32_t)tiles_n);
        });
        if (rc != LIN_EPI_OK) return rc;
    } else if (!unfused && split > 1) {
        const size_t bytes = (size_t)split * MN * sizeof(float);
        rc = ensure_workspace(h, bytes);
        if (rc != LIN_EPI_OK) return rc;
        g.out = static_cast<float *>(h->ws);
        rc = timed_launch(h, 0, [&] { launch_gemm<EPI_SPLITK_PARTIAL>(pl.cfg, g, tiles, split, s, h->reg_staging); });
        if (rc != LIN_EPI_OK) return rc;
        const float *P = static_cast<const float *>(h->ws);
        rc = timed_launch(h, 1, [&] {
            switch (kind) {
                case LIN_EPI_NONE: launch_reduce<EPI_NONE>(P, b, Y, MN, (int)N, split, g.tail, s); break;
                case LIN_EPI_SCALE_HARDTANH_GELU:
                    launch_reduce<EPI_SCALE_HARDTANH_GELU>(P, b, Y, MN, (int)N, split, g.tail, s);
                    break;
                default: launch_reduce<EPI_SWISH_SCALE>(P, b, Y, MN, (int)N, split, g.tail, s); break;
            }
        });
        if (rc != LIN_EPI_OK) return rc;
    } else if (!unfused) {
        g.out = Y;
        rc = timed_launch(h, 0, [&] {
            switch (kind) {
                case LIN_EPI_NONE: launch_gemm<EPI_NONE>(pl.cfg, g, tiles, 1, s, h->reg_staging); break;
                case LIN_EPI_SCALE_HARDTANH_GELU: launch_gemm<EPI_SCALE_HARDTANH_GELU>(pl.cfg, g, tiles, 1, s, h->reg_staging); break;
                default: launch_gemm<EPI_SWISH_SCALE>(pl.cfg, g, tiles, 1, s, h->reg_staging); break;
            }
        });
        if (rc != LIN_EPI_OK) return rc;
    } else {
        // Unfused ablation: raw y = XW^T + b to memory (Y itself for the
        // elementwise kinds, the workspace for the row-max kinds), then the
        // tail as a separate pass.  Workspace: [split partials][raw y].
        const size_t part_floats = split > 1 ? (size_t)split * MN : 0;
        const size_t raw_floats = rowmax ? (size_t)MN : 0;
        const size_t bytes = (part_floats + raw_floats) * sizeof(float);
        if (bytes) {
            rc = ensure_workspace(h, bytes);
            if (rc != LIN_EPI_OK) return rc;
        }
        float *ws = static_cast<float *>(h->ws);
        float *Yraw = rowmax ? ws + part_floats : Y;
        if (split > 1) {
            g.out = ws;
            rc = timed_launch(h, 0, [&] { launch_gemm<EPI_SPLITK_PARTIAL>(pl.cfg, g, tiles, split, s, h->reg_staging); });
            if (rc != LIN_EPI_OK) return rc;
            rc = timed_launch(h, 1, [&] { launch_reduce<EPI_NONE>(ws, b, Yraw, MN, (int)N, split, g.tail, s); });
            if (rc != LIN_EPI_OK) return rc;
        } else {
            g.out = Yraw;
            rc = timed_launch(h, 0, [&] { launch_gemm<EPI_NONE>(pl.cfg, g, tiles, 1, s, h->reg_staging); });
            if (rc != LIN_EPI_OK) return rc;
        }
        if (rowmax) {
            const int32_t pool = kind == LIN_EPI_POOL_GELU_SCALE_ROWMAX ? 16 : 1;
            const float scale = desc->scale;
            const int32_t Ni = (int32_t)N;
            rc = timed_launch(h, 2, [&] {
                hipLaunchKernelGGL(rowmax_pass_kernel, dim3((unsigned)M), dim3(256), 0, s, Yraw, (const float *)nullptr,
                                   Y, MN, Ni, 1, pool, scale,
                                   (int32_t)(N % 4 == 0 && ((uintptr_t)Yraw & 15u) == 0));
            });
        } else if (kind != LIN_EPI_NONE) {
            const int vec4 = (MN % 4 == 0) && (((uintptr_t)Y & 15u) == 0);
            int64_t blocks = ((vec4 ? MN / 4 : MN) + 255) / 256;
            if (blocks > 65536) blocks = 65536;
            if (blocks < 1) blocks = 1;
            const TailParams t = g.tail;
            rc = timed_launch(h, 2, [&] {
                if (kind == LIN_EPI_SCALE_HARDTANH_GELU)
                    hipLaunchKernelGGL((tail_inplace_kernel<EPI_SCALE_HARDTANH_GELU>), dim3((unsigned)blocks),
                                       dim3(256), 0, s, Y, MN, t, vec4);
                else
                    hipLaunchKernelGGL((tail_inplace_kernel<EPI_SWISH_SCALE>), dim3((unsigned)blocks), dim3(256), 0,
                                       s, Y, MN, t, vec4);
            });
        }
        if (rc != LIN_EPI_OK) return rc;
    }
    h->plan = plan;
    h->has_plan = true;
    return LIN_EPI_OK;
}

int lin_epi_query_plan(lin_epi_handle h, int64_t M, int64_t N, int64_t K, const lin_epi_desc *desc,
                       int32_t num_cus, lin_epi_plan *out)
{
    if (!h || !out || num_cus < 0) return LIN_EPI_EINVAL;
    const int rc = validate_desc(M, N, K, desc);
    if (rc != LIN_EPI_OK) return rc;
    if (num_cus == 0) {
        const int drc = ensure_device(h);
        if (drc != LIN_EPI_OK) return drc;
        num_cus = h->num_cus;
    }
    *out = lin_epi_plan{};
    if (M == 0 || N == 0) return LIN_EPI_OK;
    const Plan pl = choose_plan(h, M, N, K, desc->kind, num_cus);
    *out = describe(h, pl, M, N, desc->kind);
    return LIN_EPI_OK;
}

int lin_epi_scale_weights(lin_epi_handle h, int64_t N, int64_t K, const float *W, const float *b, float scale,
                          float *Ws, float *bs)
{
    if (!h) return LIN_EPI_EINVAL;
    if (N < 0 || K < 0) return LIN_EPI_EINVAL;
    if (N > INT32_MAX || K > INT32_MAX) return LIN_EPI_EINVAL;
    if (N == 0) return LIN_EPI_OK;
    if (!b || !bs) return LIN_EPI_EINVAL;
    if (K > 0 && (!W || !Ws)) return LIN_EPI_EINVAL;
    if (K % 4 != 0) return LIN_EPI_EALIGN;
    if (K > 0 && (((uintptr_t)W | (uintptr_t)Ws) & 15u)) return LIN_EPI_EALIGN;
    if (((uintptr_t)b | (uintptr_t)bs) & 3u) return LIN_EPI_EALIGN;
    int rc = ensure_device(h);
    if (rc != LIN_EPI_OK) return rc;
    const int64_t nk4 = N * K / 4;
    int64_t blocks = (std::max<int64_t>(nk4, N) + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipStream_t s = h->stream;
    return timed_launch(h, 2, [&] {
        hipLaunchKernelGGL(scale_weights_kernel, dim3((unsigned)blocks), dim3(256), 0, s, W, b, Ws, bs, nk4, N, scale);
    });
}

int lin_epi_pool_weights(lin_epi_handle h, int64_t N, int64_t K, const float *W, const float *b, int32_t pool_kernel,
                         float *Wp, float *bp)
{
    if (!h) return LIN_EPI_EINVAL;
    if (N < 0 || K < 0 || pool_kernel < 1) return LIN_EPI_EINVAL;
    if (N > INT32_MAX || K > INT32_MAX) return LIN_EPI_EINVAL;
    const int64_t L = N / pool_kernel;
    if (L == 0) return LIN_EPI_OK;
    if (!b || !bp) return LIN_EPI_EINVAL;
    if (K > 0 && (!W || !Wp)) return LIN_EPI_EINVAL;
    if (K % 4 != 0) return LIN_EPI_EALIGN;
    if (K > 0 && (((uintptr_t)W | (uintptr_t)Wp) & 15u)) return LIN_EPI_EALIGN;
    if (((uintptr_t)b | (uintptr_t)bp) & 3u) return LIN_EPI_EALIGN;
    int rc = ensure_device(h);
    if (rc != LIN_EPI_OK) return rc;
    int64_t chunks = (K / 4 + 255) / 256;
    if (chunks < 1) chunks = 1;
    if (L * chunks > INT32_MAX) return LIN_EPI_EINVAL;
    hipStream_t s = h->stream;
    const int32_t ci = (int32_t)chunks;
    return timed_launch(h, 2, [&] {
        hipLaunchKernelGGL(pool_weights_kernel, dim3((unsigned)(L * chunks)), dim3(256), 0, s, W, b, Wp, bp, K,
                           pool_kernel, ci);
    });
}

}  // extern "C"
