// C ABI of the fused fp32 linear layer (include/lin_epi.h): argument
// validation, kernel selection, workspace management and optional per-kernel
// timing.  Kernels live in gemm_mfma.hpp, gemv_mfma.hpp and epilogue.hpp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "gemm_mfma.hpp"
#include "gemv_mfma.hpp"
#include "lin_epi.h"

using namespace lin_epi;

namespace {

// Tile table.  The LDS tiles use v_mfma_f32_32x32x2_f32 and two LDS stages;
// they differ in workgroup tile and wavefront count, and the dispatcher picks
// one configuration per call (choose_plan below).  They stage 32-deep K
// steps with direct-to-LDS buffer loads (LDS figures below; rows padded to 36 floats,
// 12 % more, on the register-staged path used when a tile's rows of X or W
// span 1 GiB or more):
//   LARGE  256x256, 8 wavefronts (4x2, 64x128 each), 128 KiB LDS, 1 WG/CU
//   MID    128x256, 8 wavefronts (2x4, 64x64 each),   96 KiB LDS, 1 WG/CU
//   SMALL  128x128, 4 wavefronts (2x2, 64x64 each),   64 KiB LDS, 2 WG/CU
//   TINY    64x64,  4 wavefronts (2x2, 32x32 each),   32 KiB LDS, 4 WG/CU
//   WIDE    64x128, 4 wavefronts (2x2, 32x64 each),  48 KiB LDS, 3 WG/CU
//   TALL   128x96,  4 wavefronts (4x1, 32x96 each),  56 KiB LDS, 2 WG/CU:
//           a quarter fewer fragment reads per MFMA than WIDE, for shapes
//           whose 128x96 tiles fill rounds of two per CU
//   SKINNY  32x128, 4 wavefronts (1x4, 32x32 each),  40 KiB LDS, 4 WG/CU:
//           few rows of X against a long stream of W rows (the small-M,
//           weight-streaming regime, where HBM rather than MFMA bounds);
//           small workgroups so that two or more share a CU and keep enough
//           weight bytes in flight
//   DECODE  16x64 per wavefront, 4 independent wavefronts per workgroup, no
//           LDS (gemv_mfma.hpp): operands streamed from HBM into a register
//           ring; for M <= 16, where the layer is one read of W
using CfgLarge = TileCfg<256, 256, 32, 4, 2, 1>;
using CfgMid = TileCfg<128, 256, 32, 2, 4, 1>;
using CfgSmall = TileCfg<128, 128, 32, 2, 2, 2>;
using CfgTiny = TileCfg<64, 64, 32, 2, 2, 4>;
using CfgSkinny = TileCfg<32, 128, 32, 1, 4, 4>;
using CfgWide = TileCfg<64, 128, 32, 2, 2, 3>;
using CfgTall = TileCfg<128, 96, 32, 4, 1, 2>;

enum CfgId {
    CFG_LARGE = 0, CFG_MID = 1, CFG_SMALL = 2, CFG_TINY = 3, CFG_SKINNY = 4, CFG_DECODE = 5, CFG_WIDE = 6, CFG_TALL = 7,
    CFG_COUNT = 8
};

// The weight-streaming kernel: 16 rows of X against kGemvFN blocks of 16
// rows of W per wavefront, a ring of kGemvDepth K steps of operands in
// registers (64 W rows keep the X fragments, which every lane reloads from L2
// each step, at a quarter of the weight bytes; 4 steps of 8 KiB in flight per
// wavefront and one wavefront per SIMD streamed fastest on MI355X).
constexpr int kGemvFN = 4;
constexpr int kGemvDepth = 4;

struct CfgInfo {
    int bm, bn, bk, wgs_per_cu;
    int waves;          // wavefronts per workgroup
    double efficiency;  // fraction of the CU's 2.4 GHz fp32 MFMA peak, fitted to MI355X timings
    double thin_rate;   // relative MFMA rate of a round with fewer than two wavefronts per SIMD
};

constexpr CfgInfo kCfgs[CFG_COUNT] = {
    {CfgLarge::BM, CfgLarge::BN, CfgLarge::BK, CfgLarge::WG_PER_CU, CfgLarge::NW, 0.975, 0.95},
    {CfgMid::BM, CfgMid::BN, CfgMid::BK, CfgMid::WG_PER_CU, CfgMid::NW, 0.975, 0.95},
    {CfgSmall::BM, CfgSmall::BN, CfgSmall::BK, CfgSmall::WG_PER_CU, CfgSmall::NW, 0.960, 0.95},
    {CfgTiny::BM, CfgTiny::BN, CfgTiny::BK, CfgTiny::WG_PER_CU, CfgTiny::NW, 0.895, 0.95},
    {CfgSkinny::BM, CfgSkinny::BN, CfgSkinny::BK, CfgSkinny::WG_PER_CU, CfgSkinny::NW, 0.895, 0.95},
    {16, 16 * kGemvFN, kStepK, 4, 1, 0.50, 1.0},  // per wavefront; streams fastest with one wavefront per SIMD
    {CfgWide::BM, CfgWide::BN, CfgWide::BK, CfgWide::WG_PER_CU, CfgWide::NW, 0.950, 0.95},
    // a hair under WIDE: on the shapes both fill (1000x6000x4100) they time
    // within +-2 % of each other box to box; measured at full rate with one
    // workgroup per CU (stream-K on 768x3072x3072, 1536x1536x6144,
    // 640x5000x5000), unlike the other tiles
    {CfgTall::BM, CfgTall::BN, CfgTall::BK, CfgTall::WG_PER_CU, CfgTall::NW, 0.949, 1.0},
};
static_assert(CfgLarge::LDS_BYTES * CfgLarge::WG_PER_CU <= 160 * 1024 &&
                  CfgMid::LDS_BYTES * CfgMid::WG_PER_CU <= 160 * 1024 &&
                  CfgSmall::LDS_BYTES * CfgSmall::WG_PER_CU <= 160 * 1024 &&
                  CfgTiny::LDS_BYTES * CfgTiny::WG_PER_CU <= 160 * 1024 &&
                  CfgSkinny::LDS_BYTES * CfgSkinny::WG_PER_CU <= 160 * 1024 &&
                  CfgWide::LDS_BYTES * CfgWide::WG_PER_CU <= 160 * 1024 &&
                  CfgTall::LDS_BYTES * CfgTall::WG_PER_CU <= 160 * 1024,
              "LDS budget");

// Time-model constants of the planner, fitted (with the efficiencies above)
// to timed (shape, tail, configuration, grid) combinations on MI355X (22
// shapes from 1x4096x4096 to 8192x8192x1024, every tile with split-K 1-16
// and stream-K grids of 256-1024 workgroups), each timed after enough
// warm-up for the engine clock to have ramped up.
constexpr double kCuPeakFlops = 256.0 * 2.4e9;  // fp32 MFMA FLOP/s of one CU at the 2.4 GHz peak clock
constexpr double kRoundFixedS = 5e-6;           // per round of workgroups: first loads, epilogue, drain
constexpr double kStreamKRate = 0.95;           // stream-K ranges start at scattered K positions: little L2 reuse
constexpr double kPassFixedS = 2e-6;            // one more kernel on the stream
constexpr double kPassBytesPerS = 4e12;         // sustained HBM rate of partial-sum traffic
constexpr double kGemmBytesPerS = 5.9e12;       // sustained HBM rate of a weight-streaming MFMA tile kernel
constexpr double kSingleStreamRate = 0.7;       // fraction of it with fewer than 2 workgroups per CU
constexpr double kFixupFixedS = 3e-6;           // split tiles: release/acquire and the finishing reads
constexpr double kCuBytesPerS = 60e9;           // one workgroup reading other segments' sums
constexpr double kGemvBytesPerS = 6.1e12;       // weight-streaming kernel, one loading wavefront per SIMD

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
    size_t ws_clean = 0;  // leading workspace bytes known to be zero between runs (the arrival counters)
    int64_t split_opt = 0;
    int64_t grid_opt = 0;
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
        h->ws_clean = 0;
    }
    const size_t rounded = (bytes + (1u << 20) - 1) & ~(size_t)((1u << 20) - 1);
    if (hipMalloc(&h->ws, rounded) != hipSuccess) {
        (void)hipGetLastError();
        h->ws = nullptr;
        return LIN_EPI_ENOMEM;
    }
    h->ws_bytes = rounded;
    h->ws_clean = 0;
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
template <class Cfg, int EPI, bool SPLIT>
void launch_gemm_cfg(const GemmArgs &g, int64_t grid, hipStream_t s, bool reg_staging)
{
    const dim3 gr((unsigned)grid), block(Cfg::THREADS);
    if constexpr (Cfg::BUFLOAD) {
        // buffer loads while a tile's rows of X and W span less than the window
        if (!reg_staging && (int64_t)std::max(Cfg::BM, Cfg::BN) * g.K * 4 < kBufferWindow) {
            hipLaunchKernelGGL((gemm_epi_kernel<Cfg, EPI, true, SPLIT>), gr, block, 0, s, g);
            return;
        }
    }
    hipLaunchKernelGGL((gemm_epi_kernel<Cfg, EPI, false, SPLIT>), gr, block, 0, s, g);
}

// multi: the grid is not one workgroup per tile, so workgroups walk ranges
// of (tile, K step) iterations (the kernels with the segment loop and the
// partial-sum code)
template <int EPI>
void launch_gemm(int cfg, bool multi, const GemmArgs &g, int64_t grid, hipStream_t s, bool reg_staging)
{
    switch (cfg * 2 + (multi ? 1 : 0)) {
        case CFG_LARGE * 2: launch_gemm_cfg<CfgLarge, EPI, false>(g, grid, s, reg_staging); break;
        case CFG_LARGE * 2 + 1: launch_gemm_cfg<CfgLarge, EPI, true>(g, grid, s, reg_staging); break;
        case CFG_MID * 2: launch_gemm_cfg<CfgMid, EPI, false>(g, grid, s, reg_staging); break;
        case CFG_MID * 2 + 1: launch_gemm_cfg<CfgMid, EPI, true>(g, grid, s, reg_staging); break;
        case CFG_SMALL * 2: launch_gemm_cfg<CfgSmall, EPI, false>(g, grid, s, reg_staging); break;
        case CFG_SMALL * 2 + 1: launch_gemm_cfg<CfgSmall, EPI, true>(g, grid, s, reg_staging); break;
        case CFG_TINY * 2: launch_gemm_cfg<CfgTiny, EPI, false>(g, grid, s, reg_staging); break;
        case CFG_TINY * 2 + 1: launch_gemm_cfg<CfgTiny, EPI, true>(g, grid, s, reg_staging); break;
        case CFG_SKINNY * 2: launch_gemm_cfg<CfgSkinny, EPI, false>(g, grid, s, reg_staging); break;
        case CFG_SKINNY * 2 + 1: launch_gemm_cfg<CfgSkinny, EPI, true>(g, grid, s, reg_staging); break;
        case CFG_WIDE * 2: launch_gemm_cfg<CfgWide, EPI, false>(g, grid, s, reg_staging); break;
        case CFG_WIDE * 2 + 1: launch_gemm_cfg<CfgWide, EPI, true>(g, grid, s, reg_staging); break;
        case CFG_TALL * 2: launch_gemm_cfg<CfgTall, EPI, false>(g, grid, s, reg_staging); break;
        default: launch_gemm_cfg<CfgTall, EPI, true>(g, grid, s, reg_staging); break;
    }
}

struct Plan;
template <int EPI>
void launch_main(const Plan &pl, bool multi, const GemmArgs &g, hipStream_t s, bool reg_staging);

bool is_rowmax(int kind)
{
    return kind == LIN_EPI_POOL_GELU_SCALE_ROWMAX || kind == LIN_EPI_GELU_SCALE_ROWMAX;
}

// Shape of the work partition for a grid of G workgroups over T = tiles *
// steps iterations (schedule.hpp): how many K segments the tiles are cut
// into in all, and at most per tile.
struct SegStats {
    int64_t segments;  // sum over tiles of their segment counts
    int max_per_tile;
};

SegStats seg_stats(int64_t tiles, int steps, int64_t G)
{
    if (G == tiles) return SegStats{tiles, 1};
    if (G % tiles == 0) return SegStats{G, (int)(G / tiles)};  // split-K: S segments per tile
    // stream-K: a range boundary strictly inside a tile adds a segment
    const int64_t T = tiles * steps;
    const Partition p{steps, (int)G, 0, (int)(T / G), (int)(T % G)};
    SegStats st{tiles, 1};
    int64_t prev_t = -1;
    int run = 1;
    for (int v = 1; v < (int)G; ++v) {
        const int64_t b = range_begin(p, v);
        if (b % steps == 0) continue;
        ++st.segments;
        const int64_t t = b / steps;
        run = t == prev_t ? run + 1 : 2;
        prev_t = t;
        if (run > st.max_per_tile) st.max_per_tile = run;
    }
    return st;
}

struct Plan {
    int cfg;
    int64_t grid;  // workgroups of the GEMM kernel
    int schedule;  // 0 one tile per workgroup, 1 split-K, 2 stream-K
    int max_seg;   // largest number of K segments of one tile
    int64_t segments;
    int tiles_m, tiles_n;
    int steps;
};

// Workspace layout of one run: [arrival counters, one int per tile, then
// one per tile row for a row-max tail finished in the tile kernel, rounded
// up to 256 bytes][partial-sum slots when tiles are split: one per
// workgroup for split-K, two for stream-K][row-max partials M * tiles_n]
// [raw linear output M * N: unfused row-max tails only].
struct WsLayout {
    size_t counters, partials, rowmax, raw, total;  // byte offsets and size
};

// Floats in one partial-sum slot: the raw tile, or (tail (b) on the MFMA
// tiles) its 16-column window sums; the weight-streaming kernel publishes
// raw sums of its 16 x 16*FN block.
int64_t slot_floats(const lin_epi_ctx *h, const Plan &pl, int kind)
{
    if (pl.cfg == CFG_DECODE) return 16 * 16 * kGemvFN;
    return (int64_t)kCfgs[pl.cfg].bm * kCfgs[pl.cfg].bn /
           (!h->unfused && kind == LIN_EPI_POOL_GELU_SCALE_ROWMAX ? 16 : 1);
}

// The fused row-max tails on the MFMA tiles finish the row maxima in the
// GEMM kernel itself (the weight-streaming kernel leaves them to a pass).
bool rowmax_in_kernel(const lin_epi_ctx *h, const Plan &pl, int kind)
{
    return is_rowmax(kind) && !h->unfused && pl.cfg != CFG_DECODE;
}

WsLayout ws_layout(const lin_epi_ctx *h, const Plan &pl, int64_t M, int64_t N, int kind)
{
    WsLayout w{};
    const int64_t tiles = (int64_t)pl.tiles_m * pl.tiles_n;
    const bool split = pl.segments > tiles;
    const int64_t slot = slot_floats(h, pl, kind);
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    w.counters = 0;
    const int64_t row_counters = rowmax_in_kernel(h, pl, kind) ? pl.tiles_m : 0;
    w.partials = up((size_t)(tiles + row_counters) * sizeof(int32_t));
    // split-K never crosses a tile; a stream-K range ends in at most two
    // split tiles; the weight-streaming kernel has one slot per wavefront
    const int64_t nslots = pl.cfg == CFG_DECODE ? pl.segments : pl.schedule == 2 ? 2 * pl.grid : pl.grid;
    w.rowmax = w.partials + (split ? up((size_t)(nslots * slot) * sizeof(float)) : 0);
    const bool rm = is_rowmax(kind);
    w.raw = w.rowmax + (rm && !h->unfused ? up((size_t)(M * pl.tiles_n) * sizeof(float)) : 0);
    w.total = w.raw + (rm && h->unfused ? up((size_t)(M * N) * sizeof(float)) : 0);
    return w;
}

// Pick the tile configuration and the grid by estimated time.  For each
// configuration the candidate grids are one tile per workgroup, split-K
// with S = 2..16 equal K segments per tile (at most one per K step), and
// stream-K with one or two workgroups per matrix-core slot; then
//   busiest CU: load = ceil(G / CUs) workgroups of ceil(T / G) K steps,
//   w = WG_PER_CU of them at a time sharing its matrix pipes:
//     t_gemm = ceil(load / w) * t_round + load * n_it * 2*BM*BN*32 / (peak * eff)
//   (never less than the time to stream W and X from HBM once, 1/0.7 times
//   longer when fewer than two workgroups per CU stream); split tiles add
//     t_fix = t_fix0 + (published sums, written and read) / HBM rate
//           + (max segments - 1) * slot / one workgroup's read rate
//   and the row-max tails behind the weight-streaming kernel one finalize
//   kernel.
// Padding waste is included (a tile's work counts in full).  The fastest
// estimate wins.  LIN_EPI_OPT_SPLIT_K = 1 forbids splitting, S >= 2 forces
// S segments per tile (clamped to the K steps available);
// LIN_EPI_OPT_GRID = G forces a grid of G workgroups (clamped to T).
// Plans whose workspace exceeds max_ws are skipped; *fits reports whether
// any plan was left (with a fixed workspace a large row-max problem may
// have none).
Plan choose_plan(const lin_epi_ctx *h, int64_t M, int64_t N, int64_t K, int kind, int num_cus,
                 size_t max_ws = SIZE_MAX, bool *fits = nullptr)
{
    Plan best{CFG_SMALL, 1, 0, 1, 1, 1, 1, 1};
    double best_t = 1e300;
    bool any = false;
    const bool rowmax = is_rowmax(kind);
    const int steps = k_steps((int)K);
    // A forced weight-streaming kernel the problem cannot use (rows of W
    // spanning the buffer window) leaves the choice to the planner.
    const bool decode_ok = (int64_t)16 * kGemvFN * K * 4 < kBufferWindow;
    const int64_t tile_opt = h->tile_opt == CFG_DECODE + 1 && !decode_ok ? 0 : h->tile_opt;
    for (int c = 0; c < CFG_COUNT; ++c) {
        const CfgInfo &ci = kCfgs[c];
        if (tile_opt > 0 && c != tile_opt - 1) continue;
        if (c == CFG_DECODE) {
            // One wavefront per (X block, W block, K segment).  Time: reading
            // W once per block of 16 X rows at the streaming rate, scaled
            // down while there are fewer wavefronts than SIMDs, or the
            // busiest SIMD's MFMA work if longer.  More wavefronts than SIMDs
            // stream no faster; their extra segments only add partial sums.
            const int64_t mblocks = (M + 15) / 16, wblocks = (N + ci.bn - 1) / ci.bn;
            // W is read once per 16 rows of X: chosen automatically for at
            // most two such blocks
            if (!decode_ok || (tile_opt == 0 && mblocks > 2)) continue;
            const int64_t blocks = mblocks * wblocks;
            std::vector<int64_t> splits;
            if (h->grid_opt > 0)
                splits.push_back(std::max<int64_t>(1, std::min<int64_t>(h->grid_opt * kGemvWaves / blocks, steps)));
            else if (h->split_opt == 1)
                splits.push_back(1);
            else if (h->split_opt >= 2)
                splits.push_back(std::min<int64_t>(h->split_opt, steps));
            else
                for (int S = 1; S <= std::min(16, steps); ++S) splits.push_back(S);
            const int64_t resident = 4 * (int64_t)num_cus;
            for (int64_t S : splits) {
                const int64_t units = blocks * S;
                if (units > INT32_MAX) continue;
                const double fill = std::min(1.0, (double)units / (double)resident);
                const double t_hbm = 4.0 * ((double)mblocks * N * K + (double)M * K) / (kGemvBytesPerS * fill);
                const int64_t per_simd = (units + 4 * (int64_t)num_cus - 1) / (4 * (int64_t)num_cus);
                const double t_mfma = (double)per_simd * ((steps + S - 1) / S) * 8 * kGemvFN * 32 / (2.4e9 * ci.efficiency);
                double t = std::max(t_hbm, t_mfma) + kRoundFixedS;
                if (S > 1)
                    t += kFixupFixedS + 2.0 * (double)(units - blocks) * 4 * 16 * ci.bn / kPassBytesPerS;
                if (rowmax) t += kPassFixedS;
                const Plan cand{c, (units + kGemvWaves - 1) / kGemvWaves, S > 1 ? 1 : 0, (int)S, units,
                                (int)mblocks, (int)wblocks, steps};
                if (max_ws != SIZE_MAX && (S > 1 || rowmax) && ws_layout(h, cand, M, N, kind).total > max_ws) continue;
                if (t < best_t) {
                    best_t = t;
                    best = cand;
                    any = true;
                }
            }
            continue;
        }
        // the 32-row tile is for 17-32 rows of X (measured 25 % off the best
        // plan at 96 rows, where the time model rates it too well)
        if (c == CFG_SKINNY && tile_opt == 0 && M > 32) continue;
        const int64_t tm = (M + ci.bm - 1) / ci.bm, tn = (N + ci.bn - 1) / ci.bn;
        const int64_t tiles = tm * tn;
        const int64_t T = tiles * steps;
        std::vector<int64_t> grids;
        if (h->grid_opt > 0) {
            grids.push_back(std::min<int64_t>(h->grid_opt, T));
        } else if (h->split_opt == 1) {
            grids.push_back(tiles);
        } else if (h->split_opt >= 2) {
            grids.push_back(tiles * std::min<int64_t>(h->split_opt, steps));
        } else {
            for (int S = 1; S <= std::min(16, steps); ++S) grids.push_back(tiles * S);
            // stream-K within one round of resident workgroups (1..wgs_per_cu
            // per CU, fewer or more workgroups than tiles): grids of several
            // rounds measured markedly slower
            for (int64_t k = 1; k <= ci.wgs_per_cu; ++k) {
                const int64_t g = k * num_cus;
                if (g != tiles && g < T && g % tiles != 0) grids.push_back(g);
            }
        }
        const double slot_bytes = 4.0 * ci.bm * ci.bn / (kind == LIN_EPI_POOL_GELU_SCALE_ROWMAX ? 16 : 1);
        // The 256x256 tile's accumulators leave no room for reading back
        // whole raw partial tiles (that kernel spills), so unless forced it
        // only splits for tail (b), whose partials are pooled.
        const bool forced = h->grid_opt > 0 || h->split_opt >= 2;
        const bool raw_split_ok = c != CFG_LARGE || kind == LIN_EPI_POOL_GELU_SCALE_ROWMAX || forced;
        for (int64_t G : grids) {
            // other grids need 32-bit iteration indices (T < 2^31); the
            // 256x256 tile only splits where it does not spill
            if (G != tiles && (T > INT32_MAX || G > INT32_MAX || !raw_split_ok)) G = tiles;
            const int64_t n_it = (T + G - 1) / G;
            const int64_t load = (G + num_cus - 1) / num_cus;
            const double step_t = 2.0 * ci.bm * ci.bn * kStepK / (kCuPeakFlops * ci.efficiency);
            // the busiest CU runs its workgroups wgs_per_cu at a time; a round
            // that leaves fewer than two wavefronts per SIMD runs at the
            // tile's thin_rate
            auto rate = [&](int64_t k) { return k * ci.waves < 8 ? ci.thin_rate : 1.0; };
            const int64_t full = load / ci.wgs_per_cu, rem = load % ci.wgs_per_cu;
            const double sk = (G != tiles && G % tiles != 0) ? kStreamKRate : 1.0;
            double t = (double)(full + (rem ? 1 : 0)) * kRoundFixedS +
                       ((double)(full * ci.wgs_per_cu) * n_it * step_t / rate(ci.wgs_per_cu) +
                        (rem ? (double)rem * n_it * step_t / rate(rem) : 0.0)) / sk;
            double t_hbm = 4.0 * ((double)N * K + (double)M * K) / kGemmBytesPerS;
            if (G < 2 * (int64_t)num_cus) t_hbm /= kSingleStreamRate;
            t = std::max(t, t_hbm);
            const SegStats st = seg_stats(tiles, steps, G);
            if (st.segments > tiles)
                t += kFixupFixedS + 2.0 * (double)(st.segments - tiles) * slot_bytes / kPassBytesPerS +
                     (st.max_per_tile - 1) * slot_bytes / kCuBytesPerS;
            // (row-max tails: the tile kernel's last workgroup of each tile
            // row finishes the row, no second pass)
            const Plan cand{c, G, G == tiles ? 0 : G % tiles == 0 ? 1 : 2, st.max_per_tile, st.segments,
                            (int)tm, (int)tn, steps};
            if (max_ws != SIZE_MAX && (st.segments > tiles || rowmax) && ws_layout(h, cand, M, N, kind).total > max_ws)
                continue;
            if (t < best_t) {
                best_t = t;
                best = cand;
                any = true;
            }
        }
    }
    if (fits) *fits = any;
    return best;
}

// The GEMM of a plan: the weight-streaming kernel or an MFMA tile kernel.
template <int EPI>
void launch_main(const Plan &pl, bool multi, const GemmArgs &g, hipStream_t s, bool reg_staging)
{
    if (pl.cfg == CFG_DECODE) {
        const GemvArgs gv{g.X, g.W, g.bias,     g.out,   g.partials, g.counters, g.M, g.N,
                          g.K, g.tiles_n, (int32_t)pl.segments, g.steps, g.koff, (int32_t)pl.max_seg, g.tail};
        hipLaunchKernelGGL((gemv_mfma_kernel<EPI, kGemvFN, kGemvDepth>), dim3((unsigned)pl.grid),
                           dim3(64 * kGemvWaves), 0, s, gv);
        return;
    }
    launch_gemm<EPI>(pl.cfg, multi, g, pl.grid, s, reg_staging);
}

// The launch plan of one lin_epi_run call as the C interface reports it.
//   fused:    GEMM with the tail in its epilogue (1 kernel); the row-max
//             kinds add the finalize pass over per-tile row maxima
//   unfused:  GEMM to raw y (Y itself for the elementwise kinds, the
//             workspace for the row-max kinds), then a tail kernel (none for
//             kind 0)
lin_epi_plan describe(const lin_epi_ctx *h, const Plan &pl, int64_t M, int64_t N, int kind)
{
    lin_epi_plan p{};
    p.tile_m = kCfgs[pl.cfg].bm;
    p.tile_n = kCfgs[pl.cfg].bn;
    p.tile_k = kCfgs[pl.cfg].bk;
    p.split_k = pl.max_seg;
    p.grid_main = pl.grid;
    p.schedule = pl.schedule;
    if (h->unfused)
        p.kernels = 1 + (kind != LIN_EPI_NONE ? 1 : 0);
    else
        p.kernels = is_rowmax(kind) && !rowmax_in_kernel(h, pl, kind) ? 2 : 1;
    const WsLayout w = ws_layout(h, pl, M, N, kind);
    const bool split = pl.segments > (int64_t)pl.tiles_m * pl.tiles_n;
    p.workspace_bytes = (split || is_rowmax(kind)) ? (int64_t)w.total : 0;
    p.partial_bytes = split ? (pl.segments - (int64_t)pl.tiles_m * pl.tiles_n) * slot_floats(h, pl, kind) * 4 : 0;
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
        case LIN_EPI_ETOOBIG: return "problem needs more workspace than the fixed no-alloc scratch array holds";
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
        case LIN_EPI_OPT_GRID:
            if (value < 0 || value > INT32_MAX) return LIN_EPI_EINVAL;
            h->grid_opt = value;
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

}  // extern "C"

namespace {

// A workspace in place of the handle's own: fixed size, never (re)allocated;
// its arrival counters are cleared on every call that splits tiles.
struct FixedWs {
    char *base;
    size_t bytes;
};

int scratch_address(int dev, char **out);
extern const size_t kScratchBytesHost;

// lin_epi_run (noalloc = false) and lin_epi_run_noalloc (true): the same
// validation, plan and kernels; only where intermediates live differs.
int run_impl(lin_epi_handle h, int64_t M, int64_t N, int64_t K, const float *X, const float *W, const float *b,
             const lin_epi_desc *desc, float *Y, bool noalloc)
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
    FixedWs fixed_ws{nullptr, 0};
    const FixedWs *fixed = nullptr;
    if (noalloc) {
        rc = scratch_address(h->device, &fixed_ws.base);
        if (rc != LIN_EPI_OK) return rc;
        fixed_ws.bytes = kScratchBytesHost;
        fixed = &fixed_ws;
    }

    const bool rowmax = is_rowmax(kind);
    const bool unfused = h->unfused;
    bool fits = true;
    const Plan pl = choose_plan(h, M, N, K, kind, h->num_cus, fixed ? fixed->bytes : SIZE_MAX, &fits);
    if (!fits) return LIN_EPI_ETOOBIG;
    const int64_t tiles = (int64_t)pl.tiles_m * pl.tiles_n;
    const lin_epi_plan plan = describe(h, pl, M, N, kind);
    const WsLayout wl = ws_layout(h, pl, M, N, kind);
    const bool split = pl.segments > tiles;  // some tile is cut into K segments
    const bool multi = pl.grid != tiles;     // workgroups walk ranges (segment-loop kernel)
    const bool row_fin = rowmax_in_kernel(h, pl, kind);
    const bool counters = split || row_fin;  // arrival counters in use, zero before the launch
    hipStream_t s = h->stream;

    GemmArgs g{};
    g.X = X;
    g.W = W;
    g.bias = b;
    g.M = (int32_t)M;
    g.N = (int32_t)N;
    g.K = (int32_t)K;
    g.tiles_m = pl.tiles_m;
    g.tiles_n = pl.tiles_n;
    g.steps = pl.steps;
    g.koff = k_offset((int)K);
    g.split = pl.schedule == 1 ? (int32_t)(pl.grid / tiles) : 0;
    g.q = multi ? (int32_t)(tiles * pl.steps / pl.grid) : 0;
    g.r = multi ? (int32_t)(tiles * pl.steps % pl.grid) : 0;
    g.tail = TailParams{desc->scale, desc->ht_min, desc->ht_max};

    char *ws = nullptr;
    if ((split || rowmax) && fixed) {
        ws = fixed->base;
        if (counters) {
            // the fixed array keeps whatever the last call left: clear the
            // arrival counters (a fill kernel, not a memset)
            const int64_t n = (int64_t)(wl.partials / sizeof(int32_t));
            const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 4096);
            hipLaunchKernelGGL(zero_counters_kernel, dim3(blocks), dim3(256), 0, s, reinterpret_cast<int32_t *>(ws), n);
            if (hipGetLastError() != hipSuccess) return LIN_EPI_EHIP;
        }
        g.counters = reinterpret_cast<int32_t *>(ws + wl.counters);
        g.partials = reinterpret_cast<float *>(ws + wl.partials);
    } else if (split || rowmax) {
        rc = ensure_workspace(h, wl.total);
        if (rc != LIN_EPI_OK) return rc;
        ws = static_cast<char *>(h->ws);
        if (counters && wl.partials > h->ws_clean) {
            // arrival counters start at zero (and every run leaves them so)
            const int64_t n = (int64_t)(wl.partials / sizeof(int32_t));
            const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 4096);
            hipLaunchKernelGGL(zero_counters_kernel, dim3(blocks), dim3(256), 0, s, reinterpret_cast<int32_t *>(ws), n);
            if (hipGetLastError() != hipSuccess) return LIN_EPI_EHIP;
            h->ws_clean = wl.partials;
        }
        g.counters = reinterpret_cast<int32_t *>(ws + wl.counters);
        g.partials = reinterpret_cast<float *>(ws + wl.partials);
    }

    if (!unfused && rowmax) {
        // GEMM with the row-max epilogue -> per-(row, column tile) partials ->
        // max over column tiles: by the tile kernel's last workgroup of each
        // tile row, or (weight-streaming kernel) by a second pass.
        g.out = reinterpret_cast<float *>(ws + wl.rowmax);
        if (row_fin) {
            g.Y = Y;
            g.rowcnt = reinterpret_cast<int32_t *>(ws + wl.counters) + tiles;
        }
        rc = timed_launch(h, 0, [&] {
            if (kind == LIN_EPI_POOL_GELU_SCALE_ROWMAX)
                launch_main<EPI_POOL_GELU_SCALE_ROWMAX>(pl, multi, g, s, h->reg_staging);
            else
                launch_main<EPI_GELU_SCALE_ROWMAX>(pl, multi, g, s, h->reg_staging);
        });
        if (rc != LIN_EPI_OK) return rc;
        if (!row_fin) {
            const float *part = g.out;
            const int32_t Mi = (int32_t)M, tn = (int32_t)pl.tiles_n;
            rc = timed_launch(h, 1, [&] {
                hipLaunchKernelGGL(rowmax_finalize_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s, part, Y, Mi,
                                   tn);
            });
            if (rc != LIN_EPI_OK) return rc;
        }
    } else if (!unfused) {
        g.out = Y;
        rc = timed_launch(h, 0, [&] {
            switch (kind) {
                case LIN_EPI_NONE: launch_main<EPI_NONE>(pl, multi, g, s, h->reg_staging); break;
                case LIN_EPI_SCALE_HARDTANH_GELU:
                    launch_main<EPI_SCALE_HARDTANH_GELU>(pl, multi, g, s, h->reg_staging);
                    break;
                default: launch_main<EPI_SWISH_SCALE>(pl, multi, g, s, h->reg_staging); break;
            }
        });
        if (rc != LIN_EPI_OK) return rc;
    } else {
        // Unfused ablation: raw y = XW^T + b to memory (Y itself for the
        // elementwise kinds, the workspace for the row-max kinds), then the
        // tail as a separate pass.
        float *Yraw = rowmax ? reinterpret_cast<float *>(ws + wl.raw) : Y;
        g.out = Yraw;
        rc = timed_launch(h, 0, [&] { launch_main<EPI_NONE>(pl, multi, g, s, h->reg_staging); });
        if (rc != LIN_EPI_OK) return rc;
        if (rowmax) {
            const int32_t pool = kind == LIN_EPI_POOL_GELU_SCALE_ROWMAX ? 16 : 1;
            const float scale = desc->scale;
            const int32_t Ni = (int32_t)N;
            rc = timed_launch(h, 2, [&] {
                hipLaunchKernelGGL(rowmax_pass_kernel, dim3((unsigned)M), dim3(256), 0, s, (const float *)Yraw, Y, Ni,
                                   pool, scale, (int32_t)(N % 4 == 0));
            });
        } else if (kind != LIN_EPI_NONE) {
            const int64_t MN = M * N;
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
    // A split run leaves its counters at zero; any run that used the
    // workspace may have written everything past them.
    if (!fixed && (split || rowmax)) h->ws_clean = std::min(h->ws_clean, wl.partials);
    h->plan = plan;
    h->has_plan = true;
    return LIN_EPI_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Fixed device scratch for lin_epi_run_noalloc: every intermediate of a run
// (arrival counters, partial sums of split tiles, per-tile row maxima) in
// one file-scope device array instead of the handle's workspace.  Each GPU
// the library runs on holds its own copy until the process ends.  In host
// code the array's name is not a device address: its address on each device
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is passed to kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

const size_t kScratchBytesHost = kScratchBytes;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char *g_scratch_ptr[kMaxDevices];

int scratch_address(int dev, char **out)
{
    if (dev < 0 || dev >= kMaxDevices) return LIN_EPI_EINVAL;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess || cur != dev) return LIN_EPI_EINVAL;
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return LIN_EPI_EHIP;
        }
        g_scratch_ptr[dev] = static_cast<char *>(p);
    }
    *out = g_scratch_ptr[dev];
    return LIN_EPI_OK;
}

}  // namespace

extern "C" {

int lin_epi_run(lin_epi_handle h, int64_t M, int64_t N, int64_t K, const float *X, const float *W, const float *b,
                const lin_epi_desc *desc, float *Y)
{
    return run_impl(h, M, N, K, X, W, b, desc, Y, false);
}

int lin_epi_run_noalloc(lin_epi_handle h, int64_t M, int64_t N, int64_t K, const float *X, const float *W,
                        const float *b, const lin_epi_desc *desc, float *Y)
{
    return run_impl(h, M, N, K, X, W, b, desc, Y, true);
}

int64_t lin_epi_noalloc_scratch_bytes(void)
{
    return (int64_t)kScratchBytes;
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
