// C ABI of the fused fp32 linear layer (include/lin_epi.h): argument
// validation, kernel selection, workspace management and optional per-kernel
// timing.  Kernels live in gemm_mfma.hpp and epilogue.hpp.
#include <hip/hip_runtime.h>

#include <new>
#include <vector>

#include "gemm_mfma.hpp"
#include "lin_epi.h"

using namespace lin_epi;

namespace {

// One tile configuration: 128x128 output tile, K step 32, four wavefronts
// in a 2x2 arrangement (64x64 per wavefront = 2x2 MFMA 32x32 blocks).
constexpr int BM = 128, BN = 128, BK = 32, WAVES_M = 2, WAVES_N = 2;
constexpr int THREADS = 64 * WAVES_M * WAVES_N;

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
    bool profile = false;
    bool has_plan = false;
    lin_epi_plan plan{};
    std::vector<PendingTiming> pending;
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

template <typename Launch>
int timed_launch(lin_epi_ctx *h, int role, Launch &&launch)
{
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (h->profile) {
        if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return LIN_EPI_EHIP;
        if (hipEventRecord(e0, h->stream) != hipSuccess) return LIN_EPI_EHIP;
    }
    launch();
    if (hipGetLastError() != hipSuccess) return LIN_EPI_EHIP;
    if (h->profile) {
        if (hipEventRecord(e1, h->stream) != hipSuccess) return LIN_EPI_EHIP;
        h->pending.push_back({role, e0, e1});
    }
    return LIN_EPI_OK;
}

template <int EPI>
void launch_gemm(const GemmArgs &g, int64_t grid_x, int split, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_epi_kernel<BM, BN, BK, WAVES_M, WAVES_N, EPI>), dim3((unsigned)grid_x, (unsigned)split),
                       dim3(THREADS), 0, s, g);
}

template <int EPI>
void launch_reduce(const float *P, const float *bias, float *Y, int64_t MN, int N, int S, TailParams t,
                   hipStream_t s)
{
    int64_t blocks = (MN + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL((splitk_reduce_kernel<EPI>), dim3((unsigned)blocks), dim3(256), 0, s, P, bias, Y, MN, N, S, t);
}

// Split-K slices for the elementwise tails: only when the output tiles alone
// cannot give every compute unit two workgroups and K is long enough that
// each slice still runs many K steps.
int choose_split(const lin_epi_ctx *h, int64_t tiles, int64_t K, int kind)
{
    if (kind == LIN_EPI_POOL_GELU_SCALE_ROWMAX) return 1;
    if (h->split_opt == 1) return 1;
    if (h->split_opt >= 2) return (int)h->split_opt;
    const int64_t slots = 2 * (int64_t)h->num_cus;
    if (tiles * 2 > slots || K < 8192) return 1;
    int64_t s = slots / tiles;
    if (s > 4) s = 4;
    return (int)(s < 2 ? 1 : s);
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
            (void)hipEventDestroy(p.start);
            (void)hipEventDestroy(p.stop);
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
    if (!h || !desc) return LIN_EPI_EINVAL;
    if (M < 0 || N < 0 || K < 0) return LIN_EPI_EINVAL;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return LIN_EPI_EINVAL;
    const int kind = desc->kind;
    if (kind < LIN_EPI_NONE || kind > LIN_EPI_SWISH_SCALE) return LIN_EPI_EINVAL;
    if (kind == LIN_EPI_SCALE_HARDTANH_GELU && !(desc->ht_min <= desc->ht_max)) return LIN_EPI_EINVAL;
    if (kind == LIN_EPI_POOL_GELU_SCALE_ROWMAX) {
        if (desc->pool_kernel != 16 || desc->pool_stride != desc->pool_kernel) return LIN_EPI_ENOTSUP;
        if (N > 0 && N < 16) return LIN_EPI_ENOTSUP;
    }
    if (M == 0 || N == 0) return LIN_EPI_OK;
    if (!b || !Y) return LIN_EPI_EINVAL;
    if (K > 0 && (!X || !W)) return LIN_EPI_EINVAL;
    if (K % 4 != 0) return LIN_EPI_EALIGN;
    if (K > 0 && (((uintptr_t)X | (uintptr_t)W) & 15u)) return LIN_EPI_EALIGN;
    if (((uintptr_t)Y | (uintptr_t)b) & 3u) return LIN_EPI_EALIGN;

    int rc = ensure_device(h);
    if (rc != LIN_EPI_OK) return rc;

    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    int split = choose_split(h, tiles, K, kind);
    // every slice must own at least one K step
    int64_t k_slice = K;
    if (split > 1) {
        const int64_t steps = (K + BK - 1) / BK;
        if (split > steps) split = (int)(steps > 0 ? steps : 1);
        k_slice = ((steps + split - 1) / split) * BK;
        split = (int)((K + k_slice - 1) / k_slice);
        if (split < 1) split = 1;
    }
    if (split <= 1) {
        split = 1;
        k_slice = (K + BK - 1) / BK * BK;
        if (k_slice == 0) k_slice = BK;
    }

    GemmArgs g{};
    g.X = X;
    g.W = W;
    g.bias = b;
    g.M = (int32_t)M;
    g.N = (int32_t)N;
    g.K = (int32_t)K;
    g.k_slice = (int32_t)k_slice;
    g.tiles_m = tiles_m;
    g.tiles_n = tiles_n;
    g.tail = TailParams{desc->scale, desc->ht_min, desc->ht_max};

    lin_epi_plan plan{};
    plan.tile_m = BM;
    plan.tile_n = BN;
    plan.tile_k = BK;
    plan.split_k = split;
    plan.grid_main = tiles * split;

    hipStream_t s = h->stream;
    if (kind == LIN_EPI_POOL_GELU_SCALE_ROWMAX) {
        const size_t bytes = (size_t)M * tiles_n * sizeof(float);
        rc = ensure_workspace(h, bytes);
        if (rc != LIN_EPI_OK) return rc;
        g.out = static_cast<float *>(h->ws);
        rc = timed_launch(h, 0, [&] { launch_gemm<EPI_POOL_GELU_SCALE_ROWMAX>(g, tiles, 1, s); });
        if (rc != LIN_EPI_OK) return rc;
        const float *part = static_cast<const float *>(h->ws);
        const int32_t Mi = (int32_t)M;
        rc = timed_launch(h, 1, [&] {
            hipLaunchKernelGGL(rowmax_finalize_kernel, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, part, Y, Mi,
                               (int32_t)tiles_n);
        });
        if (rc != LIN_EPI_OK) return rc;
        plan.kernels = 2;
        plan.workspace_bytes = (int64_t)bytes;
    } else if (split > 1) {
        const size_t bytes = (size_t)split * M * N * sizeof(float);
        rc = ensure_workspace(h, bytes);
        if (rc != LIN_EPI_OK) return rc;
        g.out = static_cast<float *>(h->ws);
        rc = timed_launch(h, 0, [&] { launch_gemm<EPI_SPLITK_PARTIAL>(g, tiles, split, s); });
        if (rc != LIN_EPI_OK) return rc;
        const float *P = static_cast<const float *>(h->ws);
        const int64_t MN = M * N;
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
        plan.kernels = 2;
        plan.workspace_bytes = (int64_t)bytes;
    } else {
        g.out = Y;
        rc = timed_launch(h, 0, [&] {
            switch (kind) {
                case LIN_EPI_NONE: launch_gemm<EPI_NONE>(g, tiles, 1, s); break;
                case LIN_EPI_SCALE_HARDTANH_GELU: launch_gemm<EPI_SCALE_HARDTANH_GELU>(g, tiles, 1, s); break;
                default: launch_gemm<EPI_SWISH_SCALE>(g, tiles, 1, s); break;
            }
        });
        if (rc != LIN_EPI_OK) return rc;
        plan.kernels = 1;
        plan.workspace_bytes = 0;
    }
    h->plan = plan;
    h->has_plan = true;
    return LIN_EPI_OK;
}

}  // extern "C"
