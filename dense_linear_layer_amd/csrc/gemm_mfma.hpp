// MFMA-tiled fp32 GEMM with a fused epilogue, for gfx950 (CDNA4).
//
// Computes, for one BM x BN output tile per workgroup,
//     acc[m, n] = sum_k X[m, k] * W[n, k]        (X [M,K], W [N,K], both K-contiguous)
// with v_mfma_f32_32x32x2_f32 (fp32 products, fp32 accumulation), then
// applies the bias and the tail in registers and stores the result once.
// This is the "compute the GEMM tile into registers, apply the tail, write
// the final output" plan that page "Kimi-K2.6 l2_p53" names as the ideal
// fusion and page "Kimi-K2.6 l2_p59" sketches as a tiled kernel with staged
// input/weight tiles and a register epilogue.
//
// Data flow per workgroup (NT = 64 * WAVES_M * WAVES_N threads), two LDS
// stages (double buffer), one K step of BK per stage:
//   * global -> LDS directly (the buffer-load configurations, BK = 32):
//     buffer_load_dwordx4 ... lds writes each wavefront's 64 x 16 bytes
//     straight into LDS, 8 rows of 128 bytes per instruction, with the 16-byte
//     chunks of a row XOR-swizzled so the fragment reads are bank-conflict
//     free.  No registers and no LDS store instructions are spent on staging,
//     and a step's loads are issued a whole step ahead of their use.
//   * otherwise global -> registers -> LDS: 128-bit loads, BK/4 consecutive
//     threads per BK-float row segment (whole cache lines per wavefront), then
//     128-bit LDS stores with a row stride of BK+4 floats, so consecutive rows
//     start 4 banks apart and stores and fragment reads are conflict free.
//   * Rows past M/N and k past the slice end are zero-filled (K is a multiple
//     of 4, so a float4 is all-in or all-out): by the buffer range check where
//     buffer loads are used, else by predicated loads.
//   * LDS -> MFMA operands: the contraction index is permuted inside each
//     group of 8 k: lane l of a 32x32x2 MFMA supplies k-slot l/32, and the
//     four MFMAs of one group use components 0..3 of a float4 read at
//     k = 8g + 4*(l/32).  A and B use the same permutation, so the sum over
//     k is unchanged, and both operands come from K-contiguous 128-bit reads
//     (no transpose of the [N,K] weight is ever needed).
//
// Accumulator layout of v_mfma_f32_32x32x2_f32 (one 32x32 block, 16 VGPRs):
// lane l, register r holds C[row][col] with col = l % 32 and
// row = 8*(r/4) + 4*(l/32) + r%4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "epilogue.hpp"

namespace lin_epi {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum EpiKind : int {
    EPI_NONE = 0,
    EPI_SCALE_HARDTANH_GELU = 1,
    EPI_POOL_GELU_SCALE_ROWMAX = 2,
    EPI_SWISH_SCALE = 3,
    EPI_SPLITK_PARTIAL = 4,  // raw partial sums of one K slice, no bias/tail
    EPI_GELU_SCALE_ROWMAX = 5,  // max over columns of scale*GELU(y): tail (b) on pooled weights
};

struct GemmArgs {
    const float *X;
    const float *W;
    const float *bias;
    float *out;       // Y [M,N]; or split-K slices [S,M,N]; or row-max partials [M, tiles_n]
    int32_t M, N, K;
    int32_t k_slice;  // K elements per split-K slice (multiple of BK); >= K when not split
    int32_t tiles_m, tiles_n;
    TailParams tail;
};

// Workgroup index -> output tile, XCD-aware.  Workgroups are dispatched
// round-robin over the 8 XCDs (wg % 8), each XCD with its own L2.  The first
// 8*q workgroups (q = tiles / 8) are renumbered so that XCD x owns the
// contiguous tile range [x*q, (x+1)*q); the remainder keeps its index.  The
// tile number is then unfolded GROUP_M tile-rows at a time (column-major
// inside a group), so the workgroups resident on one XCD cover a compact
// block of tiles and share both X row panels and W column panels in L2.
template <int GROUP_M>
__device__ __forceinline__ void tile_of(int wg, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int tiles = tiles_m * tiles_n;
    const int q = tiles >> 3;
    int t = wg;
    if (wg < (q << 3)) t = (wg & 7) * q + (wg >> 3);
    const int per_group = GROUP_M * tiles_n;
    const int g = t / per_group;
    const int first_m = g * GROUP_M;
    const int gm = min(tiles_m - first_m, GROUP_M);
    const int r = t - g * per_group;
    tm = first_m + r % gm;
    tn = r / gm;
}

// A workgroup tile shape: BM x BN outputs, K step BK, WAVES_M x WAVES_N
// wavefronts each owning a (BM/WAVES_M) x (BN/WAVES_N) sub-tile, and the
// number of workgroups meant to share one compute unit (register budget).
// BUFLOAD selects direct-to-LDS buffer loads (BK = 32 only) where the
// range-checked form is usable (see gemm_epi_kernel); otherwise, and for
// tiles too large for the buffer window, operands go through registers.
template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int WG_PER_CU_, bool BUFLOAD_ = true, int STAGES_ = 2>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int WG_PER_CU = WG_PER_CU_;
    static constexpr bool BUFLOAD = BUFLOAD_;
    static constexpr int STAGES = STAGES_;  // LDS stages of the direct-to-LDS path
    static constexpr int THREADS = 64 * WAVES_M * WAVES_N;
    static constexpr int WAVES_PER_SIMD = WG_PER_CU * WAVES_M * WAVES_N / 4;
    // Direct-to-LDS path: STAGES stages of whole
    // 1 KiB blocks (8 unpadded 128-byte rows), the block count rounded up to
    // a multiple of the wavefront count.  Otherwise two stages of rows
    // padded to BK + 4 floats.
    static constexpr bool DMA = BUFLOAD;
    static_assert(!BUFLOAD || BK == 32, "the direct-to-LDS layout holds 128-byte rows");
    static constexpr int NW = WAVES_M * WAVES_N;
    static constexpr int DMA_BLOCKS = ((BM + BN) / 8 + NW - 1) / NW * NW;
    static constexpr int LDS_BYTES = DMA ? STAGES * DMA_BLOCKS * 1024 : 2 * (BM + BN) * (BK + 4) * 4;
    // The register-staged form (padded rows) may fit fewer workgroups per CU.
    static constexpr int LDS_BYTES_REG = 2 * (BM + BN) * (BK + 4) * 4;
    static constexpr int WG_PER_CU_REG = WG_PER_CU < 160 * 1024 / LDS_BYTES_REG ? WG_PER_CU : 160 * 1024 / LDS_BYTES_REG;
    static constexpr int WAVES_PER_SIMD_REG = (WG_PER_CU_REG * WAVES_M * WAVES_N + 3) / 4;
};

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt bits [3:0] and [15:14]; expcnt
// and lgkmcnt left at their maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Byte window the buffer-load path is used within: a tile's rows of X or W
// span rows * K * 4 < 2^30 bytes, so every byte offset the kernel forms
// (per-lane offset + scalar offset, the latter a row-block offset plus the K
// position) stays below 2^31, and OOB_OFFSET = 2^30 plus any scalar offset
// is past num_records yet still inside 32 bits.
constexpr int64_t kBufferWindow = 1 << 30;

template <class Cfg, int EPI, bool BUF>
__global__ void __launch_bounds__(Cfg::THREADS, BUF ? Cfg::WAVES_PER_SIMD : Cfg::WAVES_PER_SIMD_REG)
gemm_epi_kernel(GemmArgs a)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, WAVES_M = Cfg::WAVES_M, WAVES_N = Cfg::WAVES_N;
    constexpr int NT = Cfg::THREADS;
    constexpr int LDK = BK + 4;             // padded LDS row stride, floats
    constexpr int STAGE = (BM + BN) * LDK;  // floats per LDS stage
    constexpr int TM = BM / WAVES_M;        // wave tile
    constexpr int TN = BN / WAVES_N;
    constexpr int FM = TM / 32;             // 32x32 MFMA blocks per wave
    constexpr int FN = TN / 32;
    constexpr int C4 = BK / 4;                    // float4 per tile row
    constexpr int A_LD = (BM * C4 + NT - 1) / NT;  // float4 global loads per thread
    constexpr int B_LD = (BN * C4 + NT - 1) / NT;
    constexpr bool A_EVEN = A_LD * NT == BM * C4;  // else the last round is partial
    constexpr bool B_EVEN = B_LD * NT == BN * C4;
    static_assert(BK % 8 == 0 && TM % 32 == 0 && TN % 32 == 0, "tile shape");

    // Direct-to-LDS staging (DMA): buffer loads that write LDS themselves,
    // for the buffer-load configurations, all with BK = 32 (one 128-byte row
    // segment = 8 float4 chunks).  smem is stage 0 there.
    constexpr bool DMA = BUF;
    static_assert(!BUF || Cfg::DMA, "buffer loads are used on the direct-to-LDS path only");
    constexpr int DMA_STAGE = Cfg::DMA_BLOCKS * 256;  // floats per DMA stage
    __shared__ __attribute__((aligned(16))) float smem[DMA ? DMA_STAGE : 2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WAVES_N;
    const int wn = wave % WAVES_N;

    int tm, tn;
    tile_of<8>(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int M = a.M, N = a.N, K = a.K;

    const int kbeg = blockIdx.y * a.k_slice;
    const int kend = min(K, kbeg + a.k_slice);
    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

    f32x4 ra[A_LD], rb[B_LD];

    // Direct-to-LDS staging (BUF): one buffer resource over this tile's rows
    // of X and one over its rows of W, sized to the valid rows.  A read past
    // num_records returns zeros in hardware (written into LDS as zeros), so
    // rows beyond M or N need no per-load branch, and the K tail is masked by
    // swapping in an out-of-range offset.  The host uses this path only when
    // rows * K * 4 < kBufferWindow.
    constexpr int OOB_OFFSET = (int)kBufferWindow;
    const int a_bytes = BUF ? min(BM, M - m0) * K * 4 : 0, b_bytes = BUF ? min(BN, N - n0) * K * 4 : 0;
    const __amdgpu_buffer_rsrc_t rsA =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.X + (int64_t)m0 * K), (short)0, a_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsB =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.W + (int64_t)n0 * K), (short)0, b_bytes, 0x00020000);

    // Register staging (!BUF): predicated 128-bit loads, zero-filled past M,
    // N and the slice end.
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const int idx = tid + i * NT;
            const int row = idx / C4;
            const int gk = k0 + (idx % C4) * 4;
            const int gm = m0 + row;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if ((A_EVEN || idx < BM * C4) && gm < M && gk < kend)
                v = *reinterpret_cast<const f32x4 *>(a.X + (int64_t)gm * K + gk);
            ra[i] = v;
        }
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int idx = tid + i * NT;
            const int row = idx / C4;
            const int gk = k0 + (idx % C4) * 4;
            const int gn = n0 + row;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if ((B_EVEN || idx < BN * C4) && gn < N && gk < kend)
                v = *reinterpret_cast<const f32x4 *>(a.W + (int64_t)gn * K + gk);
            rb[i] = v;
        }
    };
    auto sstore = [&](int buf) {
        float *As = smem + buf * STAGE;
        float *Bs = As + BM * LDK;
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const int idx = tid + i * NT;
            if (A_EVEN || idx < BM * C4) *reinterpret_cast<f32x4 *>(As + (idx / C4) * LDK + (idx % C4) * 4) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int idx = tid + i * NT;
            if (B_EVEN || idx < BN * C4) *reinterpret_cast<f32x4 *>(Bs + (idx / C4) * LDK + (idx % C4) * 4) = rb[i];
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * 4;

    // Operand fragments of one 8-deep K group ("sub-step"), double-buffered in
    // registers so the next group's LDS reads overlap this group's MFMAs.
    constexpr int G = BK / 8;
    f32x4 fa[2][FM], fb[2][FN];
    auto read_frags = [&](int buf, int kk, f32x4 (&af)[FM], f32x4 (&bf)[FN]) {
        const float *As = smem + buf * STAGE;
        const float *Bs = As + BM * LDK;
#pragma unroll
        for (int i = 0; i < FM; ++i)
            af[i] = *reinterpret_cast<const f32x4 *>(As + (wm * TM + i * 32 + frag_row) * LDK + kk + frag_k);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            bf[j] = *reinterpret_cast<const f32x4 *>(Bs + (wn * TN + j * 32 + frag_row) * LDK + kk + frag_k);
    };
    auto mfma_group = [&](const f32x4 (&af)[FM], const f32x4 (&bf)[FN]) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][c], bf[j][c], acc[i][j], 0, 0, 0);
    };

    if constexpr (DMA) {
        // Each LDS stage holds the tile's BM rows of X then BN rows of W,
        // 128 bytes per row, unpadded, then (when the block count is not a
        // multiple of the wavefront count) padding blocks.  One
        // buffer_load ... lds instruction writes 1 KiB (64 lanes x 16 B)
        // contiguously: a block of 8 rows, lane l landing at row l/8,
        // physical chunk l%8.  Chunks are stored XOR-swizzled,
        // physical = logical ^ s(row) with s(row) = (row % 8) ^ ((row / 8) % 2),
        // so the fragment reads (32 rows, one logical chunk) hit 8 distinct
        // chunk positions per 8 rows and, with the row parity, 16 distinct
        // 16-byte slots per 16 rows: no bank conflicts at 128 or 256 bytes per
        // LDS cycle.  Lane l therefore fetches logical chunk (l%8) ^ s(row).
        constexpr int NST = Cfg::STAGES;
        static_assert(NST >= 2 && NST <= 4, "2 to 4 DMA stages");
        __shared__ __attribute__((aligned(16))) float smem1[DMA_STAGE];
        __shared__ __attribute__((aligned(16))) float smem2[NST > 2 ? DMA_STAGE : 4];
        __shared__ __attribute__((aligned(16))) float smem3[NST > 3 ? DMA_STAGE : 4];
        auto stage = [&](int st) -> float * { return st == 0 ? smem : st == 1 ? smem1 : st == 2 ? smem2 : smem3; };
        constexpr int NW = Cfg::NW;
        constexpr int NBA = BM / 8, NB = (BM + BN) / 8;  // 8-row blocks of X, of X and W
        constexpr int NL = Cfg::DMA_BLOCKS / NW;          // DMA instructions per wavefront and step
        static_assert(NW % 2 == 0 && NBA % 2 == 0, "block parity = wavefront parity");
        const int wave_u = __builtin_amdgcn_readfirstlane(wave);
        const int lr = lane >> 3;
        const int cdma = (lane & 7) ^ lr ^ (wave_u & 1);  // blocks i*NW + wave all have parity wave&1
        // Byte offset of this lane's float4 inside an 8-row block of X or W.
        const int lane_off = (lr * K + 4 * cdma) * 4;
        // Loads of K step k0 into stage st.  Past the slice end every lane is
        // out of range: the stage gets zeros and no memory is read.
        auto dma = [&](float *st, int k0) {
            // the block's row offset and k0 are wave-uniform: scalar offset
            // (the range check applies to the sum)
            const int voff = k0 + 4 * cdma < kend ? lane_off : OOB_OFFSET;
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const int blk = i * NW + wave_u;
                auto *dst = (__attribute__((address_space(3))) void *)(st + blk * 256);
                const bool all_a = (i + 1) * NW <= NBA, all_b = i * NW >= NBA && (i + 1) * NW <= NB;
                if (all_a || (!all_b && blk < NBA)) {
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, dst, 16, voff, (blk * 8 * K + k0) * 4, 0, 0);
                } else if (all_b || blk < NB) {
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, dst, 16, voff, ((blk - NBA) * 8 * K + k0) * 4, 0, 0);
                } else {  // padding block: zeros, never read
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, dst, 16, OOB_OFFSET, 0, 0, 0);
                }
            }
        };
        const int tsw = (lane >> 5) ^ (frag_row & 7) ^ ((frag_row >> 3) & 1);
        auto read_dma = [&](const float *st, int g, f32x4 (&af)[FM], f32x4 (&bf)[FN]) {
            const int ch = 4 * ((2 * g) ^ tsw);
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const f32x4 *>(st + (wm * TM + i * 32 + frag_row) * BK + ch);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[j] = *reinterpret_cast<const f32x4 *>(st + (BM + wn * TN + j * 32 + frag_row) * BK + ch);
        };
        // One K step kt (stage kt % NST): the DMA of step kt+NST-1 goes into
        // the stage step kt-1 used (every wavefront finished reading it before
        // the previous barrier), so loads are issued NST-1 steps ahead; before
        // the barrier, a wait until at most the NST-2 younger steps' loads are
        // outstanding, i.e. step kt+1 has landed (loads complete in order).
        // The DMA instructions are spread over the first group's MFMAs (one
        // per 4*FM*FN/NL MFMAs): issued back to back they would hold every
        // wavefront of the CU off the matrix pipes at the same moment, right
        // after the barrier.  The stages are separate LDS arrays and the loop
        // is unrolled by NST, so the compiler can tell a DMA target from the
        // stage being read and does not make those reads wait for the DMA.
        auto step = [&](float *cur, float *nxt, float *fre, int kt) {
            dma(fre, kbeg + (kt + NST - 1) * BK);
            read_dma(cur, 1, fa[1], fb[1]);
            mfma_group(fa[0], fb[0]);
            // scheduling groups (masks: 0x100 LDS reads, 0x008 MFMA, 0x020
            // vector-memory reads): the next group's fragment reads first,
            // then MFMAs and DMA instructions alternating
            __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);
#pragma unroll
            for (int q = 0; q < NL; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 4 * FM * FN / NL, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 1; g < G - 1; ++g) {
                read_dma(cur, g + 1, fa[(g + 1) & 1], fb[(g + 1) & 1]);
                mfma_group(fa[g & 1], fb[g & 1]);
            }
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<(NST - 2) * NL>();
            __syncthreads();
            if (kt + 1 < nk) read_dma(nxt, 0, fa[G & 1], fb[G & 1]);
            __builtin_amdgcn_sched_barrier(0);
            mfma_group(fa[(G - 1) & 1], fb[(G - 1) & 1]);
        };
        if (nk > 0) {
#pragma unroll
            for (int st = 0; st < NST - 1; ++st) dma(stage(st), kbeg + st * BK);
            wait_vmcnt<(NST - 2) * NL>();
            __syncthreads();
            read_dma(smem, 0, fa[0], fb[0]);
        }
        for (int kt0 = 0; kt0 < nk; kt0 += NST) {
#pragma unroll
            for (int u = 0; u < NST; ++u)
                if (kt0 + u < nk) step(stage(u), stage((u + 1) % NST), stage((u + NST - 1) % NST), kt0 + u);
        }
        wait_vmcnt<0>();  // the zero-filling loads past the end have landed before LDS is reused
    } else {
        // Software pipeline over K steps (one LDS stage = BK of K per step):
        //   * step kt+1's tile is written to the other LDS stage before step kt's
        //     second-to-last MFMA group, so the stores complete under MFMA work;
        //   * the registers it came from receive the global loads of step kt+2
        //     right after that group's MFMAs are issued (the issue slots before
        //     the barrier are otherwise idle), so the loads have a whole step to
        //     arrive;
        //   * the last group's MFMAs are issued after the barrier, together with
        //     the LDS reads of the next step's first group, so the matrix pipe
        //     has queued work while the barrier and those reads resolve.
        // The other stage is free to overwrite: every wavefront finished reading
        // it before the previous barrier.
        if (nk > 0) {
            gload(kbeg);
            sstore(0);
            if (nk > 1) gload(kbeg + BK);
            __syncthreads();
            read_frags(0, 0, fa[0], fb[0]);
        }
        for (int kt = 0; kt < nk; ++kt) {
            const bool more = kt + 1 < nk;
            const int buf = kt & 1;
    #pragma unroll
            for (int g = 0; g < G - 1; ++g) {
                read_frags(buf, (g + 1) * 8, fa[(g + 1) & 1], fb[(g + 1) & 1]);
                if (g == G - 2 && more) sstore(buf ^ 1);
                mfma_group(fa[g & 1], fb[g & 1]);
                if (g == G - 2 && kt + 2 < nk) gload(kbeg + (kt + 2) * BK);
            }
            // Keep the stores and the second-to-last group's MFMAs ahead of the
            // barrier, and the next step's first LDS reads ahead of the last
            // group's MFMAs (MFMAs carry no memory dependence, so the scheduler
            // would otherwise move them across the barrier).
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            if (more) read_frags(buf ^ 1, 0, fa[G & 1], fb[G & 1]);
            __builtin_amdgcn_sched_barrier(0);
            mfma_group(fa[(G - 1) & 1], fb[(G - 1) & 1]);
        }

    }

    // ------------------------------------------------------------------ epilogue
    const int col_in_block = lane & 31;
    const int row_half = (lane >> 5) * 4;

    if constexpr (EPI == EPI_SPLITK_PARTIAL) {
        float *P = a.out + (int64_t)blockIdx.y * M * N;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * TN + j * 32 + col_in_block;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + wm * TM + i * 32 + (r >> 2) * 8 + row_half + (r & 3);
                    if (m < M && n < N) P[(int64_t)m * N + n] = acc[i][j][r];
                }
        }
    } else if constexpr (EPI == EPI_POOL_GELU_SCALE_ROWMAX || EPI == EPI_GELU_SCALE_ROWMAX) {
        // Row maximum of scale*GELU over this workgroup's columns, one partial
        // per (row, column tile); a second pass takes the max over tiles.
        // With pooling (AvgPool1d(16)): a 16-wide window is 16 consecutive
        // columns, i.e. the 16 lanes of one quarter-wavefront holding the same
        // row; they are summed with butterfly shuffles, and window j is kept
        // only if it lies wholly inside N (floor mode).  Without pooling (the
        // pooled-weight variant, whose columns already are window means) every
        // column < N is a candidate.
        constexpr bool POOL = EPI == EPI_POOL_GELU_SCALE_ROWMAX;
        const int L = N >> 4;
        float bn[FN];
        bool win_ok[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * TN + j * 32 + col_in_block;
            bn[j] = n < N ? a.bias[n] : 0.f;
            win_ok[j] = POOL ? ((n0 + wn * TN + j * 32 + (col_in_block & 16)) >> 4) < L : n < N;
        }
        __syncthreads();  // LDS stages are free now; reuse them for the cross-wave max
        float *red = smem;  // [WAVES_N][BM]
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float mx = -INFINITY;
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    float v = acc[i][j][r] + bn[j];
                    if constexpr (POOL) {
                        v += __shfl_xor(v, 1);
                        v += __shfl_xor(v, 2);
                        v += __shfl_xor(v, 4);
                        v += __shfl_xor(v, 8);
                        v *= 0.0625f;
                    }
                    const float g = gelu_erf(v) * a.tail.scale;
                    mx = fmaxf(mx, win_ok[j] ? g : -INFINITY);
                }
                if constexpr (!POOL) {
                    mx = fmaxf(mx, __shfl_xor(mx, 1));
                    mx = fmaxf(mx, __shfl_xor(mx, 2));
                    mx = fmaxf(mx, __shfl_xor(mx, 4));
                    mx = fmaxf(mx, __shfl_xor(mx, 8));
                }
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                if ((lane & 31) == 0) red[wn * BM + wm * TM + i * 32 + (r >> 2) * 8 + row_half + (r & 3)] = mx;
            }
        __syncthreads();
        for (int t = tid; t < BM; t += NT) {
            const int m = m0 + t;
            if (m < M) {
                float v = red[t];
#pragma unroll
                for (int w = 1; w < WAVES_N; ++w) v = fmaxf(v, red[w * BM + t]);
                a.out[(int64_t)m * a.tiles_n + tn] = v;
            }
        }
    } else {
        using Tail = typename std::conditional<
            EPI == EPI_SCALE_HARDTANH_GELU, TailScaleHardtanhGelu,
            typename std::conditional<EPI == EPI_SWISH_SCALE, TailSwishScale, TailNone>::type>::type;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * TN + j * 32 + col_in_block;
            const bool n_ok = n < N;
            const float bn = n_ok ? a.bias[n] : 0.f;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + wm * TM + i * 32 + (r >> 2) * 8 + row_half + (r & 3);
                    if (m < M && n_ok) a.out[(int64_t)m * N + n] = Tail::apply(acc[i][j][r] + bn, a.tail);
                }
        }
    }
}

// Second pass of split-K: Y[m,n] = tail(sum_{s=0..S-1} P[s,m,n] + b[n]), the
// slices added in increasing s, so the result is the same on every run.
// With vec4 (N % 4 == 0 and Y 16-byte aligned; the workspace always is) each
// thread handles four consecutive columns of one row with 128-bit accesses.
template <int EPI>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float *P, const float *bias, float *Y,
                                                            int64_t MN, int32_t N, int32_t S, TailParams tail,
                                                            int32_t vec4)
{
    using Tail = typename std::conditional<
        EPI == EPI_SCALE_HARDTANH_GELU, TailScaleHardtanhGelu,
        typename std::conditional<EPI == EPI_SWISH_SCALE, TailSwishScale, TailNone>::type>::type;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (vec4) {
        for (; e < MN / 4; e += stride) {
            f32x4 v = reinterpret_cast<const f32x4 *>(P)[e];
            for (int k = 1; k < S; ++k) v += reinterpret_cast<const f32x4 *>(P + (int64_t)k * MN)[e];
            const int n = (int)((e * 4) % N);
#pragma unroll
            for (int c = 0; c < 4; ++c) v[c] = Tail::apply(v[c] + bias[n + c], tail);
            reinterpret_cast<f32x4 *>(Y)[e] = v;
        }
    } else {
        for (; e < MN; e += stride) {
            float v = P[e];
            for (int k = 1; k < S; ++k) v += P[(int64_t)k * MN + e];
            Y[e] = Tail::apply(v + bias[e % N], tail);
        }
    }
}

// Row-max pass over materialised sums, one workgroup (256 threads) per row m:
// y[n] = sum_{s=0..S-1} P[s, m, n] (+ b[n] when bias is given), slices added
// in order; windows of `pool` consecutive columns averaged (pool = 16:
// AvgPool1d(16), floor mode; pool = 1: every column); Y[m] = max_j scale *
// GELU(window j).  Used as the second pass of split-K for the row-max tails
// (S slices, bias) and as the tail pass of the unfused ablation (S = 1, the
// raw output already holds the bias).  Lane t of a 256-column chunk owns
// column n0 + t, so every load is coalesced; a 16-wide window is 16
// consecutive lanes (chunks start at multiples of 16) and is summed with
// butterfly shuffles.
// With vec4 (N % 4 == 0 and P 16-byte aligned) a lane owns four consecutive
// columns instead, loaded with 128-bit reads, and a window is 4 lanes.
__global__ void __launch_bounds__(256) rowmax_pass_kernel(const float *P, const float *bias, float *Y, int64_t MN,
                                                          int32_t N, int32_t S, int32_t pool, float scale,
                                                          int32_t vec4)
{
    __shared__ float red[4];
    const int64_t row = (int64_t)blockIdx.x * N;
    const int ncols = (N / pool) * pool;  // columns that belong to a whole window
    float mx = -INFINITY;
    if (vec4) {
        for (int n0 = 0; n0 < ncols; n0 += 1024) {
            const int n = n0 + 4 * (int)threadIdx.x;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (n < ncols) {
                v = *reinterpret_cast<const f32x4 *>(P + row + n);
                for (int k = 1; k < S; ++k) v += *reinterpret_cast<const f32x4 *>(P + (int64_t)k * MN + row + n);
                if (bias) {
                    v[0] += bias[n];
                    v[1] += bias[n + 1];
                    v[2] += bias[n + 2];
                    v[3] += bias[n + 3];
                }
            }
            if (pool == 16) {
                float w = (v[0] + v[1]) + (v[2] + v[3]);
                w += __shfl_xor(w, 1);
                w += __shfl_xor(w, 2);
                if (n < ncols) mx = fmaxf(mx, gelu_erf(w * 0.0625f) * scale);
            } else if (n < ncols) {
#pragma unroll
                for (int c = 0; c < 4; ++c) mx = fmaxf(mx, gelu_erf(v[c]) * scale);
            }
        }
    }
    for (int n0 = 0; !vec4 && n0 < ncols; n0 += 256) {
        const int n = n0 + (int)threadIdx.x;
        float v = 0.f;
        if (n < ncols) {
            v = P[row + n];
            for (int k = 1; k < S; ++k) v += P[(int64_t)k * MN + row + n];
            if (bias) v += bias[n];
        }
        if (pool == 16) {
            v += __shfl_xor(v, 1);
            v += __shfl_xor(v, 2);
            v += __shfl_xor(v, 4);
            v += __shfl_xor(v, 8);
            v *= 0.0625f;
        }
        if (n < ncols) mx = fmaxf(mx, gelu_erf(v) * scale);
    }
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) Y[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Second pass of tail (b): Y[m] = max over column tiles of the per-tile row
// maxima.  Max is exact, so the result does not depend on order.
__global__ void __launch_bounds__(256) rowmax_finalize_kernel(const float *part, float *Y, int32_t M,
                                                              int32_t tiles_n)
{
    const int m = blockIdx.x * blockDim.x + threadIdx.x;
    if (m >= M) return;
    const float *p = part + (int64_t)m * tiles_n;
    float v = p[0];
    for (int t = 1; t < tiles_n; ++t) v = fmaxf(v, p[t]);
    Y[m] = v;
}

// ---------------------------------------------------------------------------
// Unfused tail kernels: the same tails as separate passes over a materialised
// linear output, as the pages' own solutions run them after a library GEMM.
// They exist to measure what fusing the tail into the GEMM epilogue saves.

// Y[e] = tail(Y[e]) in place, four elements per thread when Y is 16-byte
// aligned and the length is a multiple of 4, else one.
template <int EPI>
__global__ void __launch_bounds__(256) tail_inplace_kernel(float *Y, int64_t count, TailParams tail, int vec4)
{
    using Tail = typename std::conditional<
        EPI == EPI_SCALE_HARDTANH_GELU, TailScaleHardtanhGelu,
        typename std::conditional<EPI == EPI_SWISH_SCALE, TailSwishScale, TailNone>::type>::type;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (vec4) {
        f32x4 *Y4 = reinterpret_cast<f32x4 *>(Y);
        for (; e < count / 4; e += stride) {
            f32x4 v = Y4[e];
            v[0] = Tail::apply(v[0], tail);
            v[1] = Tail::apply(v[1], tail);
            v[2] = Tail::apply(v[2], tail);
            v[3] = Tail::apply(v[3], tail);
            Y4[e] = v;
        }
    } else {
        for (; e < count; e += stride) Y[e] = Tail::apply(Y[e], tail);
    }
}

// ---------------------------------------------------------------------------
// Pooled weights for tail (b): W_p[j, :] = mean over the `pool` rows
// j*pool .. j*pool+pool-1 of W, b_p[j] = mean of the same bias entries, for
// j < floor(N / pool).  Rows are added in increasing order, then scaled by
// 1/pool.  One-dimensional grid of L * chunks workgroups: workgroup w handles
// pooled row w / chunks and 256 float4 columns starting at (w % chunks)*256.
// HBM-bound.
__global__ void __launch_bounds__(256) pool_weights_kernel(const float *W, const float *b, float *Wp, float *bp,
                                                           int64_t K, int32_t pool, int32_t chunks)
{
    const int64_t j = blockIdx.x / chunks;
    const int64_t c4 = (int64_t)(blockIdx.x % chunks) * blockDim.x + threadIdx.x;
    const float inv = 1.0f / (float)pool;
    if (c4 * 4 < K) {
        const float *src = W + (int64_t)j * pool * K + c4 * 4;
        f32x4 s = *reinterpret_cast<const f32x4 *>(src);
        for (int t = 1; t < pool; ++t) s += *reinterpret_cast<const f32x4 *>(src + (int64_t)t * K);
        *reinterpret_cast<f32x4 *>(Wp + (int64_t)j * K + c4 * 4) = s * inv;
    }
    if (blockIdx.x % chunks == 0 && threadIdx.x == 0) {
        float s = b[(int64_t)j * pool];
        for (int t = 1; t < pool; ++t) s += b[(int64_t)j * pool + t];
        bp[j] = s * inv;
    }
}

// ---------------------------------------------------------------------------
// Scale-folded weights for tail (a): Ws = scale * W (128-bit, grid-stride
// over the N*K/4 float4s), bs = scale * b.  HBM-bound.
__global__ void __launch_bounds__(256) scale_weights_kernel(const float *W, const float *b, float *Ws, float *bs,
                                                            int64_t nk4, int64_t N, float scale)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < nk4; e += stride)
        reinterpret_cast<f32x4 *>(Ws)[e] = reinterpret_cast<const f32x4 *>(W)[e] * scale;
    for (int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; n < N; n += stride) bs[n] = b[n] * scale;
}

}  // namespace lin_epi
