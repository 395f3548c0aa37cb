// MFMA-tiled fp32 GEMM with a fused epilogue, for gfx950 (CDNA4).
//
// Computes, for BM x BN output tiles,
//     acc[m, n] = sum_k X[m, k] * W[n, k]        (X [M,K], W [N,K], both K-contiguous)
// with v_mfma_f32_32x32x2_f32 (fp32 products, fp32 accumulation), then
// applies the bias and the tail in registers and stores the result once.
// This is the "compute the GEMM tile into registers, apply the tail, write
// the final output" plan that page "Kimi-K2.6 l2_p53" names as the ideal
// fusion and page "Kimi-K2.6 l2_p59" sketches as a tiled kernel with staged
// input/weight tiles and a register epilogue.
//
// Work partition (schedule.hpp): each workgroup walks a contiguous range of
// (tile, K step) iterations; a tile it computes whole gets the epilogue
// directly, a tile split over several workgroups is finished by the last of
// them to arrive, which adds the others' partial sums in K order first.
//
// Data flow per tile segment (NT = 64 * WAVES_M * WAVES_N threads), two LDS
// stages (double buffer), one K step of 32 per stage:
//   * global -> LDS directly (the buffer-load configurations):
//     buffer_load_dwordx4 ... lds writes each wavefront's 64 x 16 bytes
//     straight into LDS, 8 rows of 128 bytes per instruction, with the 16-byte
//     chunks of a row XOR-swizzled so the fragment reads are bank-conflict
//     free (dma_layout.hpp).  No registers and no LDS store instructions are
//     spent on staging, a step's loads are issued a whole step ahead of their
//     use, and the steady-state loop spends no vector instruction on them:
//     the per-lane offsets (rows past M/N masked) are the same every step.
//   * otherwise global -> registers -> LDS: 128-bit loads, 8 consecutive
//     threads per 128-byte row segment (whole cache lines per wavefront), then
//     128-bit LDS stores with a row stride of 36 floats, so consecutive rows
//     start 4 banks apart and stores and fragment reads are conflict free.
//   * Rows past M/N and K positions outside [0, K) are zero-filled (K is a
//     multiple of 4, so a float4 is all-in or all-out): by out-of-range
//     buffer offsets where buffer loads are used, else by predicated loads.
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

#include "dma_layout.hpp"
#include "epilogue.hpp"
#include "schedule.hpp"

namespace lin_epi {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Epilogue kinds; the numbering follows lin_epi_kind of the C interface.
enum EpiKind : int {
    EPI_NONE = 0,
    EPI_SCALE_HARDTANH_GELU = 1,
    EPI_POOL_GELU_SCALE_ROWMAX = 2,
    EPI_SWISH_SCALE = 3,
    EPI_GELU_SCALE_ROWMAX = 4,  // max over columns of scale*GELU(y): tail (b) on pooled weights
};

struct GemmArgs {
    const float *X;
    const float *W;
    const float *bias;
    float *out;         // Y [M,N]; or row-max partials [M, tiles_n]
    float *partials;    // partial-sum slots of split tiles (2 per workgroup)
    int32_t *counters;  // per-tile arrival counters, zero before and after every launch
    // Row-max tails: when Y is set, the last workgroup of each tile row to
    // finish takes the max over that row's per-tile partials (in `out`) and
    // writes Y [M]; rowcnt holds one arrival counter per tile row, zero
    // before and after every launch.  When Y is null a separate pass does it.
    float *Y;
    int32_t *rowcnt;
    int32_t M, N, K;
    int32_t tiles_m, tiles_n;
    int32_t steps;  // K steps per tile (k_steps(K))
    int32_t koff;   // K position of step s is koff + 32 s (k_offset(K))
    int32_t split;  // split-K segments per tile, 0 = stream-K (schedule.hpp)
    int32_t q, r;   // stream-K: tiles * steps = q * gridDim.x + r
    TailParams tail;
};

// A workgroup tile shape: BM x BN outputs, K step BK, WAVES_M x WAVES_N
// wavefronts each owning a (BM/WAVES_M) x (BN/WAVES_N) sub-tile, and the
// number of workgroups meant to share one compute unit (register budget).
// BUFLOAD selects direct-to-LDS buffer loads where the range-checked form is
// usable (see gemm_epi_kernel); otherwise, and for tiles too large for the
// buffer window, operands go through registers.
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
    static_assert(BK == kStepK, "one K step is one 128-byte row segment");
    static constexpr int NW = WAVES_M * WAVES_N;
    static constexpr int DMA_BLOCKS = ((BM + BN) / 8 + NW - 1) / NW * NW;
    static constexpr int LDS_BYTES = DMA ? STAGES * DMA_BLOCKS * 1024 : 2 * (BM + BN) * (BK + 4) * 4;
    // The register-staged form (padded rows) may fit fewer workgroups per CU.
    static constexpr int LDS_BYTES_REG = 2 * (BM + BN) * (BK + 4) * 4;
    static constexpr int WG_PER_CU_REG = WG_PER_CU < 160 * 1024 / LDS_BYTES_REG ? WG_PER_CU : 160 * 1024 / LDS_BYTES_REG;
    static constexpr int WAVES_PER_SIMD_REG = (WG_PER_CU_REG * WAVES_M * WAVES_N + 3) / 4;
    // floats in one partial-sum slot: the raw tile, or (tail (b)) its
    // 16-column window sums
    static constexpr int SLOT_FLOATS_RAW = BM * BN;
    static constexpr int SLOT_FLOATS_POOL = BM * BN / 16;
};

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt bits [3:0] and [15:14]; expcnt
// and lgkmcnt left at their maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Sum of register x[r] over the 16 lanes of each quarter-wavefront, for all
// 16 registers at once: four butterfly stages (xor 1, 2, 4, 8) that halve
// the register count each time, lanes with the stage's bit set keeping the
// odd register of each pair.  Lane 16q + u ends with the quarter's sum of
// register u.  15 exchanges instead of 4 per register.
template <int D>
__device__ __forceinline__ void halve_stage(float (&x)[16], int lane)
{
    constexpr int PAIRS = 16 / (2 * D);
    const bool upper = lane & D;
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) {
        const float keep = upper ? x[2 * p + 1] : x[2 * p];
        const float give = upper ? x[2 * p] : x[2 * p + 1];
        x[p] = keep + __shfl_xor(give, D);
    }
}

__device__ __forceinline__ float quarter_sums(float (&x)[16], int lane)
{
    halve_stage<1>(x, lane);
    halve_stage<2>(x, lane);
    halve_stage<4>(x, lane);
    halve_stage<8>(x, lane);
    return x[0];
}

// SPLIT = false: one whole tile per workgroup (grid = tiles); no segment
// loop and no partial-sum code, so these kernels keep their registers for
// the K loop.  SPLIT = true: the general partition of schedule.hpp.
template <class Cfg, int EPI, bool BUF, bool SPLIT>
__global__ void __launch_bounds__(Cfg::THREADS, BUF ? Cfg::WAVES_PER_SIMD : Cfg::WAVES_PER_SIMD_REG)
gemm_epi_kernel(GemmArgs a)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, WAVES_M = Cfg::WAVES_M, WAVES_N = Cfg::WAVES_N;
    constexpr int NT = Cfg::THREADS;
    constexpr int NW = Cfg::NW;
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
    constexpr bool POOL = EPI == EPI_POOL_GELU_SCALE_ROWMAX;
    constexpr bool ROWMAX = POOL || EPI == EPI_GELU_SCALE_ROWMAX;
    constexpr int SLOT = POOL ? Cfg::SLOT_FLOATS_POOL : Cfg::SLOT_FLOATS_RAW;
    static_assert(BK % 8 == 0 && TM % 32 == 0 && TN % 32 == 0, "tile shape");

    // Direct-to-LDS staging (DMA): NST separate LDS arrays, one per stage
    // (smem is stage 0); register staging: two padded stages in smem.
    constexpr bool DMA = BUF;
    static_assert(!BUF || Cfg::DMA, "buffer loads are used on the direct-to-LDS path only");
    constexpr int NST = Cfg::STAGES;
    static_assert(NST >= 2 && NST <= 4, "2 to 4 DMA stages");
    constexpr int DMA_STAGE = Cfg::DMA_BLOCKS * 256;  // floats per DMA stage
    __shared__ __attribute__((aligned(16))) float smem[DMA ? DMA_STAGE : 2 * STAGE];
    __shared__ __attribute__((aligned(16))) float smem1[DMA ? DMA_STAGE : 4];
    __shared__ __attribute__((aligned(16))) float smem2[DMA && NST > 2 ? DMA_STAGE : 4];
    __shared__ __attribute__((aligned(16))) float smem3[DMA && NST > 3 ? DMA_STAGE : 4];
    auto stage = [&](int st) -> float * { return st == 0 ? smem : st == 1 ? smem1 : st == 2 ? smem2 : smem3; };

    const int tid0 = threadIdx.x;
    const int wave = tid0 >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int wm = wave / WAVES_N;
    const int wn = wave % WAVES_N;
    const int M = a.M, N = a.N, K = a.K;
    const int G = gridDim.x;
    const int steps = a.steps;
    const Partition part{steps, G, a.split, a.q, a.r};

    // this workgroup's range of (tile, K step) iterations: from K step s0 of
    // tile t onwards, tile by tile (one whole tile when !SPLIT)
    const int v = virtual_wg(blockIdx.x, G);
    int it = SPLIT ? range_begin(part, v) : 0;
    const int it_end = SPLIT ? range_begin(part, v + 1) : 1;
    int t = SPLIT ? it / steps : v;
    int s0 = SPLIT ? it - t * steps : 0;

    // Operand fragments of one 8-deep K group ("sub-step"), double-buffered in
    // registers so the next group's LDS reads overlap this group's MFMAs.
    constexpr int G8 = BK / 8;
    f32x4 fa[2][FM], fb[2][FN];
    f32x16 acc[FM][FN];
    f32x4 ra[A_LD], rb[B_LD];

    auto mfma_group = [&](const f32x4 (&af)[FM], const f32x4 (&bf)[FN]) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][c], bf[j][c], acc[i][j], 0, 0, 0);
    };

    do {
        // ---------------------------------------------------- one tile segment
        // Lane-derived values are recomputed per segment (the empty asm hides
        // that they do not change), so none of them is hoisted above the
        // segment loop and kept live through the K loop.
        int tid = tid0;
        if constexpr (SPLIT) asm volatile("" : "+v"(tid));
        const int lane = tid & 63;
        const int frag_row = lane & 31;
        const int frag_k = (lane >> 5) * 4;
        const int col_in_block = lane & 31;
        const int row_half = (lane >> 5) * 4;
        const int s1 = SPLIT && it_end - it < steps - s0 ? s0 + (it_end - it) : steps;
        it += s1 - s0;
        const int nk = s1 - s0;
        int tm, tn;
        tile_coords<8>(t, a.tiles_m, a.tiles_n, tm, tn);
        const int m0 = tm * BM;
        const int n0 = tn * BN;
        const int a_rows = min(BM, M - m0), b_rows = min(BN, N - n0);

#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

        if constexpr (DMA) {
            // Each LDS stage holds the tile's BM rows of X then BN rows of W,
            // 128 bytes per row, unpadded, then padding blocks up to a multiple
            // of the wavefront count; one buffer_load ... lds instruction
            // writes one 8-row block of 1 KiB (dma_layout.hpp).  One buffer
            // resource per operand covers the tile's valid rows; for steps
            // past the segment's end a zero-length one, so those loads write
            // zeros and read no memory (a scalar select, no per-lane work).
            constexpr int NBA = BM / 8, NB = (BM + BN) / 8;  // 8-row blocks of X, of X and W
            constexpr int NL = Cfg::DMA_BLOCKS / NW;          // DMA instructions per wavefront and step
            static_assert(NW % 2 == 0 && NBA % 2 == 0, "block parity = wavefront parity");
            const int a_bytes = a_rows * K * 4, b_bytes = b_rows * K * 4;
            float *const xa = const_cast<float *>(a.X + (int64_t)m0 * K);
            float *const wb = const_cast<float *>(a.W + (int64_t)n0 * K);
            // K step s (steady state: K positions koff + 32 s .. + 31, all
            // inside [0, K) for 1 <= s < steps) into LDS stage st.
            auto dma = [&](float *st, int s) {
                const bool live = s < s1;
                const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(xa, (short)0, live ? a_bytes : 0, 0x00020000);
                const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(wb, (short)0, live ? b_bytes : 0, 0x00020000);
                const int k0 = a.koff + kStepK * s;
#pragma unroll
                for (int i = 0; i < NL; ++i) {
                    const DmaLoad ld = dma_load_of<BM, BN, NW>(i, wave_u, lane);
                    const int blk = i * NW + wave_u;
                    auto *dst = (__attribute__((address_space(3))) void *)(st + blk * 256);
                    const bool all_a = (i + 1) * NW <= NBA, all_b = i * NW >= NBA && (i + 1) * NW <= NB;
                    if (all_a || (!all_b && blk < NBA)) {
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, dst, 16, dma_voffset(ld.row, ld.chunk, 0, ld.row < a_rows, K),
                                                                 dma_soffset(blk, k0, K), 0, 0);
                    } else if (all_b || blk < NB) {
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, dst, 16, dma_voffset(ld.row, ld.chunk, 0, ld.row < b_rows, K),
                                                                 dma_soffset(blk - NBA, k0, K), 0, 0);
                    } else {  // padding block: zeros, never read
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, dst, 16, kOobOffset, 0, 0, 0);
                    }
                }
            };
            // K step 0 when K % 32 != 0: positions koff .. koff + 31 start
            // before 0, so the K shift and the K mask go in the per-lane
            // offset (the scalar offset stays non-negative).  Prologue only.
            auto dma_first = [&](float *st) {
                const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(xa, (short)0, a_bytes, 0x00020000);
                const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(wb, (short)0, b_bytes, 0x00020000);
#pragma unroll
                for (int i = 0; i < NL; ++i) {
                    const DmaLoad ld = dma_load_of<BM, BN, NW>(i, wave_u, lane);
                    const int blk = i * NW + wave_u;
                    const bool k_ok = a.koff + 4 * ld.chunk >= 0;
                    auto *dst = (__attribute__((address_space(3))) void *)(st + blk * 256);
                    if (blk < NBA) {
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            rsA, dst, 16, dma_voffset(ld.row, ld.chunk, a.koff, k_ok && ld.row < a_rows, K),
                            dma_soffset(blk, 0, K), 0, 0);
                    } else if (blk < NB) {
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            rsB, dst, 16, dma_voffset(ld.row, ld.chunk, a.koff, k_ok && ld.row < b_rows, K),
                            dma_soffset(blk - NBA, 0, K), 0, 0);
                    } else {
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, dst, 16, kOobOffset, 0, 0, 0);
                    }
                }
            };
            // physical chunk of logical chunk 2g + lane/32 in this lane's
            // fragment row (X and W fragment rows start at multiples of 32)
            const int tsw = (lane >> 5) ^ lds_swizzle(frag_row);
            auto read_dma = [&](const float *st, int g, f32x4 (&af)[FM], f32x4 (&bf)[FN]) {
                const int ch = 4 * ((2 * g) ^ tsw);
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    af[i] = *reinterpret_cast<const f32x4 *>(st + (wm * TM + i * 32 + frag_row) * BK + ch);
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    bf[j] = *reinterpret_cast<const f32x4 *>(st + (BM + wn * TN + j * 32 + frag_row) * BK + ch);
            };
            // One K step kt of the segment (stage kt % NST): the DMA of step
            // kt+NST-1 goes into the stage step kt-1 used (every wavefront
            // finished reading it before the previous barrier), so loads are
            // issued NST-1 steps ahead; before the barrier, a wait until at
            // most the NST-2 younger steps' loads are outstanding, i.e. step
            // kt+1 has landed (loads complete in order).  The DMA instructions
            // are spread over the first group's MFMAs (one per 4*FM*FN/NL
            // MFMAs): issued back to back they would hold every wavefront of
            // the CU off the matrix pipes at the same moment, right after the
            // barrier.  The stages are separate LDS arrays and the loop is
            // unrolled by NST, so the compiler can tell a DMA target from the
            // stage being read and does not make those reads wait for the DMA.
            auto step = [&](float *cur, float *nxt, float *fre, int kt) {
                dma(fre, s0 + kt + NST - 1);
                read_dma(cur, 1, fa[1], fb[1]);
                mfma_group(fa[0], fb[0]);
                // scheduling groups (masks: 0x100 LDS reads, 0x008 MFMA, 0x020
                // vector-memory reads): the next group's fragment reads first,
                // then MFMAs and DMA instructions alternating
                __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);
#pragma unroll
                for (int d = 0; d < NL; ++d) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 4 * FM * FN / NL, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int g = 1; g < G8 - 1; ++g) {
                    read_dma(cur, g + 1, fa[(g + 1) & 1], fb[(g + 1) & 1]);
                    mfma_group(fa[g & 1], fb[g & 1]);
                }
                __builtin_amdgcn_sched_barrier(0);
                wait_vmcnt<(NST - 2) * NL>();
                __syncthreads();
                if (kt + 1 < nk) read_dma(nxt, 0, fa[G8 & 1], fb[G8 & 1]);
                __builtin_amdgcn_sched_barrier(0);
                mfma_group(fa[(G8 - 1) & 1], fb[(G8 - 1) & 1]);
            };
            if (s0 == 0 && a.koff < 0)
                dma_first(stage(0));
            else
                dma(stage(0), s0);
#pragma unroll
            for (int st = 1; st < NST - 1; ++st) dma(stage(st), s0 + st);
            wait_vmcnt<(NST - 2) * NL>();
            __syncthreads();
            read_dma(smem, 0, fa[0], fb[0]);
            for (int kt0 = 0; kt0 < nk; kt0 += NST) {
#pragma unroll
                for (int u = 0; u < NST; ++u)
                    if (kt0 + u < nk) step(stage(u), stage((u + 1) % NST), stage((u + NST - 1) % NST), kt0 + u);
            }
            wait_vmcnt<0>();  // the zero-filling loads past the end have landed before LDS is reused
        } else {
            // Register staging: predicated 128-bit loads of K step s, zero
            // outside rows M/N and K positions [0, K).
            auto gload = [&](int s) {
                const int k0 = a.koff + kStepK * s;
#pragma unroll
                for (int i = 0; i < A_LD; ++i) {
                    const int idx = tid + i * NT;
                    const int row = idx / C4;
                    const int gk = k0 + (idx % C4) * 4;
                    const int gm = m0 + row;
                    f32x4 x = {0.f, 0.f, 0.f, 0.f};
                    if ((A_EVEN || idx < BM * C4) && gm < M && gk >= 0 && gk < K)
                        x = *reinterpret_cast<const f32x4 *>(a.X + (int64_t)gm * K + gk);
                    ra[i] = x;
                }
#pragma unroll
                for (int i = 0; i < B_LD; ++i) {
                    const int idx = tid + i * NT;
                    const int row = idx / C4;
                    const int gk = k0 + (idx % C4) * 4;
                    const int gn = n0 + row;
                    f32x4 x = {0.f, 0.f, 0.f, 0.f};
                    if ((B_EVEN || idx < BN * C4) && gn < N && gk >= 0 && gk < K)
                        x = *reinterpret_cast<const f32x4 *>(a.W + (int64_t)gn * K + gk);
                    rb[i] = x;
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
            // Software pipeline over K steps (one LDS stage per step):
            //   * step kt+1's tile is written to the other LDS stage before step
            //     kt's second-to-last MFMA group, so the stores complete under
            //     MFMA work;
            //   * the registers it came from receive the global loads of step
            //     kt+2 right after that group's MFMAs are issued, so the loads
            //     have a whole step to arrive;
            //   * the last group's MFMAs are issued after the barrier, together
            //     with the LDS reads of the next step's first group, so the
            //     matrix pipe has queued work while the barrier and those reads
            //     resolve.
            // The other stage is free to overwrite: every wavefront finished
            // reading it before the previous barrier.
            gload(s0);
            sstore(0);
            if (nk > 1) gload(s0 + 1);
            __syncthreads();
            read_frags(0, 0, fa[0], fb[0]);
            for (int kt = 0; kt < nk; ++kt) {
                const bool more = kt + 1 < nk;
                const int buf = kt & 1;
#pragma unroll
                for (int g = 0; g < G8 - 1; ++g) {
                    read_frags(buf, (g + 1) * 8, fa[(g + 1) & 1], fb[(g + 1) & 1]);
                    if (g == G8 - 2 && more) sstore(buf ^ 1);
                    mfma_group(fa[g & 1], fb[g & 1]);
                    if (g == G8 - 2 && kt + 2 < nk) gload(s0 + kt + 2);
                }
                // Keep the stores and the second-to-last group's MFMAs ahead of
                // the barrier, and the next step's first LDS reads ahead of the
                // last group's MFMAs (MFMAs carry no memory dependence, so the
                // scheduler would otherwise move them across the barrier).
                __builtin_amdgcn_sched_barrier(0);
                __syncthreads();
                if (more) read_frags(buf ^ 1, 0, fa[G8 & 1], fb[G8 & 1]);
                __builtin_amdgcn_sched_barrier(0);
                mfma_group(fa[(G8 - 1) & 1], fb[(G8 - 1) & 1]);
            }
        }

        // ----------------------------------------------------------- epilogue
        // Tail (b): the 16-wide pool windows of this segment's sums, lane
        // 16q + u holding window (block column half q % 2) of accumulator
        // register u; the bias belongs to the segment that starts at K step 0.
        float win[FM][FN];
        if constexpr (POOL) {
            float bn[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = n0 + wn * TN + j * 32 + col_in_block;
                bn[j] = (s0 == 0 && n < N) ? a.bias[n] : 0.f;
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    float x[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r) x[r] = acc[i][j][r] + bn[j];
                    win[i][j] = quarter_sums(x, lane);
                }
        }

        // Split tile: publish this segment's sums, and if it is the last of
        // the tile's segments to arrive, add all of them in K order.
        bool finish = s0 == 0 && s1 == steps;
        if (SPLIT && !finish) {
            // the LDS stages are free once every wavefront's loads have
            // landed; their first word carries the arrival flag
            __syncthreads();
            int &s_flag = *reinterpret_cast<int *>(smem);
            const TileSegs sg = tile_segments(part, t);
            const int nseg = sg.last - sg.first + 1;
            int *cnt = a.counters + t;
            // Partial sums travel with device-scope cache policy (sc1, as the
            // compiler emits for agent-scope atomics): stores write through the
            // XCD's L2 and loads miss in it, so the sums of a segment computed
            // on another XCD are seen without writing back or invalidating
            // whole caches.  One buffer resource per slot (offsets < 1 MiB).
            constexpr int kDeviceScope = 16;  // cache-policy bit sc1
            auto slot_rsrc = [&](int u) {
                float *base = a.partials + (int64_t)partial_slot(part, u, t) * SLOT;
                return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, SLOT * 4, 0x00020000);
            };
            const int wave_off = wave_u * (SLOT / NW) * 4;  // this wavefront's bytes in a slot
            auto store_own = [&]() {
                const __amdgpu_buffer_rsrc_t rs = slot_rsrc(v);
                if constexpr (POOL) {
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j)
                            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, win[i][j]), rs,
                                                                  ((i * FN + j) * 64 + lane) * 4, wave_off, kDeviceScope);
                } else {
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j)
#pragma unroll
                            for (int c4 = 0; c4 < 4; ++c4) {
                                const f32x4 x = {acc[i][j][4 * c4], acc[i][j][4 * c4 + 1], acc[i][j][4 * c4 + 2],
                                                 acc[i][j][4 * c4 + 3]};
                                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rs,
                                                                       (((i * FN + j) * 4 + c4) * 64 + lane) * 16,
                                                                       wave_off, kDeviceScope);
                            }
                }
            };
            // SET: sums := segment u's; else sums += segment u's.  The raw
            // sums are read in batches of BATCH MFMA blocks (4 * BATCH 128-bit
            // loads in flight), so the reads do not need a second
            // accumulator's worth of registers.
            auto combine = [&](int u, auto set_tag) {
                constexpr bool SET = decltype(set_tag)::value;
                const __amdgpu_buffer_rsrc_t rs = slot_rsrc(u);
                if constexpr (POOL) {
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j) {
                            const float x = __builtin_bit_cast(
                                float, __builtin_amdgcn_raw_buffer_load_b32(rs, ((i * FN + j) * 64 + lane) * 4, wave_off,
                                                                            kDeviceScope));
                            win[i][j] = SET ? x : win[i][j] + x;
                        }
                } else {
                    constexpr int BATCH = FM * FN > 4 ? 2 : FM * FN;
#pragma unroll
                    for (int b = 0; b < FM * FN; ++b) {
                        const int i = b / FN, j = b % FN;
#pragma unroll
                        for (int c4 = 0; c4 < 4; ++c4) {
                            const f32x4 x = __builtin_bit_cast(
                                f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, ((b * 4 + c4) * 64 + lane) * 16, wave_off,
                                                                             kDeviceScope));
#pragma unroll
                            for (int c = 0; c < 4; ++c)
                                acc[i][j][4 * c4 + c] = SET ? x[c] : acc[i][j][4 * c4 + c] + x[c];
                        }
                        if ((b + 1) % BATCH == 0) __builtin_amdgcn_sched_barrier(0);
                    }
                }
            };
            using Set = std::true_type;
            using Add = std::false_type;
            // Arrival: a segment that finds all the others already counted is
            // the last and keeps its sums in registers; otherwise it publishes
            // them (device-scope stores, every wavefront waits for them to
            // complete, then the count), and the one whose count completes the
            // tile is the last.  The counter is only touched with device-scope
            // atomics; the last segment reads the others' sums after seeing
            // the full count, with device-scope loads.
            if (tid == 0) s_flag = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nseg - 1;
            __syncthreads();
            bool last = s_flag;
            bool own_published = false;
            if (!last) {
                store_own();
                wait_vmcnt<0>();
                __syncthreads();
                if (tid == 0)
                    s_flag = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nseg - 1;
                __syncthreads();
                last = s_flag;
                own_published = true;
            }
            if (last) {
                if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                // Sum in segment order.  When this segment is the first (or
                // one of only two, where the order of one addition does not
                // matter) its sums stay in registers; otherwise they are read
                // back in their place in the order.
                const int own = v - sg.first;
                if (own == 0 || nseg == 2) {
                    for (int u = sg.first; u <= sg.last; ++u)
                        if (u != v) combine(u, Add{});
                } else {
                    if (!own_published) {
                        store_own();
                        wait_vmcnt<0>();  // read back below, in segment order
                    }
                    combine(sg.first, Set{});
                    for (int u = sg.first + 1; u <= sg.last; ++u) combine(u, Add{});
                }
                finish = true;
            }
        }

        // Row-max tails: this tile's row maxima (cross-wavefront partials in
        // red[WAVES_N][BM]) go to the per-(row, tile) partials; then, when the
        // kernel finishes the rows itself, the last of the tile row's
        // workgroups to arrive (device-scope counter, as for split tiles)
        // takes the max over the row's partials, one wavefront per row, lanes
        // over the tiles.  The partials are written and read back with
        // relaxed device-scope atomics (plain loads and stores with
        // device-scope cache policy), 64-bit addressed.
        auto publish_row_max = [&](const float *red) {
            const int rows = min(BM, M - m0);
            uint32_t *const part = reinterpret_cast<uint32_t *>(a.out + (int64_t)m0 * a.tiles_n);
            __syncthreads();
            for (int r = tid; r < rows; r += NT) {
                float x = red[r];
#pragma unroll
                for (int w = 1; w < WAVES_N; ++w) x = fmaxf(x, red[w * BM + r]);
                __hip_atomic_store(part + (int64_t)r * a.tiles_n + tn, __builtin_bit_cast(uint32_t, x), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
            if (!a.Y) return;
            wait_vmcnt<0>();
            __syncthreads();  // red is read: its first word can hold the flag
            int &s_row_last = *reinterpret_cast<int *>(smem);
            if (tid == 0)
                s_row_last = __hip_atomic_fetch_add(a.rowcnt + tm, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                             a.tiles_n - 1;
            __syncthreads();
            if (!s_row_last) return;
            if (tid == 0) __hip_atomic_store(a.rowcnt + tm, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int r = wave_u; r < rows; r += NW) {
                const uint32_t *pr = part + (int64_t)r * a.tiles_n;
                float v = -INFINITY;
                for (int t = lane; t < a.tiles_n; t += 64)
                    v = fmaxf(v, __builtin_bit_cast(float, __hip_atomic_load(pr + t, __ATOMIC_RELAXED,
                                                                             __HIP_MEMORY_SCOPE_AGENT)));
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
                if (lane == 0) a.Y[m0 + r] = v;
            }
        };

        if (finish) {
            if constexpr (POOL) {
                // Row maximum of scale * GELU(window mean) over this tile's
                // windows, one partial per (row, column tile); a second pass
                // takes the max over tiles.  Window (block j, half q % 2)
                // counts only if it lies wholly inside N (floor mode).
                const int L = N >> 4;
                const int u = lane & 15, qw = lane >> 4;  // lane 16 qw + u
                __syncthreads();  // LDS stages are free now; reuse them for the cross-wave max
                float *red = smem;  // [WAVES_N][BM]
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    float mx = -INFINITY;
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const int wcol = n0 + wn * TN + j * 32 + 16 * (qw & 1);
                        const float g = gelu_erf(win[i][j] * 0.0625f) * a.tail.scale;
                        mx = fmaxf(mx, (wcol >> 4) < L ? g : -INFINITY);
                    }
                    mx = fmaxf(mx, __shfl_xor(mx, 16));
                    if (!(qw & 1)) red[wn * BM + wm * TM + i * 32 + 8 * (u >> 2) + 4 * (qw >> 1) + (u & 3)] = mx;
                }
                publish_row_max(red);
            } else if constexpr (ROWMAX) {
                // Row maximum of scale * GELU(y) over this tile's columns (the
                // pooled-weight form, whose columns already are window means).
                float bn[FN];
                bool col_ok[FN];
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int n = n0 + wn * TN + j * 32 + col_in_block;
                    bn[j] = n < N ? a.bias[n] : 0.f;
                    col_ok[j] = n < N;
                }
                __syncthreads();
                float *red = smem;  // [WAVES_N][BM]
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float mx = -INFINITY;
#pragma unroll
                        for (int j = 0; j < FN; ++j) {
                            const float g = gelu_erf(acc[i][j][r] + bn[j]) * a.tail.scale;
                            mx = fmaxf(mx, col_ok[j] ? g : -INFINITY);
                        }
                        mx = fmaxf(mx, __shfl_xor(mx, 1));
                        mx = fmaxf(mx, __shfl_xor(mx, 2));
                        mx = fmaxf(mx, __shfl_xor(mx, 4));
                        mx = fmaxf(mx, __shfl_xor(mx, 8));
                        mx = fmaxf(mx, __shfl_xor(mx, 16));
                        if ((lane & 31) == 0) red[wn * BM + wm * TM + i * 32 + (r >> 2) * 8 + row_half + (r & 3)] = mx;
                    }
                publish_row_max(red);
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
        if constexpr (SPLIT) __syncthreads();  // LDS is reused by the next segment
        ++t;
        s0 = 0;
    } while (SPLIT && it < it_end);
}

// Second pass of the row-max tails behind the weight-streaming kernel (the
// tile kernel finishes its rows itself): Y[m] = max over column blocks of the
// per-block row maxima, one wavefront per row (lanes take every 64th partial,
// then a butterfly).  Max is exact, so the result does not depend on order.
__global__ void __launch_bounds__(256) rowmax_finalize_kernel(const float *part, float *Y, int32_t M,
                                                              int32_t tiles_n)
{
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (m >= M) return;
    const float *p = part + (int64_t)m * tiles_n;
    float v = -INFINITY;
    for (int t = lane; t < tiles_n; t += 64) v = fmaxf(v, p[t]);
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    if (lane == 0) Y[m] = v;
}

// ---------------------------------------------------------------------------
// Unfused tail kernels: the same tails as separate passes over a materialised
// linear output, as the pages' own solutions run them after a library GEMM.
// They exist to measure what fusing the tail into the GEMM epilogue saves.

// Row-max pass over a materialised linear output y [M, N] (bias included),
// one workgroup (256 threads) per row m: windows of `pool` consecutive
// columns averaged (pool = 16: AvgPool1d(16), floor mode; pool = 1: every
// column); Y[m] = max_j scale * GELU(window j).  Lane t of a 256-column
// chunk owns column n0 + t, so every load is coalesced; a 16-wide window is
// 16 consecutive lanes (chunks start at multiples of 16) and is summed with
// butterfly shuffles.  With vec4 (N % 4 == 0 and y 16-byte aligned) a lane
// owns four consecutive columns instead, loaded with 128-bit reads, and a
// window is 4 lanes.
__global__ void __launch_bounds__(256) rowmax_pass_kernel(const float *P, float *Y, int32_t N, int32_t pool,
                                                          float scale, int32_t vec4)
{
    __shared__ float red[4];
    const int64_t row = (int64_t)blockIdx.x * N;
    const int ncols = (N / pool) * pool;  // columns that belong to a whole window
    float mx = -INFINITY;
    if (vec4) {
        for (int n0 = 0; n0 < ncols; n0 += 1024) {
            const int n = n0 + 4 * (int)threadIdx.x;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (n < ncols) v = *reinterpret_cast<const f32x4 *>(P + row + n);
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
        float v = n < ncols ? P[row + n] : 0.f;
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

// Arrival counters of split tiles start at zero: cleared by a kernel (not a
// memset) whenever a workspace is (re)allocated.
__global__ void __launch_bounds__(256) zero_counters_kernel(int32_t *c, int64_t n)
{
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x)
        c[e] = 0;
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
