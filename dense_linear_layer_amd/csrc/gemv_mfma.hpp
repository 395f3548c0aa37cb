// Weight-streaming form of the fused linear layer, for few rows of X (the
// decode-size batches of page "Kimi-K2.6 l2_p59", its small-M discussion:
// with a handful of rows the layer is bound by reading W once from HBM, not
// by arithmetic).
//
// Every wavefront works alone: it owns 16 rows of X (zero-padded past M),
// FN blocks of 16 rows of W and one contiguous run of K steps, and
// multiplies them with v_mfma_f32_16x16x4_f32.  Nothing is staged in LDS and
// there is no barrier: each lane loads its own MFMA operand fragments from
// global memory straight into a ring of D K steps of registers, so a
// wavefront keeps D steps of weight loads in flight while it multiplies the
// oldest one.  That many bytes in flight per CU is what a plain streaming
// read needs to reach the HBM rate; an LDS-staged tile is limited by its
// stages.
//
// Fragments of one 32-deep K step at K position k0 (lane l, r = l % 16,
// q = l / 16): the lane loads X[m0 + r][k0 + 8q .. 8q + 7] and
// W[n0 + r][k0 + 8q .. 8q + 7] as two 128-bit halves.  MFMA (h, c) (half h,
// component c) takes k-slot q from component c of half h, so it sums
// k = k0 + 8q + 4h + c over q: the 8 MFMAs of the step cover the 32 K
// positions once, and X and W use the same assignment.  Each W row's 128
// bytes of the step are read by its 4 lanes as whole 32-byte pieces.
//
// Accumulator of one 16x16 block (4 VGPRs): lane l, register i holds
// C[4 (l / 16) + i][l % 16].
//
// Work partition: unit u = (row block of X, row block of W, K segment), one
// per wavefront; the S segments of a block split its K steps evenly and the
// last of them to finish adds the others' partial sums in segment order
// (deterministic), then applies the bias and the tail.  Rows past M or N
// and K positions outside [0, K) read as zeros (dma_layout.hpp's rule: an
// out-of-range per-lane offset against a resource sized to the valid rows).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dma_layout.hpp"
#include "epilogue.hpp"
#include "gemm_mfma.hpp"
#include "schedule.hpp"

namespace lin_epi {

struct GemvArgs {
    const float *X;
    const float *W;
    const float *bias;
    float *out;         // Y [M,N]; or row-max partials [M, wblocks]
    float *partials;    // one slot of 16 x 16*FN floats per unit
    int32_t *counters;  // per (X block, W block) arrival counters, zero before and after every launch
    int32_t M, N, K;
    int32_t wblocks;  // row blocks of W (16*FN rows each)
    int32_t units;    // mblocks * wblocks * split
    int32_t steps;    // K steps (k_steps(K))
    int32_t koff;     // K position of step s is koff + 32 s
    int32_t split;    // K segments per block
    TailParams tail;
};

constexpr int kGemvWaves = 4;  // wavefronts per workgroup (independent units)

// Rows of W per wavefront (16 * FN) and the depth D of the register ring.
template <int EPI, int FN, int D>
__global__ void __launch_bounds__(64 * kGemvWaves) gemv_mfma_kernel(GemvArgs a)
{
    constexpr int KH = 2;  // 128-bit halves per lane and step: 4 lanes x 32 bytes = one 128-byte row piece
    static_assert(16 * KH == kStepK, "one K step of the schedule");
    constexpr bool POOL = EPI == EPI_POOL_GELU_SCALE_ROWMAX;
    constexpr bool ROWMAX = POOL || EPI == EPI_GELU_SCALE_ROWMAX;
    constexpr int kDeviceScope = 16;  // cache-policy bit sc1 (see gemm_epi_kernel)
    constexpr int SLOT = 16 * 16 * FN;

    const int lane = threadIdx.x & 63;
    const int unit = __builtin_amdgcn_readfirstlane(blockIdx.x * kGemvWaves + (threadIdx.x >> 6));
    if (unit >= a.units) return;  // whole wavefronts only; the kernel has no barrier
    const int r = lane & 15, q = lane >> 4;
    const int M = a.M, N = a.N, K = a.K;
    const int S = a.split;
    const int seg = unit % S;
    const int blk = unit / S;
    const int rb = blk % a.wblocks, mb = blk / a.wblocks;
    const int n0 = rb * 16 * FN, m0 = mb * 16;
    const int wrows = min(16 * FN, N - n0), xrows = min(16, M - m0);
    const int s_begin = (int)((int64_t)seg * a.steps / S), s_end = (int)((int64_t)(seg + 1) * a.steps / S);

    // One buffer resource per operand over its valid rows; rows past them get
    // the out-of-range offset.  Steady-state offsets (K position in the scalar
    // offset) are the same every step.
    float *const xb = const_cast<float *>(a.X + (int64_t)m0 * K);
    float *const wb = const_cast<float *>(a.W + (int64_t)n0 * K);
    const int xbytes = xrows * K * 4, wbytes = wrows * K * 4;
    const int vx = r < xrows ? (r * K + 4 * KH * q) * 4 : kOobOffset;
    int vw[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) vw[j] = 16 * j + r < wrows ? ((16 * j + r) * K + 4 * KH * q) * 4 : kOobOffset;

    f32x4 xr[D][KH], wr[D][FN][KH];
    auto ld = [&](__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
        return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0));
    };
    // K step s into ring slot `slot`; steps past the segment read through
    // zero-length resources (zeros, no memory access)
    auto load = [&](int slot, int s) {
        const bool live = s < s_end;
        const __amdgpu_buffer_rsrc_t rsX = __builtin_amdgcn_make_buffer_rsrc(xb, (short)0, live ? xbytes : 0, 0x00020000);
        const __amdgpu_buffer_rsrc_t rsW = __builtin_amdgcn_make_buffer_rsrc(wb, (short)0, live ? wbytes : 0, 0x00020000);
        const int soff = (a.koff + kStepK * s) * 4;
#pragma unroll
        for (int h = 0; h < KH; ++h) xr[slot][h] = ld(rsX, vx + 16 * h, soff);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int h = 0; h < KH; ++h) wr[slot][j][h] = ld(rsW, vw[j] + 16 * h, soff);
    };
    // Step 0 when K % 32 != 0 starts before K = 0: its K shift and mask go in
    // the per-lane offsets (a float4 is wholly inside or outside [0, K)).
    auto load_first = [&](int slot) {
        const __amdgpu_buffer_rsrc_t rsX = __builtin_amdgcn_make_buffer_rsrc(xb, (short)0, xbytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rsW = __builtin_amdgcn_make_buffer_rsrc(wb, (short)0, wbytes, 0x00020000);
#pragma unroll
        for (int h = 0; h < KH; ++h) {
            const bool k_ok = a.koff + 4 * KH * q + 4 * h >= 0;
            xr[slot][h] = ld(rsX, k_ok && r < xrows ? vx + (a.koff + 4 * h) * 4 : kOobOffset, 0);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                wr[slot][j][h] = ld(rsW, k_ok && 16 * j + r < wrows ? vw[j] + (a.koff + 4 * h) * 4 : kOobOffset, 0);
        }
    };

    f32x4 acc[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The ring is filled in slot order (the scheduling barriers keep it so):
    // the loop then finds slot u's loads to be the oldest outstanding ones on
    // entry as on every later round, so each slot waits only for its own.
    if (s_begin == 0 && a.koff < 0)
        load_first(0);
    else
        load(0, s_begin);
#pragma unroll
    for (int u = 1; u < D; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        load(u, s_begin + u);
    }
    __builtin_amdgcn_sched_barrier(0);
    // Steps past s_end inside the last round hold zeros and add nothing.
    for (int s = s_begin; s < s_end; s += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
#pragma unroll
            for (int h = 0; h < KH; ++h)
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(xr[u][h][c], wr[u][j][h][c], acc[j], 0, 0, 0);
            load(u, s + u + D);
        }
    }

    // ---- K segments of one block: the last to arrive adds them in order
    if (S > 1) {
        int *cnt = a.counters + blk;
        auto slot_rsrc = [&](int u) {
            float *base = a.partials + (int64_t)u * SLOT;
            return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, SLOT * 4, 0x00020000);
        };
        auto store_own = [&]() {
            const __amdgpu_buffer_rsrc_t rs = slot_rsrc(unit);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[j]), rs, (j * 64 + lane) * 16, 0,
                                                       kDeviceScope);
        };
        auto read_slot = [&](int u, f32x4 (&x)[FN]) {
            const __amdgpu_buffer_rsrc_t rs = slot_rsrc(u);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                x[j] = __builtin_bit_cast(f32x4,
                                          __builtin_amdgcn_raw_buffer_load_b128(rs, (j * 64 + lane) * 16, 0, kDeviceScope));
        };
        const int first = blk * S;  // unit of segment 0
        // Arrival, as in gemm_epi_kernel: a segment that finds all others
        // already counted keeps its sums in registers; otherwise it
        // publishes them (device-scope stores, completed), then counts.
        // (The empty asm statements keep the compiler from moving memory
        // accesses across the counter accesses.)
        int seen = 0;
        if (lane == 0) seen = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        bool last = __shfl(seen, 0) == S - 1;
        bool published = false;
        if (!last) {
            store_own();
            wait_vmcnt<0>();
            asm volatile("" ::: "memory");
            int prev = 0;
            if (lane == 0) prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last = __shfl(prev, 0) == S - 1;
            published = true;
        }
        if (!last) return;
        if (lane == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("" ::: "memory");
        if (seg == 0 || S == 2) {
            for (int u = first; u < first + S; ++u) {
                if (u == unit) continue;
                f32x4 x[FN];
                read_slot(u, x);
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[j] += x[j];
            }
        } else {
            if (!published) {
                store_own();
                wait_vmcnt<0>();  // read back below, in segment order
            }
            read_slot(first, acc);
            for (int u = first + 1; u < first + S; ++u) {
                f32x4 x[FN];
                read_slot(u, x);
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[j] += x[j];
            }
        }
    }

    // ---- epilogue: bias and tail in registers, each output stored once
    float bn[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = n0 + 16 * j + r;
        bn[j] = n < N ? a.bias[n] : 0.f;
    }
    if constexpr (ROWMAX) {
        // row maxima over this block's columns (tail (b): over its whole
        // 16-column windows), one partial per (row, W block)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                float v = acc[j][i] + bn[j];
                if constexpr (POOL) {
                    v += __shfl_xor(v, 1);
                    v += __shfl_xor(v, 2);
                    v += __shfl_xor(v, 4);
                    v += __shfl_xor(v, 8);
                    const bool whole = n0 + 16 * j + 16 <= N;  // floor mode
                    mx = fmaxf(mx, whole ? gelu_erf(v * 0.0625f) * a.tail.scale : -INFINITY);
                } else {
                    const bool n_ok = n0 + 16 * j + r < N;
                    mx = fmaxf(mx, n_ok ? gelu_erf(v) * a.tail.scale : -INFINITY);
                }
            }
            if constexpr (!POOL) {
                mx = fmaxf(mx, __shfl_xor(mx, 1));
                mx = fmaxf(mx, __shfl_xor(mx, 2));
                mx = fmaxf(mx, __shfl_xor(mx, 4));
                mx = fmaxf(mx, __shfl_xor(mx, 8));
            }
            const int m = m0 + 4 * q + i;
            if (r == 0 && m < M) a.out[(int64_t)m * a.wblocks + rb] = mx;
        }
    } else {
        using Tail = typename std::conditional<
            EPI == EPI_SCALE_HARDTANH_GELU, TailScaleHardtanhGelu,
            typename std::conditional<EPI == EPI_SWISH_SCALE, TailSwishScale, TailNone>::type>::type;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + 16 * j + r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + 4 * q + i;
                if (m < M && n < N) a.out[(int64_t)m * N + n] = Tail::apply(acc[j][i] + bn[j], a.tail);
            }
        }
    }
}

}  // namespace lin_epi
