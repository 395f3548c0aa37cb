// Layout of the direct-to-LDS operand staging of gemm_epi_kernel: which row
// and 16-byte chunk of X or W each lane moves with each buffer_load ... lds
// instruction, the byte offsets it passes, and where the chunk lands in LDS.
//
// One K step stages BK = 32 floats (128 bytes, 8 chunks of 16 bytes) of each
// of the tile's BM rows of X and BN rows of W.  LDS holds them as 8-row
// blocks of 1 KiB: blocks 0 .. BM/8-1 are X, the next BN/8 are W, then
// padding blocks up to a multiple of the wavefront count NW.  Instruction i
// of wavefront w writes block i*NW + w; lane l lands at block row l/8,
// physical chunk l%8, and fetches the logical chunk that belongs there.
// Chunks are XOR-swizzled, physical = logical ^ swizzle(row) with
// swizzle(row) = (row % 8) ^ ((row / 8) % 2), so a fragment read (32 rows,
// one logical chunk) is bank-conflict free.
//
// Zero-filling: each operand has one buffer resource over the tile's valid
// rows (num_records = valid_rows * K * 4 bytes).  A lane whose row is past
// the valid rows, or whose K position is outside [0, K), gets the per-lane
// offset kOobOffset, which is at least num_records by itself, so the load
// returns zeros whether or not the hardware adds the scalar offset into the
// range check.  Valid lanes stay inside num_records under either rule.
// In the steady state the K position goes in the scalar offset and the
// per-lane offset (row mask included) is the same for every K step; only
// the first step of a tile, the one step that can start before K = 0 (see
// schedule.hpp), carries its K shift and K mask per lane.
//
// Every function here is host-callable too, so the CPU test suite checks
// these properties over every tile shape by enumeration.
#pragma once

#include <stdint.h>

namespace lin_epi {

// Byte window the buffer-load path is used within: a tile's rows of X or W
// span rows * K * 4 < 2^30 bytes, so every offset formed below stays under
// 2^31, and kOobOffset plus any scalar offset still fits in 32 bits.
constexpr int64_t kBufferWindow = int64_t(1) << 30;
constexpr int kOobOffset = (int)kBufferWindow;

struct DmaLoad {
    int op;     // 0 = X, 1 = W, 2 = padding block (never read)
    int blk;    // 8-row block within the operand's tile rows
    int row;    // row within the operand's tile rows (blk * 8 + lane / 8)
    int chunk;  // logical 16-byte chunk of the row's 128-byte K segment
};

// XOR swizzle of the 16-byte chunks of LDS row `row` (row counted over the
// whole stage: X rows first, then W rows).
__host__ __device__ inline int lds_swizzle(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// What lane `lane` of wavefront `wave` loads with DMA instruction i.
// NW is even and BM/8 is even, so block i*NW + wave has the wavefront's
// parity and swizzle(stage row) = (lane / 8) ^ (wave & 1).
template <int BM, int BN, int NW>
__host__ __device__ inline DmaLoad dma_load_of(int i, int wave, int lane)
{
    const int blk = i * NW + wave;
    const int lr = lane >> 3;
    const int chunk = (lane & 7) ^ lr ^ (wave & 1);
    if (blk < BM / 8) return DmaLoad{0, blk, blk * 8 + lr, chunk};
    if (blk < (BM + BN) / 8) return DmaLoad{1, blk - BM / 8, (blk - BM / 8) * 8 + lr, chunk};
    return DmaLoad{2, 0, 0, chunk};
}

// Per-lane byte offset of the chunk inside its 8-row block, kdelta K
// positions from the block's K position in the scalar offset, or kOobOffset
// when ok is false (row past the valid rows, or K position outside [0, K)).
__host__ __device__ inline int dma_voffset(int row, int chunk, int kdelta, bool ok, int K)
{
    return ok ? ((row & 7) * K + kdelta + 4 * chunk) * 4 : kOobOffset;
}

// Scalar (wave-uniform) byte offset: the start of 8-row block blk at K
// position k0.
__host__ __device__ inline int dma_soffset(int blk, int k0, int K) { return (blk * 8 * K + k0) * 4; }

}  // namespace lin_epi
