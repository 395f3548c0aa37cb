// Work partition of gemm_epi_kernel: which workgroup computes which output
// tiles over which K steps, and how split tiles are put back together.
//
// The work of one call is the iteration space of (tile, K step) pairs,
// tile-major: iteration i belongs to tile i / steps, K step i % steps, with
// T = tiles * steps iterations in all.  A grid of G workgroups (G <= T)
// divides it into G contiguous ranges, and a workgroup walks its range tile
// by tile, computing each tile it touches over a contiguous run of K steps
// (a "segment"):
//   * G = tiles: one whole tile per workgroup (data parallel).
//   * split-K, G = tiles * S (S <= steps): segment k of every tile holds K
//     steps floor(k steps / S) .. floor((k+1) steps / S) - 1, so no range
//     crosses a tile and every tile has S segments.
//   * stream-K, any other G: with T = q G + r the first r ranges hold q + 1
//     iterations and the others q (range v starts at v q + min(v, r)); ranges
//     cross tile boundaries and the work is balanced to within one K step.
// A tile computed in more than one segment is finished by whichever of its
// workgroups arrives last: every other segment leaves its partial sums in a
// slot of the workspace, and the last one adds them in segment order (so the
// result does not depend on the arrival order) and applies the epilogue.
// Split plans keep T within 32 bits, so every lookup below is 32-bit
// arithmetic; one tile per workgroup needs none.
//
// K steps: step s covers K positions koff + 32 s .. koff + 32 s + 31, with
// koff = (K % 32) - 32 when K % 32 != 0, else 0.  Every step then lies
// inside [0, K) except step 0, whose first -koff positions are before 0 and
// are zero-filled: the only partial step is the first one.
//
// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2), so physical workgroup w is renumbered to a virtual index that gives
// XCD x a contiguous block of ranges: neighbouring ranges (which share tiles,
// X row panels and W column panels) then run on the same XCD.
//
// Every function here is host-callable too; the CPU test suite enumerates
// them over many shapes and grids.
#pragma once

#include <stdint.h>

namespace lin_epi {

constexpr int kStepK = 32;  // K elements per step (one 128-byte row segment)

__host__ __device__ inline int k_steps(int K) { return K > 0 ? (K + kStepK - 1) / kStepK : 1; }
__host__ __device__ inline int k_offset(int K) { return K % kStepK ? K % kStepK - kStepK : 0; }

// Physical workgroup -> virtual index: XCD x = w % 8 gets the contiguous
// virtual block [x*q, (x+1)*q), q = G / 8; the last G % 8 keep their index.
__host__ __device__ inline int virtual_wg(int w, int G)
{
    const int q = G >> 3;
    return w < (q << 3) ? (w & 7) * q + (w >> 3) : w;
}

// A split partition: split-K when S > 0, else stream-K with T = q G + r.
struct Partition {
    int steps;  // K steps per tile
    int G;      // workgroups
    int S;      // split-K segments per tile (0: stream-K)
    int q, r;   // stream-K range lengths
};

// First iteration of virtual workgroup v's range (v = G gives T).
__host__ __device__ inline int range_begin(const Partition &p, int v)
{
    if (p.S > 0) {
        const int t = v / p.S, k = v - t * p.S;
        return t * p.steps + k * p.steps / p.S;
    }
    return v * p.q + (v < p.r ? v : p.r);
}

// The virtual workgroup whose range holds iteration i (0 <= i < T).
__host__ __device__ inline int range_owner(const Partition &p, int i)
{
    if (p.S > 0) {
        const int t = i / p.steps, s = i - t * p.steps;
        return t * p.S + ((s + 1) * p.S - 1) / p.steps;
    }
    const int c = p.r * (p.q + 1);  // iterations held by the r longer ranges
    return i < c ? i / (p.q + 1) : p.r + (i - c) / p.q;
}

// The segments of tile t: workgroups first .. last, in K order.
struct TileSegs {
    int first, last;
};
__host__ __device__ inline TileSegs tile_segments(const Partition &p, int t)
{
    if (p.S > 0) return TileSegs{t * p.S, t * p.S + p.S - 1};
    const int i0 = t * p.steps;
    return TileSegs{range_owner(p, i0), range_owner(p, i0 + p.steps - 1)};
}

// Partial-sum slot of workgroup u's segment of tile t.  Split-K: slot u.
// Stream-K: slot u for the tile u's range starts in, G + u for the tile it
// ends in (only those two of its tiles can be split; u's range starts before
// tile t exactly when t is not its first tile).
__host__ __device__ inline int partial_slot(const Partition &p, int u, int t)
{
    if (p.S > 0) return u;
    return u + (range_begin(p, u) < t * p.steps ? p.G : 0);
}

// Tile number -> (tile row, tile column): GROUP_M tile rows at a time,
// column-major inside a group, so consecutive tiles share W column panels
// and a group's X row panels stay resident.
template <int GROUP_M>
__host__ __device__ inline void tile_coords(int t, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int per_group = GROUP_M * tiles_n;
    const int g = t / per_group;
    const int first_m = g * GROUP_M;
    const int gm = tiles_m - first_m < GROUP_M ? tiles_m - first_m : GROUP_M;
    const int r = t - g * per_group;
    tm = first_m + r % gm;
    tn = r / gm;
}

}  // namespace lin_epi
