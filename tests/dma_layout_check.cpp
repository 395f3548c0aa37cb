// CPU check of the direct-to-LDS staging layout (dma_layout.hpp), compiled
// with g++ by tests/test_dma_layout.py for every tile shape in the library's
// tile table (passed as -DTILES="T(BM, BN, NW) ...").
//
// For each shape it checks, by enumeration of every DMA instruction,
// wavefront and lane:
//   * every (stage row, logical chunk) of a K step is loaded exactly once,
//     into the physical chunk logical ^ swizzle(row) that the fragment reads
//     expect, and padding blocks only follow the X and W blocks;
//   * over the K steps of schedule.hpp (step s at koff + 32 s, only step 0
//     partial), for valid rows and K positions the per-lane + scalar offset
//     addresses exactly element (row, k) and the 16 bytes lie inside the
//     resource (num_records = valid_rows * K * 4);
//   * for rows past the valid rows or K positions before 0, the per-lane
//     offset alone is >= num_records (so the load is out of range whether or
//     not the scalar offset takes part in the range check), no offset is
//     negative and the sum does not wrap 32 bits.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "dma_layout.hpp"

using namespace lin_epi;

static long g_fail = 0;
#define EXPECT(cond, ...)                          \
    do {                                           \
        if (!(cond)) {                             \
            if (g_fail < 20) {                     \
                std::printf("FAIL %s: ", #cond);   \
                std::printf(__VA_ARGS__);          \
                std::printf("\n");                 \
            }                                      \
            ++g_fail;                              \
        }                                          \
    } while (0)

template <int BM, int BN, int NW>
static void check_shape()
{
    constexpr int NBA = BM / 8, NB = (BM + BN) / 8;
    constexpr int BLOCKS = (NB + NW - 1) / NW * NW;
    constexpr int NL = BLOCKS / NW;
    std::printf("tile %dx%d, %d wavefronts, %d DMA instructions per wavefront and step\n", BM, BN, NW, NL);

    // coverage and swizzle
    std::vector<int> seen((size_t)NB * 8 * 8, 0);
    for (int i = 0; i < NL; ++i)
        for (int w = 0; w < NW; ++w)
            for (int l = 0; l < 64; ++l) {
                const DmaLoad ld = dma_load_of<BM, BN, NW>(i, w, l);
                const int blk = i * NW + w;
                const int stage_row = blk * 8 + l / 8;
                if (ld.op == 2) {
                    EXPECT(blk >= NB, "padding block %d inside the tile", blk);
                    continue;
                }
                EXPECT(blk < NB, "block %d past the tile", blk);
                EXPECT(ld.op == (blk < NBA ? 0 : 1), "operand of block %d", blk);
                EXPECT(stage_row == (ld.op == 0 ? ld.row : BM + ld.row), "row %d of block %d", ld.row, blk);
                EXPECT(ld.blk * 8 == (ld.row & ~7), "block of row %d", ld.row);
                EXPECT(ld.chunk >= 0 && ld.chunk < 8, "chunk %d", ld.chunk);
                EXPECT((l & 7) == (ld.chunk ^ lds_swizzle(stage_row)), "swizzle: lane %d row %d chunk %d", l,
                       stage_row, ld.chunk);
                seen[(size_t)stage_row * 8 + ld.chunk]++;
            }
    for (size_t e = 0; e < seen.size(); ++e) EXPECT(seen[e] == 1, "stage row %zu chunk %zu loaded %d times", e / 8, e % 8, seen[e]);

    // offsets and masking.  K steps start at koff + 32 s (schedule.hpp): the
    // steady state (k0 >= 0, the K position in the scalar offset) and the
    // first step of a K that is not a multiple of 32 (k0 = koff < 0, the K
    // shift and mask per lane, scalar offset at K position 0).
    const int Ks[] = {4, 36, 132, 4100, 8192, 32768};
    for (int K : Ks) {
        const int koff = K % 32 ? K % 32 - 32 : 0;
        const int steps = (K + 31) / 32;
        for (int op = 0; op < 2; ++op) {
            const int rows = op == 0 ? BM : BN;
            if ((int64_t)rows * K * 4 >= kBufferWindow) continue;  // the register-staged path serves these
            const int valids[] = {1, 7, 8, 9, rows / 2 + 3, rows - 1, rows};
            for (int valid : valids) {
                if (valid < 1 || valid > rows) continue;
                const int64_t nrec = (int64_t)valid * K * 4;
                for (int s = 0; s < steps; ++s) {
                    const int k0 = koff + 32 * s;
                    const bool first = s == 0 && koff < 0;
                    for (int i = 0; i < NL; ++i)
                        for (int w = 0; w < NW; ++w)
                            for (int l = 0; l < 64; ++l) {
                                const DmaLoad ld = dma_load_of<BM, BN, NW>(i, w, l);
                                if (ld.op != op) continue;
                                const int kpos = k0 + 4 * ld.chunk;  // K position of the lane's 4 floats
                                int64_t voff, soff;
                                if (first) {
                                    voff = dma_voffset(ld.row, ld.chunk, koff, ld.row < valid && koff + 4 * ld.chunk >= 0, K);
                                    soff = dma_soffset(ld.blk, 0, K);
                                } else {
                                    EXPECT(k0 >= 0 && k0 + 32 <= K, "steady step %d of K %d out of [0, K)", s, K);
                                    voff = dma_voffset(ld.row, ld.chunk, 0, ld.row < valid, K);
                                    soff = dma_soffset(ld.blk, k0, K);
                                }
                                EXPECT(soff >= 0 && soff < ((int64_t)1 << 31), "soffset %lld", (long long)soff);
                                EXPECT(voff >= 0 && voff + soff < ((int64_t)1 << 32), "offset sum wraps");
                                if (ld.row < valid && kpos >= 0) {
                                    EXPECT(kpos + 4 <= K, "K position %d past K %d", kpos, K);
                                    EXPECT(voff + soff == ((int64_t)ld.row * K + kpos) * 4, "address of row %d k %d",
                                           ld.row, kpos);
                                    EXPECT(voff + soff + 16 <= nrec && voff < nrec, "in range: row %d of %d", ld.row,
                                           valid);
                                } else {
                                    EXPECT(voff >= nrec, "masked lane in range: row %d of %d, k %d", ld.row, valid, kpos);
                                }
                            }
                }
            }
        }
    }
}

#define T(BM, BN, NW) check_shape<BM, BN, NW>();

int main()
{
    TILES
    if (g_fail) {
        std::printf("%ld failures\n", g_fail);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
