// da2_partition.cpp -- the spatial partition of a latent frame into regions of
// at most C = 64 tokens (DraftAttention2, Sec. 3.3: a ragged 2D partition with
// balanced token counts, the smallest total perimeter among candidate
// partitions, the minimum number of blocks and less than one block of
// padding per frame; App. C.2: R_f = ceil(H_v W_v / C)).
//
// Candidate family: bands of whole rows (or of whole columns) across the
// frame.  A band of h lines and length L is walked as a column snake --
// column by column, down even columns and up odd ones -- and cut into
// k = ceil(h L / C) consecutive pieces, the first (h L mod k) of them one
// token larger than the rest; every piece is connected.  A candidate is
// admissible when it gives exactly R_f regions and no piece is under 48
// tokens.  Among admissible candidates the smallest total perimeter (region
// edges against another region or the frame border) is taken; ties prefer
// row bands, then fewer bands, then a smaller first band height (then the
// next, and so on).  A dynamic program over (lines covered, regions used)
// finds it.  Regions are numbered band by band and along the snake; each
// region's tokens take its slots in raster order, the remaining slots are
// padding.  For H_v, W_v multiples of 8 the result is the 8x8 grid.
#include <stdint.h>
#include <stdlib.h>

#include <vector>

#include "da2_internal.h"

namespace da2 {
namespace {

struct Band {
    int pieces;        // regions of the band
    long perimeter;    // summed perimeter of its pieces, -1 when inadmissible
};

// Piece of each cell of an h x L band (cell (line, col) at line * L + col).
std::vector<int> snake_pieces(int h, int L)
{
    const int n = h * L, k = (n + kBlk - 1) / kBlk, q = n / k, big = n % k;
    std::vector<int> lab(n);
    int piece = 0, filled = 0;
    for (int col = 0; col < L; col++)
        for (int t = 0; t < h; t++) {
            const int line = col & 1 ? h - 1 - t : t;
            lab[line * L + col] = piece;
            if (++filled == q + (piece < big)) {
                piece++;
                filled = 0;
            }
        }
    return lab;
}

Band measure_band(int h, int L)
{
    const int n = h * L, k = (n + kBlk - 1) / kBlk;
    Band b{k, -1};
    if (n / k < kMinFill)
        return b;
    const std::vector<int> lab = snake_pieces(h, L);
    long per = 0;
    for (int line = 0; line < h; line++)
        for (int col = 0; col < L; col++) {
            const int me = lab[line * L + col];
            per += (line == 0 || lab[(line - 1) * L + col] != me);
            per += (line == h - 1 || lab[(line + 1) * L + col] != me);
            per += (col == 0 || lab[line * L + col - 1] != me);
            per += (col == L - 1 || lab[line * L + col + 1] != me);
        }
    b.perimeter = per;
    return b;
}

struct Choice {
    long perimeter = -1;
    int bands = 0;
    std::vector<int> heights;
};

// Best composition of E lines into bands of length L giving Rf regions.
Choice best_composition(int E, int L, int Rf)
{
    std::vector<Band> band(E + 1);
    for (int h = 1; h <= E; h++)
        band[h] = measure_band(h, L);
    // state (e, r): lines e .. E-1 still to cover with r regions
    const size_t W = (size_t)Rf + 1;
    std::vector<long> cost((size_t)(E + 1) * W, -1);
    std::vector<int> nb((size_t)(E + 1) * W, 0), first((size_t)(E + 1) * W, 0);
    cost[(size_t)E * W] = 0;
    for (int e = E - 1; e >= 0; e--)
        for (int r = 0; r <= Rf; r++) {
            const size_t me = (size_t)e * W + r;
            for (int h = 1; h <= E - e; h++) {
                if (band[h].perimeter < 0 || band[h].pieces > r)
                    continue;
                const size_t rest = (size_t)(e + h) * W + (r - band[h].pieces);
                if (cost[rest] < 0)
                    continue;
                const long c = band[h].perimeter + cost[rest];
                const int n = nb[rest] + 1;
                if (cost[me] < 0 || c < cost[me] || (c == cost[me] && n < nb[me])) {
                    cost[me] = c;
                    nb[me] = n;
                    first[me] = h;
                }
            }
        }
    Choice ch;
    if (cost[Rf] < 0)
        return ch;
    ch.perimeter = cost[Rf];
    ch.bands = nb[Rf];
    for (int e = 0, r = Rf; e < E;) {
        const int h = first[(size_t)e * W + r];
        ch.heights.push_back(h);
        r -= band[h].pieces;
        e += h;
    }
    return ch;
}

}  // namespace

int partition_frame(int Hv, int Wv, int32_t *tok)
{
    if (Hv < 1 || Wv < 1)
        return -1;
    const int Rf = (Hv * Wv + kBlk - 1) / kBlk;
    const Choice rows = best_composition(Hv, Wv, Rf);
    const Choice cols = best_composition(Wv, Hv, Rf);
    bool by_rows;
    if (rows.perimeter >= 0 && (cols.perimeter < 0 || rows.perimeter <= cols.perimeter))
        by_rows = true;
    else if (cols.perimeter >= 0)
        by_rows = false;
    else
        return -1;
    const Choice &ch = by_rows ? rows : cols;
    const int L = by_rows ? Wv : Hv;
    std::vector<int> region(Hv * Wv);
    int base = 0, line0 = 0;
    for (int h : ch.heights) {
        const std::vector<int> lab = snake_pieces(h, L);
        for (int line = 0; line < h; line++)
            for (int col = 0; col < L; col++) {
                const int y = by_rows ? line0 + line : col, x = by_rows ? col : line0 + line;
                region[y * Wv + x] = base + lab[line * L + col];
            }
        base += (h * L + kBlk - 1) / kBlk;
        line0 += h;
    }
    std::vector<int> fill(Rf, 0);
    for (int i = 0; i < Rf * kBlk; i++)
        tok[i] = -1;
    for (int t = 0; t < Hv * Wv; t++) {
        const int r = region[t];
        tok[r * kBlk + fill[r]++] = t;   // raster order inside the region
    }
    return Rf;
}

}  // namespace da2
