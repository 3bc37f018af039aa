// da2_partition.cpp -- the spatial partition of a latent frame into regions of
// at most C tokens, C = 64 or 128 (DraftAttention2, Sec. 3.3: a ragged 2D partition with
// balanced token counts across regions, the smallest total perimeter among
// candidate partitions, the minimum number of blocks and less than one block
// of padding per frame; App. C.2: R_f = ceil(H_v W_v / C)).
//
// Balance: with n = H_v W_v, q = floor(n / R_f) and r = n mod R_f, every
// region holds q tokens or (when r > 0) q + 1.  Candidate family: bands of
// whole rows (or of whole columns) across the frame.  A band of h lines and
// length L is walked as a column snake -- column by column, down even
// columns and up odd ones -- and cut into k consecutive pieces, the first
// (hL - kq) of them q + 1 tokens long and the rest q; a band can take k
// pieces when kq <= hL <= k(q + r?1:0).  Bands adding up to R_f pieces give
// a balanced partition (one band of all lines always does).  The smallest
// total perimeter (region edges against another region or the frame border)
// is taken; ties prefer row bands, then fewer bands, then a smaller first
// band height, then fewer pieces in it (then the next band, and so on).  A
// dynamic program over (lines covered, regions used) finds it.  Regions are
// numbered band by band and along the snake; each region's tokens take its
// slots in raster order, the remaining slots are padding.  For H_v, W_v
// multiples of 8 the result is the 8x8 grid.
//
// The attention kernels handle at most 16 padding slots per 64-slot tile,
// and a region's padding slots all lie in its last tile, so a frame whose
// regions hold fewer than C - 16 tokens is refused here.
#include <stdint.h>
#include <stdlib.h>

#include <vector>

#include "da2_internal.h"

namespace da2 {
namespace {

// Piece of each cell of an h x L band cut into k pieces of q or q + 1 tokens
// (cell (line, col) at line * L + col).
std::vector<int> snake_pieces(int h, int L, int k, int q)
{
    const int big = h * L - k * q;
    std::vector<int> lab(h * L);
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

long band_perimeter(int h, int L, int k, int q)
{
    const std::vector<int> lab = snake_pieces(h, L, k, q);
    long per = 0;
    for (int line = 0; line < h; line++)
        for (int col = 0; col < L; col++) {
            const int me = lab[line * L + col];
            per += (line == 0 || lab[(line - 1) * L + col] != me);
            per += (line == h - 1 || lab[(line + 1) * L + col] != me);
            per += (col == 0 || lab[line * L + col - 1] != me);
            per += (col == L - 1 || lab[line * L + col + 1] != me);
        }
    return per;
}

struct BandChoice {
    int h, k;
    long perimeter;
};

struct Choice {
    long perimeter = -1;
    std::vector<int> heights, pieces;
};

// Best composition of E lines into bands of length L giving Rf regions of q
// (or q + 1 when big) tokens.
Choice best_composition(int E, int L, int Rf, int q, bool big)
{
    // every band that can be cut: height h, pieces k, perimeter
    std::vector<std::vector<BandChoice>> opts(E + 1);
    for (int h = 1; h <= E; h++) {
        const long n = (long)h * L;
        const long kmax = n / q, kmin = big ? (n + q) / (q + 1) : kmax;
        for (long k = kmin; k <= kmax && k <= Rf; k++)
            if (k >= 1 && k * q <= n && n <= k * (q + (big ? 1 : 0)))
                opts[h].push_back({h, (int)k, band_perimeter(h, L, (int)k, q)});
    }
    // state (e, t): lines e .. E-1 still to cover with t regions
    const size_t W = (size_t)Rf + 1;
    std::vector<long> cost((size_t)(E + 1) * W, -1);
    std::vector<int> nb((size_t)(E + 1) * W, 0), fh((size_t)(E + 1) * W, 0), fk((size_t)(E + 1) * W, 0);
    cost[(size_t)E * W] = 0;
    for (int e = E - 1; e >= 0; e--)
        for (int t = 0; t <= Rf; t++) {
            const size_t me = (size_t)e * W + t;
            for (int h = 1; h <= E - e; h++)
                for (const BandChoice &o : opts[h]) {
                    if (o.k > t)
                        continue;
                    const size_t rest = (size_t)(e + h) * W + (t - o.k);
                    if (cost[rest] < 0)
                        continue;
                    const long c = o.perimeter + cost[rest];
                    const int n = nb[rest] + 1;
                    if (cost[me] < 0 || c < cost[me] || (c == cost[me] && n < nb[me])) {
                        cost[me] = c;
                        nb[me] = n;
                        fh[me] = h;
                        fk[me] = o.k;
                    }
                }
        }
    Choice ch;
    if (cost[Rf] < 0)
        return ch;
    ch.perimeter = cost[Rf];
    for (int e = 0, t = Rf; e < E;) {
        const size_t me = (size_t)e * W + t;
        ch.heights.push_back(fh[me]);
        ch.pieces.push_back(fk[me]);
        t -= fk[me];
        e += fh[me];
    }
    return ch;
}

}  // namespace

int partition_frame(int Hv, int Wv, int C, int32_t *tok)
{
    if (Hv < 1 || Wv < 1 || C < kBlk || C % kBlk)
        return -1;
    const int n = Hv * Wv, Rf = (n + C - 1) / C, q = n / Rf;
    const bool big = n % Rf != 0;
    if (q < C - (kBlk - kMinFill))
        return -1;
    const Choice rows = best_composition(Hv, Wv, Rf, q, big);
    const Choice cols = best_composition(Wv, Hv, Rf, q, big);
    bool by_rows;
    if (rows.perimeter >= 0 && (cols.perimeter < 0 || rows.perimeter <= cols.perimeter))
        by_rows = true;
    else if (cols.perimeter >= 0)
        by_rows = false;
    else
        return -1;
    const Choice &ch = by_rows ? rows : cols;
    const int L = by_rows ? Wv : Hv;
    std::vector<int> region(n);
    int base = 0, line0 = 0;
    for (size_t b = 0; b < ch.heights.size(); b++) {
        const int h = ch.heights[b], k = ch.pieces[b];
        const std::vector<int> lab = snake_pieces(h, L, k, q);
        for (int line = 0; line < h; line++)
            for (int col = 0; col < L; col++) {
                const int y = by_rows ? line0 + line : col, x = by_rows ? col : line0 + line;
                region[y * Wv + x] = base + lab[line * L + col];
            }
        base += k;
        line0 += h;
    }
    std::vector<int> fill(Rf, 0);
    for (int i = 0; i < Rf * C; i++)
        tok[i] = -1;
    for (int t = 0; t < n; t++) {
        const int r = region[t];
        tok[r * C + fill[r]++] = t;   // raster order inside the region
    }
    return Rf;
}

}  // namespace da2
