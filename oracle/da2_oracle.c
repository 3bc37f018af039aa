/*
 * da2_oracle.c -- plain, slow, obviously correct CPU oracle for the
 * DraftAttention2 hot path (low-resolution-guided, block-sparse, mixed
 * 16-bit / FP8 / MXFP4 / skip attention for video diffusion transformers).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant generator with the HIP library: every rule below
 * is restated from the pages, in fp64 unless a step fixes another precision.
 *
 * Sources (page titles; sections named on each page):
 *   [DA2]  "DraftAttention2: Fast Video Diffusion with Low-Resolution-Guided
 *           Mixed-Precision Attention" -- Sec. 3.1 (Eq. 1 pooled descriptors,
 *           Eq. 2 draft map, joint allocation of sparsity and precision),
 *           Sec. 3.3 (fused quantization and reordering, phased execution,
 *           cross-precision accumulation), App. B.3/B.4 (shared
 *           normalization), App. C.1 (routing and precision formats),
 *           App. C.2 (spatial packing).
 *   [DA1]  "DraftAttention: Fast Video Diffusion via Low-Resolution Attention
 *           Guidance" -- abstract (reorder, block-sparse attention, restore
 *           the original order).
 *   [Triage] "Triage: Skip, Skim, or Refine Attention Tiles in Video
 *           Diffusion Transformers" -- abstract (a skipped tile replaced by
 *           its block means).
 * Number formats: the 8-bit path takes INT8 for Q K^T ([DA2] App. C.1) with
 * the uniform nearest-integer quantizer of App. B.2, and OCP 8-bit floating
 * point (E4M3, "fn" variant: no inf, max 448) for P V; the 4-bit path takes
 * OCP Microscaling v1.0 (E2M1 elements, E8M0 scale, blocks of 32) in place of
 * the paper's NVFP4.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - token order of the input is (frame, y, x) raster;
 *   - the partition of a frame: R_f = ceil(HW/C) regions of
 *     floor(HW/R_f) or ceil(HW/R_f) tokens (balanced across the frame),
 *     C the block capacity (64 by default; App. C.2's study uses 128);
 *     candidates are bands of whole rows or columns walked as column
 *     snakes and cut into consecutive pieces; the smallest total perimeter
 *     wins; valid tokens take slots in raster order, padding slots follow
 *     (the 8x8 grid when the sides are multiples of 8);
 *   - pooled sums run over the n_a valid tokens in slot order, in fp64;
 *   - logits are fixed-order fma chains over channels 0..d-1 times 1/sqrt(d);
 *   - exp of the draft softmax is a Cody-Waite reduction (fdlibm's split of
 *     ln 2) followed by a degree-13 Taylor polynomial in Horner form;
 *   - row sums of the draft softmax are sequential over key regions;
 *   - ranking key is the bit pattern of fp32(A); ties by ascending pair index;
 *   - quotas: cumulative counts T16, T16+T8, T16+T8+T4, each rounded half up;
 *   - regions of capacity C > 64 run as C/64 tiles of 64 positions in slot
 *     order, every tile of a region pair taking the pair's tier; the
 *     quantization blocks below stay 64 tokens; block-mean tiles only at
 *     C = 64;
 *   - INT8 Q/K step amax/127 per 64-token block (code = nearest integer of
 *     x 127/amax, ties to even, the product in fp32), FP8 V scale per channel
 *     over all tokens, MXFP4 groups along channels for Q/K and along keys
 *     for V;
 *   - attention weights are taken per 64-key tile relative to the running
 *     max: the 16-bit path keeps them unquantized (App. B's bound charges
 *     quantization error to the 4- and 8-bit paths only), FP8
 *     e4m3(w * 2^8) * 2^-8, MXFP4 per 32 keys (E8M0 exponent: the smallest
 *     X with max w 2^-X <= 6); phases 16 -> 8 -> 4, then
 *     block-mean tiles (the tile's mean
 *     score q_a . k_b / sqrt(d), its mean value, n_b keys);
 *   - a text prefix: video rows take the valid prefix keys first on the
 *     16-bit path, in tiles of 64; prefix rows take every valid prefix key and
 *     every video region on the 16-bit path, in chunks of 128 tiles merged
 *     by the exact rescale.
 * Parity: every exported function is pinned by a CPU test against closed
 * forms, brute force or a library routine (see the test suite).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_BLK 64 /* tokens per tile (and per region at the default capacity C = 64) */

/* ------------------------------------------------------------------ */
/* bf16 and IEEE helpers                                               */
/* ------------------------------------------------------------------ */
static float bf16f(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t f32bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

/* ------------------------------------------------------------------ */
/* O1 layout: [DA2] Sec. 3.3 (a ragged 2D partition of each frame with  */
/* balanced token counts across regions, the smallest total perimeter   */
/* among candidate partitions, the minimum number of blocks and less    */
/* than one block of padding per frame; every region packed into one    */
/* block of C slots) and App. C.2 (R_f = ceil(H_v W_v / C)).            */
/*                                                                      */
/* Balanced: with n = H_v W_v tokens, q = floor(n / R_f) and            */
/* r = n mod R_f, every region holds q or q + 1 tokens (q only when r   */
/* is 0).  Candidates: the frame is cut into bands of whole rows, or of */
/* whole columns.  A band of h lines and length L is walked as a column */
/* snake (its columns in order, each from the band's first line to its  */
/* last for even columns and back for odd ones) and cut into k          */
/* consecutive pieces, the first (hL - kq) of them q + 1 tokens long    */
/* and the rest q; the band admits k when kq <= hL <= k(q+1) (kq = hL   */
/* when r is 0).  Pieces are runs of a path of adjacent cells, so       */
/* connected; bands summing to R_f pieces give a balanced partition.    */
/* The smallest total perimeter (edges between a region's token and a   */
/* token outside it or the frame's border) wins.  Ties: row bands before */
/* column bands, then fewer bands, then the smaller first band height,  */
/* then the fewer pieces in it (and so on).  Regions are numbered band  */
/* by band and along the snake inside a band; a region's tokens take    */
/* its slots in raster order, and the slots after them are padding.     */
/* For H_v, W_v multiples of 8 and C = 64 this is the 8x8 grid, raster  */
/* inside each square.  One band of every line always qualifies, so     */
/* every frame has a partition.                                          */
/* ------------------------------------------------------------------ */
#define OR_MEAN 1 /* tier of a block-mean tile (skip replaced by block means) */

/* Piece label of every cell of one band (h lines x L) cut into k pieces of
 * q or q + 1 tokens, lab[line*L + col]. */
static void band_pieces(int h, int L, int k, int q, int *lab)
{
    int big = h * L - k * q;   /* pieces of q + 1 tokens, first */
    int piece = 0, used = 0;
    for (int col = 0; col < L; col++)
        for (int t = 0; t < h; t++) {
            int line = (col % 2 == 0) ? t : h - 1 - t;
            lab[line * L + col] = piece;
            used++;
            if (used == q + (piece < big ? 1 : 0)) {
                piece++;
                used = 0;
            }
        }
}

/* Total perimeter of a band's pieces. */
static long band_perimeter(int h, int L, int k, int q)
{
    int n = h * L;
    int *lab = malloc(sizeof(int) * n);
    band_pieces(h, L, k, q, lab);
    long per = 0;
    for (int line = 0; line < h; line++)
        for (int col = 0; col < L; col++) {
            int me = lab[line * L + col];
            int same = 0;
            if (line > 0 && lab[(line - 1) * L + col] == me) same++;
            if (line < h - 1 && lab[(line + 1) * L + col] == me) same++;
            if (col > 0 && lab[line * L + col - 1] == me) same++;
            if (col < L - 1 && lab[line * L + col + 1] == me) same++;
            per += 4 - same;
        }
    free(lab);
    return per;
}

/* Does a band of n = hL tokens admit k pieces of q (or q + 1 when r > 0)? */
static int band_admits(int n, int k, int q, int r)
{
    if (k < 1) return 0;
    long lo = (long)k * q, hi = (long)k * (q + (r > 0 ? 1 : 0));
    return n >= lo && n <= hi;
}

/* Best band sequence of one orientation: E lines across, bands of length L,
 * exactly Rf regions of q or q + 1 tokens.  Returns the number of bands
 * (heights in hs, pieces in ks) and the perimeter in *per, or -1. */
static int best_bands(int E, int L, int Rf, int q, int r, int32_t *hs, int32_t *ks, long *per)
{
    /* perimeters of every admissible (height, pieces) band, computed once;
     * pieces k run from kmin[h] = ceil(hL/(q+1)) (hL/q when r is 0) to
     * floor(hL/q) */
    int *kmin = malloc(sizeof(int) * (E + 1)), *kcnt = malloc(sizeof(int) * (E + 1));
    size_t *koff = malloc(sizeof(size_t) * (E + 2));
    koff[1] = 0;
    for (int h = 1; h <= E; h++) {
        int n = h * L;
        kmin[h] = r > 0 ? (n + q) / (q + 1) : n / q;
        kcnt[h] = n / q - kmin[h] + 1;
        if (kcnt[h] < 0) kcnt[h] = 0;
        koff[h + 1] = koff[h] + (size_t)kcnt[h];
    }
    long *bp = malloc(sizeof(long) * (koff[E + 1] + 1));
    for (int h = 1; h <= E; h++)
        for (int j = 0; j < kcnt[h]; j++) {
            int k = kmin[h] + j;
            bp[koff[h] + j] = band_admits(h * L, k, q, r) ? band_perimeter(h, L, k, q) : -1;
        }
    /* cost[e][t]: best (perimeter, bands) covering lines e..E-1 with t regions */
    size_t S = (size_t)(E + 1) * (Rf + 1);
    long *cost = malloc(sizeof(long) * S);
    int *nb = malloc(sizeof(int) * S), *ph = malloc(sizeof(int) * S), *pk = malloc(sizeof(int) * S);
    for (size_t i = 0; i < S; i++) { cost[i] = -1; nb[i] = 0; ph[i] = 0; pk[i] = 0; }
    cost[(size_t)E * (Rf + 1) + 0] = 0;
    for (int e = E - 1; e >= 0; e--)
        for (int t = 0; t <= Rf; t++) {
            size_t me = (size_t)e * (Rf + 1) + t;
            for (int h = 1; e + h <= E; h++)
                for (int j = 0; j < kcnt[h]; j++) {
                    int k = kmin[h] + j;
                    long pb = bp[koff[h] + j];
                    if (pb < 0 || k > t) continue;
                    size_t nx = (size_t)(e + h) * (Rf + 1) + (t - k);
                    if (cost[nx] < 0) continue;
                    long c = pb + cost[nx];
                    int n = 1 + nb[nx];
                    if (cost[me] < 0 || c < cost[me] || (c == cost[me] && n < nb[me])) {
                        cost[me] = c;
                        nb[me] = n;
                        ph[me] = h;
                        pk[me] = k;
                    }
                }
        }
    int m = -1;
    if (cost[Rf] >= 0) {
        *per = cost[Rf];
        m = 0;
        for (int e = 0, t = Rf; e < E;) {
            size_t me = (size_t)e * (Rf + 1) + t;
            hs[m] = ph[me];
            ks[m] = pk[me];
            t -= pk[me];
            e += ph[me];
            m++;
        }
    }
    free(kmin); free(kcnt); free(koff); free(bp); free(cost); free(nb); free(ph); free(pk);
    return m;
}

/* The partition of an Hv x Wv frame into regions of at most C tokens:
 * orientation (0: row bands, 1: column bands), band heights and pieces
 * (capacity Hv + Wv each) and total perimeter.  Returns the number of
 * bands, or -1 for an empty frame or C < 1. */
int or_partition_bands_c(int Hv, int Wv, int C, int *orient, int32_t *bands, int32_t *pieces,
                         int64_t *perim)
{
    if (Hv <= 0 || Wv <= 0 || C < 1)
        return -1;
    int n = Hv * Wv, Rf = (n + C - 1) / C, q = n / Rf, r = n % Rf;
    int32_t *h0 = malloc(sizeof(int32_t) * (Hv + Wv)), *h1 = malloc(sizeof(int32_t) * (Hv + Wv));
    int32_t *k0 = malloc(sizeof(int32_t) * (Hv + Wv)), *k1 = malloc(sizeof(int32_t) * (Hv + Wv));
    long p0 = 0, p1 = 0;
    int m0 = best_bands(Hv, Wv, Rf, q, r, h0, k0, &p0);
    int m1 = best_bands(Wv, Hv, Rf, q, r, h1, k1, &p1);
    int m = -1;
    if (m0 >= 0 && (m1 < 0 || p0 <= p1)) {
        *orient = 0;
        memcpy(bands, h0, sizeof(int32_t) * m0);
        memcpy(pieces, k0, sizeof(int32_t) * m0);
        *perim = p0;
        m = m0;
    } else if (m1 >= 0) {
        *orient = 1;
        memcpy(bands, h1, sizeof(int32_t) * m1);
        memcpy(pieces, k1, sizeof(int32_t) * m1);
        *perim = p1;
        m = m1;
    }
    free(h0); free(h1); free(k0); free(k1);
    return m;
}

int or_partition_bands(int Hv, int Wv, int *orient, int32_t *bands, int64_t *perim)
{
    int32_t *pieces = malloc(sizeof(int32_t) * (Hv + Wv > 0 ? Hv + Wv : 1));
    int m = or_partition_bands_c(Hv, Wv, OR_BLK, orient, bands, pieces, perim);
    free(pieces);
    return m;
}

/* Slot table of one frame for block capacity C: tok[r*C + i] = y*Wv + x of
 * region r's slot i, -1 for padding; nvalid[r] = its token count.  Returns
 * R_f or -1. */
int or_partition_c(int Hv, int Wv, int C, int32_t *tok, int32_t *nvalid)
{
    int orient;
    int64_t per;
    if (Hv <= 0 || Wv <= 0 || C < 1) return -1;
    int32_t *bands = malloc(sizeof(int32_t) * (Hv + Wv)), *pieces = malloc(sizeof(int32_t) * (Hv + Wv));
    int m = or_partition_bands_c(Hv, Wv, C, &orient, bands, pieces, &per);
    if (m < 0) { free(bands); free(pieces); return -1; }
    int n = Hv * Wv, Rf = (n + C - 1) / C, q = n / Rf;
    int *reg = malloc(sizeof(int) * n);   /* region of each cell */
    int L = orient ? Hv : Wv;
    int base = 0, line0 = 0;
    for (int b = 0; b < m; b++) {
        int h = bands[b], k = pieces[b];
        int *lab = malloc(sizeof(int) * h * L);
        band_pieces(h, L, k, q, lab);
        for (int line = 0; line < h; line++)
            for (int col = 0; col < L; col++) {
                int y = orient ? col : line0 + line, x = orient ? line0 + line : col;
                reg[y * Wv + x] = base + lab[line * L + col];
            }
        free(lab);
        base += k;
        line0 += h;
    }
    for (int i = 0; i < Rf; i++)
        nvalid[i] = 0;
    for (int i = 0; i < Rf * C; i++)
        tok[i] = -1;
    for (int y = 0; y < Hv; y++)
        for (int x = 0; x < Wv; x++) {
            int g = reg[y * Wv + x];
            tok[g * C + nvalid[g]++] = y * Wv + x;
        }
    free(reg);
    free(bands);
    free(pieces);
    return Rf;
}

int or_partition(int Hv, int Wv, int32_t *tok, int32_t *nvalid)
{
    return or_partition_c(Hv, Wv, OR_BLK, tok, nvalid);
}

/* Regions of an F x Hv x Wv video at block capacity C (F R_f with
 * R_f = ceil(Hv Wv / C), App. C.2), or -1 when Hv x Wv has no partition. */
int or_regions(int F, int Hv, int Wv, int C)
{
    int orient;
    int64_t per;
    if (F <= 0 || C < 1) return -1;
    int32_t *bands = malloc(sizeof(int32_t) * (Hv + Wv > 0 ? Hv + Wv : 1));
    int32_t *pieces = malloc(sizeof(int32_t) * (Hv + Wv > 0 ? Hv + Wv : 1));
    int m = or_partition_bands_c(Hv, Wv, C, &orient, bands, pieces, &per);
    free(bands);
    free(pieces);
    return m < 0 ? -1 : F * ((Hv * Wv + C - 1) / C);
}

/* perm[pos] (pos < F R_f C) = original token index of reordered position
 * pos, -1 for padding.  Region a = f R_f + r covers frame f's region r and
 * positions a C .. a C + C - 1; its tokens take the first of them. */
int or_layout(int F, int Hv, int Wv, int C, int32_t *perm)
{
    if (or_regions(F, Hv, Wv, C) < 0)
        return -1;
    int Rf = (Hv * Wv + C - 1) / C;
    int32_t *tok = malloc(sizeof(int32_t) * Rf * C), *nv = malloc(sizeof(int32_t) * Rf);
    or_partition_c(Hv, Wv, C, tok, nv);
    for (int f = 0; f < F; f++)
        for (int i = 0; i < Rf * C; i++)
            perm[(size_t)f * Rf * C + i] = tok[i] < 0 ? -1 : f * Hv * Wv + tok[i];
    free(tok);
    free(nv);
    return 0;
}

/* ------------------------------------------------------------------ */
/* O2 pooled descriptors: [DA2] Sec. 3.1 Eq. (1), App. C.1.             */
/* X is one head, [N][d] bf16; regions of C slots.  avg[a][c] = (sum    */
/* over the region's n_a valid tokens in slot order, fp64) / n_a;       */
/* mx[a][c] = signed max over the valid tokens, first occurrence kept   */
/* on equal values.  Padding slots (perm -1) take no part.              */
/* ------------------------------------------------------------------ */
void or_pool_head(const uint16_t *X, int d, const int32_t *perm, int R, int C,
                  double *avg, float *mx)
{
    for (int a = 0; a < R; a++) {
        int na = 0;
        while (na < C && perm[(size_t)a * C + na] >= 0)
            na++;
        for (int c = 0; c < d; c++) {
            double s = 0.0;
            float m = bf16f(X[(size_t)perm[(size_t)a * C] * d + c]);
            for (int i = 0; i < na; i++) {
                float v = bf16f(X[(size_t)perm[(size_t)a * C + i] * d + c]);
                s += (double)v;
                if (v > m)
                    m = v;
            }
            avg[(size_t)a * d + c] = s / (double)na;
            mx[(size_t)a * d + c] = m;
        }
    }
}

/* ------------------------------------------------------------------ */
/* exp used by the draft softmax.  Cody-Waite reduction with the split  */
/* of ln 2 into a 32-significant-bit head and its remainder (the fdlibm */
/* constants), then the Taylor series of e^r to degree 13 in Horner     */
/* form with fma, then scaling by 2^k.  Arguments below -708 give 0 so  */
/* every nonzero result is a normal number.                             */
/* ------------------------------------------------------------------ */
static const double OR_LN2_HI = 6.93147180369123816490e-01;
static const double OR_LN2_LO = 1.90821492927058770002e-10;
static const double OR_INV_LN2 = 1.44269504088896338700e+00;

void or_exp_constants(double *out /* [3 + 14] */)
{
    out[0] = OR_LN2_HI;
    out[1] = OR_LN2_LO;
    out[2] = OR_INV_LN2;
    double fact = 1.0;
    for (int j = 0; j <= 13; j++) {
        if (j > 0)
            fact *= (double)j; /* j! is exact in double for j <= 18 */
        out[3 + j] = 1.0 / fact;
    }
}

double or_exp(double x)
{
    if (x < -708.0)
        return 0.0;
    double coef[17];
    or_exp_constants(coef);
    double k = rint(x * OR_INV_LN2);
    double r = fma(-k, OR_LN2_HI, x);
    r = fma(-k, OR_LN2_LO, r);
    double p = coef[3 + 13];
    for (int j = 12; j >= 0; j--)
        p = fma(p, r, coef[3 + j]);
    return ldexp(p, (int)k);
}

/* ------------------------------------------------------------------ */
/* O3..O5 draft map and ranking keys: [DA2] Sec. 3.1 Eq. (2), App. C.1  */
/* (both branches normalize over key regions).                          */
/* A = (1 - lambda) softmax(avgQ avgK^T / sqrt d)                        */
/*   +      lambda  softmax(maxQ maxK^T / sqrt d);                        */
/* key = bit pattern of fp32(A) (RNE).  Optionally returns A in fp64.   */
/* ------------------------------------------------------------------ */
static double fma_chain(const double *x, const double *y, int d)
{
    double acc = 0.0;
    for (int c = 0; c < d; c++)
        acc = fma(x[c], y[c], acc);
    return acc;
}

static void softmax_row_spec(const double *L, int R, double *p)
{
    double m = L[0];
    for (int b = 1; b < R; b++)
        if (L[b] > m)
            m = L[b];
    double Z = 0.0;
    for (int b = 0; b < R; b++) {
        p[b] = or_exp(L[b] - m);
        Z += p[b];
    }
    for (int b = 0; b < R; b++)
        p[b] = p[b] / Z;
}

void or_draft_keys_head(const double *qa, const double *ka, const float *qm,
                        const float *km, int R, int d, double lambda,
                        uint32_t *keys, double *A /* may be NULL */)
{
    double inv_sqrt_d = 1.0 / sqrt((double)d);
    double w0 = 1.0 - lambda;
    double *qmd = malloc(sizeof(double) * (size_t)R * d);
    double *kmd = malloc(sizeof(double) * (size_t)R * d);
    for (size_t i = 0; i < (size_t)R * d; i++) {
        qmd[i] = (double)qm[i];
        kmd[i] = (double)km[i];
    }
#pragma omp parallel
    {
        double *La = malloc(sizeof(double) * R), *Lm = malloc(sizeof(double) * R);
        double *pa = malloc(sizeof(double) * R), *pm = malloc(sizeof(double) * R);
#pragma omp for schedule(dynamic, 4)
        for (int a = 0; a < R; a++) {
            for (int b = 0; b < R; b++) {
                La[b] = fma_chain(qa + (size_t)a * d, ka + (size_t)b * d, d) * inv_sqrt_d;
                Lm[b] = fma_chain(qmd + (size_t)a * d, kmd + (size_t)b * d, d) * inv_sqrt_d;
            }
            softmax_row_spec(La, R, pa);
            softmax_row_spec(Lm, R, pm);
            for (int b = 0; b < R; b++) {
                double t0 = w0 * pa[b];
                double t1 = lambda * pm[b];
                double Ab = t0 + t1;
                keys[(size_t)a * R + b] = f32bits((float)Ab);
                if (A)
                    A[(size_t)a * R + b] = Ab;
            }
        }
        free(La);
        free(Lm);
        free(pa);
        free(pm);
    }
    free(qmd);
    free(kmd);
}

/* Logits of both branches for one head (the first step of the keys above),
 * exported so the tests can pin the fixed evaluation order. */
void or_draft_logits_head(const double *qa, const double *ka, const float *qm,
                          const float *km, int R, int d, double *La, double *Lm)
{
    double inv_sqrt_d = 1.0 / sqrt((double)d);
    double *x = malloc(sizeof(double) * d), *y = malloc(sizeof(double) * d);
    for (int a = 0; a < R; a++)
        for (int b = 0; b < R; b++) {
            La[(size_t)a * R + b] = fma_chain(qa + (size_t)a * d, ka + (size_t)b * d, d) * inv_sqrt_d;
            for (int c = 0; c < d; c++) {
                x[c] = (double)qm[(size_t)a * d + c];
                y[c] = (double)km[(size_t)b * d + c];
            }
            Lm[(size_t)a * R + b] = fma_chain(x, y, d) * inv_sqrt_d;
        }
    free(x);
    free(y);
}

/* ------------------------------------------------------------------ */
/* O6 quotas: [DA2] Sec. 3.1 (T = T16 + T8 + T4), App. C.1 (integer     */
/* quotas from precision fractions).  Budgets in basis points of n      */
/* (n = R^2 for head scope, R for row scope); the cumulative counts     */
/* T16, T16 + T8 and T16 + T8 + T4 are each rounded half up.            */
/* ------------------------------------------------------------------ */
void or_quotas(int64_t n, int32_t full_bp, int32_t hi_bp, int32_t lo_bp, int64_t *T16,
               int64_t *T8c, int64_t *Tk)
{
    *T16 = ((int64_t)full_bp * n + 5000) / 10000;
    *T8c = ((int64_t)(full_bp + hi_bp) * n + 5000) / 10000;
    *Tk = ((int64_t)(full_bp + hi_bp + lo_bp) * n + 5000) / 10000;
}

/* ------------------------------------------------------------------ */
/* O7 ranking: [DA2] Sec. 3.1 (ranking across the whole map of a head;  */
/* larger masses to higher precision: the 16-bit path for the T16       */
/* largest, 8-bit for the next T8, 4-bit for the next T4), App. C.1     */
/* (ties by region-pair index).  Order = key descending, pair index     */
/* ascending; rank < T16 -> 16, < T16+T8 -> 8, < Tk -> 4, else 0 (skip).*/
/* scope 0: one ranking over all R^2 pairs; scope 1: one per query row. */
/* ------------------------------------------------------------------ */
static int cmp_u64(const void *x, const void *y)
{
    uint64_t a = *(const uint64_t *)x, b = *(const uint64_t *)y;
    return (a > b) - (a < b);
}

static uint8_t tier_of_rank(int64_t r, int64_t T16, int64_t T8c, int64_t Tk)
{
    return r < T16 ? 16 : (r < T8c ? 8 : (r < Tk ? 4 : 0));
}

void or_rank_head(const uint32_t *keys, int R, int scope, int64_t T16, int64_t T8c, int64_t Tk,
                  uint8_t *tier)
{
    int64_t n = (int64_t)R * R;
    if (scope == 0) {
        /* composite: larger key first (complemented), then smaller index */
        uint64_t *ord = malloc(sizeof(uint64_t) * (size_t)n);
        for (int64_t i = 0; i < n; i++)
            ord[i] = ((uint64_t)(~keys[i]) << 32) | (uint64_t)i;
        qsort(ord, (size_t)n, sizeof(uint64_t), cmp_u64);
        for (int64_t r = 0; r < n; r++) {
            uint32_t idx = (uint32_t)(ord[r] & 0xffffffffu);
            tier[idx] = tier_of_rank(r, T16, T8c, Tk);
        }
        free(ord);
    } else {
        uint64_t *ord = malloc(sizeof(uint64_t) * (size_t)R);
        for (int a = 0; a < R; a++) {
            for (int b = 0; b < R; b++)
                ord[b] = ((uint64_t)(~keys[(size_t)a * R + b]) << 32) | (uint64_t)b;
            qsort(ord, (size_t)R, sizeof(uint64_t), cmp_u64);
            for (int r = 0; r < R; r++) {
                uint32_t b = (uint32_t)(ord[r] & 0xffffffffu);
                tier[(size_t)a * R + b] = tier_of_rank(r, T16, T8c, Tk);
            }
        }
        free(ord);
    }
}

/* ------------------------------------------------------------------ */
/* Plan for a whole [B,H] problem: pooling, keys, ranking, over the R   */
/* regions of block capacity C.                                         */
/* q, k: [B,H,N,d] contiguous bf16.  Outputs (each may be NULL except    */
/* keys and tier): avg [B,H,R,d] fp64 (Q then K arrays), mx f32.         */
/* Block-mean replacement (skip_means) is defined for C = 64 only.       */
/* ------------------------------------------------------------------ */
int or_plan(int B, int H, int F, int Hv, int Wv, int C, int d, const uint16_t *q,
            const uint16_t *k, int32_t full_bp, int32_t hi_bp, int32_t lo_bp, double lambda, int scope,
            int skip_means, uint32_t *keys, uint8_t *tier, double *qavg, double *kavg, float *qmx,
            float *kmx)
{
    int N = F * Hv * Wv, R = or_regions(F, Hv, Wv, C);
    if (R < 0 || (skip_means && C != OR_BLK))
        return -1;
    int32_t *perm = malloc(sizeof(int32_t) * (size_t)R * C);
    or_layout(F, Hv, Wv, C, perm);
    int64_t T16, T8c, Tk;
    or_quotas(scope == 0 ? (int64_t)R * R : (int64_t)R, full_bp, hi_bp, lo_bp, &T16, &T8c, &Tk);
    double *qa = malloc(sizeof(double) * (size_t)R * d), *ka = malloc(sizeof(double) * (size_t)R * d);
    float *qm = malloc(sizeof(float) * (size_t)R * d), *km = malloc(sizeof(float) * (size_t)R * d);
    for (int bh = 0; bh < B * H; bh++) {
        const uint16_t *qh = q + (size_t)bh * N * d, *kh = k + (size_t)bh * N * d;
        or_pool_head(qh, d, perm, R, C, qa, qm);
        or_pool_head(kh, d, perm, R, C, ka, km);
        if (qavg) memcpy(qavg + (size_t)bh * R * d, qa, sizeof(double) * (size_t)R * d);
        if (kavg) memcpy(kavg + (size_t)bh * R * d, ka, sizeof(double) * (size_t)R * d);
        if (qmx) memcpy(qmx + (size_t)bh * R * d, qm, sizeof(float) * (size_t)R * d);
        if (kmx) memcpy(kmx + (size_t)bh * R * d, km, sizeof(float) * (size_t)R * d);
        or_draft_keys_head(qa, ka, qm, km, R, d, lambda, keys + (size_t)bh * R * R, NULL);
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * H; bh++)
        or_rank_head(keys + (size_t)bh * R * R, R, scope, T16, T8c, Tk, tier + (size_t)bh * R * R);
    /* skip replacement by block means: every pair outside the quotas */
    if (skip_means)
        for (size_t i = 0; i < (size_t)B * H * R * R; i++)
            if (tier[i] == 0)
                tier[i] = OR_MEAN;
    free(qa); free(ka); free(qm); free(km); free(perm);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Number formats (OCP FP8 E4M3 "fn", OCP MX E2M1 + E8M0).              */
/* Rounding to nearest, ties to even; magnitudes above the largest      */
/* finite value saturate.  The sign bit is the sign bit of the input,   */
/* also when the magnitude rounds to zero.                              */
/* ------------------------------------------------------------------ */
double or_e4m3_value(int code)
{
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7)
        return NAN;
    double v = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp((double)m, -9);
    return s ? -v : v;
}

double or_e2m1_value(int code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double v = e ? ldexp(1.0 + m / 2.0, e - 1) : 0.5 * m;
    return s ? -v : v;
}

uint8_t or_e4m3_encode(double v)
{
    uint8_t sgn = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    if (a >= 448.0)
        return sgn | 0x7e;
    int e;
    frexp(a, &e);
    int E = e - 1;                       /* floor(log2 a) for a > 0 */
    if (a == 0.0 || E < -6)
        E = -6;                          /* subnormal spacing 2^-9 */
    double q = ldexp(1.0, E - 3);
    double r = rint(a / q) * q;          /* a / q is exact */
    if (r == 0.0)
        return sgn;
    frexp(r, &e);
    E = e - 1;
    if (E < -6)
        return sgn | (uint8_t)ldexp(r, 9);             /* subnormal: r = m 2^-9 */
    int m = (int)ldexp(r, 3 - E) - 8;                   /* r = (1 + m/8) 2^E */
    return sgn | (uint8_t)(((E + 7) << 3) | m);
}

uint8_t or_e2m1_encode(double v)
{
    uint8_t sgn = signbit(v) ? 8 : 0;
    double a = fabs(v);
    if (a >= 6.0)
        return sgn | 7;
    int e;
    frexp(a, &e);
    int E = e - 1;
    if (a == 0.0 || E < 0)
        E = 0;                           /* subnormal spacing 0.5 */
    double q = ldexp(1.0, E - 1);
    double r = rint(a / q) * q;
    if (r == 0.0)
        return sgn;
    if (r < 1.0)
        return sgn | 1;                  /* 0.5 */
    frexp(r, &e);
    E = e - 1;
    int m = (int)ldexp(r, 1 - E) - 2;    /* r = (1 + m/2) 2^E */
    return sgn | (uint8_t)(((E + 1) << 1) | m);
}

/* bfloat16 rounding of a double (8 significant bits, exponent range of
 * binary32 with its subnormals down to 2^-133), nearest with ties to even;
 * returns the rounded value.  The weights it is used on are finite and at
 * most 2^8, far below the bfloat16 maximum. */
double or_bf16_round(double v)
{
    double a = fabs(v);
    if (a == 0.0)
        return v;
    int e;
    frexp(a, &e);
    int E = e - 1;                       /* floor(log2 a) */
    if (E < -126)
        E = -126;                        /* subnormal spacing 2^-133 */
    double q = ldexp(1.0, E - 7);
    double r = rint(a / q) * q;          /* a / q exact: a power-of-two quotient */
    return signbit(v) ? -r : r;
}

/* E8M0 exponent of an MX block: floor(log2 amax) - 2 (2 = exponent of the
 * largest E2M1 power of two), clamped to the E8M0 range; amax = 0 -> -127. */
int or_mx_exponent(double amax)
{
    if (amax == 0.0)
        return -127;
    int e;
    frexp(amax, &e);
    int E = (e - 1) - 2;
    if (E < -127) E = -127;
    if (E > 127) E = 127;
    return E;
}

/* E8M0 exponent of an MX block of attention weights: the smallest X with
 * amax 2^-X <= 6, so the block maximum is never clipped -- the power-of-two
 * counterpart of the NVFP4 block scale amax / 6 that [DA2] App. C.1 names
 * for the probability-value product.  (The operand rule above clips block
 * maxima in [6, 8) 2^X to 6; a weight block holding the running maximum has
 * amax = 1 exactly, where that rule jumps from 1 to 0.75 under any rounding
 * below 1.)  amax = 0 -> -127; clamped to the E8M0 range. */
int or_mx_exponent_w(double amax)
{
    if (amax == 0.0)
        return -127;
    int e;
    double m = frexp(amax, &e);           /* amax = m 2^e, m in [0.5, 1) */
    int E = (e - 1) - 2 + (2.0 * m > 1.5 ? 1 : 0);
    if (E < -127) E = -127;
    if (E > 127) E = 127;
    return E;
}

/* ------------------------------------------------------------------ */
/* O8/O9 operand quantization: [DA2] Sec. 3.3 (fused quantization and   */
/* reordering).  All outputs are in reordered token order pos.          */
/*  Q/K INT8: one fp32 step per 64-token block: s = amax/127 (fp32      */
/*            division), code = nearest integer (ties to even) of        */
/*            fp32(x * fp32(127/amax)): App. B.2's uniform quantizer     */
/*            with no clipping ([DA2] App. C.1: INT8 for Q K^T).         */
/*  Q/K MX  : per token, per 32 channels: E8M0 + E2M1 codes of x 2^-E.  */
/*  V FP8   : one fp32 scale per channel over all N tokens.             */
/*  V MX    : per channel, per 32 consecutive keys of a block.          */
/* Codes are stored one per byte (E2M1 in the low nibble).              */
/* ------------------------------------------------------------------ */
static void fp8_scale(float amax, float *s, float *inv)
{
    if (amax == 0.0f) {
        *s = 1.0f;
        *inv = 0.0f;
    } else {
        *s = amax / 448.0f;
        *inv = 448.0f / amax;
    }
}

/* Value at reordered position pos, channel c: 0 for a padding slot. */
static float xat(const uint16_t *X, const int32_t *perm, size_t pos, int d, int c)
{
    return perm[pos] < 0 ? 0.0f : bf16f(X[(size_t)perm[pos] * d + c]);
}

/* INT8 step of a Q/K block: amax/127; an all-zero block takes step 1 and
 * zero codes. */
static void int8_scale(float amax, float *s, float *inv)
{
    if (amax == 0.0f) {
        *s = 1.0f;
        *inv = 0.0f;
    } else {
        *s = amax / 127.0f;
        *inv = 127.0f / amax;
    }
}

/* Nearest integer of an fp32 value, ties to even, within [-127, 127]
 * (|x| <= 127 up to the product's rounding, so the clamp never changes a
 * code that the rounding alone would not). */
static uint8_t int8_code(float x)
{
    double r = nearbyint((double)x);
    if (r > 127.0) r = 127.0;
    if (r < -127.0) r = -127.0;
    return (uint8_t)(int8_t)r;
}

/* Q/K of one head over Np = R 64 reordered positions (padding slots hold
 * zeros): c8 [Np][d] INT8 codes (two's complement bytes), s8 [R] steps,
 * c4 [Np][d], e4 [Np][d/32]. */
void or_quant_qk_head(const uint16_t *X, int Np, int d, const int32_t *perm,
                      uint8_t *c8, float *s8, uint8_t *c4, uint8_t *e4)
{
    int R = Np / OR_BLK;
    for (int a = 0; a < R; a++) {
        float amax = 0.0f;
        for (int i = 0; i < OR_BLK; i++)
            for (int c = 0; c < d; c++) {
                float v = fabsf(xat(X, perm, (size_t)a * OR_BLK + i, d, c));
                if (v > amax) amax = v;
            }
        float s, inv;
        int8_scale(amax, &s, &inv);
        s8[a] = s;
        for (int i = 0; i < OR_BLK; i++)
            for (int c = 0; c < d; c++) {
                float v = xat(X, perm, (size_t)a * OR_BLK + i, d, c);
                float prod = v * inv;
                c8[((size_t)a * OR_BLK + i) * d + c] = int8_code(prod);
            }
    }
    for (int pos = 0; pos < Np; pos++)
        for (int g = 0; g < d / 32; g++) {
            double amax = 0.0;
            for (int j = 0; j < 32; j++) {
                double v = fabs((double)xat(X, perm, pos, d, 32 * g + j));
                if (v > amax) amax = v;
            }
            int E = or_mx_exponent(amax);
            e4[(size_t)pos * (d / 32) + g] = (uint8_t)(E + 127);
            for (int j = 0; j < 32; j++) {
                double v = (double)xat(X, perm, pos, d, 32 * g + j);
                c4[(size_t)pos * d + 32 * g + j] = or_e2m1_encode(ldexp(v, -E));
            }
        }
}

/* V of one head (N tokens, Np positions): c8 [Np][d] codes, s8 [d] scales
 * (amax over the N tokens), c4 [Np][d] codes, e4 [R][2][d] exponents */
void or_quant_v_head(const uint16_t *X, int N, int Np, int d, const int32_t *perm,
                     uint8_t *c8, float *s8, uint8_t *c4, uint8_t *e4)
{
    int R = Np / OR_BLK;
    for (int c = 0; c < d; c++) {
        float amax = 0.0f;
        for (int n = 0; n < N; n++) {
            float v = fabsf(bf16f(X[(size_t)n * d + c]));
            if (v > amax) amax = v;
        }
        float s, inv;
        fp8_scale(amax, &s, &inv);
        s8[c] = s;
        for (int pos = 0; pos < Np; pos++) {
            float v = xat(X, perm, pos, d, c);
            float prod = v * inv;
            c8[(size_t)pos * d + c] = or_e4m3_encode((double)prod);
        }
    }
    for (int a = 0; a < R; a++)
        for (int g = 0; g < 2; g++)
            for (int c = 0; c < d; c++) {
                double amax = 0.0;
                for (int j = 0; j < 32; j++) {
                    int pos = a * OR_BLK + 32 * g + j;
                    double v = fabs((double)xat(X, perm, pos, d, c));
                    if (v > amax) amax = v;
                }
                int E = or_mx_exponent(amax);
                e4[((size_t)a * 2 + g) * d + c] = (uint8_t)(E + 127);
                for (int j = 0; j < 32; j++) {
                    int pos = a * OR_BLK + 32 * g + j;
                    double v = (double)xat(X, perm, pos, d, c);
                    c4[(size_t)pos * d + c] = or_e2m1_encode(ldexp(v, -E));
                }
            }
}

/* Whole-problem quantization into canonical layouts (Np = R C positions
 * of the R regions of capacity C, region order, padding slots included;
 * T = Np / 64 tiles of 64 positions):
 *   qk8 [B,H,Np,d] codes, qks8 [B,H,T] scales, qk4 [B,H,Np,d], qke4 [B,H,Np,d/32]
 *   v8  [B,H,Np,d],       vs8  [B,H,d],        v4  [B,H,Np,d], ve4  [B,H,T,2,d] */
int or_quant_qk(int B, int H, int F, int Hv, int Wv, int C, int d, const uint16_t *X,
                uint8_t *c8, float *s8, uint8_t *c4, uint8_t *e4)
{
    int N = F * Hv * Wv, R = or_regions(F, Hv, Wv, C);
    if (R < 0 || C % OR_BLK) return -1;
    size_t Np = (size_t)R * C;
    int32_t *perm = malloc(sizeof(int32_t) * Np);
    or_layout(F, Hv, Wv, C, perm);
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * H; bh++)
        or_quant_qk_head(X + (size_t)bh * N * d, (int)Np, d, perm, c8 + (size_t)bh * Np * d,
                         s8 + (size_t)bh * (Np / OR_BLK), c4 + (size_t)bh * Np * d,
                         e4 + (size_t)bh * Np * (d / 32));
    free(perm);
    return 0;
}

int or_quant_v(int B, int H, int F, int Hv, int Wv, int C, int d, const uint16_t *X,
               uint8_t *c8, float *s8, uint8_t *c4, uint8_t *e4)
{
    int N = F * Hv * Wv, R = or_regions(F, Hv, Wv, C);
    if (R < 0 || C % OR_BLK) return -1;
    size_t Np = (size_t)R * C;
    int32_t *perm = malloc(sizeof(int32_t) * Np);
    or_layout(F, Hv, Wv, C, perm);
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * H; bh++)
        or_quant_v_head(X + (size_t)bh * N * d, N, (int)Np, d, perm, c8 + (size_t)bh * Np * d,
                        s8 + (size_t)bh * d, c4 + (size_t)bh * Np * d,
                        e4 + (size_t)bh * (Np / OR_BLK) * 2 * d);
    free(perm);
    return 0;
}

/* ------------------------------------------------------------------ */
/* O10 attention over kept tiles: [DA2] Sec. 3.1 (all retained blocks   */
/* of a query share one softmax normalization and output), Sec. 3.3     */
/* (consecutive precision phases; shared online-softmax statistics and  */
/* accumulator), App. B.3 (w = e^{s - h}, Z^q = sum of unquantized w),  */
/* App. B.4 (O = sum(w_hat V_hat) / Z^q), App. C.1 (rows with no        */
/* retained key return zero).                                           */
/* Phases in descending precision: tier 32 (oracle-only: unquantized    */
/* operands and weights, for the invariants), tier 16 (the 16-bit path: */
/* the bf16 inputs as they are, weights unquantized), tier 8 (INT8      */
/* Q K^T, FP8 P V), tier 4 (MXFP4); tiles ascending inside a phase;     */
/* running max                                                          */
/* updated once per 64-key tile.                                        */
/* ------------------------------------------------------------------ */
typedef struct {
    int N, d, R;             /* N: reordered positions R 64 (padding included) */
    const int32_t *perm;
    int32_t *nv;             /* valid tokens of each region [R] (slots 0 .. nv-1) */
    double *qf, *kf, *vf;    /* unquantized, reordered [N][d]; padding rows 0 */
    double *q8, *k8, *v8;    /* 8-bit path dequantized: INT8 Q/K, FP8 V */
    double *q4, *k4, *v4;    /* MXFP4 dequantized */
    uint8_t *c8q, *c8k;      /* INT8 codes of Q and K, reordered [N][d] */
    float *s8q, *s8k;        /* their per-block scales [R] */
    double *qa, *ka, *va;    /* region means over the valid tokens [R][d] */
} head_ops;

/* q, k, v: one head, [Ntok][d] in token order; perm over Np = R 64
 * positions (-1 for padding). */
static void head_ops_build(head_ops *h, const uint16_t *q, const uint16_t *k,
                           const uint16_t *v, int Ntok, int Np, int d, const int32_t *perm)
{
    int N = Np, R = Np / OR_BLK;
    size_t nd = (size_t)N * d;
    h->N = N; h->d = d; h->R = R; h->perm = perm;
    h->nv = malloc(sizeof(int32_t) * R);
    for (int a = 0; a < R; a++) {
        int n = 0;
        while (n < OR_BLK && perm[a * OR_BLK + n] >= 0)
            n++;
        h->nv[a] = n;
    }
    double **arrs[9] = {&h->qf, &h->kf, &h->vf, &h->q8, &h->k8, &h->v8, &h->q4, &h->k4, &h->v4};
    for (int i = 0; i < 9; i++)
        *arrs[i] = malloc(sizeof(double) * nd);
    uint8_t *c8 = malloc(nd), *c4 = malloc(nd);
    uint8_t *e4 = malloc(nd / 32 + (size_t)R * 2 * d);
    float *s8 = malloc(sizeof(float) * (size_t)(R > d ? R : d));
    h->c8q = malloc(nd);
    h->c8k = malloc(nd);
    h->s8q = malloc(sizeof(float) * R);
    h->s8k = malloc(sizeof(float) * R);
    const uint16_t *src[3] = {q, k, v};
    double *full[3] = {h->qf, h->kf, h->vf};
    double *d8[3] = {h->q8, h->k8, h->v8};
    double *d4[3] = {h->q4, h->k4, h->v4};
    for (int t = 0; t < 3; t++) {
        for (int pos = 0; pos < N; pos++)
            for (int c = 0; c < d; c++)
                full[t][(size_t)pos * d + c] = (double)xat(src[t], perm, pos, d, c);
        if (t < 2) {
            or_quant_qk_head(src[t], N, d, perm, c8, s8, c4, e4);
            memcpy(t == 0 ? h->c8q : h->c8k, c8, nd);
            memcpy(t == 0 ? h->s8q : h->s8k, s8, sizeof(float) * R);
            for (int pos = 0; pos < N; pos++)
                for (int c = 0; c < d; c++) {
                    size_t i = (size_t)pos * d + c;
                    d8[t][i] = (double)(int8_t)c8[i] * (double)s8[pos / OR_BLK];
                    d4[t][i] = ldexp(or_e2m1_value(c4[i]), (int)e4[(size_t)pos * (d / 32) + c / 32] - 127);
                }
        } else {
            or_quant_v_head(src[t], Ntok, N, d, perm, c8, s8, c4, e4);
            for (int pos = 0; pos < N; pos++)
                for (int c = 0; c < d; c++) {
                    size_t i = (size_t)pos * d + c;
                    int a = pos / OR_BLK, g = (pos % OR_BLK) / 32;
                    d8[t][i] = or_e4m3_value(c8[i]) * (double)s8[c];
                    d4[t][i] = ldexp(or_e2m1_value(c4[i]), (int)e4[((size_t)a * 2 + g) * d + c] - 127);
                }
        }
    }
    free(c8); free(c4); free(e4); free(s8);
    double **means[3] = {&h->qa, &h->ka, &h->va};
    float *mx = malloc(sizeof(float) * (size_t)R * d);
    for (int t = 0; t < 3; t++) {
        *means[t] = malloc(sizeof(double) * (size_t)R * d);
        or_pool_head(src[t], d, perm, R, OR_BLK, *means[t], mx);
    }
    free(mx);
}

static void head_ops_free(head_ops *h)
{
    double *arrs[9] = {h->qf, h->kf, h->vf, h->q8, h->k8, h->v8, h->q4, h->k4, h->v4};
    for (int i = 0; i < 9; i++)
        free(arrs[i]);
    free(h->c8q);
    free(h->c8k);
    free(h->s8q);
    free(h->s8k);
    free(h->nv);
    free(h->qa);
    free(h->ka);
    free(h->va);
}

/* Block-mean tile (a, b) ([Triage] abstract: a skipped tile replaced by its
 * block means).  By bilinearity the mean of the tile's 64 x 64 scores is
 * the score of the mean query and the mean key, q_a . k_b / sqrt(d) (the
 * average-branch draft logit of Eq. 2, same fma chain); the tile's values
 * are replaced by the key region's mean value v_b, and the tile counts its
 * n_b valid keys. */
static double mean_logit(const head_ops *h, int a, int b)
{
    return fma_chain(h->qa + (size_t)a * h->d, h->ka + (size_t)b * h->d, h->d) / sqrt((double)h->d);
}

/* Relative precision band of a weight code decision.  The GPU path forms
 * each weight in fp32 from fp32 logits; its relative error stays below
 * 2^-16 wherever the weight is above 2^-60 (log2-domain error about
 * (|t| + |S c|) 2^-23 for |t|, |S c| <= 60, plus one ulp of exp2).  A code
 * whose value changes when w moves by that band has two correct results. */
#define OR_AMB_REL 0x1p-16

/* Alternative of one element's code inside the band: the largest change of
 * the quantized value over w (1 - delta) and w (1 + delta). */
static double band_alt_e4m3(double x, double q)
{
    double a = or_e4m3_value(or_e4m3_encode(x * (1.0 - OR_AMB_REL)));
    double b = or_e4m3_value(or_e4m3_encode(x * (1.0 + OR_AMB_REL)));
    double da = fabs(a - q), db = fabs(b - q);
    return da > db ? da : db;
}

static double band_alt_e2m1(double x, double q)
{
    double a = or_e2m1_value(or_e2m1_encode(x * (1.0 - OR_AMB_REL)));
    double b = or_e2m1_value(or_e2m1_encode(x * (1.0 + OR_AMB_REL)));
    double da = fabs(a - q), db = fabs(b - q);
    return da > db ? da : db;
}

/* Weight quantizers for one 64-key tile, w[64] in key order.  wa (may be
 * NULL) receives, per key, how far its quantized weight can move when the
 * decisions it depends on are taken anywhere in the precision band: its own
 * code, and for MXFP4 also the block exponent. */
static void quant_weights(int tier, const double *w, double *wq, double *wa)
{
    if (wa)
        for (int j = 0; j < OR_BLK; j++) wa[j] = 0.0;
    if (tier == 32) {
        for (int j = 0; j < OR_BLK; j++) wq[j] = w[j];
    } else if (tier == 16) {
        /* the 16-bit path: weights unquantized (App. B's error bound has no
         * term for it) */
        for (int j = 0; j < OR_BLK; j++) wq[j] = w[j];
    } else if (tier == 8) {
        for (int j = 0; j < OR_BLK; j++) {
            double x = ldexp(w[j], 8), q = or_e4m3_value(or_e4m3_encode(x));
            wq[j] = ldexp(q, -8);
            if (wa)
                wa[j] = ldexp(band_alt_e4m3(x, q), -8);
        }
    } else {
        for (int g = 0; g < 2; g++) {
            double amax = 0.0;
            for (int j = 0; j < 32; j++)
                if (fabs(w[32 * g + j]) > amax) amax = fabs(w[32 * g + j]);
            int E = or_mx_exponent_w(amax);
            int Elo = or_mx_exponent_w(amax * (1.0 - OR_AMB_REL));
            int Ehi = or_mx_exponent_w(amax * (1.0 + OR_AMB_REL));
            for (int j = 0; j < 32; j++) {
                double x = ldexp(w[32 * g + j], -E), q = or_e2m1_value(or_e2m1_encode(x));
                wq[32 * g + j] = ldexp(q, E);
                if (!wa)
                    continue;
                double d = ldexp(band_alt_e2m1(x, q), E);
                int Ea[2] = {Elo, Ehi};
                for (int t = 0; t < 2; t++) {
                    if (Ea[t] == E)
                        continue;
                    double xa = ldexp(w[32 * g + j], -Ea[t]);
                    double qa = ldexp(or_e2m1_value(or_e2m1_encode(xa)), Ea[t]);
                    double da = fabs(qa - wq[32 * g + j]) + ldexp(band_alt_e2m1(xa, ldexp(qa, -Ea[t])), Ea[t]);
                    if (da > d) d = da;
                }
                wa[32 * g + j] = d;
            }
        }
    }
}

/* Optional per-row trace for the tests: for every processed key (in
 * processing order) its reordered position, tier, s_hat, w, w_hat and the
 * running max after its tile. */
typedef struct {
    int64_t cap, n;
    int32_t *key;
    int32_t *tier;
    double *s, *w, *wq, *m;
    double Z;
} row_trace;

/* Online-softmax state of one query row (App. B.4): running max m, sum Z
 * of the unquantized weights, unnormalised output acc[d]; amb[d] (NULL when
 * not asked for) the same sum over the band movements wa of the weights
 * times |v|. */
typedef struct {
    double m, Z;
    double *acc;
    double *amb;
} row_acc;

/* One tile of up to 64 keys at tier p: key j < nk has operand rows
 * kt + j d and vt + j d; keys j >= nk (past the valid prefix keys, App. C.1)
 * take no part: they add no weight and do not move the running max.  s, w
 * and wq receive the tile's logits, weights and quantized weights (zero
 * past nk; s is -inf there). */
static void tile_exact(row_acc *st, int d, int p, const double *qu, const double *kt,
                       const double *vt, int nk, double *s, double *w, double *wq)
{
    double wa[OR_BLK];
    double inv_sqrt_d = 1.0 / sqrt((double)d);
    double tmax = -INFINITY;
    for (int j = 0; j < OR_BLK; j++) {
        s[j] = -INFINITY;
        if (j >= nk)
            continue;
        const double *kv = kt + (size_t)j * d;
        double dot = 0.0;
        for (int c = 0; c < d; c++)
            dot += qu[c] * kv[c];
        s[j] = dot * inv_sqrt_d;
        if (s[j] > tmax) tmax = s[j];
    }
    double mn = tmax > st->m ? tmax : st->m;
    double alpha = (st->m == -INFINITY) ? 0.0 : exp(st->m - mn);
    st->Z *= alpha;
    for (int c = 0; c < d; c++)
        st->acc[c] *= alpha;
    if (st->amb)
        for (int c = 0; c < d; c++)
            st->amb[c] *= alpha;
    for (int j = 0; j < OR_BLK; j++) {
        w[j] = j < nk ? exp(s[j] - mn) : 0.0;
        st->Z += w[j];
    }
    quant_weights(p, w, wq, st->amb ? wa : NULL);
    for (int j = 0; j < nk; j++) {
        const double *vv = vt + (size_t)j * d;
        for (int c = 0; c < d; c++)
            st->acc[c] += wq[j] * vv[c];
        if (st->amb)
            for (int c = 0; c < d; c++)
                st->amb[c] += wa[j] * fabs(vv[c]);
    }
    st->m = mn;
}

/* Text prefix of one head (App. C.1): Lp prefix tokens in their own order,
 * of which the first nv are valid keys.  Prefix interactions are computed
 * at tier pt (16: the 16-bit path; 32: unquantized, for the invariants). */
typedef struct {
    int Lp, nv, pt;
    const double *qf, *kf, *vf; /* [Lp][d] */
} prefix_ops;

/* The prefix segment of a row: tiles of 64 consecutive prefix keys,
 * ascending, the last one ragged.  Processed before the video tiles. */
static void prefix_segment(row_acc *st, int d, const prefix_ops *px, const double *qu,
                           row_trace *tr)
{
    double s[OR_BLK], w[OR_BLK], wq[OR_BLK];
    if (!px)
        return;
    for (int t = 0; OR_BLK * t < px->nv; t++) {
        int nk = px->nv - OR_BLK * t < OR_BLK ? px->nv - OR_BLK * t : OR_BLK;
        tile_exact(st, d, px->pt, qu, px->kf + (size_t)OR_BLK * t * d,
                   px->vf + (size_t)OR_BLK * t * d, nk, s, w, wq);
        if (tr) {
            for (int j = 0; j < nk && tr->n < tr->cap; j++, tr->n++) {
                tr->key[tr->n] = -1 - (OR_BLK * t + j);
                tr->tier[tr->n] = px->pt;
                tr->s[tr->n] = s[j];
                tr->w[tr->n] = w[j];
                tr->wq[tr->n] = wq[j];
                tr->m[tr->n] = st->m;
            }
        }
    }
}

static void finish_row(const row_acc *st, int d, double *out, double *amb)
{
    for (int c = 0; c < d; c++)
        out[c] = st->Z > 0.0 ? st->acc[c] / st->Z : 0.0;
    if (amb)
        for (int c = 0; c < d; c++)
            amb[c] = st->Z > 0.0 ? st->amb[c] / st->Z : 0.0;
}

/* Video query row u (reordered position): the prefix segment (if any), then
 * the phases in descending precision over the kept video tiles. */
static void attention_row(const head_ops *h, const prefix_ops *px, const uint8_t *tier_row,
                          int u, double *out, row_trace *tr, double *amb)
{
    int d = h->d, R = h->R;
    row_acc st = {-INFINITY, 0.0, calloc(d, sizeof(double)), amb ? calloc(d, sizeof(double)) : NULL};
    double s[OR_BLK], w[OR_BLK], wq[OR_BLK];
    static const int phases[4] = {32, 16, 8, 4};
    const int a = u / OR_BLK;
    prefix_segment(&st, d, px, h->qf + (size_t)u * d, tr);
    for (int ph = 0; ph < 4; ph++) {
        int p = phases[ph];
        const double *Q = p >= 16 ? h->qf : (p == 8 ? h->q8 : h->q4);
        const double *K = p >= 16 ? h->kf : (p == 8 ? h->k8 : h->k4);
        const double *V = p >= 16 ? h->vf : (p == 8 ? h->v8 : h->v4);
        for (int b = 0; b < R; b++) {
            if (tier_row[b] != p)
                continue;
            tile_exact(&st, d, p, Q + (size_t)u * d, K + (size_t)b * OR_BLK * d,
                       V + (size_t)b * OR_BLK * d, h->nv[b], s, w, wq);
            if (tr) {
                for (int j = 0; j < h->nv[b] && tr->n < tr->cap; j++, tr->n++) {
                    tr->key[tr->n] = b * OR_BLK + j;
                    tr->tier[tr->n] = p;
                    tr->s[tr->n] = s[j];
                    tr->w[tr->n] = w[j];
                    tr->wq[tr->n] = wq[j];
                    tr->m[tr->n] = st.m;
                }
            }
        }
    }
    /* block-mean tiles last, ascending (the lowest tier): one score per
     * tile, unquantized */
    for (int b = 0; b < R; b++) {
        if (tier_row[b] != OR_MEAN)
            continue;
        double sb = mean_logit(h, a, b);
        double mn = sb > st.m ? sb : st.m;
        double alpha = (st.m == -INFINITY) ? 0.0 : exp(st.m - mn);
        st.Z *= alpha;
        for (int c = 0; c < d; c++)
            st.acc[c] *= alpha;
        if (st.amb)
            for (int c = 0; c < d; c++)
                st.amb[c] *= alpha;
        double w = (double)h->nv[b] * exp(sb - mn);
        st.Z += w;
        for (int c = 0; c < d; c++)
            st.acc[c] += w * h->va[(size_t)b * d + c];
        st.m = mn;
    }
    finish_row(&st, d, out, amb);
    if (tr)
        tr->Z = st.Z;
    free(st.acc);
    free(st.amb);
}

/* Prefix query rows (App. C.1: non-sparse attention).  Their key sequence
 * is every valid prefix key (tiles of 64, the last one ragged), then every
 * video region ascending, all at the prefix tier.  The sequence is split
 * into chunks of OR_PCHUNK consecutive tiles; each chunk is an online
 * softmax of its own (running max from -inf), and the chunks' states are
 * merged by the exact rescale of App. B.4's shared normalization:
 * M = max m_c, Z = sum Z_c e^(m_c - M), acc = sum acc_c e^(m_c - M). */
#define OR_PCHUNK 128

static int prefix_tiles(const prefix_ops *px) { return (px->nv + OR_BLK - 1) / OR_BLK; }

/* Tile t of prefix row i's key sequence: rows of K and V and the count of
 * valid keys. */
static int prefix_row_tile(const head_ops *h, const prefix_ops *px, int t, const double **kt,
                           const double **vt)
{
    int np = prefix_tiles(px), d = h->d;
    if (t < np) {
        *kt = px->kf + (size_t)OR_BLK * t * d;
        *vt = px->vf + (size_t)OR_BLK * t * d;
        return px->nv - OR_BLK * t < OR_BLK ? px->nv - OR_BLK * t : OR_BLK;
    }
    *kt = h->kf + (size_t)(t - np) * OR_BLK * d;
    *vt = h->vf + (size_t)(t - np) * OR_BLK * d;
    return h->nv[t - np];
}

static void attention_prefix_row(const head_ops *h, const prefix_ops *px, int i, double *out)
{
    int d = h->d, T = prefix_tiles(px) + h->R;
    int nc = (T + OR_PCHUNK - 1) / OR_PCHUNK;
    double s[OR_BLK], w[OR_BLK], wq[OR_BLK];
    const double *qu = px->qf + (size_t)i * d;
    double *mc = malloc(sizeof(double) * nc), *zc = malloc(sizeof(double) * nc);
    double *ac = calloc((size_t)nc * d, sizeof(double));
    for (int c = 0; c < nc; c++) {
        row_acc st = {-INFINITY, 0.0, ac + (size_t)c * d, NULL};
        for (int t = c * OR_PCHUNK; t < T && t < (c + 1) * OR_PCHUNK; t++) {
            const double *kt, *vt;
            int nk = prefix_row_tile(h, px, t, &kt, &vt);
            tile_exact(&st, d, px->pt, qu, kt, vt, nk, s, w, wq);
        }
        mc[c] = st.m;
        zc[c] = st.Z;
    }
    double M = -INFINITY, Z = 0.0;
    for (int c = 0; c < nc; c++)
        if (mc[c] > M) M = mc[c];
    for (int c = 0; c < d; c++)
        out[c] = 0.0;
    for (int c = 0; c < nc; c++) {
        double f = exp(mc[c] - M);
        Z += zc[c] * f;
        for (int j = 0; j < d; j++)
            out[j] += ac[(size_t)c * d + j] * f;
    }
    for (int j = 0; j < d; j++)
        out[j] = Z > 0.0 ? out[j] / Z : 0.0;
    free(mc);
    free(zc);
    free(ac);
}

/* Tiles of a layout of block capacity C (a multiple of 64): region a's C
 * positions are the C / 64 tiles a C/64 .. a C/64 + C/64 - 1, and a region
 * pair's tier holds for each of its tile pairs.  The phases visit a row's
 * kept tiles ascending, i.e. key regions ascending and the tiles of one
 * region in slot order.  tile_tiers writes one head's [T,T] tile tiers
 * from its [R,R] region tiers (T = R C/64); for C = 64 they are the same. */
static const uint8_t *tile_tiers(const uint8_t *tier, int R, int tpr, uint8_t **buf)
{
    if (tpr == 1)
        return tier;
    int T = R * tpr;
    if (!*buf)
        *buf = malloc((size_t)T * T);
    for (int at = 0; at < T; at++)
        for (int bt = 0; bt < T; bt++)
            (*buf)[(size_t)at * T + bt] = tier[(size_t)(at / tpr) * R + bt / tpr];
    return *buf;
}

/* Block-mean tiles are defined for C = 64 only. */
static int tiers_valid(const uint8_t *tier, size_t n, int C)
{
    if (C == OR_BLK)
        return 1;
    for (size_t i = 0; i < n; i++)
        if (tier[i] == OR_MEAN)
            return 0;
    return 1;
}

/* q,k,v: [B,H,N,d] bf16; tier: [B,H,R,R] in {0,4,8,16} over the R regions
 * of block capacity C (a multiple of 64).  qblocks: nqb query tiles (64
 * positions each) evaluated for every (b,h) (NULL -> all T = R C/64).
 * out: [B,H,nqb,64,d] fp64, row (j,i) belongs to original token
 * perm[qblocks[j]*64 + i] (restore is done by the caller's indexing). */
int or_attention(int B, int H, int F, int Hv, int Wv, int C, int d, const uint16_t *q,
                 const uint16_t *k, const uint16_t *v, const uint8_t *tier, int nqb,
                 const int32_t *qblocks, double *out, double *amb)
{
    int N = F * Hv * Wv, R = or_regions(F, Hv, Wv, C);
    if (R < 0 || C % OR_BLK || !tiers_valid(tier, (size_t)B * H * R * R, C)) return -1;
    int tpr = C / OR_BLK, T = R * tpr, Np = R * C;
    int32_t *perm = malloc(sizeof(int32_t) * Np);
    uint8_t *tbuf = NULL;
    or_layout(F, Hv, Wv, C, perm);
    if (!qblocks) nqb = T;
    for (int bh = 0; bh < B * H; bh++) {
        head_ops h;
        size_t off = (size_t)bh * N * d;
        head_ops_build(&h, q + off, k + off, v + off, N, Np, d, perm);
        const uint8_t *tm = tile_tiers(tier + (size_t)bh * R * R, R, tpr, &tbuf);
#pragma omp parallel for schedule(dynamic, 8)
        for (int r = 0; r < nqb * OR_BLK; r++) {
            int j = r / OR_BLK, i = r % OR_BLK;
            int a = qblocks ? qblocks[j] : j;
            size_t ro = (((size_t)bh * nqb + j) * OR_BLK + i) * d;
            double *o = out + ro;
            if (i >= h.nv[a]) {   /* padding slot: no query */
                memset(o, 0, sizeof(double) * d);
                if (amb)
                    memset(amb + ro, 0, sizeof(double) * d);
                continue;
            }
            attention_row(&h, NULL, tm + (size_t)a * T, a * OR_BLK + i, o, NULL, amb ? amb + ro : NULL);
        }
        head_ops_free(&h);
    }
    free(perm);
    free(tbuf);
    return 0;
}

/* Trace of one query row (reordered position u) of one head.  Returns the
 * number of processed keys (may exceed cap; only cap entries are written). */
int64_t or_attention_trace(int F, int Hv, int Wv, int C, int d, const uint16_t *q,
                           const uint16_t *k, const uint16_t *v, const uint8_t *tier,
                           int u, int64_t cap, int32_t *key, int32_t *tr_tier, double *s,
                           double *w, double *wq, double *m, double *Z, double *out)
{
    int N = F * Hv * Wv, R = or_regions(F, Hv, Wv, C);
    if (R < 0 || C % OR_BLK || !tiers_valid(tier, (size_t)R * R, C)) return -1;
    int tpr = C / OR_BLK, T = R * tpr, Np = R * C;
    int32_t *perm = malloc(sizeof(int32_t) * Np);
    uint8_t *tbuf = NULL;
    or_layout(F, Hv, Wv, C, perm);
    head_ops h;
    head_ops_build(&h, q, k, v, N, Np, d, perm);
    const uint8_t *tm = tile_tiers(tier, R, tpr, &tbuf);
    row_trace tr = {cap, 0, key, tr_tier, s, w, wq, m, 0.0};
    attention_row(&h, NULL, tm + (size_t)(u / OR_BLK) * T, u, out, &tr, NULL);
    *Z = tr.Z;
    head_ops_free(&h);
    free(perm);
    free(tbuf);
    return tr.n;
}

/* ------------------------------------------------------------------ */
/* Text prefix (App. C.1): video queries keep every valid prefix key    */
/* outside the region budget, prefix queries attend to every valid key. */
/* The prefix tensors qp, kp, vp are [B,H,Lp,d] bf16; valid[b] in      */
/* [0, Lp] is the number of valid prefix keys of batch b (NULL: all).   */
/* out: the video rows as in or_attention; outp: [B,H,np,d] prefix query */
/* rows prows[0..np) (prows NULL: all Lp rows, np = Lp; outp NULL: none). */
/* pt: tier of the prefix interactions (16: the 16-bit path; 32:        */
/* unquantized, for the invariants).                                    */
/* ------------------------------------------------------------------ */
static void prefix_ops_build(prefix_ops *px, const uint16_t *qp, const uint16_t *kp,
                             const uint16_t *vp, int Lp, int nv, int d, int pt)
{
    size_t n = (size_t)Lp * d;
    double *a[3];
    const uint16_t *src[3] = {qp, kp, vp};
    for (int t = 0; t < 3; t++) {
        a[t] = malloc(sizeof(double) * (n ? n : 1));
        for (size_t i = 0; i < n; i++)
            a[t][i] = (double)bf16f(src[t][i]);
    }
    px->Lp = Lp;
    px->nv = nv < 0 ? 0 : (nv > Lp ? Lp : nv);
    px->pt = pt;
    px->qf = a[0];
    px->kf = a[1];
    px->vf = a[2];
}

static void prefix_ops_free(prefix_ops *px)
{
    free((void *)px->qf);
    free((void *)px->kf);
    free((void *)px->vf);
}

static int pfx_common(int B, int H, int F, int Hv, int Wv, int C, int d, const uint16_t *q,
                      const uint16_t *k, const uint16_t *v, int Lp, const uint16_t *qp,
                      const uint16_t *kp, const uint16_t *vp, const int32_t *valid, int pt,
                      const uint8_t *tier, int nqb, const int32_t *qblocks, int nprow,
                      const int32_t *prows, double *out, double *outp, double *amb)
{
    int N = F * Hv * Wv, R = or_regions(F, Hv, Wv, C);
    if (pt != 16 && pt != 32) return -1;
    if (R < 0 || C % OR_BLK || !tiers_valid(tier, (size_t)B * H * R * R, C)) return -1;
    int tpr = C / OR_BLK, T = R * tpr, Np = R * C;
    int32_t *perm = malloc(sizeof(int32_t) * Np);
    uint8_t *tbuf = NULL;
    or_layout(F, Hv, Wv, C, perm);
    if (!qblocks) nqb = T;
    for (int bh = 0; bh < B * H; bh++) {
        head_ops h;
        prefix_ops px;
        size_t off = (size_t)bh * N * d, poff = (size_t)bh * Lp * d;
        head_ops_build(&h, q + off, k + off, v + off, N, Np, d, perm);
        prefix_ops_build(&px, qp + poff, kp + poff, vp + poff, Lp, valid ? valid[bh / H] : Lp, d, pt);
        const uint8_t *tm = tile_tiers(tier + (size_t)bh * R * R, R, tpr, &tbuf);
#pragma omp parallel for schedule(dynamic, 8)
        for (int r = 0; r < nqb * OR_BLK; r++) {
            int j = r / OR_BLK, i = r % OR_BLK;
            int a = qblocks ? qblocks[j] : j;
            size_t o = (((size_t)bh * nqb + j) * OR_BLK + i) * d;
            if (i >= h.nv[a]) {   /* padding slot: no query */
                memset(out + o, 0, sizeof(double) * d);
                if (amb)
                    memset(amb + o, 0, sizeof(double) * d);
                continue;
            }
            attention_row(&h, &px, tm + (size_t)a * T, a * OR_BLK + i, out + o, NULL, amb ? amb + o : NULL);
        }
        if (outp) {
            int n = prows ? nprow : Lp;
#pragma omp parallel for schedule(dynamic, 1)
            for (int j = 0; j < n; j++) {
                int i = prows ? prows[j] : j;
                size_t o = ((size_t)bh * n + j) * d;
                attention_prefix_row(&h, &px, i, outp + o);
            }
        }
        prefix_ops_free(&px);
        head_ops_free(&h);
    }
    free(perm);
    free(tbuf);
    return 0;
}

int or_attention_pfx(int B, int H, int F, int Hv, int Wv, int C, int d, const uint16_t *q,
                     const uint16_t *k, const uint16_t *v, int Lp, const uint16_t *qp,
                     const uint16_t *kp, const uint16_t *vp, const int32_t *valid, int pt,
                     const uint8_t *tier, int nqb, const int32_t *qblocks, int nprow,
                     const int32_t *prows, double *out, double *outp, double *amb)
{
    return pfx_common(B, H, F, Hv, Wv, C, d, q, k, v, Lp, qp, kp, vp, valid, pt, tier, nqb, qblocks,
                      nprow, prows, out, outp, amb);
}

/* ------------------------------------------------------------------ */
/* O12 dense reference: softmax(Q K^T / sqrt d) V in fp64 over all N    */
/* keys, two passes (max, then exp and sums), for chosen original-order */
/* query rows.  out: [B,H,nrows,d].                                     */
/* ------------------------------------------------------------------ */
int or_dense(int B, int H, int N, int d, const uint16_t *q, const uint16_t *k,
             const uint16_t *v, int nrows, const int32_t *rows, double *out)
{
    double inv_sqrt_d = 1.0 / sqrt((double)d);
    for (int bh = 0; bh < B * H; bh++) {
        size_t off = (size_t)bh * N * d;
        double *kf = malloc(sizeof(double) * (size_t)N * d), *vf = malloc(sizeof(double) * (size_t)N * d);
        for (size_t i = 0; i < (size_t)N * d; i++) {
            kf[i] = bf16f(k[off + i]);
            vf[i] = bf16f(v[off + i]);
        }
#pragma omp parallel for schedule(dynamic, 4)
        for (int r = 0; r < nrows; r++) {
            double *qu = malloc(sizeof(double) * d), *s = malloc(sizeof(double) * N);
            for (int c = 0; c < d; c++)
                qu[c] = bf16f(q[off + (size_t)rows[r] * d + c]);
            double m = -INFINITY;
            for (int n = 0; n < N; n++) {
                double dot = 0.0;
                for (int c = 0; c < d; c++)
                    dot += qu[c] * kf[(size_t)n * d + c];
                s[n] = dot * inv_sqrt_d;
                if (s[n] > m) m = s[n];
            }
            double Z = 0.0;
            double *o = out + ((size_t)bh * nrows + r) * d;
            for (int c = 0; c < d; c++) o[c] = 0.0;
            for (int n = 0; n < N; n++) {
                double w = exp(s[n] - m);
                Z += w;
                for (int c = 0; c < d; c++)
                    o[c] += w * vf[(size_t)n * d + c];
            }
            for (int c = 0; c < d; c++) o[c] /= Z;
            free(qu);
            free(s);
        }
        free(kf);
        free(vf);
    }
    return 0;
}
