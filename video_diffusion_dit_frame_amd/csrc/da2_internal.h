// da2_internal.h -- private types, workspace layout and device helpers of
// libda2 (gfx950).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "da2.h"

namespace da2 {

constexpr int kBlk = 64;          // slots per tile (a region at capacity 64: one 8x8 cell)
constexpr int kMaxRegions = 8192; // tile limit (keeps R*R in 32 bits, row scope in LDS)
constexpr int kMaxTimed = 4096;   // attention calls recorded while timing
constexpr int kTargets = 3;       // ranking thresholds: T16, T16+T8, T16+T8+T4
constexpr int kPrefixChunkTiles = 128; // tiles per chunk of a prefix query row
constexpr int kMaxPrefix = 4096;  // text-prefix tokens per sequence
constexpr int kMinFill = 48;      // fewest valid tokens of a tile (at most 16 padding slots)
constexpr uint8_t kMeanTier = 1;  // tier of a block-mean tile (skip replaced by block means)

// ---------------------------------------------------------------------------
// Workspace: one region of caller memory carved into these buffers.
// Packed operand layouts (per (b,h) slice "bh", per tile a of 64 slots):
//   Q int8 : [bh][a][w=2][kc=d/64][lane=64][32 B]   B operand of S^T = K Q^T:
//            lane l holds row 32 w + l % 32, channels 64 kc + 32 (l / 32) .. +31
//   K int8 : [bh][a][m=2][kc][lane][32 B]           A operand, key rows permuted
//            (lane l: slot key_of_row(l % 32, m), the same channels)
//   *_mx   : same chunking, 16 B of E2M1 pairs per lane, one E8M0 byte per lane
//   V fp8  : [bh][a][cb=d/32][lane][32 B]           A operand of O^T = V^T P^T
//   V mx   : [bh][a][cb][lane][16 B] + E8M0 byte per lane
//   V bf16 : [bh][a][cb][t=4][lane][16 B]           A operand of the 16-bit
//            product: lane l holds channel 32cb + l%32, keys 32(l/32) + 8t .. +7
//   prefix V bf16 : [bh][tile][cb][t][lane][16 B]   the same for the text
//            prefix, tile t holding prefix keys 64t .. 64t+63 (zero past the
//            valid ones)
//   K bf16 (ragged layouts) : [bh][a][m=2][s=d/16][lane][16 B]   the key
//            image of the 16-bit products: chunk (m, s) holds for lane l key
//            slot key_of_row(l%32, m), channels 16s + 8(l/32) .. +7
//   V fp8 values : the layout of V bf16, holding the value of every FP8
//            value code (unscaled) as bf16 (exact: E4M3 has 4 significant
//            bits); the value operand of the 8-bit tier's P^T V
//   frame slot table (ragged layouts) : int32 [Rf tiles][64], token
//            y*W_v + x of each slot of the frame's regions, -1 for padding;
//            int32 [R] valid tokens of every tile
//   pooled descriptors, draft logits, keys and the tier map are per region
//            ([bh][Rg][d], [bh][Rg][Rg]); the schedule, its counts and the
//            work order per tile ([bh][R][R], [bh][R][3], [bh][R])
//   prefix partials : fp32 [bh][chunk][row][d] unnormalised outputs and
//            float2 [bh][chunk][row] (running max, sum) of the prefix query
//            rows' chunks, rows padded to ptiles*64
// ---------------------------------------------------------------------------
struct Workspace {
    size_t q8, q4, q4s, qs8;
    size_t k8, k4, k4s, ks8;
    size_t v8, v4, v4s, vs8, vamax, v16, vp16, pacc, pmz;
    size_t k16;          // bf16 key image of ragged layouts (16-bit path)
    size_t v8b;          // bf16 image of the FP8 value codes (8-bit tier P^T V)
    size_t vavg, magg, cagg;  // block-mean tiles: region mean values; per query region the
                              // gathered term (max logit, weight) and its value sum
    size_t ftok, nreg;   // ragged layouts: frame slot table, valid tokens per tile
    size_t qavg, kavg, qmax, kmax;
    size_t la, lm, rmax, zsum, keys, tier;
    size_t sched, cnt;
    size_t qord;         // attention work order: query region of each workgroup slot
    size_t rank_state, rank_hist, rank_eq;
    size_t total;
};

struct RankState {      // one per (segment, target)
    uint32_t prefix;    // selected key bits so far
    uint32_t mask;      // which bits of prefix are fixed
    uint32_t rank;      // 0-based rank still to find inside the prefix class
    uint32_t active;    // 0 when the quota is zero
};

}  // namespace da2

// Regions and tiles.  A region of capacity C holds C slots, tpr = C / 64
// tiles of 64.  Everything the attention side touches (operands, schedule,
// work order, slot tables) is per tile: R tiles, Rf per frame, and the tile
// is what the kernels call a region.  The plan side (pooled descriptors,
// draft logits and keys, ranking, tier map) is per region: Rg regions, Rfg
// per frame.  At C = 64 the two coincide.
struct da2_layout_s {
    da2_shape s;
    int N, R, Ry, Rx, BH, d;
    int Np;                   // reordered positions R*64 (padding slots included)
    int Rf;                   // tiles per frame
    int C, tpr;               // block capacity and tiles per region
    int Rg, Rfg;              // regions, regions per frame
    int ragged;               // 0: the 8x8 grid (closed form); 1: slot table
    int pmax;                 // most padding slots of any tile (0..16)
    int32_t *ftok;            // ragged: frame slot table [Rf*64] (host, owned)
    int32_t *nreg;            // ragged: valid tokens of every tile [R] (host, owned by
                              // the layout; a plan's copy of the layout does not use it)
    int64_t nchunk;           // rank chunks per head (head scope)
    int ptiles;               // 64-key tiles of the text prefix (ceil(prefix / 64))
    int pchunks;              // chunks of a prefix query row's key sequence (0: no prefix)
    da2::Workspace ws;
};

struct da2_plan_s {
    da2_layout_s L;           // its ftok is the plan's own copy
    int tables_ready;         // frame slot table uploaded to the workspace
    int32_t *nreg;            // ragged: valid tokens of every tile [R] (host)
    char *ws;
    size_t ws_bytes;
    const void *q, *k;        // inputs the plan was built on
    int ready;                // operands + schedule present
    int has_keys;             // draft keys present (da2_plan, not from tier map)
    int has16;                // the tier map may hold 16-bit tiles
    int has_mean;             // the tier map may hold block-mean tiles
    int timing;               // record events around the attention kernel
    int nev;                  // recorded event pairs
    hipEvent_t *ev;           // [2 * kMaxTimed] when timing is on
};

namespace da2 {

// Text-prefix inputs of one attention call (App. C.1).
struct PrefixIo {
    const void *qp, *kp, *vp;  // [B,H,Lp,d] bf16, the video strides
    void *op;                  // prefix query rows of the output
    const int32_t *valid;      // [B] valid prefix keys (device), or null
};

// ---------------------------------------------------------------------------
// Launchers (defined in the kernel translation units).
// ---------------------------------------------------------------------------
void launch_prep_qk(const da2_layout_s &L, const void *x, int is_key, char *ws, hipStream_t st);
// Spatial partition of one Hv x Wv frame into regions of capacity C
// (defined in da2_partition.cpp): fills tok [Rf*C] (y*Wv + x or -1) and
// returns Rf, or -1 without one.
int partition_frame(int Hv, int Wv, int C, int32_t *tok);
void launch_prep_v(const da2_layout_s &L, const void *v, int with16, int with_mean, char *ws, hipStream_t st);
void launch_prep_vp(const da2_layout_s &L, const PrefixIo &px, char *ws, hipStream_t st);
void launch_draft(const da2_layout_s &L, double lambda, char *ws, hipStream_t st);
void launch_draft_logits(const da2_layout_s &L, char *ws, hipStream_t st);
void launch_skip_means(const da2_layout_s &L, char *ws, hipStream_t st);
void launch_rank(const da2_layout_s &L, int scope, int64_t t16, int64_t t8c, int64_t tk, char *ws,
                 hipStream_t st);
void launch_schedule(const da2_layout_s &L, char *ws, hipStream_t st);
// ev: null, or two events recorded right before and right after the k_attn launch
void launch_attention(const da2_layout_s &L, char *ws, const void *q, const void *k, void *o,
                      int out_f32, const PrefixIo *px, int has_mean, hipEvent_t *ev, hipStream_t st);
void launch_debug(const da2_layout_s &L, int which, const char *ws, void *dst, hipStream_t st);
void launch_import_tier(const da2_layout_s &L, const uint8_t *src, char *ws, hipStream_t st);

}  // namespace da2
