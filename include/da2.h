/*
 * da2.h -- C ABI of libda2: the DraftAttention2 hot path on MI355X (gfx950).
 *
 * The operation (DraftAttention2: Fast Video Diffusion with Low-Resolution-
 * Guided Mixed-Precision Attention, Sec. 3.1 and App. C.1): for every head,
 * pool Q and K over the spatial regions of each latent frame (Eq. 1), build
 * the mixed average/max draft attention map over region pairs (Eq. 2), rank
 * all R^2 region pairs of the head, and give the top T16 pairs the 16-bit
 * tier (bf16 operands, unquantized weights), the next T8 the 8-bit tier (INT8
 * Q K^T, FP8 E4M3 weights and values), the next T4 the 4-bit tier (MXFP4
 * E2M1 with E8M0 scales per 32 values) and skip the
 * rest (or replace them by block means).  Attention (Sec. 3.3 "phased
 * execution", "cross-precision accumulation"; App. B.3/B.4) then evaluates
 * every kept 64x64 tile at full resolution with its tier's precision, phase
 * by phase in descending precision, sharing one online softmax and one
 * output accumulator, and writes the output in the original token order
 * ("DraftAttention: Fast Video Diffusion via Low-Resolution Attention
 * Guidance", abstract).  Text-prefix tokens of joint text-video attention
 * (App. C.1) are handled by da2_attention_prefixed.
 *
 * Conventions
 *   - Tokens of one (batch, head) are N = frames*height*width latent
 *     positions in (frame, y, x) raster order.  Each frame is partitioned
 *     into R_f = ceil(height*width/C) connected regions of balanced token
 *     counts (Sec. 3.3 ragged 2D partition, App. C.2), C the block
 *     capacity (64, or 128 as in the paper's operator study), the same for
 *     every frame; R = frames*R_f regions, numbered frame-major.  When C is
 *     64 and height and width are multiples of 8 the regions are the 8x8
 *     cells in raster order.  Inside a region its tokens take slots
 *     0..n_a-1 in raster order, and slots n_a..C-1 are padding (App. C.1:
 *     n_a excludes padding); every 64 slots of a region must hold at least
 *     48 tokens.  da2_layout_regions and da2_layout_slots describe the
 *     partition.  Pooling, the draft map and the ranking work on regions;
 *     attention works on tiles of 64 slots (a region of capacity 128 is two
 *     tiles), every tile of a region pair taking the pair's tier, and the
 *     INT8 steps of Q and K are per 64-slot tile.
 *   - Q, K, V are bfloat16 device arrays addressed as
 *     base + b*stride_b + h*stride_h + n*stride_n + c (element units, the
 *     channel index c is contiguous).  head_dim is 64 or 128.  Base pointers
 *     and strides must keep every token row 16-byte aligned.
 *   - The output O uses the same element strides in its own element type
 *     (fp32 or bf16).
 *   - Tier maps are uint8 [B, H, R, R] (query region a, key region b) with
 *     values 16 (16-bit: bf16 operands), 8 (8-bit), 4 (MXFP4), 1 (block mean)
 *     or 0 (skip); block-mean tiles need C = 64 (at C = 128 a 1 counts as
 *     an unknown value, which is a skip).  A block-mean tile ("Triage: Skip, Skim, or Refine
 *     Attention Tiles in Video Diffusion Transformers", abstract: a skipped
 *     tile replaced by its block means) scores all its query-key pairs with
 *     the mean of its scores, q_a . k_b / sqrt(d) over the valid-token means
 *     (the average-branch draft logit of Eq. 2), and counts the key region's
 *     n_b tokens with their mean value; it costs no tile product.
 *   - All calls are asynchronous on the given HIP stream.  Nothing is
 *     synchronised except where stated.  Device buffers (inputs, outputs,
 *     the workspace) belong to the caller; the library allocates only the
 *     small host objects da2_layout_t and da2_plan_t.
 *   - Errors are returned as da2_status.  Argument and shape checks happen
 *     before any launch, so a failed call writes nothing.  DA2_ERR_HIP
 *     reports a launch failure (the HIP error is left in the runtime).
 */
#ifndef DA2_H
#define DA2_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DA2_OK = 0,
    DA2_ERR_INVALID_ARG = 1,       /* null pointer, bad budget, bad dtype, misalignment */
    DA2_ERR_UNSUPPORTED_SHAPE = 2, /* head_dim not 64/128, no partition of the frame, too large */
    DA2_ERR_WORKSPACE = 3,         /* workspace smaller than da2_workspace_bytes() */
    DA2_ERR_PLAN_MISMATCH = 4,     /* q/k pointers differ from the ones the plan was built on, or no plan */
    DA2_ERR_HIP = 5                /* a kernel launch failed */
} da2_status;

typedef struct {
    int32_t batch, heads, head_dim;  /* B, H, d */
    int32_t frames, height, width;   /* F, H_v, W_v of the latent video */
    int64_t stride_b, stride_h, stride_n; /* element strides of Q/K/V/O */
    int32_t prefix;                  /* Lp: text-prefix tokens per sequence (0: none;
                                        at most 4096), see da2_attention_prefixed */
    int32_t capacity;                /* C: tokens per region, 64 or 128 (0 means 64) */
} da2_shape;

typedef struct {
    int32_t hi_bp;   /* share of region pairs in the 8-bit tier, basis points of n */
    int32_t lo_bp;   /* share in the MXFP4 tier */
    double lambda;   /* weight of the max-pooled branch of the draft map, in [0, 1] */
    int32_t scope;   /* 0: one ranking per head over n = R*R pairs (the paper's);
                        1: one ranking per query region over n = R pairs */
    int32_t full_bp; /* share in the 16-bit tier (bf16 operands, the paper's 16-bit
                        path); full_bp + hi_bp + lo_bp <= 10000 */
    int32_t skip_means; /* 0: pairs outside the quotas are skipped; 1: they become
                           block-mean tiles (tier 1, see below; C = 64 only,
                           DA2_ERR_INVALID_ARG otherwise) */
} da2_budget;

typedef struct da2_layout_s da2_layout_t;
typedef struct da2_plan_s da2_plan_t;

/* Region layout of one problem shape (App. C.2: the partition is built once
 * and reused across layers and denoising steps).  Host only, no GPU work. */
da2_status da2_layout_create(const da2_shape *shape, da2_layout_t **out);
void da2_layout_destroy(da2_layout_t *layout);

/* Regions of the layout: returns R = frames*R_f (0 for NULL) and writes R_f
 * to *regions_per_frame when it is not NULL.  Host only. */
int32_t da2_layout_regions(const da2_layout_t *layout, int32_t *regions_per_frame);

/* The partition of one frame (host destination, int32 [R_f*C]): for slot i
 * of region r, the token y*width + x it holds, or -1 for a padding slot.
 * Region r of frame f is region f*R_f + r of the tier map.  Host only. */
da2_status da2_layout_slots(const da2_layout_t *layout, int32_t *dst);

/* Bytes of device workspace a plan on this layout needs (256-byte aligned
 * base required).  Holds packed operands, draft state, tier map, schedule. */
size_t da2_workspace_bytes(const da2_layout_t *layout);

/* Bind a caller-owned device workspace to a new plan object (host only). */
da2_status da2_plan_create(const da2_layout_t *layout, void *workspace, size_t workspace_bytes,
                           da2_plan_t **out);
void da2_plan_destroy(da2_plan_t *plan);

/* da2_plan: draft-guided tier planning (Sec. 3.1, App. C.1) plus the fused
 * Q/K operand preparation (Sec. 3.3): reorder, pool, quantize Q and K to INT8
 * (App. B.2's uniform quantizer: one fp32 step amax/127 per 64-token block,
 * codes the nearest integers, ties to even) and MXFP4, score the draft map, rank
 * and assign tiers, and build the per-query-region schedule.  Quotas per
 * ranking, cumulative and each rounded half up: T16 = full_bp*n/10^4, T16 +
 * T8 = (full_bp + hi_bp)*n/10^4, T16 + T8 + T4 = (full_bp + hi_bp +
 * lo_bp)*n/10^4.  The T16 highest-scoring pairs get the 16-bit tier, the next
 * T8 the 8-bit tier, the next T4 MXFP4 (Sec. 3.1: larger draft mass, higher precision);
 * ties between equal scores go to the smaller pair index a*R+b.  q and k must
 * stay unchanged until da2_attention on this plan has run (stream order). */
da2_status da2_plan(da2_plan_t *plan, const void *q, const void *k, const da2_budget *budget,
                    hipStream_t stream);

/* Same as da2_plan but with a caller-supplied tier map (device, [B,H,R,R],
 * values in {0,1,4,8,16}; other values are treated as skip).  The draft map
 * and ranking are not run; the draft logits are (block-mean tiles use them). */
da2_status da2_plan_from_tier_map(da2_plan_t *plan, const void *q, const void *k,
                                  const uint8_t *tier_map, hipStream_t stream);

/* Copy the plan's tier map to dst (device, [B,H,R,R] uint8). */
da2_status da2_plan_tier_map(const da2_plan_t *plan, uint8_t *dst, hipStream_t stream);

/* da2_attention: V preparation (FP8 with one fp32 scale per channel over all
 * tokens; MXFP4 along keys in groups of 32 inside each region) and the
 * phased mixed-precision attention over the plan's kept tiles (16-bit phase,
 * then 8-bit, then MXFP4; Sec. 3.3), then the block-mean tiles, written to o in
 * the original token order.
 * out_dtype: 0 = bf16, 1 = fp32.  q and k must be the pointers the plan was
 * built on (DA2_ERR_PLAN_MISMATCH otherwise).  Rows whose query region keeps
 * no tile are written as zero (App. C.1).  The video tokens only: a text
 * prefix in the shape is ignored here (see da2_attention_prefixed). */
da2_status da2_attention(da2_plan_t *plan, const void *q, const void *k, const void *v, void *o,
                         int32_t out_dtype, hipStream_t stream);

/* da2_attention_prefixed: da2_attention for joint text-video attention
 * (DraftAttention2 App. C.1: prefix interactions lie outside the region
 * budget; video queries keep every valid prefix key, prefix queries use
 * non-sparse attention).  Besides the video tensors q, k, v, o of
 * da2_attention, the shape's Lp = prefix text tokens have their own bf16
 * tensors qp, kp, vp and output op, [B,H,Lp,d] addressed with the same
 * strides (for one joint tensor with the prefix first: qp = q_joint and
 * q = q_joint + Lp*stride_n).  prefix_valid: device int32 [B], the number
 * of valid prefix keys of each batch element (the first ones; values are
 * clamped to [0, Lp]), or NULL for all Lp.  Prefix keys past the valid count
 * are never read for the result (padding).
 *   Video query rows: the plan's phases preceded by one segment over the
 *   valid prefix keys in tiles of 64 (16-bit path: bf16 operands, weights
 *   unquantized); a row whose region keeps no video tile still attends
 *   to the prefix, and is zero only when there is no valid prefix key.
 *   Prefix query rows: every valid prefix key, then every video region in
 *   order, all on the 16-bit path, in chunks of 128 tiles (8192 keys), each
 *   an online softmax of its own, merged by the exact rescale of the shared
 *   normalization (App. B.4); all Lp rows are written.
 * With prefix == 0 in the shape this is da2_attention (qp, kp, vp, op,
 * prefix_valid are not used).  Otherwise qp, kp, vp and op must be non-null
 * and 16-byte aligned (DA2_ERR_INVALID_ARG). */
da2_status da2_attention_prefixed(da2_plan_t *plan, const void *q, const void *k, const void *v,
                                  void *o, const void *qp, const void *kp, const void *vp, void *op,
                                  const int32_t *prefix_valid, int32_t out_dtype,
                                  hipStream_t stream);

/* Debug exports in canonical layouts, for tests (device destination):
 *   (Np = C R reordered positions, region by region, padding slots included;
 *   T = Np / 64 tiles of 64 positions; T = R at C = 64)
 *   DA2_DBG_Q_I8 / K_I8             : INT8 codes (two's complement bytes) [B,H,Np,d]
 *   DA2_DBG_Q_I8_SCALE / K_...      : fp32 steps [B,H,T]
 *   DA2_DBG_V_FP8 / V_FP8_SCALE     : E4M3 codes [B,H,Np,d];  fp32 [B,H,d]
 *   DA2_DBG_Q_MX / K_MX / V_MX      : uint8 E2M1 codes [B,H,Np,d] (one per byte)
 *   DA2_DBG_Q_MX_SCALE / K_...      : uint8 E8M0 [B,H,Np,d/32];  V: [B,H,T,2,d]
 *   DA2_DBG_Q_AVG / K_AVG           : fp64 [B,H,R,d];  Q_MAX / K_MAX: fp32 [B,H,R,d]
 *   DA2_DBG_KEYS                    : uint32 [B,H,R,R] (bits of fp32 draft score)
 *   DA2_DBG_SCHEDULE                : int32 [B,H,T,3+T]: per query tile the tile
 *                                     counts n16, n8, n4, then the 16-bit key
 *                                     tiles ascending, then 8-bit ascending,
 *                                     then MXFP4 ascending, then -1
 * V entries are valid after da2_attention. */
enum {
    DA2_DBG_Q_I8 = 0, DA2_DBG_Q_I8_SCALE, DA2_DBG_Q_MX, DA2_DBG_Q_MX_SCALE,
    DA2_DBG_K_I8, DA2_DBG_K_I8_SCALE, DA2_DBG_K_MX, DA2_DBG_K_MX_SCALE,
    DA2_DBG_V_FP8, DA2_DBG_V_FP8_SCALE, DA2_DBG_V_MX, DA2_DBG_V_MX_SCALE,
    DA2_DBG_Q_AVG, DA2_DBG_K_AVG, DA2_DBG_Q_MAX, DA2_DBG_K_MAX,
    DA2_DBG_KEYS, DA2_DBG_SCHEDULE, DA2_DBG_COUNT
};
da2_status da2_plan_debug(const da2_plan_t *plan, int32_t which, void *dst, hipStream_t stream);

/* Bytes written by da2_plan_debug for `which` (0 for unknown values). */
size_t da2_plan_debug_bytes(const da2_layout_t *layout, int32_t which);

/* Kernel timing of the attention kernel itself (measurement aid).
 * da2_plan_timing(plan, 1) starts recording a pair of HIP events around the
 * attention kernel (k_attn alone: not the value preparation, the block-mean
 * gather or the prefix query rows) of every later da2_attention or
 * da2_attention_prefixed call on this plan (up to
 * 4096 calls; older pairs are kept, further calls are not recorded);
 * da2_plan_timing(plan, 0) stops and discards them.  da2_plan_timing_read
 * waits for the recorded events and writes up to `max` per-call durations in
 * milliseconds to `ms` (host memory), the count to *n. */
da2_status da2_plan_timing(da2_plan_t *plan, int32_t enable);
da2_status da2_plan_timing_read(da2_plan_t *plan, float *ms, int32_t max, int32_t *n);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * da2_plan followed by da2_attention in one call, on a workspace inside the
 * library instead of a caller's -- a static device array of
 * DA2_NOALLOC_BYTES on every GPU the library runs on, held until the process
 * ends.  The caller passes the layout, Q, K, V, the budget and the output as
 * for da2_plan and da2_attention (same rules, same result); the layout must
 * stay alive until the call's work on the stream has completed (its host
 * tables are copied asynchronously).  Returns DA2_ERR_WORKSPACE, before any
 * GPU work, when da2_workspace_bytes(layout) exceeds DA2_NOALLOC_BYTES, and
 * DA2_ERR_HIP when the array's device address cannot be obtained.  The call
 * allocates nothing: no hipMalloc or hipFree, no host heap.  Every call on
 * one GPU shares that GPU's array, which keeps the last call's contents
 * (every byte a call reads it first writes on the same stream): calls that
 * overlap on one GPU -- on different streams or from different threads --
 * race. */
#define DA2_NOALLOC_BYTES ((size_t)32 << 20)
da2_status da2_forward_noalloc(const da2_layout_t *layout, const void *q, const void *k, const void *v,
                               void *o, const da2_budget *budget, int32_t out_dtype, hipStream_t stream);

/* Host-side helpers (no GPU work). */
const char *da2_status_string(da2_status status);
/* Constants of the fp64 exp used by the draft softmax: ln2 head, ln2 tail,
 * 1/ln2, then the 14 Taylor coefficients 1/j!, j = 0..13 (17 doubles). */
void da2_exp_constants(double *out17);
/* The cumulative quotas the ranking uses for n pairs: t16 = T16, t8 = T16 +
 * T8, tk = T16 + T8 + T4. */
void da2_quotas(int64_t n, int32_t full_bp, int32_t hi_bp, int32_t lo_bp, int64_t *t16,
                int64_t *t8, int64_t *tk);

#ifdef __cplusplus
}
#endif
#endif /* DA2_H */
