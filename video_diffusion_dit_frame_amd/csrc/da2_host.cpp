// da2_host.cpp -- the C ABI of libda2: validation, workspace carving and the
// launch sequence of the hot path (plan: prep Q/K -> draft -> rank ->
// schedule; attention: prep V -> phased attention with fused restore).
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "da2_internal.h"
#include "da2_device.h"

using namespace da2;

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

da2_status check_shape(const da2_shape *s)
{
    if (!s)
        return DA2_ERR_INVALID_ARG;
    if (s->batch < 1 || s->heads < 1 || s->frames < 1 || s->height < 1 || s->width < 1)
        return DA2_ERR_UNSUPPORTED_SHAPE;
    if (s->head_dim != 64 && s->head_dim != 128)
        return DA2_ERR_UNSUPPORTED_SHAPE;
    if (s->capacity != 0 && s->capacity != 64 && s->capacity != 128)
        return DA2_ERR_UNSUPPORTED_SHAPE;
    if ((int64_t)s->height * s->width > 4096 * kBlk)
        return DA2_ERR_UNSUPPORTED_SHAPE;
    const int64_t C = s->capacity ? s->capacity : kBlk;
    const int64_t tiles = ((int64_t)s->height * s->width + C - 1) / C * (C / kBlk);
    if ((int64_t)s->frames * tiles > kMaxRegions || (int64_t)s->batch * s->heads > 65535)
        return DA2_ERR_UNSUPPORTED_SHAPE;
    if (s->stride_n < s->head_dim || s->stride_b < 0 || s->stride_h < 0)
        return DA2_ERR_INVALID_ARG;
    if (s->stride_n % 8 || s->stride_h % 8 || s->stride_b % 8)
        return DA2_ERR_INVALID_ARG;
    // the 16-bit phase addresses one region's key rows (8 image rows) with
    // 32-bit byte offsets from the region's first token
    if ((((int64_t)7 * s->width + 7) * s->stride_n + s->head_dim) * 2 > INT32_MAX)
        return DA2_ERR_UNSUPPORTED_SHAPE;
    // the prefix rows of one head are addressed the same way from its first
    if (s->prefix < 0 || s->prefix > kMaxPrefix)
        return DA2_ERR_UNSUPPORTED_SHAPE;
    if (s->prefix > 0 && ((int64_t)(s->prefix - 1) * s->stride_n + s->head_dim) * 2 > INT32_MAX)
        return DA2_ERR_UNSUPPORTED_SHAPE;
    return DA2_OK;
}

void carve(da2_layout_s &L)
{
    // operand arrays hold every reordered position (padding slots included);
    // R counts tiles, G regions (the plan's pieces)
    const size_t BH = L.BH, N = L.Np, R = L.R, G = L.Rg, d = L.d;
    Workspace &W = L.ws;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    W.q8 = take(BH * N * d);
    W.q4 = take(BH * N * d / 2);
    W.q4s = take(BH * N * d / 32);
    W.qs8 = take(BH * R * 4);
    W.k8 = take(BH * N * d);
    W.k4 = take(BH * N * d / 2);
    W.k4s = take(BH * N * d / 32);
    W.ks8 = take(BH * R * 4);
    W.v8 = take(BH * N * d);
    W.v4 = take(BH * N * d / 2);
    W.v4s = take(BH * N * d / 32);
    W.vs8 = take(BH * d * 4);
    W.v16 = take(BH * N * d * 2);
    W.vp16 = take(BH * (size_t)L.ptiles * kBlk * d * 2);
    W.pacc = take(BH * (size_t)L.pchunks * L.ptiles * kBlk * d * 4);
    W.pmz = take(BH * (size_t)L.pchunks * L.ptiles * kBlk * 8);
    W.k16 = take(L.ragged ? BH * N * d * 2 : 0);
    W.v8b = take(BH * N * d * 2);
    W.vavg = take(BH * R * d * 4);
    W.magg = take(BH * R * 8);
    W.cagg = take(BH * R * d * 4);
    W.ftok = take(L.ragged ? (size_t)L.Rf * kBlk * 4 : 0);
    W.nreg = take(L.ragged ? R * 4 : 0);
    W.vamax = take(BH * d * 4);
    W.qavg = take(BH * G * d * 8);
    W.kavg = take(BH * G * d * 8);
    W.qmax = take(BH * G * d * 4);
    W.kmax = take(BH * G * d * 4);
    W.la = take(BH * G * G * 8);
    W.lm = take(BH * G * G * 8);
    W.rmax = take(BH * 2 * G * 8);
    W.zsum = take(BH * 2 * G * 8);
    W.keys = take(BH * G * G * 4);
    W.tier = take(BH * G * G);
    W.sched = take(BH * R * R * 4);
    W.cnt = take(BH * R * kTargets * 4);
    W.qord = take(BH * (R + 8) * 4);   // 8 shares of ceil(units / 8) slots per head
    W.rank_state = take(BH * kTargets * sizeof(RankState));
    W.rank_hist = take(BH * kTargets * 256 * 4);
    W.rank_eq = take(BH * (size_t)L.nchunk * kTargets * 4);
    W.total = off;
}

da2_status launched()
{
    return hipGetLastError() == hipSuccess ? DA2_OK : DA2_ERR_HIP;
}

// Ragged layouts: the frame slot table and the valid-token count of every
// region go to the workspace once per plan (the plan keeps the host copies
// alive, so the asynchronous copies may complete later).
da2_status upload_tables(da2_plan_s *P, hipStream_t stream)
{
    const da2_layout_s &L = P->L;
    if (!L.ragged || P->tables_ready)
        return DA2_OK;
    if (!P->nreg) {
        P->nreg = (int32_t *)malloc(sizeof(int32_t) * L.R);
        if (!P->nreg)
            return DA2_ERR_INVALID_ARG;
        for (int a = 0; a < L.R; a++) {
            const int32_t *t = L.ftok + (a % L.Rf) * kBlk;
            int n = 0;
            while (n < kBlk && t[n] >= 0)
                n++;
            P->nreg[a] = n;
        }
    }
    if (hipMemcpyAsync(P->ws + L.ws.ftok, L.ftok, sizeof(int32_t) * L.Rf * kBlk, hipMemcpyHostToDevice,
                       stream) != hipSuccess ||
        hipMemcpyAsync(P->ws + L.ws.nreg, P->nreg, sizeof(int32_t) * L.R, hipMemcpyHostToDevice, stream) !=
            hipSuccess)
        return DA2_ERR_HIP;
    P->tables_ready = 1;
    return DA2_OK;
}

}  // namespace

extern "C" {

const char *da2_status_string(da2_status s)
{
    switch (s) {
    case DA2_OK: return "ok";
    case DA2_ERR_INVALID_ARG: return "invalid argument";
    case DA2_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case DA2_ERR_WORKSPACE: return "workspace too small or misaligned";
    case DA2_ERR_PLAN_MISMATCH: return "plan does not match these inputs";
    case DA2_ERR_HIP: return "HIP launch failure";
    }
    return "unknown status";
}

da2_status da2_layout_create(const da2_shape *shape, da2_layout_t **out)
{
    if (!out)
        return DA2_ERR_INVALID_ARG;
    da2_status st = check_shape(shape);
    if (st != DA2_OK)
        return st;
    da2_layout_s *L = (da2_layout_s *)calloc(1, sizeof(da2_layout_s));
    if (!L)
        return DA2_ERR_INVALID_ARG;
    L->s = *shape;
    L->C = shape->capacity ? shape->capacity : kBlk;
    L->tpr = L->C / kBlk;
    L->N = shape->frames * shape->height * shape->width;
    L->Ry = shape->height / 8;
    L->Rx = shape->width / 8;
    if (L->C == kBlk && shape->height % 8 == 0 && shape->width % 8 == 0) {
        // the 8x8 grid: slots follow from a closed form
        L->Rf = L->Ry * L->Rx;
        L->Rfg = L->Rf;
    } else {
        // a slot table: region r's C slots are tiles r*tpr .. r*tpr + tpr - 1
        const int Rfg = (shape->height * shape->width + L->C - 1) / L->C;
        L->ftok = (int32_t *)malloc(sizeof(int32_t) * Rfg * L->C);
        if (!L->ftok || partition_frame(shape->height, shape->width, L->C, L->ftok) != Rfg) {
            free(L->ftok);
            free(L);
            return DA2_ERR_UNSUPPORTED_SHAPE;
        }
        L->Rfg = Rfg;
        L->Rf = Rfg * L->tpr;
        L->ragged = 1;
        for (int r = 0; r < L->Rf; r++) {   // padding of every tile
            int n = 0;
            while (n < kBlk && L->ftok[r * kBlk + n] >= 0)
                n++;
            L->pmax = L->pmax > kBlk - n ? L->pmax : kBlk - n;
        }
    }
    L->R = shape->frames * L->Rf;
    L->Rg = shape->frames * L->Rfg;
    if (L->ragged) {
        L->nreg = (int32_t *)malloc(sizeof(int32_t) * L->R);
        if (!L->nreg) {
            free(L->ftok);
            free(L);
            return DA2_ERR_INVALID_ARG;
        }
        for (int a = 0; a < L->R; a++) {
            const int32_t *t = L->ftok + (a % L->Rf) * kBlk;
            int n = 0;
            while (n < kBlk && t[n] >= 0)
                n++;
            L->nreg[a] = n;
        }
    }
    L->Np = L->R * kBlk;
    L->BH = shape->batch * shape->heads;
    L->d = shape->head_dim;
    L->nchunk = ((int64_t)L->Rg * L->Rg + 4095) / 4096;
    L->ptiles = (shape->prefix + kBlk - 1) / kBlk;
    L->pchunks = L->ptiles ? (L->ptiles + L->R + kPrefixChunkTiles - 1) / kPrefixChunkTiles : 0;
    carve(*L);
    *out = L;
    return DA2_OK;
}

void da2_layout_destroy(da2_layout_t *layout)
{
    if (layout) {
        free(layout->ftok);
        free(layout->nreg);
    }
    free(layout);
}

size_t da2_workspace_bytes(const da2_layout_t *layout) { return layout ? layout->ws.total : 0; }

int32_t da2_layout_regions(const da2_layout_t *layout, int32_t *regions_per_frame)
{
    if (!layout)
        return 0;
    if (regions_per_frame)
        *regions_per_frame = layout->Rfg;
    return layout->Rg;
}

da2_status da2_layout_slots(const da2_layout_t *layout, int32_t *dst)
{
    if (!layout || !dst)
        return DA2_ERR_INVALID_ARG;
    const da2_layout_s &L = *layout;
    if (L.ragged) {
        memcpy(dst, L.ftok, sizeof(int32_t) * L.Rf * kBlk);
        return DA2_OK;
    }
    for (int r = 0; r < L.Rf; r++)
        for (int i = 0; i < kBlk; i++)
            dst[r * kBlk + i] = ((r / L.Rx) * 8 + i / 8) * L.s.width + (r % L.Rx) * 8 + i % 8;
    return DA2_OK;
}

da2_status da2_plan_create(const da2_layout_t *layout, void *workspace, size_t workspace_bytes,
                           da2_plan_t **out)
{
    if (!layout || !out)
        return DA2_ERR_INVALID_ARG;
    if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < layout->ws.total)
        return DA2_ERR_WORKSPACE;
    da2_plan_s *P = (da2_plan_s *)calloc(1, sizeof(da2_plan_s));
    if (!P)
        return DA2_ERR_INVALID_ARG;
    P->L = *layout;
    P->L.nreg = nullptr;   // the plan keeps its own count table (upload_tables)
    if (layout->ragged) {
        const size_t bytes = sizeof(int32_t) * layout->Rf * kBlk;
        P->L.ftok = (int32_t *)malloc(bytes);
        if (!P->L.ftok) {
            free(P);
            return DA2_ERR_INVALID_ARG;
        }
        memcpy(P->L.ftok, layout->ftok, bytes);
    }
    P->ws = (char *)workspace;
    P->ws_bytes = workspace_bytes;
    *out = P;
    return DA2_OK;
}

static void drop_events(da2_plan_s *P)
{
    if (P->ev) {
        for (int i = 0; i < 2 * kMaxTimed; i++)
            if (P->ev[i])
                hipEventDestroy(P->ev[i]);
        free(P->ev);
    }
    P->ev = nullptr;
    P->nev = 0;
    P->timing = 0;
}

void da2_plan_destroy(da2_plan_t *plan)
{
    if (!plan)
        return;
    drop_events(plan);
    free(plan->L.ftok);
    free(plan->nreg);
    free(plan);
}

da2_status da2_plan_timing(da2_plan_t *P, int32_t enable)
{
    if (!P)
        return DA2_ERR_INVALID_ARG;
    drop_events(P);
    if (!enable)
        return DA2_OK;
    P->ev = (hipEvent_t *)calloc(2 * kMaxTimed, sizeof(hipEvent_t));
    if (!P->ev)
        return DA2_ERR_INVALID_ARG;
    P->timing = 1;
    return DA2_OK;
}

da2_status da2_plan_timing_read(da2_plan_t *P, float *ms, int32_t max, int32_t *n)
{
    if (!P || !n || (max > 0 && !ms))
        return DA2_ERR_INVALID_ARG;
    int cnt = P->nev < max ? P->nev : max;
    for (int i = 0; i < cnt; i++) {
        if (hipEventSynchronize(P->ev[2 * i + 1]) != hipSuccess ||
            hipEventElapsedTime(&ms[i], P->ev[2 * i], P->ev[2 * i + 1]) != hipSuccess)
            return DA2_ERR_HIP;
    }
    *n = P->nev;
    return DA2_OK;
}

void da2_quotas(int64_t n, int32_t full_bp, int32_t hi_bp, int32_t lo_bp, int64_t *t16,
                int64_t *t8, int64_t *tk)
{
    *t16 = ((int64_t)full_bp * n + 5000) / 10000;
    *t8 = ((int64_t)(full_bp + hi_bp) * n + 5000) / 10000;
    *tk = ((int64_t)(full_bp + hi_bp + lo_bp) * n + 5000) / 10000;
}

da2_status da2_plan(da2_plan_t *P, const void *q, const void *k, const da2_budget *bud,
                    hipStream_t stream)
{
    if (!P || !q || !k || !bud)
        return DA2_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k))
        return DA2_ERR_INVALID_ARG;
    if (bud->hi_bp < 0 || bud->lo_bp < 0 || bud->full_bp < 0 ||
        (int64_t)bud->full_bp + bud->hi_bp + bud->lo_bp > 10000)
        return DA2_ERR_INVALID_ARG;
    if (!isfinite(bud->lambda) || bud->lambda < 0.0 || bud->lambda > 1.0)
        return DA2_ERR_INVALID_ARG;
    if (bud->scope != 0 && bud->scope != 1)
        return DA2_ERR_INVALID_ARG;
    if (bud->skip_means != 0 && bud->skip_means != 1)
        return DA2_ERR_INVALID_ARG;
    const da2_layout_s &L = P->L;
    if (bud->skip_means && L.tpr > 1)
        return DA2_ERR_INVALID_ARG;
    const int64_t n = bud->scope == 0 ? (int64_t)L.Rg * L.Rg : (int64_t)L.Rg;
    int64_t t16, t8, tk;
    da2_quotas(n, bud->full_bp, bud->hi_bp, bud->lo_bp, &t16, &t8, &tk);
    P->ready = 0;
    da2_status up = upload_tables(P, stream);
    if (up != DA2_OK)
        return up;
    launch_prep_qk(L, q, 0, P->ws, stream);
    launch_prep_qk(L, k, 1, P->ws, stream);
    launch_draft(L, bud->lambda, P->ws, stream);
    launch_rank(L, bud->scope, t16, t8, tk, P->ws, stream);
    if (bud->skip_means)
        launch_skip_means(L, P->ws, stream);
    launch_schedule(L, P->ws, stream);
    da2_status st = launched();
    if (st != DA2_OK)
        return st;
    P->q = q;
    P->k = k;
    P->ready = 1;
    P->has_keys = 1;
    P->has16 = t16 > 0;
    P->has_mean = bud->skip_means != 0;
    return DA2_OK;
}

da2_status da2_plan_from_tier_map(da2_plan_t *P, const void *q, const void *k,
                                  const uint8_t *tier_map, hipStream_t stream)
{
    if (!P || !q || !k || !tier_map)
        return DA2_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k))
        return DA2_ERR_INVALID_ARG;
    const da2_layout_s &L = P->L;
    P->ready = 0;
    da2_status up = upload_tables(P, stream);
    if (up != DA2_OK)
        return up;
    launch_prep_qk(L, q, 0, P->ws, stream);
    launch_prep_qk(L, k, 1, P->ws, stream);
    launch_import_tier(L, tier_map, P->ws, stream);
    launch_schedule(L, P->ws, stream);
    // the map may hold block-mean tiles (capacity 64 only): their scores are
    // the draft's average-branch logits
    if (L.tpr == 1)
        launch_draft_logits(L, P->ws, stream);
    da2_status st = launched();
    if (st != DA2_OK)
        return st;
    P->q = q;
    P->k = k;
    P->ready = 1;
    P->has_keys = 0;
    P->has16 = 1;  // the imported map may hold 16-bit tiles
    P->has_mean = L.tpr == 1;
    return DA2_OK;
}

da2_status da2_plan_tier_map(const da2_plan_t *P, uint8_t *dst, hipStream_t stream)
{
    if (!P || !dst)
        return DA2_ERR_INVALID_ARG;
    if (!P->ready)
        return DA2_ERR_PLAN_MISMATCH;
    const da2_layout_s &L = P->L;
    hipError_t e = hipMemcpyAsync(dst, P->ws + L.ws.tier, (size_t)L.BH * L.Rg * L.Rg,
                                  hipMemcpyDeviceToDevice, stream);
    return e == hipSuccess ? DA2_OK : DA2_ERR_HIP;
}

static da2_status attend(da2_plan_s *P, const void *q, const void *k, const void *v, void *o,
                         int32_t out_dtype, const PrefixIo *px, hipStream_t stream)
{
    if (!P || !q || !k || !v || !o)
        return DA2_ERR_INVALID_ARG;
    if (out_dtype != 0 && out_dtype != 1)
        return DA2_ERR_INVALID_ARG;
    if (!aligned16(v) || !aligned16(o))
        return DA2_ERR_INVALID_ARG;
    if (px && (!px->qp || !px->kp || !px->vp || !px->op || !aligned16(px->qp) ||
               !aligned16(px->kp) || !aligned16(px->vp) || !aligned16(px->op)))
        return DA2_ERR_INVALID_ARG;
    if (!P->ready || P->q != q || P->k != k)
        return DA2_ERR_PLAN_MISMATCH;
    const da2_layout_s &L = P->L;
    // prefix queries attend to every region on the 16-bit path
    launch_prep_v(L, v, P->has16 || px, P->has_mean, P->ws, stream);
    if (px)
        launch_prep_vp(L, *px, P->ws, stream);
    hipEvent_t *ev = nullptr;
    if (P->timing && P->nev < kMaxTimed) {
        ev = P->ev + 2 * P->nev;
        for (int i = 0; i < 2; i++)
            if (!ev[i] && hipEventCreate(&ev[i]) != hipSuccess)
                return DA2_ERR_HIP;
    }
    launch_attention(L, P->ws, q, k, o, out_dtype, px, P->has_mean, ev, stream);
    if (ev)
        P->nev++;
    return launched();
}

da2_status da2_attention(da2_plan_t *P, const void *q, const void *k, const void *v, void *o,
                         int32_t out_dtype, hipStream_t stream)
{
    return attend(P, q, k, v, o, out_dtype, nullptr, stream);
}

da2_status da2_attention_prefixed(da2_plan_t *P, const void *q, const void *k, const void *v,
                                  void *o, const void *qp, const void *kp, const void *vp, void *op,
                                  const int32_t *prefix_valid, int32_t out_dtype,
                                  hipStream_t stream)
{
    if (!P)
        return DA2_ERR_INVALID_ARG;
    if (P->L.s.prefix == 0)
        return attend(P, q, k, v, o, out_dtype, nullptr, stream);
    PrefixIo px = {qp, kp, vp, op, prefix_valid};
    return attend(P, q, k, v, o, out_dtype, &px, stream);
}

size_t da2_plan_debug_bytes(const da2_layout_t *layout, int32_t which)
{
    if (!layout)
        return 0;
    const size_t BH = layout->BH, N = layout->Np, R = layout->R, G = layout->Rg, d = layout->d;
    switch (which) {
    case DA2_DBG_Q_I8: case DA2_DBG_K_I8: case DA2_DBG_V_FP8:
    case DA2_DBG_Q_MX: case DA2_DBG_K_MX: case DA2_DBG_V_MX:
        return BH * N * d;
    case DA2_DBG_Q_I8_SCALE: case DA2_DBG_K_I8_SCALE:
        return BH * R * 4;
    case DA2_DBG_V_FP8_SCALE:
        return BH * d * 4;
    case DA2_DBG_Q_MX_SCALE: case DA2_DBG_K_MX_SCALE:
        return BH * N * d / 32;
    case DA2_DBG_V_MX_SCALE:
        return BH * R * 2 * d;
    case DA2_DBG_Q_AVG: case DA2_DBG_K_AVG:
        return BH * G * d * 8;
    case DA2_DBG_Q_MAX: case DA2_DBG_K_MAX:
        return BH * G * d * 4;
    case DA2_DBG_KEYS:
        return BH * G * G * 4;
    case DA2_DBG_SCHEDULE:
        return BH * R * (R + kTargets) * 4;
    default:
        return 0;
    }
}

da2_status da2_plan_debug(const da2_plan_t *P, int32_t which, void *dst, hipStream_t stream)
{
    if (!P || !dst || which < 0 || which >= DA2_DBG_COUNT)
        return DA2_ERR_INVALID_ARG;
    if (!P->ready)
        return DA2_ERR_PLAN_MISMATCH;
    launch_debug(P->L, which, P->ws, dst, stream);
    return launched();
}

void da2_exp_constants(double *out)
{
    out[0] = kLn2Hi;
    out[1] = kLn2Lo;
    out[2] = kInvLn2;
    for (int j = 0; j < 14; j++)
        out[3 + j] = kTaylor.c[j];
}

// ---------------------------------------------------------------------------
// Workspace inside the library, for callers that cannot allocate.  The array
// is file-scope device memory: in host code its name is only a stand-in, so
// every host use goes through the device address hipGetSymbolAddress returns,
// taken once per device with that device current and kept per device.
// ---------------------------------------------------------------------------
namespace {
__device__ __align__(256) char scratch[DA2_NOALLOC_BYTES];
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
char *scratch_dev[kMaxDevices];   // device address of scratch per device (null: not taken yet)

char *scratch_address()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return nullptr;
        scratch_dev[dev] = (char *)p;
    }
    return scratch_dev[dev];
}
}  // namespace

da2_status da2_forward_noalloc(const da2_layout_t *layout, const void *q, const void *k, const void *v,
                               void *o, const da2_budget *budget, int32_t out_dtype, hipStream_t stream)
{
    if (!layout)
        return DA2_ERR_INVALID_ARG;
    if (layout->ws.total > DA2_NOALLOC_BYTES)
        return DA2_ERR_WORKSPACE;
    char *ws = scratch_address();
    if (!ws)
        return DA2_ERR_HIP;
    // a plan on the stack over the caller's layout: the layout's own host
    // tables serve the uploads, so nothing is allocated
    da2_plan_s P;
    memset(&P, 0, sizeof(P));
    P.L = *layout;
    P.nreg = layout->nreg;
    P.ws = ws;
    P.ws_bytes = DA2_NOALLOC_BYTES;
    da2_status st = da2_plan(&P, q, k, budget, stream);
    if (st != DA2_OK)
        return st;
    return da2_attention(&P, q, k, v, o, out_dtype, stream);
}

}  // extern "C"
