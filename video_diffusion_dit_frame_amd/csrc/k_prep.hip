// k_prep.hip -- fused operand preparation (DraftAttention2, Sec. 3.3 "fused
// quantization and reordering"; App. C.2 spatial packing).
//
// k_prep_qk: one workgroup per (b, h, region).  Gathers the region's 64
// tokens (one coalesced 16-byte load per chunk, strided input), and from the
// same LDS copy emits the pooled descriptors of Eq. (1) (fp64 sum in region
// order / 64, signed max), the INT8 codes of the 8-bit path's Q K^T (App.
// C.1) with one fp32 step per block (App. B.2's uniform quantizer: step
// amax / 127, codes the nearest integers of x * (127 / amax)), and MXFP4 E2M1
// codes with one E8M0 exponent per token and 32 channels -- all written
// directly in the MFMA operand layouts the attention kernel loads.
//
// k_vamax + k_prep_v: V gets one FP8 scale per channel over all tokens (so
// the attention accumulator changes units once, at the end of the FP8 phase)
// and MXFP4 groups of 32 consecutive keys inside each region, packed as the
// A operand of O^T = V^T P^T (the value transposition folded into packing);
// when the plan has 16-bit tiles, also the bf16 values in the A-operand
// layout of the 16-bit product.
#include "da2_internal.h"
#include "da2_device.h"

namespace da2 {
namespace {

// Copy the NT x 64 x D bf16 tiles a0 .. a0 + NT - 1 into LDS (row i = slot
// i of the run; padding slots of a ragged layout are zero rows).  All slot
// lookups first, then all row loads, then the stores, so that every load of
// the 256 threads is in flight at once.
template <int D, bool RAG, int NT = 1>
__device__ __forceinline__ void load_region(const uint16_t *__restrict__ x, int64_t sn, int a0,
                                            const Geo &g, uint16_t *tile)
{
    constexpr int CH = D / 8;  // 16-byte chunks per token row
    constexpr int ITER = NT * kBlk * CH / 256;
    static_assert(ITER * 256 == NT * kBlk * CH, "whole rounds of 256 chunks");
    int n[ITER];
#pragma unroll
    for (int u = 0; u < ITER; u++) {
        const int i = (int)(threadIdx.x + 256 * u) / CH;
        n[u] = slot_token<RAG>(g, a0 + i / kBlk, i % kBlk);
    }
    uint4 v[ITER];
#pragma unroll
    for (int u = 0; u < ITER; u++) {
        const int ci = threadIdx.x + 256 * u, i = ci / CH, c8 = ci - i * CH;
        v[u] = make_uint4(0u, 0u, 0u, 0u);
        if (n[u] >= 0)
            v[u] = *reinterpret_cast<const uint4 *>(x + (int64_t)n[u] * sn + c8 * 8);
    }
#pragma unroll
    for (int u = 0; u < ITER; u++) {
        const int ci = threadIdx.x + 256 * u, i = ci / CH, c8 = ci - i * CH;
        *reinterpret_cast<uint4 *>(tile + i * D + c8 * 8) = v[u];
    }
}

template <int D, bool RAG>
__global__ __launch_bounds__(256) void k_prep_qk(const uint16_t *__restrict__ x, int64_t sb,
                                                 int64_t sh, int64_t sn, int H, int R, Geo g,
                                                 int is_key, uint8_t *__restrict__ op8,
                                                 float *__restrict__ s8, uint8_t *__restrict__ op4,
                                                 uint8_t *__restrict__ op4s,
                                                 double *__restrict__ avg, float *__restrict__ mx,
                                                 uint16_t *__restrict__ op16)
{
    constexpr int KC = D / 64;
    __shared__ __attribute__((aligned(16))) uint16_t tile[kBlk * D];
    __shared__ float red[4];
    const int a = blockIdx.x, bh = blockIdx.y;
    const int b = bh / H, h = bh - b * H;
    const uint16_t *xb = x + (int64_t)b * sb + (int64_t)h * sh;
    load_region<D, RAG>(xb, sn, a, g, tile);
    // valid tokens of the region (App. C.1: n_a excludes padding); they fill
    // the first slots
    const int na = RAG ? __syncthreads_count(threadIdx.x < kBlk && slot_token<RAG>(g, a, threadIdx.x) >= 0)
                       : kBlk;
    __syncthreads();

    const int t = threadIdx.x;
    const int64_t blk = (int64_t)bh * R + a;
    // pooled descriptors: channel t, valid tokens in slot order (regions of
    // more than one tile pool in k_pool: avg is null then)
    if (avg && t < D) {
        double s = 0.0;
        float m = bf16_to_f32(tile[t]);
        for (int i = 0; i < na; i++) {
            float v = bf16_to_f32(tile[i * D + t]);
            s += (double)v;
            if (v > m)
                m = v;
        }
        avg[blk * D + t] = s / (double)na;
        mx[blk * D + t] = m;
    }
    // ragged layouts: the bf16 key image of the 16-bit products, chunk
    // (m, s) holding for lane l slot key_of_row(l % 32, m), channels
    // 16 s + 8 (l / 32) .. + 7
    if (RAG && is_key) {
        for (int u = t; u < 2 * (D / 16) * 64; u += 256) {
            const int ms = u >> 6, l = u & 63, m = ms / (D / 16), st = ms - m * (D / 16);
            const uint4 v = *reinterpret_cast<const uint4 *>(tile + key_of_row(l & 31, m) * D + 16 * st +
                                                             8 * (l >> 5));
            *reinterpret_cast<uint4 *>(op16 + blk * (kBlk * D) + (int64_t)u * 8) = v;
        }
    }
    // operand chunks: t -> (half, kc, lane); 2*KC*64 = 2*D chunks per block,
    // 32 values each, covering the tile once.  The chunk's values are read
    // before the INT8 block step, whose absolute maximum is then the
    // workgroup's maximum of the chunks' maxima (padding rows are zeros).
    const bool chunk = t < 2 * D;
    const int half = t / (KC * 64), kc = (t / 64) % KC, l = t & 63;
    float xv[32];
    float ga = 0.0f;
    if (chunk) {
        const int row = is_key ? key_of_row(l & 31, half) : 32 * half + (l & 31);
        const uint16_t *src = tile + row * D + 64 * kc + 32 * (l >> 5);
#pragma unroll
        for (int j = 0; j < 32; j++) {
            xv[j] = bf16_to_f32(src[j]);
            ga = fmaxf(ga, __builtin_fabsf(xv[j]));
        }
    }
    float am = wave_max_f32(ga);
    if ((t & 63) == 0)
        red[t >> 6] = am;
    __syncthreads();
    am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float sc = 1.0f, inv = 0.0f;
    if (am != 0.0f) {
        sc = am / 127.0f;
        inv = 127.0f / am;
    }
    if (t == 0)
        s8[blk] = sc;

    if (chunk) {
        uint32_t w8[8];
#pragma unroll
        for (int q = 0; q < 8; q++)
            w8[q] = pack_i8x4(xv[4 * q] * inv, xv[4 * q + 1] * inv, xv[4 * q + 2] * inv, xv[4 * q + 3] * inv);
        uint4 *d8 = reinterpret_cast<uint4 *>(op8 + blk * (kBlk * D) + (int64_t)t * 32);
        d8[0] = make_uint4(w8[0], w8[1], w8[2], w8[3]);
        d8[1] = make_uint4(w8[4], w8[5], w8[6], w8[7]);
        const int E = mx_exponent(ga);
        const float scale = pow2_e8m0(E);
        uint32_t w4[4];
#pragma unroll
        for (int q = 0; q < 4; q++)
            w4[q] = pack_e2m1x8(xv + 8 * q, scale);
        *reinterpret_cast<uint4 *>(op4 + blk * (kBlk * D / 2) + (int64_t)t * 16) =
            make_uint4(w4[0], w4[1], w4[2], w4[3]);
        op4s[blk * (2 * D) + t] = (uint8_t)(E + 127);
    }
}

// Pooled descriptors of regions of tpr > 1 tiles (block capacity tpr * 64):
// one workgroup per (b, h, region) gathers the region's slots into LDS, and
// channel t sums its valid tokens in slot order (fp64, tile after tile) and
// takes their signed maximum, as k_prep_qk does for a one-tile region.  The
// valid tokens fill the region's first slots.
template <int D, int TPR>
__global__ __launch_bounds__(256) void k_pool(const uint16_t *__restrict__ x, int64_t sb, int64_t sh,
                                              int64_t sn, int H, int G, Geo g,
                                              double *__restrict__ avg, float *__restrict__ mx)
{
    __shared__ __attribute__((aligned(16))) uint16_t tile[TPR * kBlk * D];
    const int a = blockIdx.x, bh = blockIdx.y;
    const int b = bh / H, h = bh - b * H;
    const uint16_t *xb = x + (int64_t)b * sb + (int64_t)h * sh;
    constexpr int slots = TPR * kBlk;
    load_region<D, true, TPR>(xb, sn, a * TPR, g, tile);
    const int i0 = threadIdx.x;
    const int na = __syncthreads_count(i0 < slots && slot_token<true>(g, a * TPR + i0 / kBlk, i0 % kBlk) >= 0);
    const int t = threadIdx.x;
    if (t < D) {
        double s = 0.0;
        float m = bf16_to_f32(tile[t]);
        for (int i = 0; i < na; i++) {
            float v = bf16_to_f32(tile[i * D + t]);
            s += (double)v;
            if (v > m)
                m = v;
        }
        const int64_t r = (int64_t)bh * G + a;
        avg[r * D + t] = s / (double)na;
        mx[r * D + t] = m;
    }
}

// Per-channel absolute maxima of V over all tokens (atomic max on the bit
// pattern, which orders like the value for non-negative floats).
template <int D>
__global__ __launch_bounds__(256) void k_vamax(const uint16_t *__restrict__ x, int64_t sb,
                                               int64_t sh, int64_t sn, int H, int N,
                                               uint32_t *__restrict__ vamax)
{
    constexpr int CH = D / 8;           // chunks per token
    constexpr int TPI = 256 / CH;       // tokens per iteration
    constexpr int TOK = 256;            // tokens per workgroup
    __shared__ float part[TPI][D];
    const int bh = blockIdx.y;
    const int b = bh / H, h = bh - b * H;
    const uint16_t *xb = x + (int64_t)b * sb + (int64_t)h * sh;
    const int t = threadIdx.x, c8 = t % CH, ti = t / CH;
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const int n0 = blockIdx.x * TOK;
    for (int n = n0 + ti; n < min(n0 + TOK, N); n += TPI) {
        uint4 v = *reinterpret_cast<const uint4 *>(xb + (int64_t)n * sn + c8 * 8);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            m[2 * j] = fmaxf(m[2 * j], __builtin_fabsf(bf16_to_f32((uint16_t)(w[j] & 0xffffu))));
            m[2 * j + 1] = fmaxf(m[2 * j + 1], __builtin_fabsf(bf16_to_f32((uint16_t)(w[j] >> 16))));
        }
    }
#pragma unroll
    for (int j = 0; j < 8; j++)
        part[ti][c8 * 8 + j] = m[j];
    __syncthreads();
    if (t < D) {
        float r = 0.0f;
        for (int i = 0; i < TPI; i++)
            r = fmaxf(r, part[i][t]);
        atomicMax(&vamax[(int64_t)bh * D + t], __float_as_uint(r));
    }
}

template <int D, bool RAG>
__global__ __launch_bounds__(256) void k_prep_v(const uint16_t *__restrict__ x, int64_t sb,
                                                int64_t sh, int64_t sn, int H, int R, Geo g,
                                                float *__restrict__ vavg,
                                                const uint32_t *__restrict__ vamax,
                                                uint8_t *__restrict__ op8, float *__restrict__ s8,
                                                uint8_t *__restrict__ op4,
                                                uint8_t *__restrict__ op4s,
                                                uint16_t *__restrict__ op16, uint16_t *__restrict__ op8b)
{
    __shared__ __attribute__((aligned(16))) uint16_t tile[kBlk * D];
    const int a = blockIdx.x, bh = blockIdx.y;
    const int b = bh / H, h = bh - b * H;
    const uint16_t *xb = x + (int64_t)b * sb + (int64_t)h * sh;
    load_region<D, RAG>(xb, sn, a, g, tile);
    const int na = RAG ? __syncthreads_count(threadIdx.x < kBlk && slot_token<RAG>(g, a, threadIdx.x) >= 0)
                       : kBlk;
    __syncthreads();
    const int t = threadIdx.x;
    const int64_t blk = (int64_t)bh * R + a;
    // mean value of the region over its valid tokens (block-mean tiles):
    // fp64 sum in slot order, divided by n_a, rounded to fp32
    if (vavg && t < D) {
        double sum = 0.0;
        for (int i = 0; i < na; i++)
            sum += (double)bf16_to_f32(tile[i * D + t]);
        vavg[blk * D + t] = (float)(sum / (double)na);
    }
    if (t < 2 * D) {
        const int cb = t >> 6, l = t & 63;
        const int c = 32 * cb + (l & 31), k0 = 32 * (l >> 5);
        const float am = __uint_as_float(vamax[(int64_t)bh * D + c]);
        float sc = 1.0f, inv = 0.0f;
        if (am != 0.0f) {
            sc = am / 448.0f;
            inv = 448.0f / am;
        }
        if (a == 0 && l < 32)
            s8[(int64_t)bh * D + c] = sc;
        float xv[32];
        float ga = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; j++) {
            xv[j] = bf16_to_f32(tile[(k0 + j) * D + c]);
            ga = fmaxf(ga, __builtin_fabsf(xv[j]));
        }
        uint32_t w8[8];
#pragma unroll
        for (int q = 0; q < 8; q++)
            w8[q] = pack_e4m3x4(xv[4 * q] * inv, xv[4 * q + 1] * inv, xv[4 * q + 2] * inv,
                                xv[4 * q + 3] * inv);
        uint4 *d8 = reinterpret_cast<uint4 *>(op8 + blk * (kBlk * D) + (int64_t)t * 32);
        d8[0] = make_uint4(w8[0], w8[1], w8[2], w8[3]);
        d8[1] = make_uint4(w8[4], w8[5], w8[6], w8[7]);
        // the values of the FP8 codes as bf16 (exact), in the layout of the
        // bf16 operand below: the value operand of the FP8 tier's products on
        // the bf16 matrix core
#pragma unroll
        for (int q = 0; q < 4; q++)
            *reinterpret_cast<uint4 *>(op8b + ((blk * (D / 32) + cb) * 4 + q) * 512 + l * 8) =
                make_uint4(fp8_pair_bf16(w8[2 * q], 0), fp8_pair_bf16(w8[2 * q], 1), fp8_pair_bf16(w8[2 * q + 1], 0),
                           fp8_pair_bf16(w8[2 * q + 1], 1));
        const int E = mx_exponent(ga);
        const float scale = pow2_e8m0(E);
        uint32_t w4[4];
#pragma unroll
        for (int q = 0; q < 4; q++)
            w4[q] = pack_e2m1x8(xv + 8 * q, scale);
        *reinterpret_cast<uint4 *>(op4 + blk * (kBlk * D / 2) + (int64_t)t * 16) =
            make_uint4(w4[0], w4[1], w4[2], w4[3]);
        op4s[blk * (2 * D) + t] = (uint8_t)(E + 127);
        if (op16) {
            // bf16 A operand of the 16-bit product: chunk (cb, step q) holds,
            // for lane l, channel c and the 8 keys 32 (l / 32) + 8 q .. + 7
#pragma unroll
            for (int q = 0; q < 4; q++) {
                uint32_t w16[4];
#pragma unroll
                for (int j = 0; j < 4; j++)
                    w16[j] = (uint32_t)tile[(k0 + 8 * q + 2 * j) * D + c] |
                             ((uint32_t)tile[(k0 + 8 * q + 2 * j + 1) * D + c] << 16);
                *reinterpret_cast<uint4 *>(op16 + ((blk * (D / 32) + cb) * 4 + q) * 512 + l * 8) =
                    make_uint4(w16[0], w16[1], w16[2], w16[3]);
            }
        }
    }
}

// Value image of the text prefix for the 16-bit path (App. C.1): the layout
// of the regions' bf16 operand above, tile t holding prefix keys 64 t ..
// 64 t + 63; keys past the valid count of their batch element are zero, so
// their (zero) weights meet finite values.  Thread (cb, l) writes lane l of
// channel block cb.
template <int D>
__global__ __launch_bounds__(2 * D) void k_prep_vp(const uint16_t *__restrict__ x, int64_t sb, int64_t sh,
                                                   int64_t sn, int H, int Lp, int ptiles,
                                                   const int32_t *__restrict__ valid,
                                                   uint16_t *__restrict__ op16)
{
    const int t = blockIdx.x, bh = blockIdx.y;
    const int b = bh / H, h = bh - b * H;
    const int nv = valid ? min(max(valid[b], 0), Lp) : Lp;
    const uint16_t *xb = x + (int64_t)b * sb + (int64_t)h * sh;
    const int cb = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int c = 32 * cb + (l & 31), k0 = kBlk * t + 32 * (l >> 5);
    const int64_t blk = (int64_t)bh * ptiles + t;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        uint32_t w16[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int key = k0 + 8 * q + 2 * j;
            const uint32_t lo = key < nv ? xb[(int64_t)key * sn + c] : 0u;
            const uint32_t hi = key + 1 < nv ? xb[(int64_t)(key + 1) * sn + c] : 0u;
            w16[j] = lo | (hi << 16);
        }
        *reinterpret_cast<uint4 *>(op16 + ((blk * (D / 32) + cb) * 4 + q) * 512 + l * 8) =
            make_uint4(w16[0], w16[1], w16[2], w16[3]);
    }
}

__global__ void k_fill_u32(uint32_t *p, int64_t n, uint32_t v)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = v;
}

}  // namespace

Geo layout_geo(const da2_layout_s &L, const char *ws)
{
    Geo g;
    g.Ry = L.Ry;
    g.Rx = L.Rx;
    g.Hv = L.s.height;
    g.Wv = L.s.width;
    g.Rf = L.Rf;
    g.ftok = L.ragged ? (const int32_t *)(ws + L.ws.ftok) : nullptr;
    return g;
}

void launch_prep_qk(const da2_layout_s &L, const void *x, int is_key, char *ws, hipStream_t st)
{
    const Workspace &W = L.ws;
    dim3 grid(L.R, L.BH);
    const uint16_t *xp = static_cast<const uint16_t *>(x);
    uint8_t *op8 = (uint8_t *)(ws + (is_key ? W.k8 : W.q8));
    float *s8 = (float *)(ws + (is_key ? W.ks8 : W.qs8));
    uint8_t *op4 = (uint8_t *)(ws + (is_key ? W.k4 : W.q4));
    uint8_t *op4s = (uint8_t *)(ws + (is_key ? W.k4s : W.q4s));
    double *avg = (double *)(ws + (is_key ? W.kavg : W.qavg));
    float *mx = (float *)(ws + (is_key ? W.kmax : W.qmax));
    uint16_t *op16 = (uint16_t *)(ws + W.k16);
    const da2_shape &s = L.s;
    const Geo g = layout_geo(L, ws);
    // one-tile regions pool in k_prep_qk, larger ones in k_pool
    double *avg1 = L.tpr == 1 ? avg : nullptr;
#define DA2_PREP_QK(DD, RG)                                                                           \
    k_prep_qk<DD, RG><<<grid, 256, 0, st>>>(xp, s.stride_b, s.stride_h, s.stride_n, s.heads, L.R, g, is_key, \
                                            op8, s8, op4, op4s, avg1, mx, op16)
    if (L.d == 128) {
        if (L.ragged)
            DA2_PREP_QK(128, true);
        else
            DA2_PREP_QK(128, false);
    } else {
        if (L.ragged)
            DA2_PREP_QK(64, true);
        else
            DA2_PREP_QK(64, false);
    }
#undef DA2_PREP_QK
    if (L.tpr > 1) {   // capacity 128: two tiles per region
        dim3 gp(L.Rg, L.BH);
        if (L.d == 128)
            k_pool<128, 2><<<gp, 256, 0, st>>>(xp, s.stride_b, s.stride_h, s.stride_n, s.heads, L.Rg, g, avg, mx);
        else
            k_pool<64, 2><<<gp, 256, 0, st>>>(xp, s.stride_b, s.stride_h, s.stride_n, s.heads, L.Rg, g, avg, mx);
    }
}

void launch_prep_v(const da2_layout_s &L, const void *v, int with16, int with_mean, char *ws, hipStream_t st)
{
    const Workspace &W = L.ws;
    const da2_shape &s = L.s;
    const uint16_t *xp = static_cast<const uint16_t *>(v);
    uint32_t *vamax = (uint32_t *)(ws + W.vamax);
    int64_t n = (int64_t)L.BH * L.d;
    k_fill_u32<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(vamax, n, 0u);
    dim3 g1((L.N + 255) / 256, L.BH), g2(L.R, L.BH);
    uint8_t *op8 = (uint8_t *)(ws + W.v8), *op4 = (uint8_t *)(ws + W.v4),
            *op4s = (uint8_t *)(ws + W.v4s);
    uint16_t *op16 = with16 ? (uint16_t *)(ws + W.v16) : nullptr;
    uint16_t *op8b = (uint16_t *)(ws + W.v8b);
    float *s8 = (float *)(ws + W.vs8);
    float *vavg = with_mean ? (float *)(ws + W.vavg) : nullptr;
    const Geo g = layout_geo(L, ws);
#define DA2_PREP_V(DD, RG)                                                                              \
    k_prep_v<DD, RG><<<g2, 256, 0, st>>>(xp, s.stride_b, s.stride_h, s.stride_n, s.heads, L.R, g, vavg, vamax, \
                                         op8, s8, op4, op4s, op16, op8b)
    if (L.d == 128) {
        k_vamax<128><<<g1, 256, 0, st>>>(xp, s.stride_b, s.stride_h, s.stride_n, s.heads, L.N, vamax);
        if (L.ragged)
            DA2_PREP_V(128, true);
        else
            DA2_PREP_V(128, false);
    } else {
        k_vamax<64><<<g1, 256, 0, st>>>(xp, s.stride_b, s.stride_h, s.stride_n, s.heads, L.N, vamax);
        if (L.ragged)
            DA2_PREP_V(64, true);
        else
            DA2_PREP_V(64, false);
    }
#undef DA2_PREP_V
}

void launch_prep_vp(const da2_layout_s &L, const PrefixIo &px, char *ws, hipStream_t st)
{
    const da2_shape &s = L.s;
    if (s.prefix <= 0)
        return;
    dim3 grid(L.ptiles, L.BH);
    const uint16_t *xp = static_cast<const uint16_t *>(px.vp);
    uint16_t *op16 = (uint16_t *)(ws + L.ws.vp16);
    if (L.d == 128)
        k_prep_vp<128><<<grid, 256, 0, st>>>(xp, s.stride_b, s.stride_h, s.stride_n, s.heads, s.prefix,
                                             L.ptiles, px.valid, op16);
    else
        k_prep_vp<64><<<grid, 128, 0, st>>>(xp, s.stride_b, s.stride_h, s.stride_n, s.heads, s.prefix,
                                            L.ptiles, px.valid, op16);
}

}  // namespace da2
