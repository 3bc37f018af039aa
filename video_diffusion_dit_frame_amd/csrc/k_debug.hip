// k_debug.hip -- unpack the plan's internal operand layouts into canonical
// layouts for bit-exact comparison in tests (not on the hot path).
#include "da2_internal.h"
#include "da2_device.h"

namespace da2 {
namespace {

// Canonical element (bh, pos = a*64 + i, c) of a Q/K operand -> packed chunk.
__device__ __forceinline__ void qk_locate(int i, int c, int is_key, int KC, int &chunk, int &j)
{
    const int kc = c / 64, lh = (c % 64) / 32;
    j = c % 32;
    int half, row;
    if (!is_key) {
        half = i / 32;
        row = i % 32;
    } else {
        // invert key_of_row: i = 32*((row>>2)&1) + 16*m + 4*(row>>3) + (row&3)
        const int hh = i / 32, rem = i % 32;
        half = rem / 16;
        const int r = rem % 16;  // 4*(row>>3) + (row&3)
        row = 8 * (r / 4) + 4 * hh + (r % 4);
    }
    chunk = (half * KC + kc) * 64 + lh * 32 + row;
}

__global__ void k_unpack_qk(const uint8_t *op8, const uint8_t *op4, const uint8_t *op4s,
                            int is_key, int which, int d, int64_t total, uint8_t *dst)
{
    int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= total)
        return;
    const int KC = d / 64;
    if (which == 2) {  // scales [bh][pos][d/32]
        const int G = d / 32;
        const int64_t tok = e / G;
        const int g = (int)(e % G);
        const int64_t blk = tok / kBlk;
        const int i = (int)(tok % kBlk);
        int chunk, j;
        qk_locate(i, 32 * g, is_key, KC, chunk, j);
        dst[e] = op4s[blk * (2 * d) + chunk];
        return;
    }
    const int64_t tok = e / d;
    const int c = (int)(e % d);
    const int64_t blk = tok / kBlk;
    const int i = (int)(tok % kBlk);
    int chunk, j;
    qk_locate(i, c, is_key, KC, chunk, j);
    if (which == 0) {
        dst[e] = op8[blk * (kBlk * d) + (int64_t)chunk * 32 + j];
    } else {
        uint8_t byte = op4[blk * (kBlk * d / 2) + (int64_t)chunk * 16 + j / 2];
        dst[e] = (j & 1) ? (byte >> 4) : (byte & 15);
    }
}

// V: chunk = cb*64 + (k/32)*32 + c%32, byte = k%32.
__global__ void k_unpack_v(const uint8_t *op8, const uint8_t *op4, const uint8_t *op4s,
                           int which, int d, int64_t total, uint8_t *dst)
{
    int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= total)
        return;
    if (which == 2) {  // [bh][a][2][d]
        const int c = (int)(e % d);
        const int g = (int)((e / d) % 2);
        const int64_t blk = e / (2 * d);
        const int chunk = (c / 32) * 64 + g * 32 + c % 32;
        dst[e] = op4s[blk * (2 * d) + chunk];
        return;
    }
    const int64_t tok = e / d;
    const int c = (int)(e % d);
    const int64_t blk = tok / kBlk;
    const int k = (int)(tok % kBlk);
    const int chunk = (c / 32) * 64 + (k / 32) * 32 + c % 32;
    const int j = k % 32;
    if (which == 0) {
        dst[e] = op8[blk * (kBlk * d) + (int64_t)chunk * 32 + j];
    } else {
        uint8_t byte = op4[blk * (kBlk * d / 2) + (int64_t)chunk * 16 + j / 2];
        dst[e] = (j & 1) ? (byte >> 4) : (byte & 15);
    }
}

__global__ void k_unpack_sched(const int32_t *sched, const int32_t *cnt, int R, int64_t rows,
                               int32_t *dst)
{
    int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t W = R + kTargets;
    if (e >= rows * W)
        return;
    const int64_t row = e / W;
    const int j = (int)(e % W);
    const int n = cnt[row * kTargets] + cnt[row * kTargets + 1] + cnt[row * kTargets + 2];
    int32_t v;
    if (j < kTargets)
        v = cnt[row * kTargets + j];
    else
        v = (j - kTargets) < n ? (int32_t)sched[row * R + (j - kTargets)] : -1;
    dst[e] = v;
}

}  // namespace

void launch_debug(const da2_layout_s &L, int which, const char *ws, void *dst, hipStream_t st)
{
    const Workspace &W = L.ws;
    const int d = L.d;
    const int64_t nd = (int64_t)L.BH * L.Np * d;
    auto grid = [](int64_t n) { return (unsigned)((n + 255) / 256); };
    uint8_t *o = (uint8_t *)dst;
    switch (which) {
    case DA2_DBG_Q_I8: case DA2_DBG_Q_MX: case DA2_DBG_Q_MX_SCALE:
    case DA2_DBG_K_I8: case DA2_DBG_K_MX: case DA2_DBG_K_MX_SCALE: {
        const int is_key = which >= DA2_DBG_K_I8;
        const int kind = (which - (is_key ? DA2_DBG_K_I8 : DA2_DBG_Q_I8));  // 0 int8, 2 mx, 3 mx scale
        const int wk = kind == 0 ? 0 : (kind == 2 ? 1 : 2);
        const int64_t total = wk == 2 ? nd / 32 : nd;
        k_unpack_qk<<<grid(total), 256, 0, st>>>(
            (const uint8_t *)(ws + (is_key ? W.k8 : W.q8)), (const uint8_t *)(ws + (is_key ? W.k4 : W.q4)),
            (const uint8_t *)(ws + (is_key ? W.k4s : W.q4s)), is_key, wk, d, total, o);
        break;
    }
    case DA2_DBG_V_FP8: case DA2_DBG_V_MX: case DA2_DBG_V_MX_SCALE: {
        const int wk = which == DA2_DBG_V_FP8 ? 0 : (which == DA2_DBG_V_MX ? 1 : 2);
        const int64_t total = wk == 2 ? (int64_t)L.BH * L.R * 2 * d : nd;
        k_unpack_v<<<grid(total), 256, 0, st>>>((const uint8_t *)(ws + W.v8), (const uint8_t *)(ws + W.v4),
                                                (const uint8_t *)(ws + W.v4s), wk, d, total, o);
        break;
    }
    case DA2_DBG_Q_I8_SCALE:
        hipMemcpyAsync(dst, ws + W.qs8, sizeof(float) * L.BH * L.R, hipMemcpyDeviceToDevice, st);
        break;
    case DA2_DBG_K_I8_SCALE:
        hipMemcpyAsync(dst, ws + W.ks8, sizeof(float) * L.BH * L.R, hipMemcpyDeviceToDevice, st);
        break;
    case DA2_DBG_V_FP8_SCALE:
        hipMemcpyAsync(dst, ws + W.vs8, sizeof(float) * L.BH * d, hipMemcpyDeviceToDevice, st);
        break;
    case DA2_DBG_Q_AVG:
        hipMemcpyAsync(dst, ws + W.qavg, sizeof(double) * L.BH * L.Rg * d, hipMemcpyDeviceToDevice, st);
        break;
    case DA2_DBG_K_AVG:
        hipMemcpyAsync(dst, ws + W.kavg, sizeof(double) * L.BH * L.Rg * d, hipMemcpyDeviceToDevice, st);
        break;
    case DA2_DBG_Q_MAX:
        hipMemcpyAsync(dst, ws + W.qmax, sizeof(float) * L.BH * L.Rg * d, hipMemcpyDeviceToDevice, st);
        break;
    case DA2_DBG_K_MAX:
        hipMemcpyAsync(dst, ws + W.kmax, sizeof(float) * L.BH * L.Rg * d, hipMemcpyDeviceToDevice, st);
        break;
    case DA2_DBG_KEYS:
        hipMemcpyAsync(dst, ws + W.keys, sizeof(uint32_t) * L.BH * L.Rg * L.Rg, hipMemcpyDeviceToDevice, st);
        break;
    case DA2_DBG_SCHEDULE: {
        const int64_t rows = (int64_t)L.BH * L.R;
        k_unpack_sched<<<grid(rows * (L.R + kTargets)), 256, 0, st>>>(
            (const int32_t *)(ws + W.sched), (const int32_t *)(ws + W.cnt), L.R, rows, (int32_t *)dst);
        break;
    }
    default:
        break;
    }
}

}  // namespace da2
