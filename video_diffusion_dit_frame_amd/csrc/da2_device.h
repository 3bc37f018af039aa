// da2_device.h -- device helpers shared by the libda2 kernels: bf16 access,
// region geometry, exact FP8 / MXFP4 encoders for operand preparation and the
// fp64 exp of the draft softmax.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da2 {

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Original token index of position i (0..63) of region a.  Regions are the
// 8x8 cells of every frame, frame-major then raster; tokens in raster order.
__device__ __forceinline__ int region_token(int a, int i, int Ry, int Rx, int Hv, int Wv)
{
    int f = a / (Ry * Rx);
    int r = a - f * Ry * Rx;
    int ry = r / Rx, rx = r - ry * Rx;
    return (f * Hv + ry * 8 + (i >> 3)) * Wv + rx * 8 + (i & 7);
}

// Region geometry of a layout: the 8x8 grid (ftok null), or a ragged
// partition given by its frame slot table (token y*Wv + x of each slot of
// the frame's Rf regions, -1 for a padding slot; valid slots first).
struct Geo {
    int Ry, Rx, Hv, Wv, Rf;
    const int32_t *ftok;
};

// Original token index of slot i of region a, or -1 for a padding slot.
template <bool RAG>
__device__ __forceinline__ int slot_token(const Geo &g, int a, int i)
{
    if (!RAG)
        return region_token(a, i, g.Ry, g.Rx, g.Hv, g.Wv);
    const int f = a / g.Rf, r = a - f * g.Rf;
    const int t = g.ftok[r * 64 + i];
    return t < 0 ? -1 : f * g.Hv * g.Wv + t;
}

// Logical key (0..63) held in row i (0..31) of the key operand of MFMA half m.
// The 32x32 accumulator puts row i at register 4*(i/8) + i%4 of lane half
// (i/4)%2; this permutation makes lane half hf own keys 32*hf .. 32*hf+31,
// slot s = 16*m + register, so one lane holds a whole 32-key MX group.
__device__ __forceinline__ int key_of_row(int i, int m)
{
    return 32 * ((i >> 2) & 1) + 16 * m + 4 * (i >> 3) + (i & 3);
}

// floor(log2 x) for finite x > 0 (normal or subnormal fp32).
__device__ __forceinline__ int floor_log2_f32(float x)
{
    uint32_t u = __float_as_uint(x);
    int e = (int)((u >> 23) & 0xffu);
    if (e)
        return e - 127;
    return (31 - __builtin_clz(u & 0x7fffffu)) - 149;
}

// E8M0 block exponent of an MX block with largest magnitude amax:
// floor(log2 amax) - 2, clamped to [-127, 127]; amax = 0 gives -127.
__device__ __forceinline__ int mx_exponent(float amax)
{
    if (amax == 0.0f)
        return -127;
    int E = floor_log2_f32(amax) - 2;
    return E < -127 ? -127 : (E > 127 ? 127 : E);
}

// Four E4M3 codes (x0 in the low byte) from the hardware conversion: nearest
// with ties to even, subnormals kept, sign kept on zero; inputs here never
// exceed 448 by more than a rounding error, so no saturation is needed.
__device__ __forceinline__ uint32_t pack_e4m3x4(float x0, float x1, float x2, float x3)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
}

// Four INT8 codes: the nearest integers of x (ties to even), two's
// complement bytes, x0 in the low byte.  Callers pass |x| <= 127 up to one
// fp32 rounding; the clamp keeps any such value on the code the rounding
// names.
__device__ __forceinline__ int i8_code(float x)
{
    return (int)__builtin_rintf(fminf(fmaxf(x, -127.0f), 127.0f));
}

__device__ __forceinline__ uint32_t pack_i8x4(float x0, float x1, float x2, float x3)
{
    return ((uint32_t)i8_code(x0) & 0xffu) | (((uint32_t)i8_code(x1) & 0xffu) << 8) |
           (((uint32_t)i8_code(x2) & 0xffu) << 16) | ((uint32_t)i8_code(x3) << 24);
}

// Two E4M3 codes (bytes 2 hi and 2 hi + 1 of c) as their values in bf16, low
// half first.  Exact: an E4M3 value has at most 4 significant bits and lies
// in the bf16 range, so the top half of its fp32 pattern is the value.
__device__ __forceinline__ uint32_t fp8_pair_bf16(uint32_t c, int hi)
{
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    const v2bf r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c, 1.0f, true)
                      : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c, 1.0f, false);
    return __builtin_bit_cast(uint32_t, r);
}

// The fp32 value 2^E for an E8M0 exponent E in [-127, 127] (2^-127 is
// subnormal).
__device__ __forceinline__ float pow2_e8m0(int E)
{
    return E > -127 ? __uint_as_float((uint32_t)(E + 127) << 23) : __uint_as_float(0x00400000u);
}

// Eight E2M1 codes of x[j] / 2^E (x[0] in the low nibble) from the hardware
// scaled conversion: the quotient by a power of two is exact, rounded to the
// nearest code with ties to even, saturating at 6, sign kept on zero.
__device__ __forceinline__ uint32_t pack_e2m1x8(const float *x, float scale)
{
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[0], x[1], scale, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[2], x[3], scale, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[4], x[5], scale, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[6], x[7], scale, 3);
    return w;
}

// ---------------------------------------------------------------------------
// fp64 exp of the draft softmax.  Cody-Waite: k = rint(x / ln 2) through the
// rounded reciprocal, r = x - k ln2 with ln 2 split into a 32-bit head and a
// tail (fdlibm's split), then e^r by its Taylor series to degree 13 in Horner
// form with fused multiply-adds, then 2^k.  Below -708 the result is 0, so
// every nonzero value is normal.
// ---------------------------------------------------------------------------
constexpr double kLn2Hi = 0x1.62e42feep-1;
constexpr double kLn2Lo = 0x1.a39ef35793c76p-33;
constexpr double kInvLn2 = 0x1.71547652b82fep+0;

struct TaylorTable {
    double c[14];
    constexpr TaylorTable() : c()
    {
        double f = 1.0;
        for (int j = 0; j < 14; j++) {
            if (j)
                f = f * (double)j;
            c[j] = 1.0 / f;
        }
    }
};
constexpr TaylorTable kTaylor{};

__device__ __forceinline__ double exp_draft(double x)
{
    if (x < -708.0)
        return 0.0;
    double k = __builtin_rint(x * kInvLn2);
    double r = __builtin_fma(-k, kLn2Hi, x);
    r = __builtin_fma(-k, kLn2Lo, r);
    double p = kTaylor.c[13];
#pragma unroll
    for (int j = 12; j >= 0; j--)
        p = __builtin_fma(p, r, kTaylor.c[j]);
    return __builtin_ldexp(p, (int)k);
}

// Block-wide reductions for 256-thread blocks (4 waves of 64).
__device__ __forceinline__ float wave_max_f32(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

}  // namespace da2

struct da2_layout_s;
namespace da2 {
// The region geometry of a layout whose workspace starts at ws.
Geo layout_geo(const ::da2_layout_s &L, const char *ws);
}  // namespace da2
