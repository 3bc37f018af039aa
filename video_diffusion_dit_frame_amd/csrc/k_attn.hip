// k_attn.hip -- phased mixed-precision block-sparse attention (DraftAttention2,
// Sec. 3.3 "phased execution" and "cross-precision accumulation", App. B.3 /
// B.4 shared normalization, App. C.1 empty rows) on gfx950 matrix cores.
//
// One workgroup = one query region (64 queries) of one (b, h); wave w owns
// queries 32w .. 32w+31.  The quantized products use 32x32x64 f8f6f4 MFMAs,
// the 16-bit ones 32x32x16 bf16 MFMAs, all in the transposed form
//     S^T = K Q^T      (A = key rows, B = queries, k = channels)
//     O^T = V^T P^T    (A = channels, B = queries, k = keys)
// so every lane holds one query: its softmax statistics never leave the lane
// except for one exchange with the partner lane (l ^ 32) per tile.  Key rows
// are stored permuted inside each region (see key_of_row) so that the S^T
// accumulator hands each lane a whole 32-key group, which is exactly the B
// operand chunk of the P^T V product and exactly one MX block of P.
//
// 16-bit phase (tiles of the schedule's 16-bit list, ascending): S from the
// bf16 inputs as they are (exact products, fp32 sums), c4 = log2(e)/sqrt(d);
// e = 2^(S c4 + 8 - m); Z += e; P = bf16(e) (nearest even); acc += P^T V in
// real units.  Phase boundary, when FP8 tiles follow: acc[c] /= sV[c].
// FP8 phase (tiles of the schedule's FP8 list, ascending): S from FP8 codes,
// c8 = sQ sK log2(e)/sqrt(d); running max m per 64-key tile; e = 2^(S c8 + 8
// - m) = 256 w; Z += e; P = e4m3(e); acc += P^T V8 (codes; V's per-channel
// scale is left out).  Phase boundary: acc[c] *= sV[c] (the change of units).
// MXFP4 phase: S from scaled MXFP4 MFMAs, c4 = log2(e)/sqrt(d); P gets one
// E8M0 exponent per 32 keys (floor(log2 max) - 2 of the group's largest e);
// acc += P^T V4 with both block scales applied by the MFMA.  Epilogue:
// O = acc / Z (256 cancels), zero when no tile is kept; rows are written
// straight to their original token positions (restore).
#include "da2_internal.h"
#include "da2_device.h"

namespace da2 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

struct AttnArgs {
    const uint8_t *q8, *q4, *q4s;
    const float *qs8;
    const uint8_t *k8, *k4, *k4s;
    const float *ks8;
    const uint8_t *v8, *v4, *v4s;
    const float *vs8;
    const uint16_t *q, *k;  // bf16 inputs (16-bit phase)
    const uint8_t *v16;     // bf16 value operand (16-bit phase)
    int kspan;              // bytes from a region's first key row past its last
    // text prefix (App. C.1): Lp rows of Q/K/O at qp/kp/outp (same strides),
    // their value images (ptiles tiles of 64 keys per head) and the valid
    // counts per batch element (null: all Lp valid); Lp = 0: no prefix
    const uint16_t *qp, *kp;
    const uint8_t *vp16;
    const int32_t *pvalid;
    void *outp;
    int Lp, ptiles, pkspan;
    // prefix query rows: per (b, h), chunk and row (padded to ptiles * 64)
    // the chunk's running max, sum and unnormalised output
    float *pacc;
    float2 *pmz;
    int pchunks;
    // region geometry; ragged layouts also give each region's valid tokens
    // and the bf16 key image of the 16-bit products
    Geo geo;
    const int32_t *nreg;
    const uint8_t *k16;
    // block-mean tiles (null when the plan has none): per query region the
    // gathered term -- max logit M (log2 units) and weight z -- and its
    // value sum [d]
    const float2 *magg;
    const float *cagg;
    const int32_t *sched;
    const int32_t *cnt;
    const int32_t *qord;  // [bh][j]: query region of work slot j
    void *out;
    int64_t osb, osh, osn;
    int out_f32;
    int H, R, Ry, Rx, Hv, Wv, BH;
    float c4;  // log2(e) / sqrt(d)
};

__device__ __forceinline__ v8bf as_bf16x8(v4u x) { return __builtin_bit_cast(v8bf, x); }

__device__ __forceinline__ v4u lds_v4u(const uint8_t *p) { return *reinterpret_cast<const v4u *>(p); }

__device__ __forceinline__ float pair_max(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ v8i load32(const uint8_t *p)
{
    const uint4 *q = reinterpret_cast<const uint4 *>(p);
    uint4 a = q[0], b = q[1];
    v8i r;
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
    r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
    return r;
}

__device__ __forceinline__ v8i load16(const uint8_t *p)
{
    uint4 a = *reinterpret_cast<const uint4 *>(p);
    v8i r;
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
    r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
    return r;
}

typedef __attribute__((address_space(3))) void lds_void;

// Loads from wave-uniform addresses through the constant address space, so
// they become scalar loads that do not share the vector-memory counter the
// tile prefetch waits on.
__device__ __forceinline__ int sload_i32(const int32_t *p)
{
    return *(const __attribute__((address_space(4))) int32_t *)p;
}

__device__ __forceinline__ float sload_f32(const float *p)
{
    return *(const __attribute__((address_space(4))) float *)p;
}

__device__ __forceinline__ v8i lds32(const uint8_t *p)
{
    const uint4 *q = reinterpret_cast<const uint4 *>(p);
    uint4 a = q[0], b = q[1];
    v8i r;
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
    r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
    return r;
}

// A value the compiler may take from any register: the high half of a
// 16-byte (FP4) matrix operand and the first packing target of a P word are
// never read, so they need no instruction to set them.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wuninitialized"
__device__ __forceinline__ int any_int()
{
    int x;
    return x;
}
__device__ __forceinline__ v16f any_v16f()
{
    v16f x;
    return x;
}
#pragma clang diagnostic pop

__device__ __forceinline__ v8i lds16(const uint8_t *p)
{
    uint4 a = *reinterpret_cast<const uint4 *>(p);
    v8i r;
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
    r[4] = any_int(); r[5] = any_int(); r[6] = any_int(); r[7] = any_int();
    return r;
}

// Key/value operands of one head as buffer resources: a copy then addresses
// its tile with one scalar offset and a fixed per-lane offset, with no
// per-copy vector address arithmetic; reads past the head's bytes return 0.
struct Src {
    __amdgpu_buffer_rsrc_t k8, k4, k4s, v8, v4, v4s;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const uint8_t *base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, (int)bytes, 0x00020000);
}

template <int D>
__device__ __forceinline__ Src head_sources(const AttnArgs &A, int64_t hbase, int R)
{
    Src s;
    s.k8 = head_rsrc(A.k8 + hbase * (kBlk * D), (int64_t)R * kBlk * D);
    s.k4 = head_rsrc(A.k4 + hbase * (kBlk * D / 2), (int64_t)R * kBlk * D / 2);
    s.k4s = head_rsrc(A.k4s + hbase * (2 * D), (int64_t)R * 2 * D);
    s.v8 = head_rsrc(A.v8 + hbase * (kBlk * D), (int64_t)R * kBlk * D);
    s.v4 = head_rsrc(A.v4 + hbase * (kBlk * D / 2), (int64_t)R * kBlk * D / 2);
    s.v4s = head_rsrc(A.v4s + hbase * (2 * D), (int64_t)R * 2 * D);
    return s;
}

// Copy UNITS kilobytes at byte offset off of a resource to LDS dst with
// direct-to-LDS buffer loads; wave w of the two copies units w, w+2, ...
// Each unit is one instruction: 64 lanes x 16 bytes landing at dst + 16 l.
template <int UNITS>
__device__ __forceinline__ void copy_kb(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint8_t *dst, int w,
                                        uint32_t loff16)
{
#pragma unroll
    for (int j = 0; j < UNITS / 2; j++) {
        const int u = 2 * j + w;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + u * 1024), 16, loff16,
                                                 off + u * 1024, 0, 0);
    }
}

// Copy 4 bytes per active lane (lane l -> dst + 4 l).
__device__ __forceinline__ void copy_dword(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint8_t *dst,
                                           uint32_t loff4)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)dst, 4, loff4, off, 0, 0);
}

// LDS images.  Keys and values travel in separate double-buffered streams:
// the key operand of tile i+1 is needed while tile i's weights are formed
// (its logits are computed one tile ahead, so the matrix core works while the
// vector unit runs the softmax), the value operand of tile i only at the end
// of tile i.  Per buffer (D = head dim):
//   FP8 key    [0, 64D)  codes                    value [0, 64D) codes
//   MXFP4 key  [0, 32D)  codes, [32D, 34D) E8M0   value [0, 32D) codes, [32D, 34D) E8M0
// kb is the key region inside the head.
template <int D, bool FP8>
__device__ __forceinline__ void issue_k(const Src &S, int kb, uint8_t *dst, int w, int l)
{
    const uint32_t lo = (uint32_t)l;
    if (FP8) {
        copy_kb<kBlk * D / 1024>(S.k8, (uint32_t)kb * (kBlk * D), dst, w, lo * 16u);
    } else {
        copy_kb<kBlk * D / 2048>(S.k4, (uint32_t)kb * (kBlk * D / 2), dst, w, lo * 16u);
        if (w == 0 && l * 4 < 2 * D)
            copy_dword(S.k4s, (uint32_t)kb * (2 * D), dst + 32 * D, lo * 4u);
    }
}

template <int D, bool FP8>
__device__ __forceinline__ void issue_v(const Src &S, int kb, uint8_t *dst, int w, int l)
{
    const uint32_t lo = (uint32_t)l;
    if (FP8) {
        copy_kb<kBlk * D / 1024>(S.v8, (uint32_t)kb * (kBlk * D), dst, w, lo * 16u);
    } else {
        copy_kb<kBlk * D / 2048>(S.v4, (uint32_t)kb * (kBlk * D / 2), dst, w, lo * 16u);
        if (w == 1 && l * 4 < 2 * D)
            copy_dword(S.v4s, (uint32_t)kb * (2 * D), dst + 32 * D, lo * 4u);
    }
}

// Rescale of the running statistics when a tile raises a row maximum;
// skipped when no lane's maximum moved (the factor would be exactly 1).
template <int CB>
__device__ __forceinline__ void rescale(v16f (&acc)[CB], float &z, float alpha)
{
    if (__any(alpha != 1.0f)) {
        z *= alpha;
#pragma unroll
        for (int cb = 0; cb < CB; cb++)
            acc[cb] *= alpha;
    }
}

// Register operands of one tile.
template <int D>
struct KRegs {
    v8i k[2][D / 64];   // per (key half, 64-channel step)
    int ks[2][D / 64];  // MXFP4 exponents
};

template <int D>
struct VRegs {
    v8i v[D / 32];      // per 32-channel block
    int vs[D / 32];     // MXFP4 exponents
};

template <int D, bool FP8>
__device__ __forceinline__ void read_k(const uint8_t *b, int l, KRegs<D> &K)
{
    constexpr int KC = D / 64;
#pragma unroll
    for (int mm = 0; mm < 2; mm++)
#pragma unroll
        for (int kc = 0; kc < KC; kc++) {
            const int chunk = (mm * KC + kc) * 64 + l;
            if (FP8) {
                K.k[mm][kc] = lds32(b + chunk * 32);
            } else {
                K.k[mm][kc] = lds16(b + chunk * 16);
                K.ks[mm][kc] = b[32 * D + chunk];
            }
        }
}

template <int D, bool FP8>
__device__ __forceinline__ void read_k_half(const uint8_t *b, int l, int mm, KRegs<D> &K)
{
    constexpr int KC = D / 64;
#pragma unroll
    for (int kc = 0; kc < KC; kc++) {
        const int chunk = (mm * KC + kc) * 64 + l;
        if (FP8) {
            K.k[mm][kc] = lds32(b + chunk * 32);
        } else {
            K.k[mm][kc] = lds16(b + chunk * 16);
            K.ks[mm][kc] = b[32 * D + chunk];
        }
    }
}

template <int D, bool FP8>
__device__ __forceinline__ void read_v_range(const uint8_t *b, int l, int c0, int c1, VRegs<D> &V)
{
#pragma unroll
    for (int cb = c0; cb < c1; cb++) {
        const int chunk = cb * 64 + l;
        if (FP8) {
            V.v[cb] = lds32(b + chunk * 32);
        } else {
            V.v[cb] = lds16(b + chunk * 16);
            V.vs[cb] = b[32 * D + chunk];
        }
    }
}

template <int D, bool FP8>
__device__ __forceinline__ void read_v(const uint8_t *b, int l, VRegs<D> &V)
{
    constexpr int CB = D / 32;
#pragma unroll
    for (int cb = 0; cb < CB; cb++) {
        const int chunk = cb * 64 + l;
        if (FP8) {
            V.v[cb] = lds32(b + chunk * 32);
        } else {
            V.v[cb] = lds16(b + chunk * 16);
            V.vs[cb] = b[32 * D + chunk];
        }
    }
}

// Logits S^T = K Q^T of one tile (FP8 codes, or MXFP4 with block scales).
// The query operand qv[kc] holds the FP8 codes of its 64 channels, or the
// MXFP4 codes in dwords 0-3 and the E8M0 exponent in dword 4.
template <int D, bool FP8>
__device__ __forceinline__ void logits(const KRegs<D> &K, const v8i (&qv)[D / 64], v16f (&s)[2])
{
    constexpr int KC = D / 64;
    s[0] = (v16f){};
    s[1] = (v16f){};
#pragma unroll
    for (int kc = 0; kc < KC; kc++)
#pragma unroll
        for (int mm = 0; mm < 2; mm++) {
            if (FP8)
                s[mm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(K.k[mm][kc], qv[kc], s[mm], 0, 0, 0, 0,
                                                                       0, 0);
            else
                s[mm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(K.k[mm][kc], qv[kc], s[mm], 4, 4, 0,
                                                                       K.ks[mm][kc], 0, qv[kc][4]);
        }
}

// Largest of the 32 logits a lane holds: two independent chains of
// three-input maxima, joined at the end.
__device__ __forceinline__ float lane_max(const v16f (&s)[2])
{
    float a = fmaxf(s[0][0], s[0][1]), b = fmaxf(s[1][0], s[1][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) {
        a = fmaxf(fmaxf(a, s[0][r]), s[0][r + 1]);
        b = fmaxf(fmaxf(b, s[1][r]), s[1][r + 1]);
    }
    return fmaxf(a, b);
}

// Running-max update of one tile: m = max(m, tile max * c), al = 2^(m_old -
// m_new) (the factor the statistics of earlier tiles owe), Z *= al.  Returns
// the bias 8 - m that puts the tile's weights in units of 2^-8.
__device__ __forceinline__ float new_max(float tmax, float c, float &m, float &z, float &al)
{
    const float mnew = fmaxf(m, tmax * c);
    al = __builtin_amdgcn_exp2f(m - mnew);
    m = mnew;
    z *= al;
    return 8.0f - mnew;
}

// FP8 weight word Q of one tile (logits s[Q / 4][4 (Q % 4) .. + 3]):
// e = 2^(S c8 + 8 - m) = 256 w, Z += e, P word Q = e4m3(e) (four keys) of the
// B operand of P^T V.
template <int Q>
__device__ __forceinline__ void weight_word_fp8(const v16f (&s)[2], float c8, float bias, float &z, v8i &p)
{
    constexpr int mm = Q >> 2, r0 = 4 * (Q & 3);
    const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mm][r0 + 0], c8, bias));
    const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mm][r0 + 1], c8, bias));
    const float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mm][r0 + 2], c8, bias));
    const float e3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mm][r0 + 3], c8, bias));
    z += (e0 + e1) + (e2 + e3);
    int wd = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, any_int(), false);
    p[Q] = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, wd, true);
}

// MXFP4 block exponent of this lane's 32-key group: floor(log2(max e)) - 2,
// where the group's largest logit is gm and the tile's is mx (tm = mx c).
// The group holding the running maximum has max e = 2^8 exactly (w = 1), so
// its exponent is fixed at 6 instead of being read from a rounded exp2 that
// may land just below the power of two.
__device__ __forceinline__ int fp4_exponent(float gm, float mx, float tm, float m, float c, float bias)
{
    if (gm == mx && m == tm)
        return 127 + 6;
    const float emax = __builtin_amdgcn_exp2f(__builtin_fmaf(gm, c, bias));
    const int ef = (int)((__float_as_uint(emax) >> 23) & 0xffu) - 2;
    return ef < 0 ? 0 : ef;
}

// MXFP4 weight word Q of one tile (slots 8 Q .. 8 Q + 7 of the lane's 32-key
// group, logits s[Q / 2][8 (Q % 2) .. + 7]), with c = log2(e)/sqrt(d) and the
// group's scale 2^(ef - 127).
template <int Q>
__device__ __forceinline__ void weight_word_fp4(const v16f (&s)[2], float c, float bias, float pscale, float &z,
                                                v8i &p)
{
    constexpr int mm = Q >> 1, r0 = 8 * (Q & 1);
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        e[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mm][r0 + j], c, bias));
        z += e[j];
    }
    uint32_t wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((uint32_t)any_int(), e[0], e[1], pscale, 0);
    wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, e[2], e[3], pscale, 1);
    wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, e[4], e[5], pscale, 2);
    p[Q] = (int)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, e[6], e[7], pscale, 3);
}

// Logits of key half mm of one tile (S^T = K Q^T, FP8 codes, or MXFP4 with
// block scales; query operand as in logits).
template <int D, bool FP8>
__device__ __forceinline__ void logits_half(const KRegs<D> &K, int mm, const v8i (&qv)[D / 64], v16f &s)
{
    constexpr int KC = D / 64;
    s = (v16f){};
#pragma unroll
    for (int kc = 0; kc < KC; kc++) {
        if (FP8)
            s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(K.k[mm][kc], qv[kc], s, 0, 0, 0, 0, 0, 0);
        else
            s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(K.k[mm][kc], qv[kc], s, 4, 4, 0, K.ks[mm][kc],
                                                               0, qv[kc][4]);
    }
}

// Wait until at most n vector-memory operations of this wave are pending
// (expcnt and lgkmcnt left alone).
__device__ __forceinline__ constexpr int vm_wait(int n)
{
    return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// 1 KB chunk c of a 16-bit tile image held in two buffers of D/16 chunks.
template <int D>
__device__ __forceinline__ uint8_t *chunk16(uint8_t *b0, uint8_t *b1, int c)
{
    return (c < D / 16 ? b0 : b1) + (c % (D / 16)) * 1024;
}

// Key tiles of the 16-bit path.  A key source says which tile the i-th step
// takes, copies that tile's key image (64 key rows x D channels, bf16,
// gathered straight from K: chunk (m, s) holds for lane l key row
// key_of_row(l % 32, m), channels 16 s + 8 (l / 32) .. + 7) into this wave's
// half of the key buffers, and locates the value images (the bf16 operand
// written by the V preparation, one 64 x D image per tile).
//
// Video regions of one head: the schedule's 16-bit list, or (DENSE) the
// regions first, first + 1, ... in order.  On the 8x8 grid the key rows are
// gathered straight from K (a fixed byte offset per lane from the region's
// first token); a ragged layout copies the bf16 key image its K preparation
// wrote and masks the region's padding slots.
template <int D, bool DENSE, bool RAG>
struct VideoKeys16 {
    static constexpr bool kMasked = RAG;
    const int32_t *list;
    int first;
    const uint16_t *kh;            // K of this head
    const uint8_t *vbase;          // value images of the head's regions
    int64_t vbytes;
    const uint8_t *kimg;           // ragged: key images of the head's regions
    const int32_t *nreg;           // ragged: valid tokens per region
    uint32_t koff;                 // grid: this lane's byte offset from a region's first token;
                                   // ragged: this lane's byte offset in a key-image chunk
    int kspan, Ry, Rx, Hv, Wv, w;
    int64_t osn;

    __device__ __forceinline__ VideoKeys16(const AttnArgs &A, const int32_t *list_, int first_, int64_t hoff,
                                           int64_t hbase, int w_, int l)
        : list(list_), first(first_), kh(A.k + hoff), nreg(A.nreg), kspan(A.kspan), Ry(A.Ry), Rx(A.Rx),
          Hv(A.Hv), Wv(A.Wv), w(w_), osn(A.osn)
    {
        if (RAG) {
            koff = (uint32_t)l * 16u;
        } else {
            // wave w gathers the key rows of half m = w
            const int kpos = key_of_row(l & 31, w_);
            koff = (uint32_t)((((kpos >> 3) * A.Wv + (kpos & 7)) * A.osn + 8 * (l >> 5)) * 2);
        }
        vbase = A.v16 + hbase * (kBlk * D * 2);
        vbytes = (int64_t)A.R * kBlk * D * 2;
        kimg = A.k16 + hbase * (kBlk * D * 2);
    }
    __device__ __forceinline__ int id(int i) const { return DENSE ? first + i : sload_i32(list + i); }
    __device__ __forceinline__ int valid(int kb) const { return RAG ? sload_i32(nreg + kb) : kBlk; }
    __device__ __forceinline__ void issue_key(int kb, uint8_t *dst) const
    {
        if (RAG) {
            // chunks (w, s) of the region's key image: 1 KB each
            const __amdgpu_buffer_rsrc_t ksrc = head_rsrc(kimg, vbytes);
#pragma unroll
            for (int s = 0; s < D / 16; s++)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ksrc, (lds_void *)(dst + s * 1024), 16, koff,
                                                         (uint32_t)kb * (kBlk * D * 2) + (w * (D / 16) + s) * 1024,
                                                         0, 0);
        } else {
            const int t0 = region_token(kb, 0, Ry, Rx, Hv, Wv);
            const __amdgpu_buffer_rsrc_t ksrc = head_rsrc((const uint8_t *)(kh + (int64_t)t0 * osn), kspan);
#pragma unroll
            for (int s = 0; s < D / 16; s++)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ksrc, (lds_void *)(dst + s * 1024), 16, koff, 32 * s,
                                                         0, 0);
        }
    }
};

// Text-prefix keys of one head (App. C.1): tile t holds prefix keys
// 64 t .. 64 t + 63, of which the first nv - 64 t are valid; the steps take
// tiles first, first + 1, ...  Rows past the valid ones are read from the
// last valid row (their logits are masked, so only the address matters);
// their value rows are zero in the value image.
template <int D>
struct PrefixKeys16 {
    static constexpr bool kMasked = true;
    int first;
    __amdgpu_buffer_rsrc_t ksrc;   // prefix K rows of this head
    const uint8_t *vbase;          // prefix value images of this head
    int64_t vbytes;
    int kpos, nv;
    uint32_t lane_off;             // channel offset of this lane, bytes
    int64_t osn;

    __device__ __forceinline__ PrefixKeys16(const AttnArgs &A, int first_, int64_t hoff, int bh, int nv_, int w,
                                            int l)
        : first(first_), nv(nv_), osn(A.osn)
    {
        kpos = key_of_row(l & 31, w);
        lane_off = (uint32_t)(16 * (l >> 5));
        ksrc = head_rsrc((const uint8_t *)(A.kp + hoff), A.pkspan);
        vbase = A.vp16 + (int64_t)bh * A.ptiles * (kBlk * D * 2);
        vbytes = (int64_t)A.ptiles * kBlk * D * 2;
    }
    __device__ __forceinline__ int id(int i) const { return first + i; }
    __device__ __forceinline__ int valid(int kb) const { return nv - kBlk * kb; }
    __device__ __forceinline__ void issue_key(int kb, uint8_t *dst) const
    {
        const int row = min(kBlk * kb + kpos, nv - 1);
        const uint32_t off = (uint32_t)(row * osn * 2) + lane_off;
#pragma unroll
        for (int s = 0; s < D / 16; s++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ksrc, (lds_void *)(dst + s * 1024), 16, off, 32 * s, 0, 0);
    }
};

// This wave's queries as B operands of the 16-bit logits (lane l: query row
// qr, channels 16 s + 8 (l / 32) .. + 7 of step s).
template <int D>
__device__ __forceinline__ void load_q16(const uint16_t *qr, int l, v4u (&q16)[D / 16])
{
#pragma unroll
    for (int s = 0; s < D / 16; s++)
        q16[s] = *reinterpret_cast<const v4u *>(qr + 8 * (l >> 5) + 16 * s);
}

// 16-bit path over n tiles of a key source (ascending).  A tile's key image
// fills both key buffers (half m in buffer m), its value image both value
// buffers.  The two streams overlap each other's use: the value copy of tile
// i runs under tile i's logits and softmax, the key copy of tile i+1 under
// tile i's softmax and P^T V.  Key and value buffers are distinct LDS
// variables, so the compiler knows a copy into one never feeds reads of the
// other.  Semantics per tile: S from the bf16 operands as they are (exact
// products, fp32 sums); masked keys get S = -inf; m = max(m, max S c4);
// e = 2^(S c4 + 8 - m); Z += e; P = bf16(e) (nearest even); acc += P^T V.
template <int D, class Keys>
__device__ __forceinline__ void run16(const AttnArgs &A, uint8_t *kb0, uint8_t *kb1, uint8_t *vb0,
                                      uint8_t *vb1, const Keys &K, int n16, const v4u (&q16)[D / 16],
                                      int w, int l, v16f (&acc)[D / 32], float &m, float &z)
{
    constexpr int KS = D / 16;                 // 16-channel steps of QK^T
    constexpr int CB = D / 32;
    constexpr int NK = KS;                     // key copies per wave and tile
    const int hf = l >> 5;
    const __amdgpu_buffer_rsrc_t vsrc = head_rsrc(K.vbase, K.vbytes);
    int kb = K.id(0);
    int kbn = n16 > 1 ? K.id(1) : 0;
    K.issue_key(kb, w ? kb1 : kb0);
    for (int i = 0; i < n16; i++) {
        // key image of tile i complete (both waves' halves); both waves are
        // done with the value buffer
        __builtin_amdgcn_s_waitcnt(vm_wait(0));
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kBlk * D * 2 / 2048; j++) {
            // unit 2j + w lies in the first buffer exactly when j < D / 32
            const int u = 2 * j + w;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                vsrc, (lds_void *)((j < D / 32 ? vb0 : vb1) + (u % (D / 16)) * 1024), 16, (uint32_t)l * 16u,
                (uint32_t)kb * (kBlk * D * 2) + u * 1024, 0, 0);
        }
        v16f sc[2];
        sc[0] = (v16f){};
        sc[1] = (v16f){};
#pragma unroll
        for (int s = 0; s < KS; s++)
#pragma unroll
            for (int mm = 0; mm < 2; mm++)
                sc[mm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    as_bf16x8(lds_v4u(chunk16<D>(kb0, kb1, mm * KS + s) + l * 16)), as_bf16x8(q16[s]), sc[mm], 0,
                    0, 0);
        // both waves are done with the key buffer: refill it with tile i+1
        __syncthreads();
        const bool more = i + 1 < n16;
        if (more)
            K.issue_key(kbn, w ? kb1 : kb0);
        if (Keys::kMasked) {
            // register r of half mm holds key 32 hf + 16 mm + r
            const int nk = K.valid(kb);
            if (nk < kBlk) {
#pragma unroll
                for (int mm = 0; mm < 2; mm++)
#pragma unroll
                    for (int r = 0; r < 16; r++)
                        if (32 * hf + 16 * mm + r >= nk)
                            sc[mm][r] = -__builtin_huge_valf();
            }
        }
        const float c = A.c4;
        const float mnew = fmaxf(m, pair_max(lane_max(sc)) * c);
        rescale<CB>(acc, z, __builtin_amdgcn_exp2f(m - mnew));
        m = mnew;
        const float bias = 8.0f - mnew;
        // P^T chunk t: this lane's keys 32 hf + 8 t .. + 7 (slots 8 t ..)
        v4u p[4];
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const int mm = t >> 1, r0 = 8 * (t & 1);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[mm][r0 + 2 * j], c, bias));
                const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[mm][r0 + 2 * j + 1], c, bias));
                z += e0 + e1;
                p[t][j] = (uint32_t)f32_to_bf16(e0) | ((uint32_t)f32_to_bf16(e1) << 16);
            }
        }
        // value image of tile i complete: only the key copy may still run
        if (more)
            __builtin_amdgcn_s_waitcnt(vm_wait(NK));
        else
            __builtin_amdgcn_s_waitcnt(vm_wait(0));
        __syncthreads();
#pragma unroll
        for (int cb = 0; cb < CB; cb++)
#pragma unroll
            for (int t = 0; t < 4; t++)
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    as_bf16x8(lds_v4u(chunk16<D>(vb0, vb1, cb * 4 + t) + l * 16)), as_bf16x8(p[t]), acc[cb], 0, 0,
                    0);
        kb = kbn;
        if (i + 2 < n16)
            kbn = K.id(i + 2);
    }
    // the next segment or phase refills both buffers
    __syncthreads();
}

// O = acc / Z for this lane's query, written at element offset obase of the
// output (this lane's channels 32 cb + 8 g + 4 hf .. + 3).
template <int D>
__device__ __forceinline__ void store_row(const AttnArgs &A, void *out, int64_t obase, const v16f (&acc)[D / 32],
                                          float inv, int hf)
{
#pragma unroll
    for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int c0 = 32 * cb + 8 * g + 4 * hf;
            float o0 = acc[cb][4 * g] * inv, o1 = acc[cb][4 * g + 1] * inv;
            float o2 = acc[cb][4 * g + 2] * inv, o3 = acc[cb][4 * g + 3] * inv;
            if (A.out_f32) {
                *reinterpret_cast<float4 *>((float *)out + obase + c0) = make_float4(o0, o1, o2, o3);
            } else {
                uint2 pk;
                pk.x = (uint32_t)f32_to_bf16(o0) | ((uint32_t)f32_to_bf16(o1) << 16);
                pk.y = (uint32_t)f32_to_bf16(o2) | ((uint32_t)f32_to_bf16(o3) << 16);
                *reinterpret_cast<uint2 *>((uint16_t *)out + obase + c0) = pk;
            }
        }
}

// Valid prefix keys of batch element b: the caller's count clamped to
// [0, Lp] (all Lp when no counts are given).
__device__ __forceinline__ int prefix_valid(const AttnArgs &A, int b)
{
    if (A.Lp == 0)
        return 0;
    if (!A.pvalid)
        return A.Lp;
    return min(max(sload_i32(A.pvalid + b), 0), A.Lp);
}

// Instruction order inside one region of a step's main block: its LDS reads
// first, then its matrix products spread through its vector instructions, so
// the wave never waits for the matrix core to accept a product while it has
// vector work to issue.
__device__ __forceinline__ void region_pattern()
{
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // LDS reads
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
#pragma unroll
    for (int j = 0; j < 2; j++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
    }
}

// Padding slots of a ragged key region take no part: slots n .. 63 (at most
// PMAX of them, n >= 48) are registers n - 48 .. 15 of logit half 1 on the
// lanes of half 1 (slot 32 hf + 16 m + r is register r of half m).
template <int PMAX>
__device__ __forceinline__ void mask_padding(v16f &s1, int n, int hf)
{
    const bool upper = hf != 0;
#pragma unroll
    for (int r = 16 - PMAX; r < 16; r++) {
        const bool pad = upper & (48 + r >= n);
        s1[r] = pad ? -__builtin_huge_valf() : s1[r];
    }
}

// One attention workgroup's state: two waves, one query region (wave w owns
// queries 32 w .. 32 w + 31).  RAG: ragged layout (slot tables); PMAX: most
// padding slots of a key region (0, 4 or 16).
template <int D, bool RAG, int PMAX>
struct Attn {
    static constexpr int KC = D / 64;   // 64-channel steps of QK^T
    static constexpr int CB = D / 32;   // 32-channel blocks of the output
    const AttnArgs &A;
    // key and value buffers, two of each; four distinct LDS variables, so
    // that the compiler can tell a copy into one from a read of another
    uint8_t *kb0, *kb1, *vb0, *vb1;
    const int32_t *list;   // key regions of the tiles, in phase order
    int64_t hbase;
    Src src;
    int n8, n, w, l, hf, bh;
    int64_t qblk;
    float qs;
    v8i qv[KC];   // this wave's queries in the format of the next logits (see logits)
    v16f acc[CB];
    float m, z;
    // Software pipeline state.  Step i forms the weights of tile i while the
    // matrix core computes the logits of tile i+1 and P^T V of tile i-1, so
    // the logits (S) and the weights (P, with the MXFP4 exponent e) live in
    // two register sets each, used by steps of alternating parity.
    v16f S0[2], S1[2];
    v8i P0, P1;
    int E0, E1;
    float al;           // factor acc owes before the next P^T V (running-max change)
    int kr0, kr1, kr2;  // key regions of tiles i, i+1, i+2 (wave-uniform)
    int nk0;            // valid tokens of tile i's key region (PMAX > 0)
    float c8;           // FP8 logit scale of tile i

    __device__ __forceinline__ void vunits(bool to_fp8)
    {
        // change of value units: real <-> FP8 codes (per-channel V scale).
        // The scales are loaded where they are used (volatile): loaded once
        // for both uses, they would stay in 64 registers through the phases.
        const volatile float4 *vs = reinterpret_cast<const volatile float4 *>(A.vs8 + (int64_t)bh * D);
#pragma unroll
        for (int cb = 0; cb < CB; cb++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const float4 sv = const_cast<const float4 &>(vs[(32 * cb + 8 * g + 4 * hf) / 4]);
                const float f[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
                for (int t = 0; t < 4; t++)
                    acc[cb][4 * g + t] = to_fp8 ? acc[cb][4 * g + t] / f[t] : acc[cb][4 * g + t] * f[t];
            }
    }

    // acc *= al before the next P^T V; with UNIT the FP8 -> real change of
    // value units is applied as well (the product about to be added is the
    // first MXFP4 one).
    template <bool UNIT>
    __device__ __forceinline__ void settle()
    {
        if (UNIT) {
#pragma unroll
            for (int cb = 0; cb < CB; cb++)
                acc[cb] *= al;
            vunits(false);
        } else if (__any(al != 1.0f)) {
#pragma unroll
            for (int cb = 0; cb < CB; cb++)
                acc[cb] *= al;
        }
    }

    template <bool FP8>
    __device__ __forceinline__ void pv_range(const VRegs<D> &V, const v8i &p, int ef, int c0, int c1)
    {
        if (FP8) {
#pragma unroll
            for (int cb = c0; cb < c1; cb++)
                acc[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(V.v[cb], p, acc[cb], 0, 0, 0, 0, 0, 0);
        } else {
#pragma unroll
            for (int cb = c0; cb < c1; cb++)
                acc[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(V.v[cb], p, acc[cb], 4, 4, 0,
                                                                         V.vs[cb], 0, ef);
        }
    }

    // Step i, kinds KP (tile i-1), KCUR (tile i), KN (tile i+1) true for FP8.
    // On entry sc holds the logits of tile i, pp / ep the weights of tile i-1
    // (zero before the first tile), al the factor acc owes before their
    // product.  The refills go first: K(i+2)
    // into K(i)'s buffer kw and V(i) into V(i-2)'s buffer vw, both read for
    // the last time in step i-1.  Then K(i+1) and V(i-1) are read from kr and
    // vr, each half just before its products.  The last step computes logits
    // of a stale key image, which are never used (kinds KN = KCUR there).
    template <bool KP, bool KCUR, bool KN, bool UNIT>
    __device__ __forceinline__ void step(int i, v16f (&sc)[2], v16f (&sn)[2], const v8i &pp, int ep,
                                         v8i &pc, int &ec, const uint8_t *__restrict__ kr,
                                         uint8_t *__restrict__ kw, const uint8_t *__restrict__ vr,
                                         uint8_t *__restrict__ vw)
    {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        settle<UNIT>();
        if (i + 2 < n) {
            if (i + 2 < n8)
                issue_k<D, true>(src, kr2, kw, w, l);
            else
                issue_k<D, false>(src, kr2, kw, w, l);
        }
        issue_v<D, KCUR>(src, kr0, vw, w, l);
        VRegs<D> V;
        KRegs<D> K;
        // main block: weights of tile i on the vector unit, products of tiles
        // i-1 and i+1 on the matrix core, in regions fenced from each other.
        // Each region reads the operands of the next region's products from
        // LDS, issues its own products (operands read by the region before)
        // and forms a quarter of the weights:
        //   R0: running max; read V blocks [0, CB/2)
        //   R1: P^T V blocks [0, CB/2);  read V blocks [CB/2, CB); weights 1/4
        //   R2: P^T V blocks [CB/2, CB); read K half 0;          weights 2/4
        //   R3: logits half 0 (into the registers of the logits weights 1/4
        //       and 2/4 consumed);        read K half 1;          weights 3/4
        //   R4: logits half 1;                                    weights 4/4
        float c, bias, pscale = 0.0f;
        if (PMAX > 0)
            mask_padding<PMAX>(sc[1], nk0, hf);
        if (KCUR) {
            c = c8;
            bias = new_max(pair_max(lane_max(sc)), c, m, z, al);
        } else {
            c = A.c4;
            const float gm = lane_max(sc);
            const float mx = pair_max(gm);
            bias = new_max(mx, c, m, z, al);
            ec = fp4_exponent(gm, mx, mx * c, m, c, bias);
            pscale = ec ? __uint_as_float((uint32_t)ec << 23) : __uint_as_float(0x00400000u);
        }
        read_v_range<D, KP>(vr, l, 0, CB / 2, V);
        __builtin_amdgcn_sched_barrier(0);
        // R1
        pv_range<KP>(V, pp, ep, 0, CB / 2);
        read_v_range<D, KP>(vr, l, CB / 2, CB, V);
        if (KCUR) {
            weight_word_fp8<0>(sc, c, bias, z, pc);
            weight_word_fp8<1>(sc, c, bias, z, pc);
        } else {
            weight_word_fp4<0>(sc, c, bias, pscale, z, pc);
        }
        region_pattern();
        __builtin_amdgcn_sched_barrier(0);
        // R2
        pv_range<KP>(V, pp, ep, CB / 2, CB);
        read_k_half<D, KN>(kr, l, 0, K);
        if (KCUR) {
            weight_word_fp8<2>(sc, c, bias, z, pc);
            weight_word_fp8<3>(sc, c, bias, z, pc);
        } else {
            weight_word_fp4<1>(sc, c, bias, pscale, z, pc);
        }
        region_pattern();
        __builtin_amdgcn_sched_barrier(0);
        // R3
        logits_half<D, KN>(K, 0, qv, sn[0]);
        read_k_half<D, KN>(kr, l, 1, K);
        if (KCUR) {
            weight_word_fp8<4>(sc, c, bias, z, pc);
            weight_word_fp8<5>(sc, c, bias, z, pc);
        } else {
            weight_word_fp4<2>(sc, c, bias, pscale, z, pc);
        }
        region_pattern();
        __builtin_amdgcn_sched_barrier(0);
        // R4
        logits_half<D, KN>(K, 1, qv, sn[1]);
        if (KCUR) {
            weight_word_fp8<6>(sc, c, bias, z, pc);
            weight_word_fp8<7>(sc, c, bias, z, pc);
        } else {
            weight_word_fp4<3>(sc, c, bias, pscale, z, pc);
            pc[4] = any_int(); pc[5] = any_int(); pc[6] = any_int(); pc[7] = any_int();
        }
        region_pattern();
        // Z, the packed weights and the next logits are complete within the
        // step: otherwise the compiler sinks their additions, conversions and
        // products into the next step (keeping every weight of this tile live
        // across the barrier, or serializing the next row maximum behind the
        // products).
        asm volatile("" ::"v"(z), "v"(pc), "v"(sn[0]), "v"(sn[1]));
        // wave-uniform values of the next step, loaded without branches so
        // that the main block stays one scheduling region (indices past the
        // list are clamped; such values and the logit scale of an MXFP4 tile
        // are never used)
        kr0 = kr1;
        kr1 = kr2;
        kr2 = sload_i32(list + min(i + 3, n - 1));
        c8 = (qs * sload_f32(A.ks8 + hbase + kr0)) * A.c4;
        if (PMAX > 0)
            nk0 = sload_i32(A.nreg + kr0);
    }

    // Step i with the register sets and buffers of an even or an odd step.
    template <bool KP, bool KCUR, bool KN, bool UNIT>
    __device__ __forceinline__ void step_even(int i)
    {
        step<KP, KCUR, KN, UNIT>(i, S0, S1, P1, E1, P0, E0, kb1, kb0, vb1, vb0);
    }

    template <bool KP, bool KCUR, bool KN, bool UNIT>
    __device__ __forceinline__ void step_odd(int i)
    {
        step<KP, KCUR, KN, UNIT>(i, S1, S0, P0, E0, P1, E1, kb0, kb1, vb0, vb1);
    }

    template <bool ODD, bool KP, bool KCUR, bool KN, bool UNIT>
    __device__ __forceinline__ void step_par(int i)
    {
        if (ODD)
            step_odd<KP, KCUR, KN, UNIT>(i);
        else
            step_even<KP, KCUR, KN, UNIT>(i);
    }

    // Queries of this wave in one format, loaded when the first logits of
    // that format are due, into the one query operand set.
    __device__ __forceinline__ void load_q8()
    {
#pragma unroll
        for (int kc = 0; kc < KC; kc++)
            qv[kc] = load32(A.q8 + qblk * (kBlk * D) + ((w * KC + kc) * 64 + l) * 32);
    }

    // (volatile: a second load before the MXFP4 loop gives the loop its
    // own short live range instead of one spanning the phase boundary)
    __device__ __forceinline__ void load_q4()
    {
#pragma unroll
        for (int kc = 0; kc < KC; kc++) {
            const int chunk = (w * KC + kc) * 64 + l;
            const uint4 c = const_cast<const uint4 &>(
                *reinterpret_cast<const volatile uint4 *>(A.q4 + qblk * (kBlk * D / 2) + chunk * 16));
            qv[kc][0] = c.x;
            qv[kc][1] = c.y;
            qv[kc][2] = c.z;
            qv[kc][3] = c.w;
            qv[kc][4] = *(const volatile uint8_t *)(A.q4s + qblk * (2 * D) + chunk);
        }
    }

    // FP8 tiles [0, n8), then MXFP4 tiles [n8, n).  Step i uses the register
    // sets and buffers of parity (i + off) % 2, with off = 1 - n8 % 2: the
    // last FP8 step is then always even, so every step's sets and buffers are
    // fixed at compile time (a lead-in step absorbs the choice).
    __device__ __forceinline__ void quantized_phases()
    {
        if (n == 0)
            return;
        if (n8 > 0)
            load_q8();
        else
            load_q4();
        const bool off = !(n8 & 1);
        // prologue: keys of tiles 0 and 1, logits of tile 0
        kr0 = sload_i32(list);
        kr1 = n > 1 ? sload_i32(list + 1) : 0;
        kr2 = n > 2 ? sload_i32(list + 2) : 0;
        uint8_t *k0 = off ? kb1 : kb0, *k1 = off ? kb0 : kb1;
        if (n8 > 0)
            issue_k<D, true>(src, kr0, k0, w, l);
        else
            issue_k<D, false>(src, kr0, k0, w, l);
        if (n > 1) {
            if (n8 > 1)
                issue_k<D, true>(src, kr1, k1, w, l);
            else
                issue_k<D, false>(src, kr1, k1, w, l);
        }
        c8 = n8 > 0 ? (qs * sload_f32(A.ks8 + hbase + kr0)) * A.c4 : 0.0f;
        if (PMAX > 0)
            nk0 = sload_i32(A.nreg + kr0);
        // step 0 multiplies P = 0 into the value buffer of the other parity:
        // clear it so that no stale code can make a NaN
        uint8_t *vz = off ? vb0 : vb1;
#pragma unroll
        for (int u = 0; u < kBlk * D / (128 * 16); u++)
            *reinterpret_cast<v4u *>(vz + (u * 128 + threadIdx.x) * 16) = (v4u){};
        P0 = (v8i){};
        P1 = (v8i){};
        E0 = 127;
        E1 = 127;
        al = 1.0f;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        {
            KRegs<D> K;
            if (n8 > 0) {
                read_k<D, true>(k0, l, K);
                if (off)
                    logits<D, true>(K, qv, S1);
                else
                    logits<D, true>(K, qv, S0);
            } else {
                read_k<D, false>(k0, l, K);
                logits<D, false>(K, qv, S1);   // n8 = 0: off
            }
        }
        int i = 0;
        if (n8 > 0) {
            // FP8 steps whose successor is FP8, except the last FP8 step
            if (off) {
                step_odd<true, true, true, false>(0);
                i = 1;
            }
            for (; i < n8 - 1; i += 2) {
                step_even<true, true, true, false>(i);
                step_odd<true, true, true, false>(i + 1);
            }
            // the last FP8 step (even), then the first MXFP4 step (odd) and
            // the step adding the first MXFP4 product (even)
            if (n8 == n) {
                step_even<true, true, true, false>(i++);
            } else {
                load_q4();
                step_even<true, true, false, false>(i++);
                step_odd<true, false, false, false>(i++);
                if (i < n)
                    step_even<false, false, false, true>(i++);
            }
        }
        // MXFP4 steps, starting odd
        if (n8 > 0 && i + 1 < n)
            load_q4();
        for (; i + 1 < n; i += 2) {
            step_odd<false, false, false, false>(i);
            step_even<false, false, false, false>(i + 1);
        }
        if (i < n)
            step_odd<false, false, false, false>(i);
        // drain: P^T V of the last tile, and the change of value units when
        // the last product added is an FP8 one, or when the first MXFP4
        // product is the last
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const bool last8 = n - 1 < n8;
        const bool lodd = (n - 1 + (int)off) & 1;
        VRegs<D> V;
        const v8i pl = lodd ? P1 : P0;   // by value: a reference would keep both sets in memory
        const int el = lodd ? E1 : E0;
        if (last8) {
            settle<false>();
            read_v<D, true>(lodd ? vb1 : vb0, l, V);
            pv<true>(V, pl, el);
            vunits(false);
        } else {
            if (n - 1 == n8 && n8 > 0)
                settle<true>();
            else
                settle<false>();
            read_v<D, false>(lodd ? vb1 : vb0, l, V);
            pv<false>(V, pl, el);
        }
    }

    template <bool FP8>
    __device__ __forceinline__ void pv(const VRegs<D> &V, const v8i &p, int ef)
    {
        pv_range<FP8>(V, p, ef, 0, CB);
    }

    // 16-bit segments of query region a: the text-prefix keys (np tiles, nv
    // valid keys), then the schedule's 16-bit key regions
    __device__ __forceinline__ void phase16(const int32_t *list16, int n16, int np, int nv, int a)
    {
        const int bb = bh / A.H, hh = bh - bb * A.H;
        const int64_t hoff = (int64_t)bb * A.osb + (int64_t)hh * A.osh;
        v4u q16[D / 16];
        int qt = slot_token<RAG>(A.geo, a, 32 * w + (l & 31));
        if (qt < 0)   // padding slot: any valid row (its output is not written)
            qt = slot_token<RAG>(A.geo, a, 0);
        load_q16<D>(A.q + hoff + (int64_t)qt * A.osn, l, q16);
        if (np > 0)
            run16<D>(A, kb0, kb1, vb0, vb1, PrefixKeys16<D>(A, 0, hoff, bh, nv, w, l), np, q16, w, l, acc, m, z);
        if (n16 > 0)
            run16<D>(A, kb0, kb1, vb0, vb1, VideoKeys16<D, false, RAG>(A, list16, 0, hoff, hbase, w, l), n16, q16,
                     w, l, acc, m, z);
    }

    // O = acc / Z for this wave's 32 queries of region a, written straight to
    // their original token positions (the restore).  The region's block-mean
    // tiles enter first, as one key of logit M, weight z_a and value sum c_a.
    __device__ __forceinline__ void epilogue(int a)
    {
        if (A.magg) {
            const int64_t ra = (int64_t)bh * A.R + a;
            const float2 mz = A.magg[ra];
            if (mz.y > 0.0f) {
                const float mnew = fmaxf(m, mz.x);
                const float f = __builtin_amdgcn_exp2f(m - mnew), g = __builtin_amdgcn_exp2f(mz.x + 8.0f - mnew);
                z = z * f + (hf ? 0.0f : mz.y * g);   // z is summed over the lane pair
                const float *cv = A.cagg + ra * D + 4 * hf;
#pragma unroll
                for (int cb = 0; cb < CB; cb++)
#pragma unroll
                    for (int gq = 0; gq < 4; gq++) {
                        const float4 c4v = *reinterpret_cast<const float4 *>(cv + 32 * cb + 8 * gq);
                        acc[cb][4 * gq] = acc[cb][4 * gq] * f + c4v.x * g;
                        acc[cb][4 * gq + 1] = acc[cb][4 * gq + 1] * f + c4v.y * g;
                        acc[cb][4 * gq + 2] = acc[cb][4 * gq + 2] * f + c4v.z * g;
                        acc[cb][4 * gq + 3] = acc[cb][4 * gq + 3] * f + c4v.w * g;
                    }
                m = mnew;
            }
        }
        const float zt = pair_sum(z);
        const float inv = zt > 0.0f ? 1.0f / zt : 0.0f;
        const int qi = 32 * w + (l & 31);
        const int tok = slot_token<RAG>(A.geo, a, qi);
        const int b = bh / A.H, h = bh - b * A.H;
        const int64_t obase = (int64_t)b * A.osb + (int64_t)h * A.osh + (int64_t)tok * A.osn;
        if (tok >= 0)
            store_row<D>(A, A.out, obase, acc, inv, hf);
    }

    __device__ __forceinline__ void init(int w_, int bh_, int64_t qblk_)
    {
        w = w_;
        l = threadIdx.x & 63;
        hf = l >> 5;
        bh = bh_;
        qblk = qblk_;
        qs = A.qs8[qblk_];
        hbase = (int64_t)bh_ * A.R;
        src = head_sources<D>(A, hbase, A.R);
#pragma unroll
        for (int cb = 0; cb < CB; cb++)
            acc[cb] = (v16f){};
        m = -__builtin_huge_valf();
        z = 0.0f;
    }
};

// One query region per workgroup: 16-bit phase (if any), then the FP8 and
// MXFP4 phases.
template <int D, bool RAG, int PMAX>
__global__ __launch_bounds__(128, 2) void k_attn(const AttnArgs A)
{
    __shared__ __attribute__((aligned(1024))) uint8_t kb0[kBlk * D];
    __shared__ __attribute__((aligned(1024))) uint8_t kb1[kBlk * D];
    __shared__ __attribute__((aligned(1024))) uint8_t vb0[kBlk * D];
    __shared__ __attribute__((aligned(1024))) uint8_t vb1[kBlk * D];

    // XCD-aware work mapping.  Workgroups are dealt to the 8 XCDs round robin
    // (block L runs on XCD L % 8).  Every XCD walks the heads in the same
    // order and takes its own contiguous eighth (work slots j) of each head's
    // query regions, so all XCDs work on the same head at a time and that
    // head's key/value tiles (about 31 MB for a 720p Wan layer) stay in the
    // shared last-level cache.  The plan's work order maps a slot to its
    // query region (k_qorder: the share's regions are frame-fastest, ranked
    // by kept tile count).
    const int R = A.R;
    const int span = (R + 7) / 8;
    const int xcd = (int)(blockIdx.x & 7), kk = (int)(blockIdx.x >> 3);
    const int bh = kk / span;
    const int j = xcd * span + (kk - bh * span);
    if (j >= R)
        return;
    const int a = sload_i32(A.qord + (int64_t)bh * R + j);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t qblk = (int64_t)bh * R + a;

    Attn<D, RAG, PMAX> S{A, kb0, kb1, vb0, vb1};
    S.init(w, bh, qblk);
    const int n16 = sload_i32(A.cnt + qblk * kTargets);
    const int n8 = sload_i32(A.cnt + qblk * kTargets + 1);
    S.n8 = n8;
    S.n = n8 + sload_i32(A.cnt + qblk * kTargets + 2);
    S.list = A.sched + qblk * R + n16;
    const int nv = prefix_valid(A, bh / A.H);
    const int np = (nv + kBlk - 1) / kBlk;
    if (n16 > 0 || np > 0) {
        S.phase16(A.sched + qblk * R, n16, np, nv, a);
        if (n8 > 0)
            S.vunits(true);   // phase boundary: real units -> FP8 value units
    }
    S.quantized_phases();
    S.epilogue(a);
}

// Prefix query rows (App. C.1: non-sparse attention).  A row's key sequence
// is its valid prefix tiles, then every video region in order, all on the
// 16-bit path; it is cut into chunks of kPrefixChunkTiles consecutive tiles.
// One workgroup takes 64 rows of one (b, h) (wave w owning rows 32 w ..
// 32 w + 31) and one chunk, runs its own online softmax over the chunk and
// leaves the chunk's state (running max m, sum Z, unnormalised output) for
// the merge.  Rows past Lp (the last workgroup's tail) compute on a copy of
// row Lp - 1 and are not written.
template <int D, bool RAG>
__device__ __forceinline__ void prefix_rows(const AttnArgs &A, uint8_t *kb0, uint8_t *kb1, uint8_t *vb0,
                                            uint8_t *vb1, int pb, int bh, int c, int w, int l)
{
    const int b = bh / A.H, h = bh - b * A.H;
    const int64_t hoff = (int64_t)b * A.osb + (int64_t)h * A.osh;
    const int row = kBlk * pb + 32 * w + (l & 31);
    v4u q16[D / 16];
    load_q16<D>(A.qp + hoff + (int64_t)min(row, A.Lp - 1) * A.osn, l, q16);
    v16f acc[D / 32];
#pragma unroll
    for (int cb = 0; cb < D / 32; cb++)
        acc[cb] = (v16f){};
    float m = -__builtin_huge_valf(), z = 0.0f;
    const int nv = prefix_valid(A, b);
    const int np = (nv + kBlk - 1) / kBlk;
    const int t0 = c * kPrefixChunkTiles, t1 = min(t0 + kPrefixChunkTiles, np + A.R);
    if (t0 < np)
        run16<D>(A, kb0, kb1, vb0, vb1, PrefixKeys16<D>(A, t0, hoff, bh, nv, w, l), min(t1, np) - t0, q16, w,
                 l, acc, m, z);
    const int r0 = max(t0, np) - np, r1 = t1 - np;
    if (r1 > r0)
        run16<D>(A, kb0, kb1, vb0, vb1, VideoKeys16<D, true, RAG>(A, nullptr, r0, hoff, (int64_t)bh * A.R, w, l),
                 r1 - r0, q16, w, l, acc, m, z);
    const float zt = pair_sum(z);
    if (row < A.Lp) {
        const int64_t slot = ((int64_t)bh * A.pchunks + c) * (A.ptiles * kBlk) + row;
        float *dst = A.pacc + slot * D;
        const int hf = l >> 5;
#pragma unroll
        for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
            for (int g = 0; g < 4; g++)
                *reinterpret_cast<float4 *>(dst + 32 * cb + 8 * g + 4 * hf) =
                    make_float4(acc[cb][4 * g], acc[cb][4 * g + 1], acc[cb][4 * g + 2], acc[cb][4 * g + 3]);
        if (hf == 0)
            A.pmz[slot] = make_float2(m, zt);
    }
}

template <int D, bool RAG>
__global__ __launch_bounds__(128, 2) void k_attn_prefix(const AttnArgs A)
{
    __shared__ __attribute__((aligned(1024))) uint8_t kb0[kBlk * D];
    __shared__ __attribute__((aligned(1024))) uint8_t kb1[kBlk * D];
    __shared__ __attribute__((aligned(1024))) uint8_t vb0[kBlk * D];
    __shared__ __attribute__((aligned(1024))) uint8_t vb1[kBlk * D];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    prefix_rows<D, RAG>(A, kb0, kb1, vb0, vb1, (int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z, w,
                        (int)(threadIdx.x & 63));
}

// Block-mean tiles of a query region ([Triage] abstract: a skipped tile
// replaced by its block means): tile (a, b) scores all its queries with the
// mean of its token scores, the average-branch draft logit s_ab = q_a . k_b /
// sqrt(d), and counts the key region's n_b tokens with their mean value v_b.
// The region's mean tiles gather into one term: t_b = fp32(s_ab log2 e),
// M = max t_b, z = sum n_b 2^(t_b - M), c = sum n_b 2^(t_b - M) v_b, c
// summed in key order.  One 64-thread workgroup per (b, h) and kMeanRows
// consecutive query regions; thread t owns D / 64 consecutive channels.  Per
// chunk of 64 key regions thread t forms the weights of key region b0 + t
// for every row into LDS, then each mean value is read once and applied to
// all the rows.
constexpr int kMeanRows = 16;

template <int D>
__global__ __launch_bounds__(64) void k_mean_agg(const uint8_t *__restrict__ tier, const double *__restrict__ la,
                                                  const int32_t *__restrict__ nreg, int R,
                                                  const float *__restrict__ vavg, float2 *__restrict__ magg,
                                                  float *__restrict__ cagg)
{
    constexpr int CPT = D / 64;   // channels per thread
    __shared__ __attribute__((aligned(16))) float wt[64][kMeanRows];
    const int a0 = blockIdx.x * kMeanRows, bh = blockIdx.y, t = threadIdx.x;
    const int nq = min(kMeanRows, R - a0);
    const int64_t row0 = (int64_t)bh * R + a0;
    constexpr double kL2e = 1.4426950408889634;
    float M[kMeanRows];
#pragma unroll
    for (int q = 0; q < kMeanRows; q++) {
        float m = -__builtin_huge_valf();
        if (q < nq) {
            const uint8_t *trow = tier + (row0 + q) * R;
            const double *lrow = la + (row0 + q) * R;
            for (int b = t; b < R; b += 64)
                if (trow[b] == kMeanTier)
                    m = fmaxf(m, (float)(lrow[b] * kL2e));
        }
        for (int o = 32; o > 0; o >>= 1)
            m = fmaxf(m, __shfl_xor(m, o));
        M[q] = m;
    }
    float z[kMeanRows], c[kMeanRows][CPT];
#pragma unroll
    for (int q = 0; q < kMeanRows; q++) {
        z[q] = 0.0f;
#pragma unroll
        for (int u = 0; u < CPT; u++)
            c[q][u] = 0.0f;
    }
    const float *vhead = vavg + (int64_t)bh * R * D + t * CPT;
    for (int b0 = 0; b0 < R; b0 += 64) {
        const int b = b0 + t;
        const float nb = b < R ? (float)(nreg ? nreg[b] : kBlk) : 0.0f;
#pragma unroll
        for (int q = 0; q < kMeanRows; q++) {
            float w = 0.0f;
            if (q < nq && b < R && tier[(row0 + q) * R + b] == kMeanTier)
                w = nb * __builtin_amdgcn_exp2f((float)(la[(row0 + q) * R + b] * kL2e) - M[q]);
            z[q] += w;
            wt[t][q] = w;
        }
        __syncthreads();
        const int n = min(64, R - b0);
#pragma unroll 4
        for (int j = 0; j < n; j++) {
            float v[CPT];
            if (CPT == 2) {
                const float2 v2 = *reinterpret_cast<const float2 *>(vhead + (int64_t)(b0 + j) * D);
                v[0] = v2.x;
                v[CPT - 1] = v2.y;
            } else {
                v[0] = vhead[(int64_t)(b0 + j) * D];
            }
            // an absent tile has weight 0 and leaves c unchanged (v is finite)
#pragma unroll
            for (int q = 0; q < kMeanRows; q++)
#pragma unroll
                for (int u = 0; u < CPT; u++)
                    c[q][u] = __builtin_fmaf(wt[j][q], v[u], c[q][u]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < kMeanRows; q++) {
        float zz = z[q];
        for (int o = 32; o > 0; o >>= 1)
            zz += __shfl_xor(zz, o);
        if (t == 0 && q < nq)
            magg[row0 + q] = make_float2(M[q], zz);
    }
#pragma unroll
    for (int q = 0; q < kMeanRows; q++)
        if (q < nq) {
            if (CPT == 2)
                *reinterpret_cast<float2 *>(cagg + (row0 + q) * D + t * CPT) = make_float2(c[q][0], c[q][CPT - 1]);
            else
                cagg[(row0 + q) * D + t] = c[q][0];
        }
}

// Merge of a prefix row's chunks (App. B.4's shared normalization across
// parts): M = max m_c, Z = sum Z_c 2^(m_c - M), O = sum acc_c 2^(m_c - M) / Z
// (m in log2 units).  Thread: one row, 4 consecutive channels.
template <int D>
__global__ __launch_bounds__(256) void k_prefix_merge(const AttnArgs A)
{
    constexpr int TPR = D / 4;   // threads per row
    const int bh = blockIdx.y;
    const int row = blockIdx.x * (256 / TPR) + (int)threadIdx.x / TPR;
    const int c0 = 4 * ((int)threadIdx.x % TPR);
    if (row >= A.Lp)
        return;
    const int64_t rows = (int64_t)A.ptiles * kBlk;
    const int64_t base = (int64_t)bh * A.pchunks * rows + row;
    float M = -__builtin_huge_valf();
    for (int c = 0; c < A.pchunks; c++)
        M = fmaxf(M, A.pmz[base + c * rows].x);
    float Z = 0.0f;
    float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int c = 0; c < A.pchunks; c++) {
        const float2 mz = A.pmz[base + c * rows];
        const float f = __builtin_amdgcn_exp2f(mz.x - M);
        const float4 a = *reinterpret_cast<const float4 *>(A.pacc + (base + c * rows) * D + c0);
        Z += mz.y * f;
        o.x += a.x * f;
        o.y += a.y * f;
        o.z += a.z * f;
        o.w += a.w * f;
    }
    const float inv = Z > 0.0f ? 1.0f / Z : 0.0f;
    const int b = bh / A.H, h = bh - b * A.H;
    const int64_t obase = (int64_t)b * A.osb + (int64_t)h * A.osh + (int64_t)row * A.osn + c0;
    if (A.out_f32) {
        *reinterpret_cast<float4 *>((float *)A.outp + obase) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
    } else {
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(o.x * inv) | ((uint32_t)f32_to_bf16(o.y * inv) << 16);
        pk.y = (uint32_t)f32_to_bf16(o.z * inv) | ((uint32_t)f32_to_bf16(o.w * inv) << 16);
        *reinterpret_cast<uint2 *>((uint16_t *)A.outp + obase) = pk;
    }
}

}  // namespace

void launch_attention(const da2_layout_s &L, char *ws, const void *q, const void *k, void *o,
                      int out_f32, const PrefixIo *px, int has_mean, hipEvent_t *ev, hipStream_t st)
{
    const Workspace &W = L.ws;
    AttnArgs A;
    A.q8 = (const uint8_t *)(ws + W.q8);
    A.q4 = (const uint8_t *)(ws + W.q4);
    A.q4s = (const uint8_t *)(ws + W.q4s);
    A.qs8 = (const float *)(ws + W.qs8);
    A.k8 = (const uint8_t *)(ws + W.k8);
    A.k4 = (const uint8_t *)(ws + W.k4);
    A.k4s = (const uint8_t *)(ws + W.k4s);
    A.ks8 = (const float *)(ws + W.ks8);
    A.v8 = (const uint8_t *)(ws + W.v8);
    A.v4 = (const uint8_t *)(ws + W.v4);
    A.v4s = (const uint8_t *)(ws + W.v4s);
    A.vs8 = (const float *)(ws + W.vs8);
    A.q = (const uint16_t *)q;
    A.k = (const uint16_t *)k;
    A.v16 = (const uint8_t *)(ws + W.v16);
    A.kspan = (int)(((int64_t)7 * L.s.width + 7) * L.s.stride_n + L.d) * 2;
    A.sched = (const int32_t *)(ws + W.sched);
    A.cnt = (const int32_t *)(ws + W.cnt);
    A.qord = (const int32_t *)(ws + W.qord);
    A.out = o;
    A.osb = L.s.stride_b;
    A.osh = L.s.stride_h;
    A.osn = L.s.stride_n;
    A.out_f32 = out_f32;
    A.H = L.s.heads;
    A.R = L.R;
    A.Ry = L.Ry;
    A.Rx = L.Rx;
    A.Hv = L.s.height;
    A.Wv = L.s.width;
    A.BH = L.BH;
    A.c4 = (float)(1.4426950408889634 / __builtin_sqrt((double)L.d));
    A.Lp = px ? L.s.prefix : 0;
    A.ptiles = L.ptiles;
    A.qp = px ? (const uint16_t *)px->qp : nullptr;
    A.kp = px ? (const uint16_t *)px->kp : nullptr;
    A.vp16 = (const uint8_t *)(ws + W.vp16);
    A.pvalid = px ? px->valid : nullptr;
    A.outp = px ? px->op : nullptr;
    A.pkspan = A.Lp > 0 ? (int)(((int64_t)(A.Lp - 1) * L.s.stride_n + L.d) * 2) : 0;
    A.pacc = (float *)(ws + W.pacc);
    A.pmz = (float2 *)(ws + W.pmz);
    A.pchunks = L.pchunks;
    A.geo = layout_geo(L, ws);
    A.nreg = (const int32_t *)(ws + W.nreg);
    A.k16 = (const uint8_t *)(ws + W.k16);
    A.magg = nullptr;
    A.cagg = nullptr;
    if (has_mean) {
        A.magg = (const float2 *)(ws + W.magg);
        A.cagg = (const float *)(ws + W.cagg);
        const int32_t *nreg = L.ragged ? (const int32_t *)(ws + W.nreg) : nullptr;
        dim3 mg((L.R + kMeanRows - 1) / kMeanRows, L.BH);
        if (L.d == 128)
            k_mean_agg<128><<<mg, 64, 0, st>>>((const uint8_t *)(ws + W.tier), (const double *)(ws + W.la),
                                                nreg, L.R, (const float *)(ws + W.vavg), (float2 *)(ws + W.magg),
                                                (float *)(ws + W.cagg));
        else
            k_mean_agg<64><<<mg, 64, 0, st>>>((const uint8_t *)(ws + W.tier), (const double *)(ws + W.la), nreg,
                                              L.R, (const float *)(ws + W.vavg), (float2 *)(ws + W.magg),
                                              (float *)(ws + W.cagg));
    }
    dim3 grid(8 * ((L.R + 7) / 8) * L.BH);
    // kernel variant: the 8x8 grid, or a ragged layout whose key regions
    // have no padding, at most 4 or at most 16 padding slots
    const int pm = !L.ragged ? -1 : (L.pmax == 0 ? 0 : (L.pmax <= 4 ? 4 : 16));
#define DA2_ATTN(DD)                                                    \
    do {                                                                \
        if (pm < 0)                                                     \
            k_attn<DD, false, 0><<<grid, 128, 0, st>>>(A);              \
        else if (pm == 0)                                               \
            k_attn<DD, true, 0><<<grid, 128, 0, st>>>(A);               \
        else if (pm == 4)                                               \
            k_attn<DD, true, 4><<<grid, 128, 0, st>>>(A);               \
        else                                                            \
            k_attn<DD, true, 16><<<grid, 128, 0, st>>>(A);              \
    } while (0)
    if (ev)
        hipEventRecord(ev[0], st);
    if (L.d == 128)
        DA2_ATTN(128);
    else
        DA2_ATTN(64);
    if (ev)
        hipEventRecord(ev[1], st);
#undef DA2_ATTN
    if (A.Lp > 0) {
        dim3 pgrid((A.Lp + kBlk - 1) / kBlk, L.BH, L.pchunks);
        if (L.d == 128) {
            if (L.ragged)
                k_attn_prefix<128, true><<<pgrid, 128, 0, st>>>(A);
            else
                k_attn_prefix<128, false><<<pgrid, 128, 0, st>>>(A);
            k_prefix_merge<128><<<dim3((A.Lp + 7) / 8, L.BH), 256, 0, st>>>(A);
        } else {
            if (L.ragged)
                k_attn_prefix<64, true><<<pgrid, 128, 0, st>>>(A);
            else
                k_attn_prefix<64, false><<<pgrid, 128, 0, st>>>(A);
            k_prefix_merge<64><<<dim3((A.Lp + 15) / 16, L.BH), 256, 0, st>>>(A);
        }
    }
}

}  // namespace da2
