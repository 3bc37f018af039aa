// k_attn.hip -- phased mixed-precision block-sparse attention (DraftAttention2,
// Sec. 3.3 "phased execution" and "cross-precision accumulation", App. B.3 /
// B.4 shared normalization, App. C.1 empty rows) on gfx950 matrix cores.
//
// One workgroup = one query region (64 queries) of one (b, h); wave w owns
// queries 32w .. 32w+31.  Every product runs in the transposed form
//     S^T = K Q^T      (A = key rows, B = queries, k = channels)
//     O^T = V^T P^T    (A = channels, B = queries, k = keys)
// so every lane holds one query: its softmax statistics never leave the lane
// except for one exchange with the partner lane (l ^ 32) per tile.  Key rows
// are stored permuted inside each region (key_of_row) so that the S^T
// accumulator hands each lane a whole 32-key group, which is exactly the B
// operand chunk of the P^T V product and exactly one MX block of P.
//
// Phases, each over its tiles in ascending key region (one running max per
// 64-key tile, one normalizer Z of the unquantized weights, one output
// accumulator; App. B.3/B.4):
//   16-bit: S from the bf16 inputs as they are; w unquantized (App. B's
//           error bound has no term for this path), carried into P^T V as
//           two bf16 products, P = hi + lo, hi = bf16(w), lo = bf16(w - hi).
//   8-bit:  S from INT8 codes of Q and K on the integer matrix core (exact
//           int32 sums); P = e4m3(256 w) (the 256 applied by the scaled
//           conversion) times the FP8 codes of V.  That product runs on the
//           bf16 matrix core over the exact bf16 values of both codes: the
//           gfx950 FP8 matrix instructions keep only about 13 bits of each
//           product group below its largest product.  V's per-channel scale
//           and the 256 are the accumulator's units inside the phase,
//           changed once at each boundary.
//   MXFP4:  S from scaled MXFP4 products; P gets one E8M0 exponent per 32
//           keys (the smallest X with max w 2^-X <= 6); acc += P^T V4.
// Epilogue: O = acc / Z, zero when no tile is kept; rows are written straight
// to their original token positions (restore).
//
// Softmax arithmetic.  A logit is w = 2^(S c - M) with c the tile's scale
// (log2 units per unit of the product) and M the row's running maximum.  M
// is kept as an unevaluated sum mh + ml.  Every product's accumulator starts
// at -R, R = mh / c in product units, so the matrix core returns D = S - R
// with a rounding relative to the small difference, not to S (logits of
// video DiTs carry a large per-query constant); the first tile of a row is
// multiplied twice, the first time to find R.  Then t = fma(D, c, b) with a
// per-row bias b = R c - M computed in double-float arithmetic (or, for a row
// whose maximum this tile raises, the new maximum), and w = 2^t <= 1.
#include "da2_internal.h"
#include "da2_device.h"

namespace da2 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v2s __attribute__((ext_vector_type(2)));

struct AttnArgs {
    const uint8_t *q8, *q4, *q4s;
    const float *qs8;
    const uint8_t *k4, *k4s;
    const float *ks8;
    const uint8_t *k8;      // INT8 key operand tiles (8-bit tier logits)
    const uint8_t *v8b;     // bf16 values of the FP8 value codes (16-bit value layout)
    const uint8_t *v4, *v4s;
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
    float c4h, c4l;  // log2(e) / sqrt(d) as an unevaluated sum
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

// A value the compiler may take from any register: the high half of a
// 16-byte (FP4) matrix operand is never read, so it needs no instruction to
// set it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wuninitialized"
__device__ __forceinline__ int any_int()
{
    int x;
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

// A product accumulator holding -R in every element (the lane's query).
__device__ __forceinline__ v16f splat_neg(float R)
{
    v16f x;
#pragma unroll
    for (int r = 0; r < 16; r++)
        x[r] = -R;
    return x;
}

// ---------------------------------------------------------------------------
// Softmax statistics of one query row (this lane's), log2 units.
// ---------------------------------------------------------------------------
struct Row {
    float mh, ml;   // running maximum M = mh + ml; mh = -inf before the first tile
    float z;        // sum of the unquantized weights 2^(S c - M)
};

// Scale of a tile's products in log2 units, c = ch + cl, and 1 / ch (rough).
struct Scale {
    float ch, cl, inv;
};

__device__ __forceinline__ Scale scale_c4(const AttnArgs &A)
{
    return Scale{A.c4h, A.c4l, __builtin_amdgcn_rcpf(A.c4h)};
}

// c = sq sk c4 for FP8 codes: the product of the two block scales is exact as
// a + ae; c keeps the terms of (a + ae)(c4h + c4l) down to the fp32 rounding
// of the small ones.
__device__ __forceinline__ Scale scale_fp8(float sq, float sk, const AttnArgs &A)
{
    const float a = sq * sk, ae = __builtin_fmaf(sq, sk, -a);
    const float h = a * A.c4h;
    const float l = __builtin_fmaf(a, A.c4h, -h) + __builtin_fmaf(a, A.c4l, ae * A.c4h);
    return Scale{h, l, __builtin_amdgcn_rcpf(h)};
}

// Product offset of a row for a tile of scale c: R = M / c (0 before the
// first tile; the first tile finds its own R).
__device__ __forceinline__ float row_offset(const Row &r, const Scale &c)
{
    return r.mh == -__builtin_huge_valf() ? 0.0f : r.mh * c.inv;
}

// Running-max update of one tile whose products were offset by R and whose
// largest D = S - R over valid keys is dm.  B = R c - M is formed exactly
// enough to be small and precise (p + pe = R ch exactly).  A row whose
// maximum the tile raises takes M' = R c + fl(dm ch) (so the tile's largest
// weight is 2^(tiny) ~ 1) and owes its earlier statistics al = 2^(M - M');
// the others keep M.  Returns the bias b of t = fma(D, ch, b); raised tells
// whether M moved.
__device__ __forceinline__ float tile_update(Row &r, const Scale &c, float R, float dm, float &al, bool &raised)
{
    const float p = R * c.ch, pe = __builtin_fmaf(R, c.ch, -p);
    const float B = ((p - r.mh) + pe) + __builtin_fmaf(R, c.cl, -r.ml);   // +inf before the first tile
    const float tm = __builtin_fmaf(dm, c.ch, B);
    raised = tm > 0.0f;
    float b = B;
    al = 1.0f;
    if (raised) {
        const float u = dm * c.ch;
        // M' = p + u + (pe + R cl), renormalised
        const float s = p + u, bb = s - p;
        const float err = (p - (s - bb)) + (u - bb);
        const float lo = err + __builtin_fmaf(R, c.cl, pe);
        const float hi = s + lo;
        r.ml = lo - (hi - s);
        r.mh = hi;
        al = __builtin_amdgcn_exp2f(-tm);   // 0 before the first tile
        b = -u;
    }
    r.z *= al;
    return b;
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

// Rescale of the running statistics when a tile raises a row maximum;
// skipped when no lane's maximum moved (the factor would be exactly 1).
template <int CB>
__device__ __forceinline__ void rescale(v16f (&acc)[CB], float al)
{
    if (__any(al != 1.0f)) {
#pragma unroll
        for (int cb = 0; cb < CB; cb++)
            acc[cb] *= al;
    }
}

// Two bf16 values (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b)
{
    typedef float v2f __attribute__((ext_vector_type(2)));
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, v2bf));
}

// Four E4M3 codes of 256 e (the scale 2^-8 of the conversion divides).
__device__ __forceinline__ int pk_fp8_256(float e0, float e1, float e2, float e3)
{
    v2s w = {0, 0};
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, e0, e1, 0x1p-8f, false);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, e2, e3, 0x1p-8f, true);
    return __builtin_bit_cast(int, w);
}

// MXFP4 block exponent (biased) of this lane's 32-key group, whose largest
// logit is gm: the smallest X with max e 2^-X <= 6 (the block maximum is
// never clipped, as with an NVFP4 scale of amax / 6).  With max e = m 2^k,
// m in [1, 2): X = k - 2, plus 1 when m > 1.5.  Zero and subnormal maxima
// take the smallest exponent.
__device__ __forceinline__ int fp4_exponent(float gm, float c, float bias)
{
    const uint32_t u = __float_as_uint(__builtin_amdgcn_exp2f(__builtin_fmaf(gm, c, bias)));
    const int ef = (int)(u >> 23) - 2 + ((u & 0x7fffffu) > 0x400000u ? 1 : 0);
    return ef < 0 ? 0 : ef;
}

// MXFP4 weight word Q of one tile (slots 8 Q .. 8 Q + 7 of the lane's 32-key
// group, logits s[Q / 2][8 (Q % 2) .. + 7]), with the group's scale
// 2^(ef - 127).
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

// ---------------------------------------------------------------------------
// Copies of key/value tiles into LDS.
// ---------------------------------------------------------------------------
// Key/value operands of one head as buffer resources: a copy then addresses
// its tile with one scalar offset and a fixed per-lane offset, with no
// per-copy vector address arithmetic; reads past the head's bytes return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const uint8_t *base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, (int)bytes, 0x00020000);
}

// Copy UNITS kilobytes at byte offset off of a resource to LDS dst with
// direct-to-LDS buffer loads; wave w of the NW copies units w, w+NW, ...
// Each unit is one instruction: 64 lanes x 16 bytes landing at dst + 16 l.
template <int UNITS, int NW>
__device__ __forceinline__ void copy_kb(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint8_t *dst, int w,
                                        uint32_t loff16)
{
#pragma unroll
    for (int j = 0; j < (UNITS + NW - 1) / NW; j++) {
        const int u = NW * j + w;
        if (UNITS % NW == 0 || u < UNITS)   // fewer units than waves (d = 64, four waves)
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

// MXFP4 key and value tiles of one head.
struct Src {
    __amdgpu_buffer_rsrc_t k4, k4s, v4, v4s;
};

template <int D>
__device__ __forceinline__ Src head_sources(const AttnArgs &A, int64_t hbase, int R)
{
    Src s;
    s.k4 = head_rsrc(A.k4 + hbase * (kBlk * D / 2), (int64_t)R * kBlk * D / 2);
    s.k4s = head_rsrc(A.k4s + hbase * (2 * D), (int64_t)R * 2 * D);
    s.v4 = head_rsrc(A.v4 + hbase * (kBlk * D / 2), (int64_t)R * kBlk * D / 2);
    s.v4s = head_rsrc(A.v4s + hbase * (2 * D), (int64_t)R * 2 * D);
    return s;
}

// LDS images of the MXFP4 phase, in separate double-buffered key and value
// streams (D = head dim): key [0, 32D) codes, [32D, 34D) E8M0; value the same.
template <int D, int NW>
__device__ __forceinline__ void issue_k4(const Src &S, int kb, uint8_t *dst, int w, int l)
{
    copy_kb<kBlk * D / 2048, NW>(S.k4, (uint32_t)kb * (kBlk * D / 2), dst, w, (uint32_t)l * 16u);
    if (w == 0 && l * 4 < 2 * D)
        copy_dword(S.k4s, (uint32_t)kb * (2 * D), dst + 32 * D, (uint32_t)l * 4u);
}

template <int D, int NW>
__device__ __forceinline__ void issue_v4(const Src &S, int kb, uint8_t *dst, int w, int l)
{
    copy_kb<kBlk * D / 2048, NW>(S.v4, (uint32_t)kb * (kBlk * D / 2), dst, w, (uint32_t)l * 16u);
    if (w == 1 && l * 4 < 2 * D)
        copy_dword(S.v4s, (uint32_t)kb * (2 * D), dst + 32 * D, (uint32_t)l * 4u);
}

// Register operands of one MXFP4 tile.
template <int D>
struct KRegs {
    v8i k[2][D / 64];   // per (key half, 64-channel step); codes in dwords 0-3
    int ks[2][D / 64];  // E8M0 exponents
};

template <int D>
struct VRegs {
    v8i v[D / 32];      // per 32-channel block
    int vs[D / 32];
};

template <int D>
__device__ __forceinline__ void read_k4(const uint8_t *b, int l, int mm, KRegs<D> &K)
{
#pragma unroll
    for (int kc = 0; kc < D / 64; kc++) {
        const int chunk = (mm * (D / 64) + kc) * 64 + l;
        K.k[mm][kc] = lds16(b + chunk * 16);
        K.ks[mm][kc] = b[32 * D + chunk];
    }
}

template <int D>
__device__ __forceinline__ void read_v4(const uint8_t *b, int l, int c0, int c1, VRegs<D> &V)
{
#pragma unroll
    for (int cb = c0; cb < c1; cb++) {
        const int chunk = cb * 64 + l;
        V.v[cb] = lds16(b + chunk * 16);
        V.vs[cb] = b[32 * D + chunk];
    }
}

// Logits of key half mm of an MXFP4 tile (S^T = K Q^T with block scales),
// accumulator starting at neg (-R).  The query operand qv[kc] holds the MXFP4
// codes in dwords 0-3 and the E8M0 exponent in dword 4.
template <int D>
__device__ __forceinline__ v16f logits4_half(const KRegs<D> &K, int mm, const v8i (&qv)[D / 64], const v16f &neg)
{
    v16f s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(K.k[mm][0], qv[0], neg, 4, 4, 0, K.ks[mm][0], 0,
                                                            qv[0][4]);
#pragma unroll
    for (int kc = 1; kc < D / 64; kc++)
        s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(K.k[mm][kc], qv[kc], s, 4, 4, 0, K.ks[mm][kc], 0,
                                                           qv[kc][4]);
    return s;
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

// ---------------------------------------------------------------------------
// Key sources of the tiles that run on the bf16 matrix core.  A key source
// says which tile the i-th step takes, copies that tile's key image (64 key
// rows x D channels as bf16: chunk (m, s) holds for lane l key row
// key_of_row(l % 32, m), channels 16 s + 8 (l / 32) .. + 7; chunk (m, s) in
// key buffer m) -- wave w of NW copying its share of the chunks -- and
// tells how many of its keys are valid.
// ---------------------------------------------------------------------------
// Video regions of one head: the schedule's list, or (DENSE) the regions
// first, first + 1, ... in order.  IMG: copy a prepared key image (the FP8
// tier's code values, or a ragged layout's 16-bit keys); otherwise (16-bit
// tier on the 8x8 grid) the rows are gathered straight from K at a fixed
// byte offset per lane from the region's first token.  RAG: mask the
// region's padding slots.
template <int D, bool DENSE, bool IMG, bool RAG, int NW = 2>
struct VideoKeys {
    static_assert(IMG || NW == 2, "the gathered grid image is copied by two waves");
    static constexpr bool kMasked = RAG;
    static constexpr int kCopies = D / 8 / NW;   // copies per wave and tile
    static constexpr int kWaves = NW;
    const int32_t *list;
    int first;
    const uint16_t *kh;            // K of this head
    const uint8_t *kimg;           // key images of the head's regions
    const uint8_t *vbase;          // 16-bit value images of the head's regions
    int64_t vbytes;
    const int32_t *nreg;           // ragged: valid tokens per region
    uint32_t koff;                 // image: this lane's byte offset in a chunk; grid: from a region's first token
    int kspan, Ry, Rx, Hv, Wv, w;
    int64_t osn, ibytes;

    __device__ __forceinline__ VideoKeys(const AttnArgs &A, const uint8_t *img, const int32_t *list_, int first_,
                                         int64_t hoff, int64_t hbase, int w_, int l)
        : list(list_), first(first_), kh(A.k + hoff), nreg(A.nreg), kspan(A.kspan), Ry(A.Ry), Rx(A.Rx),
          Hv(A.Hv), Wv(A.Wv), w(w_), osn(A.osn)
    {
        if (IMG) {
            koff = (uint32_t)l * 16u;
        } else {
            // wave w gathers the key rows of half m = w
            const int kpos = key_of_row(l & 31, w_);
            koff = (uint32_t)((((kpos >> 3) * A.Wv + (kpos & 7)) * A.osn + 8 * (l >> 5)) * 2);
        }
        kimg = img ? img + hbase * (kBlk * D * 2) : nullptr;
        ibytes = (int64_t)A.R * kBlk * D * 2;
        vbase = A.v16 + hbase * (kBlk * D * 2);
        vbytes = ibytes;
    }
    __device__ __forceinline__ int id(int i) const { return DENSE ? first + i : sload_i32(list + i); }
    __device__ __forceinline__ int valid(int kb) const { return RAG ? sload_i32(nreg + kb) : kBlk; }
    __device__ __forceinline__ void issue_key(int kb, uint8_t *kb0, uint8_t *kb1) const
    {
        if (IMG) {
            // chunks w kCopies .. of the region's key image: 1 KB each
            const __amdgpu_buffer_rsrc_t ksrc = head_rsrc(kimg, ibytes);
#pragma unroll
            for (int s = 0; s < kCopies; s++) {
                const int ch = w * kCopies + s;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ksrc, (lds_void *)chunk16<D>(kb0, kb1, ch), 16, koff,
                                                         (uint32_t)kb * (kBlk * D * 2) + ch * 1024, 0, 0);
            }
        } else {
            uint8_t *dst = w ? kb1 : kb0;
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
template <int D, int NW = 2>
struct PrefixKeys {
    static constexpr bool kMasked = true;
    static constexpr int kCopies = D / 8 / NW;   // copies per wave and tile: half m, chunks s0 ..
    static constexpr int kWaves = NW;
    int first;
    __amdgpu_buffer_rsrc_t ksrc;   // prefix K rows of this head
    const uint8_t *vbase;          // prefix value images of this head
    int64_t vbytes;
    int kpos, nv, m, s0;
    uint32_t lane_off;             // channel offset of this lane, bytes
    int64_t osn;

    __device__ __forceinline__ PrefixKeys(const AttnArgs &A, int first_, int64_t hoff, int bh, int nv_, int w,
                                          int l)
        : first(first_), nv(nv_), osn(A.osn)
    {
        m = w / (NW / 2);
        s0 = (w % (NW / 2)) * kCopies;
        kpos = key_of_row(l & 31, m);
        lane_off = (uint32_t)(16 * (l >> 5));
        ksrc = head_rsrc((const uint8_t *)(A.kp + hoff), A.pkspan);
        vbase = A.vp16 + (int64_t)bh * A.ptiles * (kBlk * D * 2);
        vbytes = (int64_t)A.ptiles * kBlk * D * 2;
    }
    __device__ __forceinline__ int id(int i) const { return first + i; }
    __device__ __forceinline__ int valid(int kb) const { return nv - kBlk * kb; }
    __device__ __forceinline__ void issue_key(int kb, uint8_t *kb0, uint8_t *kb1) const
    {
        const int row = min(kBlk * kb + kpos, nv - 1);
        const uint32_t off = (uint32_t)(row * osn * 2) + lane_off;
        uint8_t *dst = m ? kb1 : kb0;
#pragma unroll
        for (int s = s0; s < s0 + kCopies; s++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ksrc, (lds_void *)(dst + s * 1024), 16, off, 32 * s, 0, 0);
    }
};

// INT8 key tiles of the schedule's video regions of one head (the 8-bit
// tier): the prepared operand of region kb, [m][kc][lane][32 B] (lane l: slot
// key_of_row(l % 32, m), channels 64 kc + 32 (l / 32) .. + 31), 1 KB chunks;
// wave w of NW copies chunks w kCopies .. into the key buffer.
template <int D, bool RAG, int NW = 2>
struct Int8Keys {
    static constexpr bool kMasked = RAG;
    static constexpr int kCopies = D / 16 / NW;   // 1 KB chunks per wave and tile
    const int32_t *list;
    const int32_t *nreg;
    const uint8_t *vbase;          // bf16 values of the FP8 value codes of the head's regions
    int64_t vbytes;
    __amdgpu_buffer_rsrc_t ksrc;
    uint32_t loff;
    int w;

    __device__ __forceinline__ Int8Keys(const AttnArgs &A, const int32_t *list_, int64_t hbase, int w_, int l)
        : list(list_), nreg(A.nreg), loff((uint32_t)l * 16u), w(w_)
    {
        ksrc = head_rsrc(A.k8 + hbase * (kBlk * D), (int64_t)A.R * kBlk * D);
        vbase = A.v8b + hbase * (kBlk * D * 2);
        vbytes = (int64_t)A.R * kBlk * D * 2;
    }
    __device__ __forceinline__ int id(int i) const { return sload_i32(list + i); }
    __device__ __forceinline__ int valid(int kb) const { return RAG ? sload_i32(nreg + kb) : kBlk; }
    __device__ __forceinline__ void issue_key(int kb, uint8_t *dst) const
    {
#pragma unroll
        for (int s = 0; s < kCopies; s++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ksrc, (lds_void *)(dst + (w * kCopies + s) * 1024), 16, loff,
                                                     (uint32_t)kb * (kBlk * D) + (w * kCopies + s) * 1024, 0, 0);
    }
};

// This wave's queries as B operands of the bf16 logits (lane l: query row qr,
// channels 16 s + 8 (l / 32) .. + 7 of step s).
template <int D>
__device__ __forceinline__ void load_q16(const uint16_t *qr, int l, v4u (&q16)[D / 16])
{
#pragma unroll
    for (int s = 0; s < D / 16; s++)
        q16[s] = *reinterpret_cast<const v4u *>(qr + 8 * (l >> 5) + 16 * s);
}

// This wave's INT8 query codes as B operands of the integer logits, in
// entries 0 .. D/32 - 1 of the operand array: entry 2 kc + j holds bytes
// 16 j .. 16 j + 15 of chunk (w, kc, lane), the same split as the key tiles.
template <int D>
__device__ __forceinline__ void load_q8(const uint8_t *q8blk, int w, int l, v4u (&q)[D / 16])
{
#pragma unroll
    for (int kc = 0; kc < D / 64; kc++) {
        const uint8_t *p = q8blk + ((w * (D / 64) + kc) * 64 + l) * 32;
        q[2 * kc] = *reinterpret_cast<const v4u *>(p);
        q[2 * kc + 1] = *reinterpret_cast<const v4u *>(p + 16);
    }
}

// bf16 logits of one tile from the key image in kb0 / kb1, accumulators
// starting at neg.
template <int D>
__device__ __forceinline__ void logits16(uint8_t *kb0, uint8_t *kb1, const v4u (&q16)[D / 16], int l,
                                         const v16f &neg, v16f (&sc)[2])
{
    constexpr int KS = D / 16;
#pragma unroll
    for (int mm = 0; mm < 2; mm++)
        sc[mm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            as_bf16x8(lds_v4u(chunk16<D>(kb0, kb1, mm * KS) + l * 16)), as_bf16x8(q16[0]), neg, 0, 0, 0);
#pragma unroll
    for (int s = 1; s < KS; s++)
#pragma unroll
        for (int mm = 0; mm < 2; mm++)
            sc[mm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                as_bf16x8(lds_v4u(chunk16<D>(kb0, kb1, mm * KS + s) + l * 16)), as_bf16x8(q16[s]), sc[mm], 0, 0,
                0);
}

// Keys of a tile past its valid count take no part (register r of half mm
// holds key 32 hf + 16 mm + r).
__device__ __forceinline__ void mask_keys(v16f (&sc)[2], int nk, int hf)
{
    if (nk < kBlk) {
#pragma unroll
        for (int mm = 0; mm < 2; mm++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                if (32 * hf + 16 * mm + r >= nk)
                    sc[mm][r] = -__builtin_huge_valf();
    }
}

// Tiles of the 16-bit tier on the bf16 matrix core: logits from the bf16
// inputs, P = w as the pair hi + lo of bf16 values, real units.  n tiles of
// a key source, ascending; q holds the query rows.  A tile's key image fills
// both key buffers (half m in buffer m), its value image both value buffers.
// The value copy of tile i runs under tile i's logits and softmax, the key
// copy of tile i+1 under tile i's softmax and P^T V.  Key and value buffers
// are distinct LDS variables, so the compiler knows a copy into one never
// feeds reads of the other.
template <int D, class Keys>
__device__ __forceinline__ void run_bf16(uint8_t *kb0, uint8_t *kb1, uint8_t *vb0, uint8_t *vb1, const Keys &K,
                                         int n, const v4u (&q)[D / 16], const Scale &c, int w, int l,
                                         v16f (&acc)[D / 32], Row &row)
{
    constexpr int CB = D / 32;
    constexpr int NK = Keys::kCopies;              // key copies per wave and tile
    constexpr int NW = Keys::kWaves;
    constexpr int VB = kBlk * D * 2;               // value image of a tile
    const int hf = l >> 5;
    const __amdgpu_buffer_rsrc_t vsrc = head_rsrc(K.vbase, K.vbytes);
    int kb = K.id(0);
    int kbn = n > 1 ? K.id(1) : 0;
    K.issue_key(kb, kb0, kb1);
    for (int i = 0; i < n; i++) {
        // key image of tile i complete (both waves' halves); both waves are
        // done with the value buffer
        __builtin_amdgcn_s_waitcnt(vm_wait(0));
        __syncthreads();
#pragma unroll
        for (int j = 0; j < VB / 1024 / NW; j++) {
            const int u = NW * j + w;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vsrc, (lds_void *)chunk16<D>(vb0, vb1, u), 16, (uint32_t)l * 16u,
                                                     (uint32_t)kb * VB + u * 1024, 0, 0);
        }
        const int nk = Keys::kMasked ? K.valid(kb) : kBlk;
        v16f sc[2];
        float R;
        if (__builtin_amdgcn_readfirstlane(row.mh == -__builtin_huge_valf() ? 1 : 0)) {
            // first tile of the row: find its offset from a first product
            logits16<D>(kb0, kb1, q, l, v16f{}, sc);
            if (Keys::kMasked)
                mask_keys(sc, nk, hf);
            R = pair_max(lane_max(sc));
        } else {
            R = row_offset(row, c);
        }
        logits16<D>(kb0, kb1, q, l, splat_neg(R), sc);
        // both waves are done with the key buffer: refill it with tile i+1
        __syncthreads();
        const bool more = i + 1 < n;
        if (more)
            K.issue_key(kbn, kb0, kb1);
        if (Keys::kMasked)
            mask_keys(sc, nk, hf);
        float al;
        bool raised;
        const float bias = tile_update(row, c, R, pair_max(lane_max(sc)), al, raised);
        rescale<CB>(acc, al);
        // P^T chunk t: this lane's keys 32 hf + 8 t .. + 7 (slots 8 t ..), as
        // hi and residual lo
        v4u ph[4], pl[4];
        float z = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const int mm = t >> 1, r0 = 8 * (t & 1);
            float e[8];
#pragma unroll
            for (int j = 0; j < 8; j++)
                e[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[mm][r0 + j], c.ch, bias));
            z += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const uint32_t h = pk_bf16(e[2 * j], e[2 * j + 1]);
                ph[t][j] = h;
                pl[t][j] = pk_bf16(e[2 * j] - __uint_as_float(h << 16), e[2 * j + 1] - __uint_as_float(h & 0xffff0000u));
            }
        }
        row.z += z;
        // value image of tile i complete: only the key copy may still run
        if (more)
            __builtin_amdgcn_s_waitcnt(vm_wait(NK));
        else
            __builtin_amdgcn_s_waitcnt(vm_wait(0));
        __syncthreads();
#pragma unroll
        for (int cb = 0; cb < CB; cb++)
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const v8bf vv = as_bf16x8(lds_v4u(chunk16<D>(vb0, vb1, cb * 4 + t) + l * 16));
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, as_bf16x8(ph[t]), acc[cb], 0, 0, 0);
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, as_bf16x8(pl[t]), acc[cb], 0, 0, 0);
            }
        kb = kbn;
        if (i + 2 < n)
            kbn = K.id(i + 2);
    }
    // the next segment or phase refills the buffers
    __syncthreads();
}

template <int N>
struct Par {
    static constexpr int value = N;
};

// Tiles of the 8-bit tier, software pipelined: integer logits from the INT8
// codes on the integer matrix core (c = sq sk c4 per tile), P = e4m3(256 w) as
// bf16 times the exact bf16 values of the FP8 value codes on the bf16 matrix
// core (units 256 / sV).  n tiles of the schedule's list, ascending.
//   Step i forms the weights of tile i on the vector unit while the matrix
// cores compute P^T V of tile i-1 and the logits of tile i+1.  The INT8 key
// tile (both halves) sits in kb0; the value images of even tiles go to the
// pair (vb0, vb1), of odd tiles to (kb1, xb).  Step i copies V(i) into its
// pair (last read by step i-1), reads K(i+1) from kb0 and issues its logits,
// then, once both waves are done reading kb0, copies K(i+2): every copy has
// about a step to land.
template <int D, bool RAG, int NW>
__device__ __forceinline__ void run_i8(const AttnArgs &A, uint8_t *kb0, uint8_t *kb1, uint8_t *vb0, uint8_t *vb1,
                                       uint8_t *xb, const int32_t *lst, int n, const v4u (&q)[D / 16], float qs,
                                       int64_t hbase, int w, int l, v16f (&acc)[D / 32], Row &row)
{
    constexpr int CB = D / 32;
    constexpr int VB = kBlk * D * 2;               // value image of a tile
    const int hf = l >> 5;
    const Int8Keys<D, RAG, NW> K(A, lst, hbase, w, l);
    const __amdgpu_buffer_rsrc_t vsrc = head_rsrc(K.vbase, K.vbytes);
    v16f Sa[2], Sb[2];   // logits of tiles of alternating parity
    v4u P[4];            // bf16 weights of the previous tile, then of this one
    float R, al = 1.0f;
    int kr0 = sload_i32(lst), kr1 = n > 1 ? sload_i32(lst + 1) : 0, kr2 = n > 2 ? sload_i32(lst + 2) : 0;
    int nk0 = RAG ? sload_i32(A.nreg + kr0) : kBlk;

    auto issue_value = [&](int kbv, uint8_t *b0, uint8_t *b1) {
#pragma unroll
        for (int j = 0; j < VB / 1024 / NW; j++) {
            const int u = NW * j + w;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vsrc, (lds_void *)chunk16<D>(b0, b1, u), 16, (uint32_t)l * 16u,
                                                     (uint32_t)kbv * VB + u * 1024, 0, 0);
        }
    };
    // integer logits of the tile in kb0, accumulators starting at -Ri
    auto logits = [&](int Ri, v16f (&sn)[2]) {
        v16i s[2];
        v16i neg;
#pragma unroll
        for (int j = 0; j < 16; j++)
            neg[j] = -Ri;
#pragma unroll
        for (int e = 0; e < D / 32; e++) {
            v4i k[2];
#pragma unroll
            for (int mm = 0; mm < 2; mm++)
                k[mm] = __builtin_bit_cast(v4i, lds_v4u(kb0 + mm * 32 * D + ((e >> 1) * 64 + l) * 32 + 16 * (e & 1)));
#pragma unroll
            for (int mm = 0; mm < 2; mm++)
                s[mm] = __builtin_amdgcn_mfma_i32_32x32x32_i8(k[mm], __builtin_bit_cast(v4i, q[e]), e ? s[mm] : neg, 0,
                                                             0, 0);
        }
#pragma unroll
        for (int mm = 0; mm < 2; mm++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                sn[mm][r] = (float)s[mm][r];
    };
    // R' = M / c rounded to an integer within the exact range of the sums
    auto offset = [&](const Scale &c) {
        return __builtin_rintf(fminf(fmaxf(row_offset(row, c), -0x1p22f), 0x1p22f));
    };
    // P^T V of the previous tile (weights P) from the pair (v0, v1)
    auto pv = [&](uint8_t *v0, uint8_t *v1) {
#pragma unroll
        for (int cb = 0; cb < CB; cb++) {
            v4u vv[4];
#pragma unroll
            for (int t = 0; t < 4; t++)
                vv[t] = lds_v4u(chunk16<D>(v0, v1, cb * 4 + t) + l * 16);
#pragma unroll
            for (int t = 0; t < 4; t++)
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vv[t]), as_bf16x8(P[t]), acc[cb], 0, 0, 0);
        }
    };
    auto settle = [&]() {
        if (__any(al != 1.0f)) {
#pragma unroll
            for (int cb = 0; cb < CB; cb++)
                acc[cb] *= al;
        }
    };
    // step i of parity PAR: sc the logits of tile i (offset R), P the
    // weights of tile i-1, al the factor acc owes before their product.
    // FIRST: step 0, with no earlier tile to multiply.
    auto step = [&](auto par, auto first, int i, v16f (&sc)[2], v16f (&sn)[2]) {
        constexpr int PAR = decltype(par)::value;
        constexpr bool FIRST = decltype(first)::value != 0;
        uint8_t *vw0 = PAR ? kb1 : vb0, *vw1 = PAR ? xb : vb1;   // pair of tile i
        uint8_t *vr0 = PAR ? vb0 : kb1, *vr1 = PAR ? vb1 : xb;   // pair of tile i-1
        // K(i+1) and V(i-1) complete; both waves are done with step i-1
        __builtin_amdgcn_s_waitcnt(vm_wait(0));
        __syncthreads();
        settle();
        issue_value(kr0, vw0, vw1);
        if (RAG)
            mask_keys(sc, nk0, hf);
        // running max of tile i; the offset and logits of tile i+1 (on the
        // last step from a stale key image: computed, never used)
        const Scale c = scale_fp8(qs, sload_f32(A.ks8 + hbase + kr0), A);
        bool raised;
        float al_i;
        const float bias = tile_update(row, c, R, pair_max(lane_max(sc)), al_i, raised);
        const float Rn = offset(scale_fp8(qs, sload_f32(A.ks8 + hbase + kr1), A));
        logits((int)Rn, sn);
        // both waves are done reading kb0: refill it with tile i+2
        __syncthreads();
        if (i + 2 < n)
            K.issue_key(kr2, kb0);
        // main block, one region per quarter t of the tile's 32 logits per
        // lane: the products of key chunk t of P^T V of tile i-1 (weights
        // P[t], value operands read at the top of the region) spread through
        // the quarter's unquantized weights 2^t (in place of its logits);
        // then the quarter's weight codes (bf16 images of e4m3(256 w)) go
        // into P[t], whose old value the products have read.  Every output
        // block still adds its key chunks in the order 0, 1, 2, 3.
        float z = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const int mm = t >> 1, r0 = 8 * (t & 1);
            v4u vv[CB];
            if (!FIRST) {
#pragma unroll
                for (int cb = 0; cb < CB; cb++)
                    vv[cb] = lds_v4u(chunk16<D>(vr0, vr1, cb * 4 + t) + l * 16);
            }
#pragma unroll
            for (int j = 0; j < 8; j++)
                sc[mm][r0 + j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[mm][r0 + j], c.ch, bias));
            z += ((sc[mm][r0] + sc[mm][r0 + 1]) + (sc[mm][r0 + 2] + sc[mm][r0 + 3])) +
                 ((sc[mm][r0 + 4] + sc[mm][r0 + 5]) + (sc[mm][r0 + 6] + sc[mm][r0 + 7]));
            if (!FIRST) {
#pragma unroll
                for (int cb = 0; cb < CB; cb++)
                    acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vv[cb]), as_bf16x8(P[t]), acc[cb],
                                                                     0, 0, 0);
            }
            const uint32_t w0 = (uint32_t)pk_fp8_256(sc[mm][r0], sc[mm][r0 + 1], sc[mm][r0 + 2], sc[mm][r0 + 3]);
            const uint32_t w1 = (uint32_t)pk_fp8_256(sc[mm][r0 + 4], sc[mm][r0 + 5], sc[mm][r0 + 6], sc[mm][r0 + 7]);
            P[t][0] = fp8_pair_bf16(w0, 0);
            P[t][1] = fp8_pair_bf16(w0, 1);
            P[t][2] = fp8_pair_bf16(w1, 0);
            P[t][3] = fp8_pair_bf16(w1, 1);
            if (!FIRST) {
                __builtin_amdgcn_sched_group_barrier(0x100, CB, 0);   // value reads
                __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
#pragma unroll
                for (int j = 0; j < CB; j++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 24 / CB, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // keep the weights in this block: sunk past the next step's barrier
        // they would leave the products above nothing to overlap with
        asm volatile("" ::"v"(z), "v"(P[0]), "v"(P[1]), "v"(P[2]), "v"(P[3]));
        row.z += z;
        al = al_i;
        R = Rn;
        kr0 = kr1;
        kr1 = kr2;
        kr2 = sload_i32(lst + min(i + 3, n - 1));
        if (RAG)
            nk0 = sload_i32(A.nreg + kr0);
    };

    // prologue: the logits of tile 0 (a fresh row first finds its offset)
    K.issue_key(kr0, kb0);
    __builtin_amdgcn_s_waitcnt(vm_wait(0));
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(row.mh == -__builtin_huge_valf() ? 1 : 0)) {
        logits(0, Sa);
        if (RAG)
            mask_keys(Sa, nk0, hf);
        R = pair_max(lane_max(Sa));
    } else {
        R = offset(scale_fp8(qs, sload_f32(A.ks8 + hbase + kr0), A));
    }
    logits((int)R, Sa);
    __syncthreads();
    if (n > 1)
        K.issue_key(kr1, kb0);
    step(Par<0>{}, Par<1>{}, 0, Sa, Sb);
    int i = 1;
    for (; i + 1 < n; i += 2) {
        step(Par<1>{}, Par<0>{}, i, Sb, Sa);
        step(Par<0>{}, Par<0>{}, i + 1, Sa, Sb);
    }
    if (i < n)
        step(Par<1>{}, Par<0>{}, i, Sb, Sa);
    // drain: P^T V of the last tile
    __builtin_amdgcn_s_waitcnt(vm_wait(0));
    __syncthreads();
    settle();
    if ((n - 1) & 1)
        pv(kb1, xb);
    else
        pv(vb0, vb1);
    // the next phase refills the buffers
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
template <int D, bool RAG, int PMAX, int NW>
struct Attn {
    static constexpr int KC = D / 64;   // 64-channel steps of QK^T
    static constexpr int CB = D / 32;   // 32-channel blocks of the output
    const AttnArgs &A;
    // key and value buffers, two of each, and a fifth buffer (the 8-bit
    // tier's second value pair is kb1 + xb); distinct LDS variables, so that
    // the compiler can tell a copy into one from a read of another
    uint8_t *kb0, *kb1, *vb0, *vb1, *xb;
    const int32_t *list;   // key regions of the MXFP4 tiles, ascending
    int64_t hbase;
    Src src;
    int n, w, wq, l, hf, bh;   // w: this wave's share of the copies (of NW); wq: its 32 rows of the query tile
    int64_t qblk;
    float qs;
    v8i qv[KC];   // this wave's queries: MXFP4 codes (dwords 0-3) and exponent (dword 4)
    v16f acc[CB];
    Row row;
    // Software pipeline state of the MXFP4 phase.  Step i forms the weights
    // of tile i while the matrix core computes the logits of tile i+1 and
    // P^T V of tile i-1, so the logits (S) and the weights (P, with the MXFP4
    // exponent e) live in two register sets each, used by steps of
    // alternating parity.
    v16f S0[2], S1[2];
    v8i P0, P1;
    int E0, E1;
    v16f negR;          // -R, the accumulator start of the next logits
    float R;            // offset of the logits held in the current set
    float al;           // factor acc owes before the next P^T V (running-max change)
    int kr0, kr1, kr2;  // key regions of tiles i, i+1, i+2 (wave-uniform)
    int nk0;            // valid tokens of tile i's key region (PMAX > 0)

    // change of value units around the 8-bit phase: real <-> 256 / sV (the
    // FP8 value codes and the 256 of the weight codes).  The scales are
    // loaded where they are used (volatile): loaded once for both uses, they
    // would stay in 64 registers through the phases.
    __device__ __forceinline__ void vunits(bool to_fp8)
    {
        const volatile float4 *vs = reinterpret_cast<const volatile float4 *>(A.vs8 + (int64_t)bh * D);
#pragma unroll
        for (int cb = 0; cb < CB; cb++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const float4 sv = const_cast<const float4 &>(vs[(32 * cb + 8 * g + 4 * hf) / 4]);
                const float f[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    const float u = f[t] * 0x1p-8f;
                    acc[cb][4 * g + t] = to_fp8 ? acc[cb][4 * g + t] / u : acc[cb][4 * g + t] * u;
                }
            }
    }

    // acc *= al before the next P^T V
    __device__ __forceinline__ void settle()
    {
        if (__any(al != 1.0f)) {
#pragma unroll
            for (int cb = 0; cb < CB; cb++)
                acc[cb] *= al;
        }
    }

    __device__ __forceinline__ void pv_range(const VRegs<D> &V, const v8i &p, int ef, int c0, int c1)
    {
#pragma unroll
        for (int cb = c0; cb < c1; cb++)
            acc[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(V.v[cb], p, acc[cb], 4, 4, 0, V.vs[cb], 0, ef);
    }

    // MXFP4 step i.  On entry sc holds the logits of tile i (offset R), pp /
    // ep the weights of tile i-1 (zero before the first tile), al the factor
    // acc owes before their product.  The refills go first: K(i+2) into
    // K(i)'s buffer kw and V(i) into V(i-2)'s buffer vw, both read for the
    // last time in step i-1.  Then K(i+1) and V(i-1) are read from kr and vr,
    // each half just before its products.  The last step computes logits of a
    // stale key image, which are never used.
    __device__ __forceinline__ void step(int i, v16f (&sc)[2], v16f (&sn)[2], const v8i &pp, int ep, v8i &pc,
                                         int &ec, const uint8_t *__restrict__ kr, uint8_t *__restrict__ kw,
                                         const uint8_t *__restrict__ vr, uint8_t *__restrict__ vw)
    {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        settle();
        if (i + 2 < n)
            issue_k4<D, NW>(src, kr2, kw, w, l);
        issue_v4<D, NW>(src, kr0, vw, w, l);
        VRegs<D> V;
        KRegs<D> K;
        // main block: weights of tile i on the vector unit, products of tiles
        // i-1 and i+1 on the matrix core, in regions fenced from each other.
        // Each region reads the operands of the next region's products from
        // LDS, issues its own products (operands read by the region before)
        // and forms a quarter of the weights:
        //   R0: running max; offset of the next logits; read V [0, CB/2)
        //   R1: P^T V blocks [0, CB/2);  read V blocks [CB/2, CB); weights 1/4
        //   R2: P^T V blocks [CB/2, CB); read K half 0;          weights 2/4
        //   R3: logits half 0 (into the registers of the logits weights 1/4
        //       and 2/4 consumed);        read K half 1;          weights 3/4
        //   R4: logits half 1;                                    weights 4/4
        if (PMAX > 0)
            mask_padding<PMAX>(sc[1], nk0, hf);
        const Scale c = scale_c4(A);
        const float gm = lane_max(sc);
        const float dm = pair_max(gm);
        bool raised;
        const float bias = tile_update(row, c, R, dm, al, raised);
        ec = fp4_exponent(gm, c.ch, bias);
        const float pscale = ec ? __uint_as_float((uint32_t)ec << 23) : __uint_as_float(0x00400000u);
        // the next logits start at -R' (R' = M / c), refreshed when a maximum
        // moved (a branch: the empty asm keeps the compiler from turning the
        // refresh into sixteen selects on every step)
        if (__any(raised)) {
            R = row_offset(row, c);
            asm volatile("" ::: "memory");
            negR = splat_neg(R);
        }
        read_v4<D>(vr, l, 0, CB / 2, V);
        __builtin_amdgcn_sched_barrier(0);
        // R1
        pv_range(V, pp, ep, 0, CB / 2);
        read_v4<D>(vr, l, CB / 2, CB, V);
        float z = 0.0f;
        weight_word_fp4<0>(sc, c.ch, bias, pscale, z, pc);
        region_pattern();
        __builtin_amdgcn_sched_barrier(0);
        // R2
        pv_range(V, pp, ep, CB / 2, CB);
        read_k4<D>(kr, l, 0, K);
        weight_word_fp4<1>(sc, c.ch, bias, pscale, z, pc);
        region_pattern();
        __builtin_amdgcn_sched_barrier(0);
        // R3
        sn[0] = logits4_half<D>(K, 0, qv, negR);
        read_k4<D>(kr, l, 1, K);
        weight_word_fp4<2>(sc, c.ch, bias, pscale, z, pc);
        region_pattern();
        __builtin_amdgcn_sched_barrier(0);
        // R4
        sn[1] = logits4_half<D>(K, 1, qv, negR);
        weight_word_fp4<3>(sc, c.ch, bias, pscale, z, pc);
        pc[4] = any_int(); pc[5] = any_int(); pc[6] = any_int(); pc[7] = any_int();
        region_pattern();
        row.z += z;
        // Z, the packed weights and the next logits are complete within the
        // step: otherwise the compiler sinks their additions, conversions and
        // products into the next step (keeping every weight of this tile live
        // across the barrier, or serializing the next row maximum behind the
        // products).
        asm volatile("" ::"v"(row.z), "v"(pc), "v"(sn[0]), "v"(sn[1]));
        // wave-uniform values of the next step, loaded without branches so
        // that the main block stays one scheduling region (indices past the
        // list are clamped; such values are never used)
        kr0 = kr1;
        kr1 = kr2;
        kr2 = sload_i32(list + min(i + 3, n - 1));
        if (PMAX > 0)
            nk0 = sload_i32(A.nreg + kr0);
    }

    __device__ __forceinline__ void step_even(int i) { step(i, S0, S1, P1, E1, P0, E0, kb1, kb0, vb1, vb0); }
    __device__ __forceinline__ void step_odd(int i) { step(i, S1, S0, P0, E0, P1, E1, kb0, kb1, vb0, vb1); }

    // (volatile: the load right before the MXFP4 loop gives the loop its own
    // short live range)
    __device__ __forceinline__ void load_q4()
    {
#pragma unroll
        for (int kc = 0; kc < KC; kc++) {
            const int chunk = (wq * KC + kc) * 64 + l;
            const uint4 c = const_cast<const uint4 &>(
                *reinterpret_cast<const volatile uint4 *>(A.q4 + qblk * (kBlk * D / 2) + chunk * 16));
            qv[kc][0] = c.x;
            qv[kc][1] = c.y;
            qv[kc][2] = c.z;
            qv[kc][3] = c.w;
            qv[kc][4] = *(const volatile uint8_t *)(A.q4s + qblk * (2 * D) + chunk);
            qv[kc][5] = any_int(); qv[kc][6] = any_int(); qv[kc][7] = any_int();
        }
    }

    // MXFP4 tiles [0, n), step i with the register sets and buffers of parity
    // i % 2.
    __device__ __forceinline__ void fp4_phase()
    {
        if (n == 0)
            return;
        load_q4();
        kr0 = sload_i32(list);
        kr1 = n > 1 ? sload_i32(list + 1) : 0;
        kr2 = n > 2 ? sload_i32(list + 2) : 0;
        issue_k4<D, NW>(src, kr0, kb0, w, l);
        if (n > 1)
            issue_k4<D, NW>(src, kr1, kb1, w, l);
        if (PMAX > 0)
            nk0 = sload_i32(A.nreg + kr0);
        // step 0 multiplies P = 0 into the value buffer of the other parity:
        // clear it so that no stale code can make a NaN
#pragma unroll
        for (int u = 0; u < kBlk * D / (NW * 64 * 16); u++)
            *reinterpret_cast<v4u *>(vb1 + (u * NW * 64 + threadIdx.x) * 16) = (v4u){};
        P0 = (v8i){};
        P1 = (v8i){};
        E0 = 127;
        E1 = 127;
        al = 1.0f;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        {
            KRegs<D> K;
            read_k4<D>(kb0, l, 0, K);
            read_k4<D>(kb0, l, 1, K);
            const Scale c = scale_c4(A);
            if (__builtin_amdgcn_readfirstlane(row.mh == -__builtin_huge_valf() ? 1 : 0)) {
                // first tile of the row: find its offset from a first product
                const v16f zero = {};
                S0[0] = logits4_half<D>(K, 0, qv, zero);
                S0[1] = logits4_half<D>(K, 1, qv, zero);
                if (PMAX > 0)
                    mask_padding<PMAX>(S0[1], nk0, hf);
                R = pair_max(lane_max(S0));
            } else {
                R = row_offset(row, c);
            }
            negR = splat_neg(R);
            S0[0] = logits4_half<D>(K, 0, qv, negR);
            S0[1] = logits4_half<D>(K, 1, qv, negR);
        }
        int i = 0;
        for (; i + 1 < n; i += 2) {
            step_even(i);
            step_odd(i + 1);
        }
        if (i < n)
            step_even(i);
        // drain: P^T V of the last tile
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const bool lodd = (n - 1) & 1;
        VRegs<D> V;
        const v8i pl = lodd ? P1 : P0;   // by value: a reference would keep both sets in memory
        const int el = lodd ? E1 : E0;
        settle();
        read_v4<D>(lodd ? vb1 : vb0, l, 0, CB, V);
        pv_range(V, pl, el, 0, CB);
        __syncthreads();
    }

    // Phases whose P^T V runs on the bf16 matrix core: the text-prefix keys
    // (np tiles, nv valid keys) and the schedule's 16-bit key regions, then
    // its 8-bit key regions.
    __device__ __forceinline__ void bf16_phases(const int32_t *list16, int n16, const int32_t *list8, int n8, int np,
                                                int nv, int a)
    {
        const int bb = bh / A.H, hh = bh - bb * A.H;
        const int64_t hoff = (int64_t)bb * A.osb + (int64_t)hh * A.osh;
        v4u q16[D / 16];
        if (np > 0 || n16 > 0) {
            int qt = slot_token<RAG>(A.geo, a, 32 * wq + (l & 31));
            if (qt < 0)   // padding slot: any valid row (its output is not written)
                qt = slot_token<RAG>(A.geo, a, 0);
            load_q16<D>(A.q + hoff + (int64_t)qt * A.osn, l, q16);
            if (np > 0)
                run_bf16<D>(kb0, kb1, vb0, vb1, PrefixKeys<D, NW>(A, 0, hoff, bh, nv, w, l), np, q16, scale_c4(A), w, l,
                            acc, row);
            if (n16 > 0)
                run_bf16<D>(kb0, kb1, vb0, vb1, VideoKeys<D, false, RAG, RAG, NW>(A, A.k16, list16, 0, hoff, hbase, w, l),
                            n16, q16, scale_c4(A), w, l, acc, row);
        }
        if (n8 > 0) {
            vunits(true);
            load_q8<D>(A.q8 + qblk * (kBlk * D), wq, l, q16);
            run_i8<D, RAG, NW>(A, kb0, kb1, vb0, vb1, xb, list8, n8, q16, qs, hbase, w, l, acc, row);
            vunits(false);
        }
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
                const float mnew = fmaxf(row.mh, mz.x);
                const float f = __builtin_amdgcn_exp2f(row.mh - mnew), g = __builtin_amdgcn_exp2f(mz.x - mnew);
                row.z = row.z * f + (hf ? 0.0f : mz.y * g);   // z is summed over the lane pair
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
                row.mh = mnew;
            }
        }
        const float zt = pair_sum(row.z);
        const float inv = zt > 0.0f ? 1.0f / zt : 0.0f;
        const int qi = 32 * wq + (l & 31);
        const int tok = slot_token<RAG>(A.geo, a, qi);
        const int b = bh / A.H, h = bh - b * A.H;
        const int64_t obase = (int64_t)b * A.osb + (int64_t)h * A.osh + (int64_t)tok * A.osn;
        if (tok >= 0)
            store_row<D>(A, A.out, obase, acc, inv, hf);
    }

    __device__ __forceinline__ void init(int w_, int bh_, int64_t qblk_)
    {
        w = w_;
        wq = NW == 4 ? (w_ & 1) : w_;
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
        row.mh = -__builtin_huge_valf();
        row.ml = 0.0f;
        row.z = 0.0f;
    }
};

// One query region per workgroup: 16-bit phase (text prefix, then 16-bit
// tiles), 8-bit phase, MXFP4 phase, epilogue.  NW = 2: a region of one tile,
// two waves of 32 rows.  NW = 4 (block capacity 128): a region of two tiles
// with the same key list, four waves; every copied key and value tile then
// serves 128 query rows.
template <int D, bool RAG, int PMAX, int NW>
__global__ __launch_bounds__(64 * NW, 2) void k_attn(const AttnArgs A)
{
    __shared__ __attribute__((aligned(1024))) uint8_t kb0[kBlk * D];
    __shared__ __attribute__((aligned(1024))) uint8_t kb1[kBlk * D];
    __shared__ __attribute__((aligned(1024))) uint8_t vb0[kBlk * D];
    __shared__ __attribute__((aligned(1024))) uint8_t vb1[kBlk * D];
    __shared__ __attribute__((aligned(1024))) uint8_t xb[kBlk * D];

    // XCD-aware work mapping.  Workgroups are dealt to the 8 XCDs round robin
    // (block L runs on XCD L % 8).  Every XCD walks the heads in the same
    // order and takes its own eighth (work slots j) of each head's query
    // regions, so all XCDs work on the same head at a time and that head's
    // key/value tiles (about 31 MB for a 720p Wan layer) stay in the shared
    // last-level cache.  The plan's work order maps a slot to its query
    // region (k_qorder: an XCD's eighth of a head holds regions of about the
    // same kept tile count, largest first; -1 marks an empty slot).
    const int R = A.R;                           // tiles
    const int QU = NW == 4 ? R / 2 : R;          // query regions
    const int span = (QU + 7) / 8;
    const int xcd = (int)(blockIdx.x & 7), kk = (int)(blockIdx.x >> 3);
    const int bh = kk / span;
    const int j = xcd * span + (kk - bh * span);
    const int au = sload_i32(A.qord + (int64_t)bh * 8 * span + j);
    if (au < 0)   // an empty slot of the last share
        return;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int a = NW == 4 ? 2 * au + (w >> 1) : au;   // this wave's query tile
    const int64_t qblk = (int64_t)bh * R + a;

    Attn<D, RAG, PMAX, NW> S{A, kb0, kb1, vb0, vb1, xb};
    S.init(w, bh, qblk);
    const int n16 = sload_i32(A.cnt + qblk * kTargets);
    const int n8 = sload_i32(A.cnt + qblk * kTargets + 1);
    S.n = sload_i32(A.cnt + qblk * kTargets + 2);
    const int32_t *list16 = A.sched + qblk * R;
    S.list = list16 + n16 + n8;
    const int nv = prefix_valid(A, bh / A.H);
    const int np = (nv + kBlk - 1) / kBlk;
    if (n16 > 0 || n8 > 0 || np > 0)
        S.bf16_phases(list16, n16, list16 + n16, n8, np, nv, a);
    S.fp4_phase();
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
    const int64_t hbase = (int64_t)bh * A.R;
    const int row = kBlk * pb + 32 * w + (l & 31);
    v4u q16[D / 16];
    load_q16<D>(A.qp + hoff + (int64_t)min(row, A.Lp - 1) * A.osn, l, q16);
    v16f acc[D / 32];
#pragma unroll
    for (int cb = 0; cb < D / 32; cb++)
        acc[cb] = (v16f){};
    Row st{-__builtin_huge_valf(), 0.0f, 0.0f};
    const int nv = prefix_valid(A, b);
    const int np = (nv + kBlk - 1) / kBlk;
    const int t0 = c * kPrefixChunkTiles, t1 = min(t0 + kPrefixChunkTiles, np + A.R);
    if (t0 < np)
        run_bf16<D>(kb0, kb1, vb0, vb1, PrefixKeys<D, 2>(A, t0, hoff, bh, nv, w, l), min(t1, np) - t0, q16,
                    scale_c4(A), w, l, acc, st);
    const int r0 = max(t0, np) - np, r1 = t1 - np;
    if (r1 > r0)
        run_bf16<D>(kb0, kb1, vb0, vb1, VideoKeys<D, true, RAG, RAG>(A, A.k16, nullptr, r0, hoff, hbase, w, l),
                    r1 - r0, q16, scale_c4(A), w, l, acc, st);
    const float zt = pair_sum(st.z);
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
            A.pmz[slot] = make_float2(st.mh, zt);
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
    A.k4 = (const uint8_t *)(ws + W.k4);
    A.k4s = (const uint8_t *)(ws + W.k4s);
    A.ks8 = (const float *)(ws + W.ks8);
    A.k8 = (const uint8_t *)(ws + W.k8);
    A.v8b = (const uint8_t *)(ws + W.v8b);
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
    {
        // log2(e) / sqrt(d) as an unevaluated sum of two floats
        const double c4 = 1.4426950408889634 / __builtin_sqrt((double)L.d);
        A.c4h = (float)c4;
        A.c4l = (float)(c4 - (double)A.c4h);
    }
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
    // one workgroup per query region: one tile and two waves, or (capacity
    // 128) two tiles and four waves
    const int QU = L.tpr == 2 ? L.Rg : L.R;
    dim3 grid(8 * ((QU + 7) / 8) * L.BH);
    // kernel variant: the 8x8 grid, or a ragged layout whose key regions
    // have no padding, at most 4 or at most 16 padding slots
    const int pm = !L.ragged ? -1 : (L.pmax == 0 ? 0 : (L.pmax <= 4 ? 4 : 16));
#define DA2_ATTN(DD)                                                    \
    do {                                                                \
        if (L.tpr == 2) {                                               \
            if (pm == 0)                                                \
                k_attn<DD, true, 0, 4><<<grid, 256, 0, st>>>(A);        \
            else if (pm == 4)                                           \
                k_attn<DD, true, 4, 4><<<grid, 256, 0, st>>>(A);        \
            else                                                        \
                k_attn<DD, true, 16, 4><<<grid, 256, 0, st>>>(A);       \
        } else if (pm < 0)                                              \
            k_attn<DD, false, 0, 2><<<grid, 128, 0, st>>>(A);           \
        else if (pm == 0)                                               \
            k_attn<DD, true, 0, 2><<<grid, 128, 0, st>>>(A);            \
        else if (pm == 4)                                               \
            k_attn<DD, true, 4, 2><<<grid, 128, 0, st>>>(A);            \
        else                                                            \
            k_attn<DD, true, 16, 2><<<grid, 128, 0, st>>>(A);           \
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
