// k_plan.hip -- draft scoring, ranking and scheduling (DraftAttention2,
// Sec. 3.1 Eq. (2) and "joint allocation of sparsity and precision"; App. C.1
// routing).
//
// Scores must be bit-identical run to run and against an fp64 reference, so
// every floating-point step has a fixed order: logits are fused multiply-add
// chains over channels 0..d-1 times 1/sqrt(d) (on the fp64 matrix core, whose
// accumulation is exactly such a chain); row maxima (order-free);
// exponentials by the shared Cody-Waite/Taylor exp; row sums strictly
// sequential over key regions; p = e / Z; A = (1-lambda) p_avg + lambda p_max
// with separate products; the ranking key is the bit pattern of fp32(A).
//
// Ranking (head scope) is an exact radix select on the 32-bit keys for the
// T16-th, (T16+T8)-th and (T16+T8+T4)-th largest (8-bit digits, four
// histogram passes), followed by a pass that resolves equal keys by
// ascending pair index a*R+b with a chunked prefix count.  Row scope does the
// same per query region inside one workgroup.  The schedule lists, per query
// region, the 16-bit key regions in ascending order, then the FP8 ones, then
// the MXFP4 ones.
#include <type_traits>

#include "da2_internal.h"
#include "da2_device.h"

namespace da2 {
namespace {

constexpr int kChunk = 4096;   // keys per rank workgroup (256 threads x 16)

__global__ void k_fill_words(uint32_t *p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Logits: La = avgQ avgK^T / sqrt(d), Lm = maxQ maxK^T / sqrt(d), fp64, on the
// fp64 matrix core.  v_mfma_f64_16x16x4f64 adds its four products to the
// accumulator as four fused multiply-adds in ascending k (each rounded), so
// feeding channels in ascending order makes every accumulator exactly the
// fma chain over channels 0..d-1 that the scores are defined by.
// Operand layouts of the instruction: A lane l = (row l%16, k l/16), B lane
// l = (k l/16, column l%16), accumulator lane l register r = (row 4r + l/16,
// column l%16).
// One workgroup (4 waves, 2x2) computes a 128x128 tile of one branch; each
// wave a 64x64 block as 4x4 accumulators.  Channels are staged through LDS
// 32 at a time, transposed so that an operand is one conflict-free read;
// the next stage's global loads are in flight while a stage's products run.
// ---------------------------------------------------------------------------
typedef double v4d __attribute__((ext_vector_type(4)));

// Order-preserving map of (non-NaN) doubles to unsigned integers, so that an
// integer atomic maximum is the floating-point maximum.  0 is below every
// encoded value.
__device__ __forceinline__ unsigned long long ord64(double x)
{
    const unsigned long long u = (unsigned long long)__double_as_longlong(x);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ double unord64(unsigned long long e)
{
    const unsigned long long u = (e >> 63) ? (e & 0x7fffffffffffffffull) : ~e;
    return __longlong_as_double((long long)u);
}

// One stage (CK channels of 128 rows of each operand) of one branch, held in
// registers between its global load and its store to LDS, so that the loads
// of stage s + 1 are in flight while the products of stage s run.
template <int D, bool MAXB>
struct LogitStage {
    static constexpr int TM = 128, CK = 32;
    static constexpr int NV = MAXB ? TM * CK / 4 / 256 : TM * CK / 2 / 256;  // vectors per thread
    typename std::conditional<MAXB, float4, double2>::type x[NV], y[NV];

    // Vector e of the stage: 16 consecutive rows per 16 lanes, and the
    // row's channel vectors over the lane groups, so that the transposing
    // LDS stores of one 16-lane group go to 16 consecutive rows (distinct
    // banks) while the global loads still read 64 contiguous bytes per row.
    static constexpr int VPR = MAXB ? CK / 4 : CK / 2;   // vectors per row
    __device__ __forceinline__ static int row_of(int e) { return (e & 15) + 16 * (e / (16 * VPR)); }

    __device__ __forceinline__ void load(const void *qb_, const void *kb_, int a0, int b0, int R, int c0, int t)
    {
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int e = t + 256 * i;
            if (MAXB) {
                const float *qb = (const float *)qb_, *kb = (const float *)kb_;
                const int r = row_of(e), c = 4 * ((e >> 4) & (CK / 4 - 1));
                float4 xv = make_float4(0.f, 0.f, 0.f, 0.f), yv = make_float4(0.f, 0.f, 0.f, 0.f);
                if (a0 + r < R)
                    xv = *reinterpret_cast<const float4 *>(qb + (int64_t)(a0 + r) * D + c0 + c);
                if (b0 + r < R)
                    yv = *reinterpret_cast<const float4 *>(kb + (int64_t)(b0 + r) * D + c0 + c);
                x[i] = *reinterpret_cast<decltype(&x[i])>(&xv);
                y[i] = *reinterpret_cast<decltype(&y[i])>(&yv);
            } else {
                const double *qb = (const double *)qb_, *kb = (const double *)kb_;
                const int r = row_of(e), c = 2 * ((e >> 4) & (CK / 2 - 1));
                double2 xv = make_double2(0.0, 0.0), yv = make_double2(0.0, 0.0);
                if (a0 + r < R)
                    xv = *reinterpret_cast<const double2 *>(qb + (int64_t)(a0 + r) * D + c0 + c);
                if (b0 + r < R)
                    yv = *reinterpret_cast<const double2 *>(kb + (int64_t)(b0 + r) * D + c0 + c);
                x[i] = *reinterpret_cast<decltype(&x[i])>(&xv);
                y[i] = *reinterpret_cast<decltype(&y[i])>(&yv);
            }
        }
    }

    template <int PITCH>
    __device__ __forceinline__ void store(double (*sq)[PITCH], double (*sk)[PITCH], int t) const
    {
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int e = t + 256 * i;
            if (MAXB) {
                const int r = row_of(e), c = 4 * ((e >> 4) & (CK / 4 - 1));
                const float4 xv = *reinterpret_cast<const float4 *>(&x[i]);
                const float4 yv = *reinterpret_cast<const float4 *>(&y[i]);
                sq[c][r] = xv.x; sq[c + 1][r] = xv.y; sq[c + 2][r] = xv.z; sq[c + 3][r] = xv.w;
                sk[c][r] = yv.x; sk[c + 1][r] = yv.y; sk[c + 2][r] = yv.z; sk[c + 3][r] = yv.w;
            } else {
                const int r = row_of(e), c = 2 * ((e >> 4) & (CK / 2 - 1));
                const double2 xv = *reinterpret_cast<const double2 *>(&x[i]);
                const double2 yv = *reinterpret_cast<const double2 *>(&y[i]);
                sq[c][r] = xv.x; sq[c + 1][r] = xv.y;
                sk[c][r] = yv.x; sk[c + 1][r] = yv.y;
            }
        }
    }
};

template <int D, bool MAXB>
__device__ __forceinline__ void logits_tile(const double *__restrict__ qa, const double *__restrict__ ka,
                                            const float *__restrict__ qm, const float *__restrict__ km, int R,
                                            double inv_sqrt_d, double *__restrict__ La, double *__restrict__ Lm,
                                            unsigned long long *__restrict__ rmax, int bh, int a0, int b0,
                                            double (*sq)[132], double (*sk)[132])
{
    constexpr int CK = 32;
    const int t = threadIdx.x, l = t & 63, wv = t >> 6, wa = wv >> 1, wb = wv & 1;
    const void *qb = MAXB ? (const void *)(qm + (int64_t)bh * R * D) : (const void *)(qa + (int64_t)bh * R * D);
    const void *kb = MAXB ? (const void *)(km + (int64_t)bh * R * D) : (const void *)(ka + (int64_t)bh * R * D);
    v4d acc[4][4];
#pragma unroll
    for (int g = 0; g < 4; g++)
#pragma unroll
        for (int h = 0; h < 4; h++)
            acc[g][h] = (v4d){0.0, 0.0, 0.0, 0.0};
    LogitStage<D, MAXB> st;
    st.load(qb, kb, a0, b0, R, 0, t);
    for (int c0 = 0; c0 < D; c0 += CK) {
        __syncthreads();
        st.template store<132>(sq, sk, t);
        __syncthreads();
        if (c0 + CK < D)
            st.load(qb, kb, a0, b0, R, c0 + CK, t);
#pragma unroll 2
        for (int s4 = 0; s4 < CK; s4 += 4) {
            const int c = s4 + (l >> 4), r = l & 15;
            double av[4], bv[4];
#pragma unroll
            for (int g = 0; g < 4; g++) {
                av[g] = sq[c][64 * wa + 16 * g + r];
                bv[g] = sk[c][64 * wb + 16 * g + r];
            }
#pragma unroll
            for (int g = 0; g < 4; g++)
#pragma unroll
                for (int h = 0; h < 4; h++)
                    acc[g][h] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[g], bv[h], acc[g][h], 0, 0, 0);
        }
    }
    // Store row-major and fold the row maxima into rmax with an
    // order-preserving integer atomic maximum.
    double *L = (MAXB ? Lm : La) + (int64_t)bh * R * R;
    unsigned long long *rm = rmax + ((int64_t)bh * 2 + MAXB) * R;
#pragma unroll
    for (int g = 0; g < 4; g++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int i = a0 + 64 * wa + 16 * g + 4 * r + (l >> 4);
            double mx = -__builtin_huge_val();
#pragma unroll
            for (int h = 0; h < 4; h++) {
                const int j = b0 + 64 * wb + 16 * h + (l & 15);
                const double v = acc[g][h][r] * inv_sqrt_d;
                if (i < R && j < R) {
                    L[(int64_t)i * R + j] = v;
                    mx = fmax(mx, v);
                }
            }
            // lanes l and l ^ 1, 2, 4, 8 hold the same row
            mx = fmax(mx, __shfl_xor(mx, 1, 16));
            mx = fmax(mx, __shfl_xor(mx, 2, 16));
            mx = fmax(mx, __shfl_xor(mx, 4, 16));
            mx = fmax(mx, __shfl_xor(mx, 8, 16));
            if ((l & 15) == 0 && i < R)
                atomicMax(rm + i, ord64(mx));
        }
}

template <int D>
__global__ __launch_bounds__(256, 2) void k_logits(const double *__restrict__ qa,
                                                const double *__restrict__ ka,
                                                const float *__restrict__ qm,
                                                const float *__restrict__ km, int R,
                                                double inv_sqrt_d, double *__restrict__ La,
                                                double *__restrict__ Lm,
                                                unsigned long long *__restrict__ rmax)
{
    __shared__ double sq[32][132], sk[32][132];
    const int b0 = blockIdx.x * 128, a0 = blockIdx.y * 128;
    const int bh = blockIdx.z >> 1, maxb = blockIdx.z & 1;
    if (maxb)
        logits_tile<D, true>(qa, ka, qm, km, R, inv_sqrt_d, La, Lm, rmax, bh, a0, b0, sq, sk);
    else
        logits_tile<D, false>(qa, ka, qm, km, R, inv_sqrt_d, La, Lm, rmax, bh, a0, b0, sq, sk);
}

// ---------------------------------------------------------------------------
// Row sums of one branch's exponentials for 64 query regions: Z is added
// strictly in key order (Z = (((e_0 + e_1) + e_2) + ...)).  Per chunk of 64
// key regions all four waves form the exponentials (coalesced row reads)
// into LDS, transposed, then wave 0 adds its lane's (row's) 64 values in
// order.  The next chunk's 16 logits per lane are loaded into registers
// before the current chunk's exponentials, so the row reads stay in flight
// through the exponentials and the in-order sum.
// ---------------------------------------------------------------------------
constexpr int kRowsumRows = 64 / 4;  // logits per lane per chunk

__device__ __forceinline__ void rowsum_load(const double *__restrict__ L, int R, int a0, int b,
                                            int wv, double (&x)[kRowsumRows])
{
#pragma unroll
    for (int i = 0; i < kRowsumRows; i++) {
        const int r = wv + 4 * i;
        x[i] = (a0 + r < R && b < R) ? L[(int64_t)r * R + b] : 0.0;
    }
}

__global__ __launch_bounds__(256) void k_rowsum(const double *__restrict__ La,
                                                const double *__restrict__ Lm, int R,
                                                const unsigned long long *__restrict__ rmax,
                                                double *__restrict__ zsum)
{
    __shared__ double es[64][65];
    __shared__ double mrow[64];
    const int a0 = blockIdx.x * 64, bh = blockIdx.y, br = blockIdx.z;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int64_t rbase = ((int64_t)bh * 2 + br) * R + a0;
    if (t < 64)
        mrow[t] = a0 + t < R ? unord64(rmax[rbase + t]) : 0.0;
    const double *L = (br ? Lm : La) + ((int64_t)bh * R + a0) * R;
    double cur[kRowsumRows], nxt[kRowsumRows] = {};
    rowsum_load(L, R, a0, lane, wv, cur);
    double z = 0.0;
    __syncthreads();
    for (int b0 = 0; b0 < R; b0 += 64) {
        const int b = b0 + lane;
        if (b0 + 64 < R)
            rowsum_load(L, R, a0, b + 64, wv, nxt);
#pragma unroll
        for (int i = 0; i < kRowsumRows; i++) {
            const int r = wv + 4 * i;
            es[lane][r] = (a0 + r < R && b < R) ? exp_draft(cur[i] - mrow[r]) : 0.0;
        }
        __syncthreads();
        if (wv == 0) {
            const int nb = R - b0 < 64 ? R - b0 : 64;
            for (int k = 0; k < nb; k++)
                z += es[k][lane];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kRowsumRows; i++)
            cur[i] = nxt[i];
    }
    if (wv == 0 && a0 + lane < R)
        zsum[rbase + lane] = z;
}

// ---------------------------------------------------------------------------
// Probabilities, mixture and ranking keys, elementwise over region pairs:
// p = e / Z per branch (e recomputed bit-identically), A = (1 - lambda) p_avg
// + lambda p_max with separate products, key = bits(fp32(A)).  One workgroup
// per query region; each thread loads kKeysUnroll pairs' logits before
// forming their keys, to keep enough reads in flight.
// ---------------------------------------------------------------------------
constexpr int kKeysUnroll = 4;

__global__ __launch_bounds__(256) void k_keys(const double *__restrict__ La,
                                              const double *__restrict__ Lm, int R, double lambda,
                                              const unsigned long long *__restrict__ rmax,
                                              const double *__restrict__ zsum,
                                              uint32_t *__restrict__ keys)
{
    const int a = blockIdx.x, bh = blockIdx.y;
    const int64_t r = (int64_t)bh * 2 * R + a;
    const double ma = unord64(rmax[r]), mm = unord64(rmax[r + R]);
    const double za = zsum[r], zm = zsum[r + R];
    const int64_t row = ((int64_t)bh * R + a) * R;
    const double w0 = 1.0 - lambda;
    for (int b0 = threadIdx.x; b0 < R; b0 += 256 * kKeysUnroll) {
        double xa[kKeysUnroll], xm[kKeysUnroll];
#pragma unroll
        for (int u = 0; u < kKeysUnroll; u++) {
            const int b = b0 + 256 * u;
            xa[u] = b < R ? La[row + b] : 0.0;
            xm[u] = b < R ? Lm[row + b] : 0.0;
        }
#pragma unroll
        for (int u = 0; u < kKeysUnroll; u++) {
            const int b = b0 + 256 * u;
            if (b < R) {
                const double pa = exp_draft(xa[u] - ma) / za;
                const double pm = exp_draft(xm[u] - mm) / zm;
                const double t0 = w0 * pa;
                const double t1 = lambda * pm;
                const double A = t0 + t1;
                keys[row + b] = __float_as_uint((float)A);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Row sums and keys in one pass, for region counts up to 256 * kSoftmaxNJMax:
// one workgroup per kSoftmaxRows query regions of a head.  Every thread
// forms the exponentials of its NJ key regions (b = t + 256 j) of both
// branches and both rows once and keeps them in registers.  The row sums go
// through LDS one 256-key chunk at a time: the workgroup writes chunk j, and
// one lane per (row, branch) adds it to its running sum strictly in key
// order (the same Z as k_rowsum).  Then every thread turns its registers
// into p = e / Z, the mixture and the key, as k_keys does.  The logits are
// read from HBM once and each exponential is formed once; the small LDS
// footprint leaves room for eight workgroups per CU, whose in-order sums
// run side by side.
// ---------------------------------------------------------------------------
constexpr int kSoftmaxRows = 2;    // query regions per workgroup
constexpr int kSoftmaxNJMax = 8;   // key chunks of 256 per row (R <= 2048)

template <int NJ>
__global__ __launch_bounds__(256) void k_softmax_keys(const double *__restrict__ La,
                                                      const double *__restrict__ Lm, int R, double lambda,
                                                      const unsigned long long *__restrict__ rmax,
                                                      double *__restrict__ zsum, uint32_t *__restrict__ keys)
{
    constexpr int NC = 2 * kSoftmaxRows;  // (row, branch) chains: c = 2 g + br
    __shared__ double es[NC][257];        // one chunk; odd pitch: the summing lanes hit distinct banks
    __shared__ double zs[NC];
    const int a0 = blockIdx.x * kSoftmaxRows, bh = blockIdx.y, t = threadIdx.x;
    double e[NC][NJ];
#pragma unroll
    for (int c = 0; c < NC; c++) {
        const int a = a0 + (c >> 1), br = c & 1;
        const double *L = (br ? Lm : La) + ((int64_t)bh * R + (a < R ? a : 0)) * R;
        double x[NJ];
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            const int b = t + 256 * j;
            x[j] = (a < R && b < R) ? L[b] : 0.0;
        }
        const double m = a < R ? unord64(rmax[((int64_t)bh * 2 + br) * R + a]) : 0.0;
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            const int b = t + 256 * j;
            e[c][j] = (a < R && b < R) ? exp_draft(x[j] - m) : 0.0;
        }
    }
    const bool summer = t < NC && a0 + (t >> 1) < R;
    double z = 0.0;
#pragma unroll
    for (int j = 0; j < NJ; j++) {
        if (j)
            __syncthreads();   // chunk j - 1 consumed
#pragma unroll
        for (int c = 0; c < NC; c++)
            es[c][t] = e[c][j];
        __syncthreads();
        if (summer) {
            const int nb = R - 256 * j < 256 ? R - 256 * j : 256;
            const double *row = es[t];
            int i = 0;
            for (; i + 8 <= nb; i += 8) {
                double v[8];
#pragma unroll
                for (int u = 0; u < 8; u++)
                    v[u] = row[i + u];
#pragma unroll
                for (int u = 0; u < 8; u++)
                    z += v[u];
            }
            for (; i < nb; i++)
                z += row[i];
        }
    }
    if (summer) {
        zs[t] = z;
        zsum[((int64_t)bh * 2 + (t & 1)) * R + a0 + (t >> 1)] = z;
    }
    __syncthreads();
    const double w0 = 1.0 - lambda;
#pragma unroll
    for (int g = 0; g < kSoftmaxRows; g++) {
        const int a = a0 + g;
        if (a >= R)
            break;
        const double za = zs[2 * g], zm = zs[2 * g + 1];
        uint32_t *kr = keys + ((int64_t)bh * R + a) * R;
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            const int b = t + 256 * j;
            if (b < R) {
                const double pa = e[2 * g][j] / za;
                const double pm = e[2 * g + 1][j] / zm;
                const double t0 = w0 * pa;
                const double t1 = lambda * pm;
                const double A = t0 + t1;
                kr[b] = __float_as_uint((float)A);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Head-scope radix select for the kTargets cumulative thresholds T16,
// T16 + T8 and T16 + T8 + T4 at once.
// ---------------------------------------------------------------------------
__global__ void k_rank_init(RankState *__restrict__ st, uint32_t *__restrict__ hist, int nseg,
                            int64_t t16, int64_t t8c, int64_t tk)
{
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < nseg * kTargets) {
        const int tg = i % kTargets;
        const int64_t T = tg == 0 ? t16 : (tg == 1 ? t8c : tk);
        RankState s;
        s.prefix = 0;
        s.mask = 0;
        s.rank = T > 0 ? (uint32_t)(T - 1) : 0u;
        s.active = T > 0 ? 1u : 0u;
        st[i] = s;
    }
    for (int j = i; j < nseg * kTargets * 256; j += gridDim.x * blockDim.x)
        hist[j] = 0;
}

__global__ __launch_bounds__(256) void k_rank_hist(const uint32_t *__restrict__ keys,
                                                   int64_t seglen, int64_t nchunk,
                                                   const RankState *__restrict__ st,
                                                   uint32_t *__restrict__ hist, int shift)
{
    __shared__ uint32_t h[kTargets][256];
    const int seg = blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * kChunk;
    const int t = threadIdx.x;
    RankState s[kTargets];
#pragma unroll
    for (int tg = 0; tg < kTargets; tg++) {
        h[tg][t] = 0;
        s[tg] = st[seg * kTargets + tg];
    }
    __syncthreads();
    // all of the thread's keys are loaded first; each thread then counts
    // runs of equal digits itself and adds a run with one LDS atomic (the
    // leading digits of nearby keys mostly agree)
    const uint32_t *kp = keys + (int64_t)seg * seglen;
    constexpr int J = kChunk / 256;
    uint32_t kv[J];
#pragma unroll
    for (int j = 0; j < J; j++) {
        const int64_t i = c0 + j * 256 + t;
        kv[j] = i < seglen ? kp[i] : 0u;
    }
    uint32_t last[kTargets], run[kTargets];
#pragma unroll
    for (int tg = 0; tg < kTargets; tg++) {
        last[tg] = 0u;
        run[tg] = 0u;
    }
#pragma unroll
    for (int j = 0; j < J; j++) {
        if (c0 + j * 256 + t < seglen) {
            const uint32_t k = kv[j];
            const uint32_t dg = (k >> shift) & 255u;
#pragma unroll
            for (int tg = 0; tg < kTargets; tg++)
                if (s[tg].active && ((k ^ s[tg].prefix) & s[tg].mask) == 0) {
                    if (run[tg] != 0u && dg != last[tg])
                        atomicAdd(&h[tg][last[tg]], run[tg]);
                    run[tg] = (run[tg] != 0u && dg == last[tg]) ? run[tg] + 1u : 1u;
                    last[tg] = dg;
                }
        }
    }
#pragma unroll
    for (int tg = 0; tg < kTargets; tg++)
        if (run[tg] != 0u)
            atomicAdd(&h[tg][last[tg]], run[tg]);
    __syncthreads();
    uint32_t *g = hist + (int64_t)seg * kTargets * 256;
#pragma unroll
    for (int tg = 0; tg < kTargets; tg++)
        if (h[tg][t])
            atomicAdd(&g[tg * 256 + t], h[tg][t]);
}

// One workgroup per segment: pick the digit holding the wanted rank (keys in
// descending order), fix it in the prefix, clear the histogram.
__global__ __launch_bounds__(256) void k_rank_select(RankState *__restrict__ st,
                                                     uint32_t *__restrict__ hist, int shift)
{
    __shared__ uint32_t scan[256];
    const int seg = blockIdx.x, t = threadIdx.x;
    for (int tg = 0; tg < kTargets; tg++) {
        RankState s = st[seg * kTargets + tg];
        uint32_t *g = hist + ((int64_t)seg * kTargets + tg) * 256;
        const int dg = 255 - t;  // thread t owns digit 255 - t (descending order)
        uint32_t cnt = g[dg];
        scan[t] = cnt;
        __syncthreads();
        for (int o = 1; o < 256; o <<= 1) {
            uint32_t v = t >= o ? scan[t - o] : 0u;
            __syncthreads();
            scan[t] += v;
            __syncthreads();
        }
        uint32_t incl = scan[t], excl = incl - cnt;
        if (s.active && excl <= s.rank && s.rank < incl) {
            s.prefix |= (uint32_t)dg << shift;
            s.mask |= 255u << shift;
            s.rank -= excl;
            st[seg * kTargets + tg] = s;
        }
        __syncthreads();
        g[dg] = 0;
        __syncthreads();
    }
}

// Count keys equal to each threshold per chunk.
__global__ __launch_bounds__(256) void k_rank_eqcount(const uint32_t *__restrict__ keys,
                                                      int64_t seglen, int64_t nchunk,
                                                      const RankState *__restrict__ st,
                                                      uint32_t *__restrict__ eq)
{
    const int seg = blockIdx.y, t = threadIdx.x;
    const int64_t c0 = (int64_t)blockIdx.x * kChunk;
    RankState s[kTargets];
    uint32_t n[kTargets];
#pragma unroll
    for (int tg = 0; tg < kTargets; tg++) {
        s[tg] = st[seg * kTargets + tg];
        n[tg] = 0;
    }
    const uint32_t *kp = keys + (int64_t)seg * seglen;
    constexpr int J = kChunk / 256;
    uint32_t kv[J];
#pragma unroll
    for (int j = 0; j < J; j++) {
        const int64_t i = c0 + j * 256 + t;
        kv[j] = i < seglen ? kp[i] : 0u;
    }
#pragma unroll
    for (int j = 0; j < J; j++) {
        if (c0 + j * 256 + t < seglen) {
#pragma unroll
            for (int tg = 0; tg < kTargets; tg++)
                n[tg] += (s[tg].active && kv[j] == s[tg].prefix);
        }
    }
    __shared__ uint32_t r[kTargets][4];
#pragma unroll
    for (int tg = 0; tg < kTargets; tg++) {
        n[tg] = wave_sum_u32(n[tg]);
        if ((t & 63) == 0)
            r[tg][t >> 6] = n[tg];
    }
    __syncthreads();
    if (t < kTargets)
        eq[((int64_t)seg * nchunk + blockIdx.x) * kTargets + t] = r[t][0] + r[t][1] + r[t][2] + r[t][3];
}

// Exclusive prefix of the equal-key counts over the chunks of each segment,
// in place: eq[seg][c][tg] becomes the number of keys equal to threshold tg
// in chunks 0 .. c-1.  One workgroup per segment walks its chunks 256 at a
// time with a carried total.
__global__ __launch_bounds__(256) void k_rank_eqscan(uint32_t *__restrict__ eq, int64_t nchunk)
{
    __shared__ uint32_t wsum[kTargets][4];
    const int seg = blockIdx.x, t = threadIdx.x, lane = t & 63, wv = t >> 6;
    uint32_t carry[kTargets] = {};
    for (int64_t c0 = 0; c0 < nchunk; c0 += 256) {
        const int64_t c = c0 + t;
        uint32_t *e = eq + ((int64_t)seg * nchunk + c) * kTargets;
        uint32_t v[kTargets], x[kTargets];
#pragma unroll
        for (int tg = 0; tg < kTargets; tg++) {
            v[tg] = c < nchunk ? e[tg] : 0u;
            x[tg] = v[tg];
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1)
#pragma unroll
            for (int tg = 0; tg < kTargets; tg++) {
                const uint32_t y = __shfl_up(x[tg], o, 64);
                x[tg] += lane >= o ? y : 0u;
            }
        if (lane == 63)
#pragma unroll
            for (int tg = 0; tg < kTargets; tg++)
                wsum[tg][wv] = x[tg];
        __syncthreads();
#pragma unroll
        for (int tg = 0; tg < kTargets; tg++) {
            uint32_t off = carry[tg];
            for (int w = 0; w < wv; w++)
                off += wsum[tg][w];
            if (c < nchunk)
                e[tg] = off + x[tg] - v[tg];
            carry[tg] += wsum[tg][0] + wsum[tg][1] + wsum[tg][2] + wsum[tg][3];
        }
        __syncthreads();
    }
}

// Tier of a key from its membership in the cumulative top sets.
__device__ __forceinline__ uint8_t tier_of(const bool (&in)[kTargets])
{
    return in[0] ? 16 : (in[1] ? 8 : (in[2] ? 4 : 0));
}

// Final tier per key: above a threshold, or equal to it and among the first
// `rank + 1` equal keys by pair index.  Thread t of the chunk's workgroup
// takes keys c0 + 256 j + t (coalesced); in pair-index order the chunk's
// keys run j-major, then wave, then lane.  The equal keys before a key are
// those of earlier chunks (eq, already an exclusive prefix over chunks), of
// earlier rows j, of earlier waves in row j and of lower lanes in its own
// wave (a ballot): per target one ballot and one popcount per row j and
// wave, exchanged once through LDS.
__global__ __launch_bounds__(256) void k_rank_tier(const uint32_t *__restrict__ keys,
                                                   int64_t seglen, int64_t nchunk,
                                                   const RankState *__restrict__ st,
                                                   const uint32_t *__restrict__ eq,
                                                   uint8_t *__restrict__ tier)
{
    constexpr int J = kChunk / 256;
    __shared__ uint32_t base[kTargets];
    __shared__ __attribute__((aligned(16))) uint32_t wcnt[kTargets][J][4];   // equal keys per (row j, wave)
    const int seg = blockIdx.y, t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int64_t ch = blockIdx.x;
    RankState s[kTargets];
#pragma unroll
    for (int tg = 0; tg < kTargets; tg++)
        s[tg] = st[seg * kTargets + tg];
    const int64_t c0 = ch * kChunk;
    const uint32_t *kp = keys + (int64_t)seg * seglen;
    uint32_t kv[J];
#pragma unroll
    for (int j = 0; j < J; j++) {
        const int64_t i = c0 + j * 256 + t;
        kv[j] = i < seglen ? kp[i] : 0u;
    }
    // equal keys in earlier chunks of this segment
    if (t < kTargets)
        base[t] = eq[((int64_t)seg * nchunk + ch) * kTargets + t];
    const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int j = 0; j < J; j++) {
        const bool valid = c0 + j * 256 + t < seglen;
#pragma unroll
        for (int tg = 0; tg < kTargets; tg++) {
            const uint64_t m = __ballot(valid && s[tg].active && kv[j] == s[tg].prefix);
            if (lane == 0)
                wcnt[tg][j][wv] = (uint32_t)__popcll(m);
        }
    }
    __syncthreads();
    uint32_t r[kTargets];
#pragma unroll
    for (int tg = 0; tg < kTargets; tg++)
        r[tg] = base[tg];
    uint8_t *tp = tier + (int64_t)seg * seglen;
#pragma unroll
    for (int j = 0; j < J; j++) {
        const int64_t i = c0 + j * 256 + t;
        const bool valid = i < seglen;
        const uint32_t k = kv[j];
        bool in[kTargets];
#pragma unroll
        for (int tg = 0; tg < kTargets; tg++) {
            const uint4 wc = *reinterpret_cast<const uint4 *>(&wcnt[tg][j][0]);
            const uint32_t before = (wv > 0 ? wc.x : 0u) + (wv > 1 ? wc.y : 0u) + (wv > 2 ? wc.z : 0u);
            const bool e = valid && s[tg].active && k == s[tg].prefix;
            const uint64_t m = __ballot(e);
            const uint32_t rank = r[tg] + before + (uint32_t)__popcll(m & lt);
            in[tg] = s[tg].active && (k > s[tg].prefix || (e && rank <= s[tg].rank));
            r[tg] += wc.x + wc.y + wc.z + wc.w;
        }
        if (valid)
            tp[i] = tier_of(in);
    }
}

// ---------------------------------------------------------------------------
// Row scope: one workgroup per query region, keys of the row in LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rank_rows(const uint32_t *__restrict__ keys, int R,
                                                   int64_t t16, int64_t t8c, int64_t tk,
                                                   uint8_t *__restrict__ tier)
{
    extern __shared__ uint32_t row[];
    __shared__ uint32_t hist[256], scan[256];
    __shared__ RankState s[kTargets];
    const int64_t seg = blockIdx.x;
    const int t = threadIdx.x;
    for (int b = t; b < R; b += 256)
        row[b] = keys[seg * R + b];
    if (t < kTargets) {
        const int64_t T = t == 0 ? t16 : (t == 1 ? t8c : tk);
        s[t].prefix = 0;
        s[t].mask = 0;
        s[t].rank = T > 0 ? (uint32_t)(T - 1) : 0u;
        s[t].active = T > 0;
    }
    __syncthreads();
    for (int tg = 0; tg < kTargets; tg++) {
        for (int shift = 24; shift >= 0; shift -= 8) {
            hist[t] = 0;
            __syncthreads();
            RankState cur = s[tg];
            for (int b = t; b < R; b += 256) {
                uint32_t k = row[b];
                if (cur.active && ((k ^ cur.prefix) & cur.mask) == 0)
                    atomicAdd(&hist[(k >> shift) & 255u], 1u);
            }
            __syncthreads();
            const int dg = 255 - t;
            uint32_t cnt = hist[dg];
            scan[t] = cnt;
            __syncthreads();
            for (int o = 1; o < 256; o <<= 1) {
                uint32_t v = t >= o ? scan[t - o] : 0u;
                __syncthreads();
                scan[t] += v;
                __syncthreads();
            }
            uint32_t incl = scan[t], excl = incl - cnt;
            if (cur.active && excl <= cur.rank && cur.rank < incl) {
                s[tg].prefix = cur.prefix | ((uint32_t)dg << shift);
                s[tg].mask = cur.mask | (255u << shift);
                s[tg].rank = cur.rank - excl;
            }
            __syncthreads();
        }
    }
    // resolve ties in index order: thread t owns keys [t*per, (t+1)*per)
    const int per = (R + 255) / 256;
    const int bb = t * per;
    uint32_t e[kTargets];
#pragma unroll
    for (int tg = 0; tg < kTargets; tg++)
        e[tg] = 0;
    for (int j = 0; j < per; j++) {
        int b = bb + j;
        if (b < R)
#pragma unroll
            for (int tg = 0; tg < kTargets; tg++)
                e[tg] += (s[tg].active && row[b] == s[tg].prefix);
    }
    __shared__ uint32_t sc2[kTargets][256];
#pragma unroll
    for (int tg = 0; tg < kTargets; tg++)
        sc2[tg][t] = e[tg];
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        uint32_t v[kTargets];
#pragma unroll
        for (int tg = 0; tg < kTargets; tg++)
            v[tg] = t >= o ? sc2[tg][t - o] : 0u;
        __syncthreads();
#pragma unroll
        for (int tg = 0; tg < kTargets; tg++)
            sc2[tg][t] += v[tg];
        __syncthreads();
    }
    uint32_t r[kTargets];
#pragma unroll
    for (int tg = 0; tg < kTargets; tg++)
        r[tg] = sc2[tg][t] - e[tg];
    for (int j = 0; j < per; j++) {
        int b = bb + j;
        if (b >= R)
            break;
        uint32_t k = row[b];
        bool in[kTargets];
#pragma unroll
        for (int tg = 0; tg < kTargets; tg++) {
            in[tg] = false;
            if (s[tg].active) {
                if (k > s[tg].prefix)
                    in[tg] = true;
                else if (k == s[tg].prefix) {
                    in[tg] = r[tg] <= s[tg].rank;
                    r[tg]++;
                }
            }
        }
        tier[seg * R + b] = tier_of(in);
    }
}

// ---------------------------------------------------------------------------
// Schedule: per query tile, the key tiles of its region's 16-bit key regions
// ascending, then 8-bit ascending, then MXFP4 ascending; counts n16, n8, n4
// of tiles.  The tier map is per region pair (G regions of tpr tiles each);
// a kept key region b contributes its tiles b tpr .. b tpr + tpr - 1 in
// order.  One wave per query tile (blockIdx.x); the tiles of one region
// get the same list.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_schedule(const uint8_t *__restrict__ tier, int R, int tpr,
                                                 int32_t *__restrict__ sched,
                                                 int32_t *__restrict__ cnt)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t rowl[];   // R bytes, rounded up to 16
    const int T = R * tpr;                                  // tiles per head
    const int64_t row = (int64_t)blockIdx.y * T + blockIdx.x;
    const int l = threadIdx.x;
    const uint8_t *tg = tier + ((int64_t)blockIdx.y * R + blockIdx.x / tpr) * R;
    // stage the row in LDS: dword reads when the row starts on a dword
    int b4 = 0;
    if ((reinterpret_cast<uintptr_t>(tg) & 3) == 0) {
        const uint32_t *t4 = reinterpret_cast<const uint32_t *>(tg);
        const int nw = R >> 2;
#pragma unroll 4
        for (int w = l; w < nw; w += 64)
            reinterpret_cast<uint32_t *>(rowl)[w] = t4[w];
        b4 = nw << 2;
    }
    for (int b = b4 + l; b < R; b += 64)
        rowl[b] = tg[b];
    __syncthreads();
    const uint8_t *tr = rowl;
    uint32_t n16 = 0, n8 = 0, n4 = 0;
    for (int b = l; b < R; b += 64) {
        uint8_t v = tr[b];
        n16 += v == 16;
        n8 += v == 8;
        n4 += v == 4;
    }
    n16 = wave_sum_u32(n16);
    n8 = wave_sum_u32(n8);
    n4 = wave_sum_u32(n4);
    int32_t *out = sched + row * T;
    uint32_t o16 = 0, o8 = n16, o4 = n16 + n8;   // in regions
    for (int b0 = 0; b0 < R; b0 += 64) {
        int b = b0 + l;
        uint8_t v = b < R ? tr[b] : 0;
        uint64_t m16 = __ballot(v == 16), m8 = __ballot(v == 8), m4 = __ballot(v == 4);
        uint64_t lt = (l == 0) ? 0ull : (~0ull >> (64 - l));
        int pos = -1;
        if (v == 16)
            pos = o16 + __popcll(m16 & lt);
        if (v == 8)
            pos = o8 + __popcll(m8 & lt);
        if (v == 4)
            pos = o4 + __popcll(m4 & lt);
        if (pos >= 0)
            for (int j = 0; j < tpr; j++)
                out[pos * tpr + j] = b * tpr + j;
        o16 += __popcll(m16);
        o8 += __popcll(m8);
        o4 += __popcll(m4);
    }
    if (l == 0) {
        cnt[row * kTargets] = (int32_t)(n16 * tpr);
        cnt[row * kTargets + 1] = (int32_t)(n8 * tpr);
        cnt[row * kTargets + 2] = (int32_t)(n4 * tpr);
    }
}

// Attention work order.  The attention kernel deals its workgroups to the 8
// XCDs round robin; XCD x takes work slots j = x*span .. x*span + span - 1
// (span = ceil(U/8) units) of every head.  A head's units (query regions of
// tpr tiles; a unit's first tile holds its counts) are ranked by kept tile
// count, largest first, ties in frame-fastest order (regions at one spatial
// position in consecutive latent frames keep largely the same key regions),
// and cut into 8 shares of span consecutive ranks.  A share holds units of
// about the same length: run together on one XCD, they walk their ascending
// key lists at about the same pace, so their tile reads meet in that XCD's
// L2.  XCD x takes share (x + h) mod 8 of head h, so over the heads every XCD
// gets every share.  Slots of ranks past the last unit hold -1.
// Grid: (ceil(U / 256), heads); U ints of LDS.
__global__ __launch_bounds__(256) void k_qorder(const int32_t *__restrict__ cnt, int U, int RF, int tpr,
                                                int32_t *__restrict__ qord)
{
    // one sort key per unit: tile count above (< 2^16), then the unit's
    // frame-fastest position reversed (< U <= 2^13), so that the rank is the
    // number of larger keys
    extern __shared__ uint32_t okey[];
    const int bh = (int)blockIdx.y, span = (U + 7) / 8, NF = U / RF;
    const int64_t row0 = (int64_t)bh * U;
    for (int a = threadIdx.x; a < U; a += 256) {
        const int32_t *c = cnt + ((row0 + a) * tpr) * kTargets;
        const uint32_t len = (uint32_t)(c[0] + c[1] + c[2]), fa = (uint32_t)((a % RF) * NF + a / RF);
        okey[a] = (len << 16) | (0xffffu - fa);
    }
    __syncthreads();
    int32_t *q = qord + (int64_t)bh * 8 * span;
    const int rot = bh % 8;
    const int a = (int)blockIdx.x * 256 + (int)threadIdx.x;
    if (a < U) {
        const uint32_t me = okey[a];
        int r = 0;
        for (int b = 0; b < U; b++)
            r += okey[b] > me;
        const int sh = r / span, i = r - sh * span;
        q[((sh - rot + 8) % 8) * span + i] = a;
    }
    // the 8 span - U (at most 7) ranks past the last unit: empty slots
    if (blockIdx.x == 0 && (int)threadIdx.x < 8 * span - U) {
        const int r = U + (int)threadIdx.x, sh = r / span, i = r - sh * span;
        q[((sh - rot + 8) % 8) * span + i] = -1;
    }
}

// Imported tier map: unknown values are skips; block-mean tiles exist at
// capacity 64 only (means: whether they are known).
__global__ void k_copy_tier(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int64_t n, int means)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        uint8_t v = src[i];
        dst[i] = (v == 16 || v == 8 || v == 4 || (means && v == kMeanTier)) ? v : 0;
    }
}

}  // namespace

// Skip replacement: every pair the ranking left out becomes a block-mean tile.
__global__ void k_skip_means_kernel(uint8_t *__restrict__ tier, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n && tier[i] == 0)
        tier[i] = kMeanTier;
}

void launch_skip_means(const da2_layout_s &L, char *ws, hipStream_t st)
{
    const int64_t n = (int64_t)L.BH * L.Rg * L.Rg;
    k_skip_means_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>((uint8_t *)(ws + L.ws.tier), n);
}

// The draft logits alone (both branches), e.g. for the block-mean tiles of
// an imported tier map.
void launch_draft_logits(const da2_layout_s &L, char *ws, hipStream_t st)
{
    const Workspace &W = L.ws;
    const double inv_sqrt_d = 1.0 / __builtin_sqrt((double)L.d);
    const int T2 = (L.Rg + 127) / 128;
    double *La = (double *)(ws + W.la), *Lm = (double *)(ws + W.lm);
    unsigned long long *rmax = (unsigned long long *)(ws + W.rmax);
    const int64_t nmax = (int64_t)L.BH * 2 * L.Rg * 2;  // as 32-bit words
    k_fill_words<<<(unsigned)((nmax + 255) / 256), 256, 0, st>>>((uint32_t *)rmax, nmax);
    dim3 g(T2, T2, 2 * L.BH);
    if (L.d == 128)
        k_logits<128><<<g, 256, 0, st>>>((const double *)(ws + W.qavg), (const double *)(ws + W.kavg),
                                         (const float *)(ws + W.qmax), (const float *)(ws + W.kmax),
                                         L.Rg, inv_sqrt_d, La, Lm, rmax);
    else
        k_logits<64><<<g, 256, 0, st>>>((const double *)(ws + W.qavg), (const double *)(ws + W.kavg),
                                        (const float *)(ws + W.qmax), (const float *)(ws + W.kmax),
                                        L.Rg, inv_sqrt_d, La, Lm, rmax);
}

void launch_draft(const da2_layout_s &L, double lambda, char *ws, hipStream_t st)
{
    const Workspace &W = L.ws;
    const int T = (L.Rg + 63) / 64;
    double *La = (double *)(ws + W.la), *Lm = (double *)(ws + W.lm);
    unsigned long long *rmax = (unsigned long long *)(ws + W.rmax);
    double *zsum = (double *)(ws + W.zsum);
    uint32_t *keys = (uint32_t *)(ws + W.keys);
    launch_draft_logits(L, ws, st);
    const int nj = (L.Rg + 255) / 256;
    if (nj <= kSoftmaxNJMax) {
        const dim3 g((L.Rg + kSoftmaxRows - 1) / kSoftmaxRows, L.BH);
        switch (nj) {
        case 1: k_softmax_keys<1><<<g, 256, 0, st>>>(La, Lm, L.Rg, lambda, rmax, zsum, keys); break;
        case 2: k_softmax_keys<2><<<g, 256, 0, st>>>(La, Lm, L.Rg, lambda, rmax, zsum, keys); break;
        case 3: k_softmax_keys<3><<<g, 256, 0, st>>>(La, Lm, L.Rg, lambda, rmax, zsum, keys); break;
        case 4: k_softmax_keys<4><<<g, 256, 0, st>>>(La, Lm, L.Rg, lambda, rmax, zsum, keys); break;
        case 5: k_softmax_keys<5><<<g, 256, 0, st>>>(La, Lm, L.Rg, lambda, rmax, zsum, keys); break;
        case 6: k_softmax_keys<6><<<g, 256, 0, st>>>(La, Lm, L.Rg, lambda, rmax, zsum, keys); break;
        default: k_softmax_keys<8><<<g, 256, 0, st>>>(La, Lm, L.Rg, lambda, rmax, zsum, keys); break;
        }
        return;
    }
    k_rowsum<<<dim3(T, L.BH, 2), 256, 0, st>>>(La, Lm, L.Rg, rmax, zsum);
    k_keys<<<dim3(L.Rg, L.BH), 256, 0, st>>>(La, Lm, L.Rg, lambda, rmax, zsum, keys);
}

void launch_rank(const da2_layout_s &L, int scope, int64_t t16, int64_t t8c, int64_t tk, char *ws,
                 hipStream_t st)
{
    const Workspace &W = L.ws;
    const uint32_t *keys = (const uint32_t *)(ws + W.keys);
    uint8_t *tier = (uint8_t *)(ws + W.tier);
    if (scope == 1) {
        k_rank_rows<<<(unsigned)((int64_t)L.BH * L.Rg), 256, sizeof(uint32_t) * L.Rg, st>>>(
            keys, L.Rg, t16, t8c, tk, tier);
        return;
    }
    RankState *rs = (RankState *)(ws + W.rank_state);
    uint32_t *hist = (uint32_t *)(ws + W.rank_hist), *eq = (uint32_t *)(ws + W.rank_eq);
    const int64_t seglen = (int64_t)L.Rg * L.Rg;
    const int64_t nchunk = L.nchunk;
    k_rank_init<<<(L.BH * kTargets * 256 + 255) / 256, 256, 0, st>>>(rs, hist, L.BH, t16, t8c, tk);
    dim3 g((unsigned)nchunk, L.BH);
    for (int shift = 24; shift >= 0; shift -= 8) {
        k_rank_hist<<<g, 256, 0, st>>>(keys, seglen, nchunk, rs, hist, shift);
        k_rank_select<<<L.BH, 256, 0, st>>>(rs, hist, shift);
    }
    k_rank_eqcount<<<g, 256, 0, st>>>(keys, seglen, nchunk, rs, eq);
    k_rank_eqscan<<<L.BH, 256, 0, st>>>(eq, nchunk);
    k_rank_tier<<<g, 256, 0, st>>>(keys, seglen, nchunk, rs, eq, tier);
}

void launch_schedule(const da2_layout_s &L, char *ws, hipStream_t st)
{
    const Workspace &W = L.ws;
    k_schedule<<<dim3(L.R, L.BH), 64, (L.Rg + 15) & ~15, st>>>((const uint8_t *)(ws + W.tier), L.Rg, L.tpr,
                                                (int32_t *)(ws + W.sched), (int32_t *)(ws + W.cnt));
    // work order over query regions: tiles at capacity 64, pairs of tiles
    // (one four-wave workgroup each) at capacity 128
    const int U = L.tpr == 2 ? L.Rg : L.R, UF = L.tpr == 2 ? L.Rfg : L.Rf;
    k_qorder<<<dim3((U + 255) / 256, L.BH), 256, sizeof(int32_t) * U, st>>>((const int32_t *)(ws + W.cnt), U, UF,
                                                                            L.tpr, (int32_t *)(ws + W.qord));
}

void launch_import_tier(const da2_layout_s &L, const uint8_t *src, char *ws, hipStream_t st)
{
    int64_t n = (int64_t)L.BH * L.Rg * L.Rg;
    k_copy_tier<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(src, (uint8_t *)(ws + L.ws.tier), n,
                                                             L.tpr == 1);
}

}  // namespace da2
