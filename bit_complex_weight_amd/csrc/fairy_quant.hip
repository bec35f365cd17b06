// fairy_quant.hip -- offline steps of the layer on gfx950:
//   widely-linear conversion   [Fairy2i article §2.1]
//   PhaseQuant codes, exact per-axis scales, recursive residual stages
//                              [Fairy2i article §3.1, §3.2, §4.1]
//   packing 16 codes per uint32
// All kernels are streaming (HBM-bound); they are launched on the caller's
// stream and allocate nothing.
#include "fairy_internal.h"

#include <mutex>
#include <type_traits>

namespace fairy {
namespace {

constexpr int kThreads = 256;

int grid_for(int64_t work, int per_block, int cap)
{
    int64_t g = (work + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return (int)g;
}

// ---------------------------------------------------------------------------
// Widely-linear conversion.  Each output is (a +- b)/2 of two fp32 inputs,
// formed exactly in fp64 and rounded once to fp32 (fp64 sum then fp32 rounding
// equals direct fp32 rounding because 53 >= 2*24+2; halving is exact).
// One thread converts four consecutive columns of one row.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float half_sum(float a, float b) { return (float)(((double)a + (double)b) * 0.5); }
__device__ __forceinline__ float half_diff(float a, float b) { return (float)(((double)a - (double)b) * 0.5); }

__global__ __launch_bounds__(kThreads) void k_real_to_complex4(const float4* __restrict__ R, int64_t n,
                                                               int64_t m4, float4* __restrict__ ure,
                                                               float4* __restrict__ uim,
                                                               float4* __restrict__ wre,
                                                               float4* __restrict__ wim)
{
    const int64_t ld = 2 * m4;
    for (int64_t i = blockIdx.y; i < n; i += gridDim.y) {
        for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < m4;
             j += (int64_t)gridDim.x * blockDim.x) {
            const float4 r11 = R[i * ld + j];
            const float4 r12 = R[i * ld + m4 + j];
            const float4 r21 = R[(n + i) * ld + j];
            const float4 r22 = R[(n + i) * ld + m4 + j];
            const int64_t o = i * m4 + j;
            ure[o] = make_float4(half_sum(r11.x, r22.x), half_sum(r11.y, r22.y), half_sum(r11.z, r22.z),
                                 half_sum(r11.w, r22.w));
            uim[o] = make_float4(half_diff(r21.x, r12.x), half_diff(r21.y, r12.y),
                                 half_diff(r21.z, r12.z), half_diff(r21.w, r12.w));
            wre[o] = make_float4(half_diff(r11.x, r22.x), half_diff(r11.y, r22.y),
                                 half_diff(r11.z, r22.z), half_diff(r11.w, r22.w));
            wim[o] = make_float4(half_sum(r12.x, r21.x), half_sum(r12.y, r21.y), half_sum(r12.z, r21.z),
                                 half_sum(r12.w, r21.w));
        }
    }
}

__global__ __launch_bounds__(kThreads) void k_real_to_complex1(const float* __restrict__ R, int64_t n,
                                                               int64_t m, float* __restrict__ ure,
                                                               float* __restrict__ uim,
                                                               float* __restrict__ wre,
                                                               float* __restrict__ wim)
{
    const int64_t ld = 2 * m;
    for (int64_t i = blockIdx.y; i < n; i += gridDim.y) {
        for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < m;
             j += (int64_t)gridDim.x * blockDim.x) {
            const float r11 = R[i * ld + j], r12 = R[i * ld + m + j];
            const float r21 = R[(n + i) * ld + j], r22 = R[(n + i) * ld + m + j];
            const int64_t o = i * m + j;
            ure[o] = half_sum(r11, r22);
            uim[o] = half_diff(r21, r12);
            wre[o] = half_diff(r11, r22);
            wim[o] = half_sum(r12, r21);
        }
    }
}

// ---------------------------------------------------------------------------
// PhaseQuant
// ---------------------------------------------------------------------------
// Quadrant of arg(a + ib) by exact comparisons: floor(2 theta/pi + 1/2) mod 4;
// on |a| == |b| the floor sends theta = 45, 135, -135, -45 degrees to
// codes 1, 2, 3, 0; zero (either sign) -> 0.
// Stated per axis: the code lies on the imaginary axis (odd code) when
// |b| > |a|, or on a tie of non-zero parts with equal signs (a == b != 0:
// 45 and -135 degrees); its sign (code >= 2) is that of the part on its
// axis, compared with 0, so a zero element (real axis, +0 or -0) gets code 0.
// Inputs are finite.  Written with comparisons and selects only: a branch
// per element would diverge inside the wave.
struct Phase {
    bool im;   // code on the imaginary axis (code & 1)
    bool neg;  // code >= 2
    float v;   // the part on the code's axis (b if im, else a)
};

__device__ __forceinline__ Phase phase_of(float a, float b)
{
    Phase ph;
    // bitwise on the comparisons: no short-circuit, so no exec-mask branch
    ph.im = (fabsf(b) > fabsf(a)) | ((a == b) & (a != 0.0f));
    ph.v = ph.im ? b : a;
    ph.neg = ph.v < 0.0f;
    return ph;
}

__device__ __forceinline__ uint32_t phase_code(const Phase& ph) { return (uint32_t)ph.im | ((uint32_t)ph.neg << 1); }

// R <- R - (s_re Re(i^c) + i s_im Im(i^c)), one fp32 operation on the code's
// axis: codes 0 / 1 subtract the scale, codes 2 / 3 subtract its negation
// (x - (-s) is the same IEEE operation as x + s).
__device__ __forceinline__ void residual_step(float& a, float& b, const Phase& ph, float s_re, float s_im)
{
    const float s = ph.im ? s_im : s_re;
    const float nv = ph.v - (ph.neg ? -s : s);
    a = ph.im ? a : nv;
    b = ph.im ? nv : b;
}

// Workspace per stage: 2 axes x 256 exponent buckets (uint64) + 2 counts.
// Bucket eb of an axis holds the sum of the 24-bit integer significands of
// the magnitudes whose biased exponent is eb (subnormals in bucket 1), so the
// axis sum is exactly  sum_eb bucket[eb] * 2^(eb-150).  Integer sums are
// order-independent: scales do not depend on launch shape or scheduling.
constexpr int kBuckets = 512;
constexpr int kStageWords = kBuckets + 2;

__global__ void k_fill_u64(unsigned long long* __restrict__ p, int64_t count)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0ull;
}

// Stage K: recompute R_K from W with the scales of stages < K (already on
// the device; K is a template parameter, so the residual steps are straight
// code), write code_K, and add |R_K| on the code's axis into the stage's
// exponent buckets.  V = 4: each thread takes 4 consecutive elements (float4
// loads, one 32-bit store of 4 codes); V = 1 for unaligned arrays.
// A block accumulates into kCopies interleaved LDS copies of the buckets,
// then adds its nonzero buckets into global copy blockIdx % kGlobalCopies of
// the stage's workspace (integer atomics: exact and order-independent; the
// copies keep the blocks of a launch from contending on ~40 hot addresses).
// The per-axis element counts are summed over the wave first and added by
// one lane: a per-lane atomic on one LDS address is turned by the compiler
// into a scalar loop over the wave's lanes, which cost more than the
// element work.
// Lanes of a wave mostly hit the same ~10 exponent buckets, and 64-bit LDS
// atomics on one address are served one at a time: 8 interleaved copies
// (32 KiB per block) cut those collisions; 2 copies measured ~7% slower.
constexpr int kCopies = 8;
constexpr int kGlobalCopies = 16;
constexpr int kStageBlocks = 1024;
constexpr int kMaxStages = 8;

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// One element of stage K: K residual steps with the earlier stages' scales,
// then its code; |part on the code's axis| goes into its exponent bucket
// (C interleaved LDS copies, this thread's copy `copy`): the exponent field
// ex (at least 1: subnormals go to bucket 1) and the 24-bit integer
// significand (mag - ex<<23 + 2^23 is man + 2^23 for a normal value and man
// for a subnormal one).  The add is unconditional (adding 0 for a zero
// magnitude changes nothing).
template <int K, int C>
__device__ __forceinline__ uint32_t pq_element(float a, float b, const float* sre, const float* sim,
                                               unsigned long long* s_buck, int copy, uint32_t& n_im)
{
#pragma unroll
    for (int j = 0; j < K; ++j) residual_step(a, b, phase_of(a, b), sre[j], sim[j]);
    const Phase ph = phase_of(a, b);
    n_im += ph.im;
    const uint32_t mag = __float_as_uint(ph.v) & 0x7FFFFFFFu;
    const uint32_t mx = mag > 0x800000u ? mag : 0x800000u;
    const uint32_t sig = mag - (mx & 0x7F800000u) + 0x800000u;
    atomicAdd(&s_buck[((ph.im ? 256u : 0u) + (mx >> 23)) * C + copy], (unsigned long long)sig);
    return phase_code(ph);
}

// End of a block: the per-axis element counts (summed over each wave, added
// by one lane into s_cnt), then the block's non-zero buckets into global
// copy g of the stage's workspace.
template <int C>
__device__ __forceinline__ void pq_flush(const unsigned long long* s_buck, unsigned long long* s_cnt,
                                         uint32_t n_re, uint32_t n_im, unsigned long long* g)
{
    const uint32_t n_re_w = wave_sum_u32(n_re), n_im_w = wave_sum_u32(n_im);
    if ((threadIdx.x & 63) == 0) {
        atomicAdd(&s_cnt[0], (unsigned long long)n_re_w);
        atomicAdd(&s_cnt[1], (unsigned long long)n_im_w);
    }
    __syncthreads();
    for (int t = threadIdx.x; t < kBuckets; t += blockDim.x) {
        unsigned long long v = 0ull;
#pragma unroll
        for (int c = 0; c < C; ++c) v += s_buck[t * C + c];
        if (v) atomicAdd(&g[t], v);
    }
    if (threadIdx.x < 2 && s_cnt[threadIdx.x]) atomicAdd(&g[kBuckets + threadIdx.x], s_cnt[threadIdx.x]);
}

template <int V, int K>
__global__ __launch_bounds__(kThreads) void k_pq_stage(const float* __restrict__ w_re,
                                                       const float* __restrict__ w_im, int64_t count,
                                                       const float* __restrict__ scales,
                                                       uint8_t* __restrict__ codes,
                                                       unsigned long long* __restrict__ ws)
{
    typedef typename std::conditional<V == 4, float4, float>::type vec_t;
    typedef typename std::conditional<V == 4, uint32_t, uint8_t>::type code_t;
    __shared__ unsigned long long s_buck[kBuckets * kCopies];
    __shared__ unsigned long long s_cnt[2];
    for (int t = threadIdx.x; t < kBuckets * kCopies; t += blockDim.x) s_buck[t] = 0ull;
    if (threadIdx.x < 2) s_cnt[threadIdx.x] = 0ull;
    // the scales of the earlier stages (uniform values)
    float sre[K > 0 ? K : 1], sim[K > 0 ? K : 1];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        sre[j] = scales[2 * j];
        sim[j] = scales[2 * j + 1];
    }
    __syncthreads();
    const int copy = threadIdx.x % kCopies;
    const int64_t nv = count / V;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const vec_t* vr = reinterpret_cast<const vec_t*>(w_re);
    const vec_t* vi = reinterpret_cast<const vec_t*>(w_im);
    code_t* cout = reinterpret_cast<code_t*>(codes + (int64_t)K * count);
    uint32_t n_im = 0, n_all = 0;
    auto element = [&](float a, float b) -> uint32_t {
        return pq_element<K, kCopies>(a, b, sre, sim, s_buck, copy, n_im);
    };
    auto vec = [&](const vec_t ra, const vec_t rb) -> code_t {
        n_all += V;
        if constexpr (V == 4) {
            uint32_t p = element(ra.x, rb.x);
            p |= element(ra.y, rb.y) << 8;
            p |= element(ra.z, rb.z) << 16;
            p |= element(ra.w, rb.w) << 24;
            return p;
        } else {
            return (code_t)element(ra, rb);
        }
    };
    // Whole tiles of kUnroll grid-stride steps: every thread has all of
    // them, whose loads are issued before any is processed; then the rest
    // one step at a time.
    constexpr int kUnroll = 4;
    const int64_t tile = kUnroll * stride;
    const int64_t full = nv / tile;
    int64_t iv0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t t = 0; t < full; ++t, iv0 += tile) {
        vec_t ra[kUnroll], rb[kUnroll];
#pragma unroll
        for (int q = 0; q < kUnroll; ++q) {
            ra[q] = vr[iv0 + q * stride];
            rb[q] = vi[iv0 + q * stride];
        }
#pragma unroll
        for (int q = 0; q < kUnroll; ++q) cout[iv0 + q * stride] = vec(ra[q], rb[q]);
    }
    for (int64_t iv = iv0; iv < nv; iv += stride) cout[iv] = vec(vr[iv], vi[iv]);
    pq_flush<kCopies>(s_buck, s_cnt, n_all - n_im, n_im,
                      ws + ((int64_t)K * kGlobalCopies + blockIdx.x % kGlobalCopies) * kStageWords);
}

// Stage K for both matrices of a real layer, read straight from R [2n][2m]:
// U = ((R11 + R22) + i (R21 - R12)) / 2 and W = ((R11 - R22) + i (R12 + R21)) / 2
// are formed per element by the conversion's own half_sum / half_diff, then
// each goes through pq_element with its own scales and buckets.  Codes and
// bucket sums therefore equal those of the conversion followed by the stage
// kernel on U and on W, and the U, W planes are never written.  V = 4: four
// consecutive columns (16-byte aligned R); a block holds both matrices'
// buckets in LDS, four copies each.
constexpr int kCopiesR = 4;

template <int V, int K>
__global__ __launch_bounds__(kThreads) void k_pq_real_stage(const float* __restrict__ R, int64_t n, int64_t m,
                                                            const float* __restrict__ sc_u,
                                                            const float* __restrict__ sc_w,
                                                            uint8_t* __restrict__ codes_u,
                                                            uint8_t* __restrict__ codes_w,
                                                            unsigned long long* __restrict__ ws_u,
                                                            unsigned long long* __restrict__ ws_w)
{
    typedef typename std::conditional<V == 4, float4, float>::type vec_t;
    typedef typename std::conditional<V == 4, uint32_t, uint8_t>::type code_t;
    __shared__ unsigned long long s_buck[2][kBuckets * kCopiesR];
    __shared__ unsigned long long s_cnt[2][2];
    for (int t = threadIdx.x; t < 2 * kBuckets * kCopiesR; t += blockDim.x) (&s_buck[0][0])[t] = 0ull;
    if (threadIdx.x < 4) (&s_cnt[0][0])[threadIdx.x] = 0ull;
    float sre_u[K > 0 ? K : 1], sim_u[K > 0 ? K : 1], sre_w[K > 0 ? K : 1], sim_w[K > 0 ? K : 1];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        sre_u[j] = sc_u[2 * j];
        sim_u[j] = sc_u[2 * j + 1];
        sre_w[j] = sc_w[2 * j];
        sim_w[j] = sc_w[2 * j + 1];
    }
    __syncthreads();
    const int copy = threadIdx.x % kCopiesR;
    const int64_t count = n * m;
    const uint32_t mv = (uint32_t)(m / V);       // vectors per row of U / W
    const uint32_t nv = (uint32_t)(count / V);   // count < 2^32
    const int64_t ldv = 2 * (int64_t)mv;         // vectors per row of R
    const vec_t* Rv = reinterpret_cast<const vec_t*>(R);
    code_t* cu = reinterpret_cast<code_t*>(codes_u + (int64_t)K * count);
    code_t* cw = reinterpret_cast<code_t*>(codes_w + (int64_t)K * count);
    uint32_t n_im_u = 0, n_im_w = 0, n_all = 0;
    auto one = [&](float r11, float r12, float r21, float r22, uint32_t& cu1, uint32_t& cw1) {
        cu1 = pq_element<K, kCopiesR>(half_sum(r11, r22), half_diff(r21, r12), sre_u, sim_u, s_buck[0], copy,
                                      n_im_u);
        cw1 = pq_element<K, kCopiesR>(half_diff(r11, r22), half_sum(r12, r21), sre_w, sim_w, s_buck[1], copy,
                                      n_im_w);
    };
    // vector iv of U / W: row i = iv / mv, vector column j; its R vectors
    // are R11 = (i, j), R12 = (i, mv + j), R21 = (n + i, j), R22 = (n + i, mv + j)
    auto vec = [&](uint32_t iv) {
        const uint32_t i = iv / mv, j = iv - i * mv;
        const int64_t top = (int64_t)i * ldv + j, bot = ((int64_t)n + i) * ldv + j;
        const vec_t r11 = Rv[top], r12 = Rv[top + mv], r21 = Rv[bot], r22 = Rv[bot + mv];
        n_all += V;
        if constexpr (V == 4) {
            uint32_t pu = 0u, pw = 0u, a, b;
            one(r11.x, r12.x, r21.x, r22.x, a, b); pu |= a;       pw |= b;
            one(r11.y, r12.y, r21.y, r22.y, a, b); pu |= a << 8;  pw |= b << 8;
            one(r11.z, r12.z, r21.z, r22.z, a, b); pu |= a << 16; pw |= b << 16;
            one(r11.w, r12.w, r21.w, r22.w, a, b); pu |= a << 24; pw |= b << 24;
            cu[iv] = pu;
            cw[iv] = pw;
        } else {
            uint32_t a, b;
            one(r11, r12, r21, r22, a, b);
            cu[iv] = (code_t)a;
            cw[iv] = (code_t)b;
        }
    };
    // 64-bit loop index (nv + stride may pass 2^32); iv < nv < 2^32 inside
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t iv = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; iv < (int64_t)nv; iv += stride)
        vec((uint32_t)iv);
    const int64_t gcopy = ((int64_t)K * kGlobalCopies + blockIdx.x % kGlobalCopies) * kStageWords;
    pq_flush<kCopiesR>(s_buck[0], s_cnt[0], n_all - n_im_u, n_im_u, ws_u + gcopy);
    pq_flush<kCopiesR>(s_buck[1], s_cnt[1], n_all - n_im_w, n_im_w, ws_w + gcopy);
}

// Exact mean -> fp32, nearest even.
// N = sum_eb bucket[eb] * 2^(eb-1) is the sum of the magnitudes in units of
// 2^-149 (< 2^311), the mean is N / cnt * 2^-149 with cnt < 2^32.
// Let T = bitlen(N), E = max(0, T - 64), Ntop = N >> E (exactly N when
// N < 2^64, which covers every subnormal result).  With Q1 = Ntop / cnt and
// r1 = Ntop % cnt,  N / cnt = Q1 * 2^E + d  with 0 <= d < 2^E and d = 0 iff
// r1 == 0 and the low E bits of N are zero.  Q1 has >= 32 significant bits
// when E > 0, so Q1 plus that sticky bit decide the rounding exactly.
constexpr int kLimbs = 10;  // 320 bits

constexpr int kFinThreads = 256;  // one thread per exponent bucket of an axis
constexpr int kFinParts = 16;     // threads per limb (a power of two dividing 64)
static_assert(64 % kFinParts == 0 && (kFinParts & (kFinParts - 1)) == 0, "a limb's threads share one wave");

// The exact mean of one axis rounded to fp32: limb q of N is lsum[q] (each
// below 2^40, so the carries are taken here), cnt the number of entries.
__device__ float exact_mean_f32(const unsigned long long (&lsum)[kLimbs], unsigned long long cnt)
{
    float result = 0.0f;
    if (cnt != 0ull) {
        uint32_t N[kLimbs];
        unsigned long long carry = 0ull;
#pragma unroll
        for (int q = 0; q < kLimbs; ++q) {
            const unsigned long long t = lsum[q] + carry;
            N[q] = (uint32_t)t;
            carry = t >> 32;
        }
        int T = 0;
#pragma unroll
        for (int q = 0; q < kLimbs; ++q)
            if (N[q]) T = 32 * q + (32 - __clz(N[q]));
        if (T > 0) {
            const int E = T > 64 ? T - 64 : 0;
            // Ntop = N >> E and the sticky bit of the shifted-out part
            unsigned long long top = 0ull;
            bool low = false;
#pragma unroll
            for (int q = 0; q < kLimbs; ++q) {
                const int pos = 32 * q - E;  // bit position of limb q inside Ntop
                const unsigned long long v = N[q];
                if (pos >= 64 || pos <= -32) {
                    if (pos <= -32 && v) low = true;
                } else if (pos >= 0) {
                    top |= v << pos;
                } else {
                    top |= v >> (-pos);
                    if (v & ((1ull << (-pos)) - 1ull)) low = true;
                }
            }
            const unsigned long long Q1 = top / cnt, r1 = top % cnt;
            const bool sticky0 = low || r1 != 0ull;
            // value = (Q1 + frac) * 2^(E - 149);  keep 24 bits (or the subnormal LSB 2^-149)
            const int L1 = 64 - __clzll(Q1);
            int shift = L1 - 24;
            if (shift < -E) shift = -E;  // LSB weight may not fall below 2^-149
            // shift >= 0 always: E > 0 gives L1 >= 32, E == 0 clamps shift at 0
            unsigned long long kept;
            bool rbit, sticky;
            if (shift > 0) {
                kept = Q1 >> shift;
                rbit = (Q1 >> (shift - 1)) & 1ull;
                sticky = sticky0 || (shift > 1 && (Q1 & ((1ull << (shift - 1)) - 1ull)));
            } else {
                // E == 0: Q1 = floor(N / cnt) exactly; the discarded part is r1 / cnt
                kept = Q1;
                rbit = 2ull * r1 >= cnt;
                sticky = 2ull * r1 > cnt;
            }
            if (rbit && (sticky || (kept & 1ull))) kept += 1ull;
            int ex = shift + E - 149;  // value = kept * 2^ex
            if (kept == (1ull << 24)) { kept >>= 1; ex += 1; }
            uint32_t bits = 0u;
            if (kept >= (1ull << 23)) bits = ((uint32_t)(ex + 150) << 23) | (uint32_t)(kept - (1ull << 23));
            else bits = (uint32_t)kept;  // subnormal: ex == -149
            result = __uint_as_float(bits);
        }
    }
    return result;
}

// Two blocks per matrix, one per axis.  Thread t owns exponent bucket t of the axis:
// it adds the bucket's global copies (all loads at once), cuts
// bucket * 2^(t-1) into 32-bit limb pieces, and the pieces of each limb are
// added by kFinParts threads from LDS, then across those threads' lanes
// (integer sums: exact in any order); one thread then divides by the count
// and rounds.
__global__ __launch_bounds__(kFinThreads) void k_pq_finalize(const unsigned long long* __restrict__ ws_a, int32_t k,
                                                              float* __restrict__ scales_a,
                                                              const unsigned long long* __restrict__ ws_b,
                                                              float* __restrict__ scales_b)
{
    // blockIdx.y picks the matrix (a second one only for a real layer's U, W)
    const unsigned long long* ws = blockIdx.y ? ws_b : ws_a;
    float* scales = blockIdx.y ? scales_b : scales_a;
    __shared__ unsigned long long s_piece[kLimbs][kFinThreads];
    __shared__ unsigned long long s_lsum[kLimbs];
    __shared__ unsigned long long s_cnt[kGlobalCopies];
    const int axis = blockIdx.x;
    const int eb = threadIdx.x;
    const unsigned long long* g0 = ws + (int64_t)k * kGlobalCopies * kStageWords;
    unsigned long long cv[kGlobalCopies];
#pragma unroll
    for (int c = 0; c < kGlobalCopies; ++c) cv[c] = g0[(int64_t)c * kStageWords + 256 * axis + eb];
    // the copies of the axis's count, one per thread, in the same round of loads
    if (eb < kGlobalCopies) s_cnt[eb] = g0[(int64_t)eb * kStageWords + kBuckets + axis];
    unsigned long long v = 0ull;
#pragma unroll
    for (int c = 0; c < kGlobalCopies; ++c) v += cv[c];
    if (eb == 0) v = 0ull;  // bucket 0 is never used (subnormals are in bucket 1)
    // v * 2^(eb-1), seen limb by limb (limb q holds bits 32q .. 32q+31)
#pragma unroll
    for (int q = 0; q < kLimbs; ++q) {
        const int sh = eb - 1 - 32 * q;
        uint32_t piece;
        if (sh >= 32 || sh <= -64) piece = 0u;
        else if (sh >= 0) piece = (uint32_t)(v << sh);
        else piece = (uint32_t)(v >> (-sh));
        s_piece[q][eb] = piece;
    }
    __syncthreads();
    {
        // thread t < kLimbs * kFinParts sums every kFinParts-th piece of limb
        // t / kFinParts; the kFinParts threads of a limb are consecutive lanes
        // of one wave and finish the sum with a butterfly
        const int q = threadIdx.x / kFinParts, part = threadIdx.x % kFinParts;
        unsigned long long acc = 0ull;
        if (q < kLimbs) {
#pragma unroll
            for (int i = 0; i < kFinThreads / kFinParts; ++i) acc += s_piece[q][part + kFinParts * i];
        }
#pragma unroll
        for (int off = kFinParts / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
        if (q < kLimbs && part == 0) s_lsum[q] = acc;
    }
    __syncthreads();
    if (threadIdx.x != 0) return;
    unsigned long long lsum[kLimbs];
#pragma unroll
    for (int q = 0; q < kLimbs; ++q) lsum[q] = s_lsum[q];
    unsigned long long cnt = 0ull;
#pragma unroll
    for (int c = 0; c < kGlobalCopies; ++c) cnt += s_cnt[c];
    scales[2 * k + axis] = exact_mean_f32(lsum, cnt);
}

__global__ __launch_bounds__(kThreads) void k_pq_resid(const float* __restrict__ w_re,
                                                       const float* __restrict__ w_im, int64_t count,
                                                       int32_t stages, const float* __restrict__ scales,
                                                       float* __restrict__ r_re, float* __restrict__ r_im)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x) {
        float a = w_re[i], b = w_im[i];
        for (int j = 0; j < stages; ++j) residual_step(a, b, phase_of(a, b), scales[2 * j], scales[2 * j + 1]);
        if (r_re) r_re[i] = a;
        if (r_im) r_im[i] = b;
    }
}

// ---------------------------------------------------------------------------
// Packing.  One thread per output word; reads the word's 16 codes as one
// 16-byte load (m % 16 == 0, 16-byte aligned codes).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t tiled_bit(int t) { return (t & 1) ? (uint32_t)(31 - t) : (uint32_t)(14 - t); }

__device__ __forceinline__ void load16(const uint8_t* p, uint8_t out[16])
{
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int t = 0; t < 16; ++t) out[t] = (uint8_t)(w[t >> 2] >> (8 * (t & 3)));
}

// ROW16: one thread per output word (consecutive threads, consecutive words
// of one plane row: coalesced both ways).
__global__ __launch_bounds__(kThreads) void k_pack_row16(const uint8_t* __restrict__ codes,
                                                         uint32_t* __restrict__ out, int64_t nwords)
{
    for (int64_t wi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; wi < nwords;
         wi += (int64_t)gridDim.x * blockDim.x) {
        // word wi covers codes 16 wi .. 16 wi + 15 of the [planes][rows][m] array
        uint8_t c[16];
        load16(codes + 16 * wi, c);
        uint32_t word = 0u;
#pragma unroll
        for (int t = 0; t < 16; ++t) word |= ((uint32_t)c[t] & 3u) << (2 * t);
        out[wi] = word;
    }
}

__global__ __launch_bounds__(kThreads) void k_unpack_row16(const uint32_t* __restrict__ in,
                                                           uint8_t* __restrict__ codes, int64_t nwords)
{
    for (int64_t wi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; wi < nwords;
         wi += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t word = in[wi];
        uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int t = 0; t < 16; ++t) o[t >> 2] |= ((word >> (2 * t)) & 3u) << (8 * (t & 3));
        *reinterpret_cast<uint4*>(codes + 16 * wi) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// TILED64, one thread per (row, 64-column group, plane), planes fastest:
// the thread reads the group's 64 codes of its plane (64 contiguous bytes,
// four 16-byte loads issued together) and writes that plane's 16-byte unit,
// so a wave's stores cover 1 KiB of the output in order and its loads 16
// groups of each plane.  (One thread per group walking the planes one at a
// time kept only 64 bytes per thread in flight.)  I is the index type:
// 32-bit unless the unit count needs more.
__device__ __forceinline__ uint32_t pack_word16(const uint4 v)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t word = 0u;
#pragma unroll
    for (int t = 0; t < 16; ++t) word |= ((w[t >> 2] >> (8 * (t & 3))) & 3u) << tiled_bit(t);
    return word;
}

template <typename I>
__global__ __launch_bounds__(kThreads) void k_pack_tiled(const uint8_t* __restrict__ codes, int32_t planes,
                                                         int64_t rows, int64_t m, uint32_t* __restrict__ out)
{
    const I G = (I)((m + 63) / 64);
    const I total = (I)rows * G * (I)planes;
    const I pl = (I)planes;
    for (I t = (I)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (I)gridDim.x * blockDim.x) {
        const I i = t / pl;
        const int p = (int)(t - i * pl);
        const I r = i / G, g = i - r * G;
        const int64_t c0 = 64 * (int64_t)g;
        const uint4* src = reinterpret_cast<const uint4*>(codes + ((int64_t)p * rows + (int64_t)r) * m + c0);
        uint4 v[4];
        if (m - c0 >= 64) {
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = src[u];
        } else {
            const int nw = (int)((m - c0) >> 4);  // valid 16-column words (m % 16 == 0)
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = (u < nw) ? src[u] : make_uint4(0, 0, 0, 0);
        }
        uint4 o;
        o.x = pack_word16(v[0]);
        o.y = pack_word16(v[1]);
        o.z = pack_word16(v[2]);
        o.w = pack_word16(v[3]);
        reinterpret_cast<uint4*>(out)[t] = o;  // unit (r, g) of plane p: (i * planes + p) = t
    }
}

// The inverse, with the same thread mapping: one 16-byte unit in, the
// group's 64 codes of that plane out.
template <typename I>
__global__ __launch_bounds__(kThreads) void k_unpack_tiled(const uint32_t* __restrict__ in, int32_t planes,
                                                           int64_t rows, int64_t m, uint8_t* __restrict__ codes)
{
    const I G = (I)((m + 63) / 64);
    const I total = (I)rows * G * (I)planes;
    const I pl = (I)planes;
    for (I t = (I)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (I)gridDim.x * blockDim.x) {
        const I i = t / pl;
        const int p = (int)(t - i * pl);
        const I r = i / G, g = i - r * G;
        const int64_t c0 = 64 * (int64_t)g;
        const int nw = (m - c0) >= 64 ? 4 : (int)((m - c0) >> 4);
        const uint4 wv = reinterpret_cast<const uint4*>(in)[t];
        const uint32_t words[4] = {wv.x, wv.y, wv.z, wv.w};
        uint4* dst = reinterpret_cast<uint4*>(codes + ((int64_t)p * rows + (int64_t)r) * m + c0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (u >= nw) break;
            uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int k = 0; k < 16; ++k) o[k >> 2] |= ((words[u] >> tiled_bit(k)) & 3u) << (8 * (k & 3));
            dst[u] = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_real_to_complex(const float* R, int64_t n, int64_t m, float* u_re, float* u_im,
                                  float* w_re, float* w_im, hipStream_t s)
{
    const bool vec = (m % 4 == 0) && ((((uintptr_t)R) | ((uintptr_t)u_re) | ((uintptr_t)u_im) |
                                       ((uintptr_t)w_re) | ((uintptr_t)w_im)) % 16 == 0);
    const int64_t cols = vec ? m / 4 : m;
    dim3 grid(grid_for(cols, kThreads, 64), (unsigned)(n < 65535 ? n : 65535));
    if (vec)
        hipLaunchKernelGGL(k_real_to_complex4, grid, dim3(kThreads), 0, s, (const float4*)R, n, m / 4,
                           (float4*)u_re, (float4*)u_im, (float4*)w_re, (float4*)w_im);
    else
        hipLaunchKernelGGL(k_real_to_complex1, grid, dim3(kThreads), 0, s, R, n, m, u_re, u_im, w_re, w_im);
    return hipGetLastError();
}

namespace {
// stage k's kernel (k residual steps before its code)
template <int V>
hipError_t launch_stage(int32_t k, int grid, const float* w_re, const float* w_im, int64_t count, const float* scales,
                        uint8_t* codes, unsigned long long* ws, hipStream_t s)
{
    const dim3 g(grid), b(kThreads);
    switch (k) {
    case 0: hipLaunchKernelGGL((k_pq_stage<V, 0>), g, b, 0, s, w_re, w_im, count, scales, codes, ws); break;
    case 1: hipLaunchKernelGGL((k_pq_stage<V, 1>), g, b, 0, s, w_re, w_im, count, scales, codes, ws); break;
    case 2: hipLaunchKernelGGL((k_pq_stage<V, 2>), g, b, 0, s, w_re, w_im, count, scales, codes, ws); break;
    case 3: hipLaunchKernelGGL((k_pq_stage<V, 3>), g, b, 0, s, w_re, w_im, count, scales, codes, ws); break;
    case 4: hipLaunchKernelGGL((k_pq_stage<V, 4>), g, b, 0, s, w_re, w_im, count, scales, codes, ws); break;
    case 5: hipLaunchKernelGGL((k_pq_stage<V, 5>), g, b, 0, s, w_re, w_im, count, scales, codes, ws); break;
    case 6: hipLaunchKernelGGL((k_pq_stage<V, 6>), g, b, 0, s, w_re, w_im, count, scales, codes, ws); break;
    case 7: hipLaunchKernelGGL((k_pq_stage<V, 7>), g, b, 0, s, w_re, w_im, count, scales, codes, ws); break;
    default: return hipErrorInvalidValue;
    }
    static_assert(kMaxStages == 8, "one case per stage");
    return hipGetLastError();
}
}  // namespace

size_t phasequant_workspace_bytes(int32_t stages)
{
    return (size_t)stages * kGlobalCopies * kStageWords * sizeof(unsigned long long);
}

hipError_t launch_phasequant(const float* w_re, const float* w_im, int64_t count, int32_t stages,
                             uint8_t* codes, float* scales, float* resid_re, float* resid_im,
                             void* workspace, hipStream_t s)
{
    unsigned long long* ws = (unsigned long long*)workspace;
    const int64_t nws = (int64_t)stages * kGlobalCopies * kStageWords;
    hipLaunchKernelGGL(k_fill_u64, dim3(grid_for(nws, kThreads, 256)), dim3(kThreads), 0, s, ws, nws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const bool vec = count % 4 == 0 && ((((uintptr_t)w_re) | ((uintptr_t)w_im) | ((uintptr_t)codes)) % 16 == 0);
    const int grid = grid_for(vec ? count / 4 : count, kThreads, kStageBlocks);
    for (int32_t k = 0; k < stages; ++k) {
        if ((e = vec ? launch_stage<4>(k, grid, w_re, w_im, count, scales, codes, ws, s)
                     : launch_stage<1>(k, grid, w_re, w_im, count, scales, codes, ws, s)) != hipSuccess)
            return e;
        hipLaunchKernelGGL(k_pq_finalize, dim3(2, 1), dim3(kFinThreads), 0, s, (const unsigned long long*)ws, k, scales,
                           (const unsigned long long*)nullptr, (float*)nullptr);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (resid_re || resid_im) {
        hipLaunchKernelGGL(k_pq_resid, dim3(grid), dim3(kThreads), 0, s, w_re, w_im, count, stages,
                           (const float*)scales, resid_re, resid_im);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

namespace {
template <int V>
hipError_t launch_real_stage(int32_t k, int grid, const float* R, int64_t n, int64_t m, const float* sc_u,
                             const float* sc_w, uint8_t* codes_u, uint8_t* codes_w, unsigned long long* ws_u,
                             unsigned long long* ws_w, hipStream_t s)
{
    const dim3 g(grid), b(kThreads);
    switch (k) {
#define FAIRY_REAL_STAGE(K)                                                                                      \
    case K:                                                                                                      \
        hipLaunchKernelGGL((k_pq_real_stage<V, K>), g, b, 0, s, R, n, m, sc_u, sc_w, codes_u, codes_w, ws_u, ws_w); \
        break;
        FAIRY_REAL_STAGE(0)
        FAIRY_REAL_STAGE(1)
        FAIRY_REAL_STAGE(2)
        FAIRY_REAL_STAGE(3)
        FAIRY_REAL_STAGE(4)
        FAIRY_REAL_STAGE(5)
        FAIRY_REAL_STAGE(6)
        FAIRY_REAL_STAGE(7)
#undef FAIRY_REAL_STAGE
    default: return hipErrorInvalidValue;
    }
    static_assert(kMaxStages == 8, "one case per stage");
    return hipGetLastError();
}
}  // namespace

size_t phasequant_real_workspace_bytes(int32_t stages) { return 2 * phasequant_workspace_bytes(stages); }

hipError_t launch_phasequant_real(const float* R, int64_t n, int64_t m, int32_t stages, uint8_t* codes,
                                  float* scales, void* workspace, hipStream_t s)
{
    const int64_t count = n * m;
    const int64_t per = (int64_t)stages * kGlobalCopies * kStageWords;  // one matrix's words
    unsigned long long* ws_u = (unsigned long long*)workspace;
    unsigned long long* ws_w = ws_u + per;
    hipLaunchKernelGGL(k_fill_u64, dim3(grid_for(2 * per, kThreads, 256)), dim3(kThreads), 0, s, ws_u, 2 * per);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // U planes 0..S-1 and scales [0, 2S); W planes S..2S-1 and scales [2S, 4S)
    uint8_t* codes_u = codes;
    uint8_t* codes_w = codes + (int64_t)stages * count;
    float* sc_u = scales;
    float* sc_w = scales + 2 * stages;
    const bool vec = m % 4 == 0 && ((uintptr_t)R % 16 == 0) && ((uintptr_t)codes % 4 == 0) && count % 4 == 0;
    const int grid = grid_for(vec ? count / 4 : count, kThreads, kStageBlocks);
    for (int32_t k = 0; k < stages; ++k) {
        if ((e = vec ? launch_real_stage<4>(k, grid, R, n, m, sc_u, sc_w, codes_u, codes_w, ws_u, ws_w, s)
                     : launch_real_stage<1>(k, grid, R, n, m, sc_u, sc_w, codes_u, codes_w, ws_u, ws_w, s)) !=
            hipSuccess)
            return e;
        hipLaunchKernelGGL(k_pq_finalize, dim3(2, 2), dim3(kFinThreads), 0, s, (const unsigned long long*)ws_u, k,
                           sc_u, (const unsigned long long*)ws_w, sc_w);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// PhaseQuant without a caller workspace: the exponent buckets live in this
// file-scope device array, sized for the most stages a call may ask for.
// Each GPU holds its own copy until the process ends.  Host code never uses
// the array's name as a device address: its address on the current device
// comes from hipGetSymbolAddress, once per device, and that pointer is what
// the kernels receive.  Every call clears the buckets it uses (a fill kernel,
// not a memset) before the first stage, so the array's previous contents do
// not matter; calls that overlap on one GPU share the array and race.
// ---------------------------------------------------------------------------
constexpr size_t kPqScratchBytes = (size_t)kMaxStages * kGlobalCopies * kStageWords * sizeof(unsigned long long);
static __device__ __align__(256) unsigned char scratch[kPqScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

size_t phasequant_scratch_bytes() { return kPqScratchBytes; }

hipError_t phasequant_scratch(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

int64_t packed_words(int64_t rows, int64_t m, int32_t planes, int32_t layout)
{
    if (layout == FAIRY_LAYOUT_ROW16) return (int64_t)planes * rows * (m / 16);
    return rows * ((m + 63) / 64) * planes * 4;
}

hipError_t launch_pack(const uint8_t* codes, int32_t planes, int64_t rows, int64_t m, int32_t layout,
                       uint32_t* packed, hipStream_t s)
{
    if (layout == FAIRY_LAYOUT_TILED64) {
        const int64_t total = rows * ((m + 63) / 64) * planes;
        const dim3 grid(grid_for(total, kThreads, 65536)), block(kThreads);
        if (total + (int64_t)65536 * kThreads < ((int64_t)1 << 32))
            hipLaunchKernelGGL(k_pack_tiled<uint32_t>, grid, block, 0, s, codes, planes, rows, m, packed);
        else
            hipLaunchKernelGGL(k_pack_tiled<uint64_t>, grid, block, 0, s, codes, planes, rows, m, packed);
        return hipGetLastError();
    }
    const int64_t nw = packed_words(rows, m, planes, layout);
    hipLaunchKernelGGL(k_pack_row16, dim3(grid_for(nw, kThreads, 8192)), dim3(kThreads), 0, s, codes, packed, nw);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint32_t* packed, int32_t planes, int64_t rows, int64_t m, int32_t layout,
                         uint8_t* codes, hipStream_t s)
{
    if (layout == FAIRY_LAYOUT_TILED64) {
        const int64_t total = rows * ((m + 63) / 64) * planes;
        const dim3 grid(grid_for(total, kThreads, 65536)), block(kThreads);
        if (total + (int64_t)65536 * kThreads < ((int64_t)1 << 32))
            hipLaunchKernelGGL(k_unpack_tiled<uint32_t>, grid, block, 0, s, packed, planes, rows, m, codes);
        else
            hipLaunchKernelGGL(k_unpack_tiled<uint64_t>, grid, block, 0, s, packed, planes, rows, m, codes);
        return hipGetLastError();
    }
    const int64_t nw = packed_words(rows, m, planes, layout);
    hipLaunchKernelGGL(k_unpack_row16, dim3(grid_for(nw, kThreads, 8192)), dim3(kThreads), 0, s, packed, codes, nw);
    return hipGetLastError();
}

}  // namespace fairy
