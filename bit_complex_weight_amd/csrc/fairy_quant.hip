// fairy_quant.hip -- offline steps of the layer on gfx950:
//   widely-linear conversion   [Fairy2i article §2.1]
//   PhaseQuant codes, exact per-axis scales, recursive residual stages
//                              [Fairy2i article §3.1, §3.2, §4.1]
//   packing 16 codes per uint32
// All kernels are streaming (HBM-bound); they are launched on the caller's
// stream and allocate nothing.
#include "fairy_internal.h"

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
__device__ __forceinline__ uint32_t phase_code(float a, float b)
{
    const float A = fabsf(a), B = fabsf(b);
    if (A > B) return a > 0.0f ? 0u : 2u;
    if (B > A) return b > 0.0f ? 1u : 3u;
    if (A == 0.0f) return 0u;
    return a > 0.0f ? (b > 0.0f ? 1u : 0u) : (b > 0.0f ? 2u : 3u);
}

// R <- R - (s_re Re(i^c) + i s_im Im(i^c)), one fp32 operation on the code's axis.
__device__ __forceinline__ void residual_step(float& a, float& b, uint32_t c, float s_re, float s_im)
{
    if (c == 0u) a = a - s_re;
    else if (c == 2u) a = a + s_re;
    else if (c == 1u) b = b - s_im;
    else b = b + s_im;
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

// Stage k: recompute R_k from W with the scales of stages < k (already on
// the device), write code_k, and add |R_k| on the code's axis into the
// stage's exponent buckets (block-local LDS buckets, flushed once per block).
// Stage k: recompute R_k from W with the scales of stages < k (already on
// the device), write code_k, and add |R_k| on the code's axis into the
// stage's exponent buckets.  V = 4: each thread takes 4 consecutive elements
// (float4 loads, one 32-bit store of 4 codes); V = 1 for unaligned arrays.
// A block accumulates into kCopies interleaved LDS copies of the buckets,
// then adds its nonzero buckets into global copy blockIdx % kGlobalCopies of
// the stage's workspace (integer atomics: exact and order-independent; the
// copies keep the blocks of a launch from contending on ~40 hot addresses).
constexpr int kCopies = 2;
constexpr int kGlobalCopies = 16;
constexpr int kStageBlocks = 1024;

template <int V>
__global__ __launch_bounds__(kThreads) void k_pq_stage(const float* __restrict__ w_re,
                                                       const float* __restrict__ w_im, int64_t count,
                                                       int32_t k, const float* __restrict__ scales,
                                                       uint8_t* __restrict__ codes,
                                                       unsigned long long* __restrict__ ws)
{
    typedef typename std::conditional<V == 4, float4, float>::type vec_t;
    typedef typename std::conditional<V == 4, uint32_t, uint8_t>::type code_t;
    __shared__ unsigned long long s_buck[kBuckets * kCopies];
    __shared__ unsigned long long s_cnt[2];
    for (int t = threadIdx.x; t < kBuckets * kCopies; t += blockDim.x) s_buck[t] = 0ull;
    if (threadIdx.x < 2) s_cnt[threadIdx.x] = 0ull;
    __syncthreads();

    float sre[8], sim[8];
    for (int j = 0; j < k; ++j) {
        sre[j] = scales[2 * j];
        sim[j] = scales[2 * j + 1];
    }
    const int copy = threadIdx.x % kCopies;
    const int64_t nv = count / V;
    const vec_t* vr = reinterpret_cast<const vec_t*>(w_re);
    const vec_t* vi = reinterpret_cast<const vec_t*>(w_im);
    code_t* cout = reinterpret_cast<code_t*>(codes + (int64_t)k * count);
    uint32_t n_im = 0, n_all = 0;
    for (int64_t iv = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; iv < nv;
         iv += (int64_t)gridDim.x * blockDim.x) {
        const vec_t ra = vr[iv], rb = vi[iv];
        float av[V], bv[V];
        if constexpr (V == 4) {
            av[0] = ra.x; av[1] = ra.y; av[2] = ra.z; av[3] = ra.w;
            bv[0] = rb.x; bv[1] = rb.y; bv[2] = rb.z; bv[3] = rb.w;
        } else {
            av[0] = ra;
            bv[0] = rb;
        }
        uint32_t cpack = 0;
#pragma unroll
        for (int e = 0; e < V; ++e) {
            float a = av[e], b = bv[e];
            for (int j = 0; j < k; ++j) residual_step(a, b, phase_code(a, b), sre[j], sim[j]);
            const uint32_t c = phase_code(a, b);
            cpack |= c << (8 * e);
            const uint32_t axis = c & 1u;
            n_im += axis;
            const uint32_t bits = __float_as_uint(axis ? fabsf(b) : fabsf(a));
            const uint32_t ex = bits >> 23, man = bits & 0x7FFFFFu;
            const uint32_t sig = ex ? (man | 0x800000u) : man;
            if (sig) atomicAdd(&s_buck[(axis * 256u + (ex ? ex : 1u)) * kCopies + copy], (unsigned long long)sig);
        }
        n_all += V;
        cout[iv] = (code_t)cpack;
    }
    if (n_all - n_im) atomicAdd(&s_cnt[0], (unsigned long long)(n_all - n_im));
    if (n_im) atomicAdd(&s_cnt[1], (unsigned long long)n_im);
    __syncthreads();
    unsigned long long* g = ws + ((int64_t)k * kGlobalCopies + blockIdx.x % kGlobalCopies) * kStageWords;
    for (int t = threadIdx.x; t < kBuckets; t += blockDim.x) {
        unsigned long long v = 0ull;
#pragma unroll
        for (int c = 0; c < kCopies; ++c) v += s_buck[t * kCopies + c];
        if (v) atomicAdd(&g[t], v);
    }
    if (threadIdx.x < 2 && s_cnt[threadIdx.x]) atomicAdd(&g[kBuckets + threadIdx.x], s_cnt[threadIdx.x]);
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

constexpr int kFinThreads = 256;

__global__ __launch_bounds__(kFinThreads) void k_pq_finalize(const unsigned long long* __restrict__ ws, int32_t k,
                                                              float* __restrict__ scales)
{
    // 128 threads per axis; thread j splits buckets 2j and 2j+1 into 32-bit
    // limb pieces, then a tree in LDS adds each limb over the 128 threads
    // (fixed order, integer: exact)
    __shared__ unsigned long long s_red[kFinThreads][kLimbs];
    __shared__ unsigned long long s_part[2][kLimbs];
    __shared__ unsigned long long s_b[kStageWords];
    const int axis = threadIdx.x >> 7;
    const int j = threadIdx.x & 127;
    // buckets and counts: the sum of the stage's global copies
    const unsigned long long* g0 = ws + (int64_t)k * kGlobalCopies * kStageWords;
    for (int t = threadIdx.x; t < kStageWords; t += blockDim.x) {
        unsigned long long v = 0ull;
        for (int c = 0; c < kGlobalCopies; ++c) v += g0[(int64_t)c * kStageWords + t];
        s_b[t] = v;
    }
    __syncthreads();
    const unsigned long long* g = s_b;
    unsigned long long part[kLimbs];
#pragma unroll
    for (int q = 0; q < kLimbs; ++q) part[q] = 0ull;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int eb = 2 * j + h;
        const unsigned long long v = (eb >= 1) ? g[256 * axis + eb] : 0ull;
        if (!v) continue;
        // v * 2^(eb-1), seen limb by limb (limb q holds bits 32q .. 32q+31)
#pragma unroll
        for (int q = 0; q < kLimbs; ++q) {
            const int sh = eb - 1 - 32 * q;
            uint32_t piece;
            if (sh >= 32 || sh <= -64) piece = 0u;
            else if (sh >= 0) piece = (uint32_t)(v << sh);
            else piece = (uint32_t)(v >> (-sh));
            part[q] += piece;
        }
    }
#pragma unroll
    for (int q = 0; q < kLimbs; ++q) s_red[threadIdx.x][q] = part[q];
    __syncthreads();
    for (int w = 64; w >= 1; w >>= 1) {
        if (j < w) {
#pragma unroll
            for (int q = 0; q < kLimbs; ++q) s_red[threadIdx.x][q] += s_red[threadIdx.x + w][q];
        }
        __syncthreads();
    }
    if (j == 0) {
#pragma unroll
        for (int q = 0; q < kLimbs; ++q) s_part[axis][q] = s_red[threadIdx.x][q];
    }
    __syncthreads();
    const int L = j;
    if (L != 0) return;
    const unsigned long long cnt = g[kBuckets + axis];
    float result = 0.0f;
    if (cnt != 0ull) {
        uint32_t N[kLimbs];
        unsigned long long carry = 0ull;
#pragma unroll
        for (int q = 0; q < kLimbs; ++q) {
            const unsigned long long t = s_part[axis][q] + carry;
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
    scales[2 * k + axis] = result;
}

__global__ __launch_bounds__(kThreads) void k_pq_resid(const float* __restrict__ w_re,
                                                       const float* __restrict__ w_im, int64_t count,
                                                       int32_t stages, const float* __restrict__ scales,
                                                       float* __restrict__ r_re, float* __restrict__ r_im)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x) {
        float a = w_re[i], b = w_im[i];
        for (int j = 0; j < stages; ++j) residual_step(a, b, phase_code(a, b), scales[2 * j], scales[2 * j + 1]);
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

__global__ __launch_bounds__(kThreads) void k_pack(const uint8_t* __restrict__ codes, int32_t planes,
                                                   int64_t rows, int64_t m, int32_t layout,
                                                   uint32_t* __restrict__ out, int64_t nwords)
{
    const int64_t G = (m + 63) / 64;
    for (int64_t wi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; wi < nwords;
         wi += (int64_t)gridDim.x * blockDim.x) {
        int64_t p, r, c0;
        if (layout == FAIRY_LAYOUT_ROW16) {
            const int64_t wpr = m / 16;
            const int64_t pr = wi / wpr;
            c0 = (wi - pr * wpr) * 16;
            p = pr / rows;
            r = pr - p * rows;
        } else {
            const int64_t u = wi & 3;
            const int64_t q = wi >> 2;
            p = q % planes;
            const int64_t rg = q / planes;
            const int64_t g = rg % G;
            r = rg / G;
            c0 = 64 * g + 16 * u;
        }
        uint32_t word = 0u;
        if (c0 < m) {
            uint8_t c[16];
            load16(codes + (p * rows + r) * m + c0, c);
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const uint32_t bitpos = (layout == FAIRY_LAYOUT_ROW16) ? (uint32_t)(2 * t) : tiled_bit(t);
                word |= ((uint32_t)c[t] & 3u) << bitpos;
            }
        }
        out[wi] = word;
    }
}

__global__ __launch_bounds__(kThreads) void k_unpack(const uint32_t* __restrict__ in, int32_t planes,
                                                     int64_t rows, int64_t m, int32_t layout,
                                                     uint8_t* __restrict__ codes, int64_t nwords)
{
    const int64_t G = (m + 63) / 64;
    for (int64_t wi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; wi < nwords;
         wi += (int64_t)gridDim.x * blockDim.x) {
        int64_t p, r, c0;
        if (layout == FAIRY_LAYOUT_ROW16) {
            const int64_t wpr = m / 16;
            const int64_t pr = wi / wpr;
            c0 = (wi - pr * wpr) * 16;
            p = pr / rows;
            r = pr - p * rows;
        } else {
            const int64_t u = wi & 3;
            const int64_t q = wi >> 2;
            p = q % planes;
            const int64_t rg = q / planes;
            const int64_t g = rg % G;
            r = rg / G;
            c0 = 64 * g + 16 * u;
        }
        if (c0 >= m) continue;
        const uint32_t word = in[wi];
        uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const uint32_t bitpos = (layout == FAIRY_LAYOUT_ROW16) ? (uint32_t)(2 * t) : tiled_bit(t);
            o[t >> 2] |= ((word >> bitpos) & 3u) << (8 * (t & 3));
        }
        *reinterpret_cast<uint4*>(codes + (p * rows + r) * m + c0) = make_uint4(o[0], o[1], o[2], o[3]);
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
        if (vec)
            hipLaunchKernelGGL(k_pq_stage<4>, dim3(grid), dim3(kThreads), 0, s, w_re, w_im, count, k,
                               (const float*)scales, codes, ws);
        else
            hipLaunchKernelGGL(k_pq_stage<1>, dim3(grid), dim3(kThreads), 0, s, w_re, w_im, count, k,
                               (const float*)scales, codes, ws);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(k_pq_finalize, dim3(1), dim3(kFinThreads), 0, s, (const unsigned long long*)ws, k, scales);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (resid_re || resid_im) {
        hipLaunchKernelGGL(k_pq_resid, dim3(grid), dim3(kThreads), 0, s, w_re, w_im, count, stages,
                           (const float*)scales, resid_re, resid_im);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
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
    const int64_t nw = packed_words(rows, m, planes, layout);
    hipLaunchKernelGGL(k_pack, dim3(grid_for(nw, kThreads, 8192)), dim3(kThreads), 0, s, codes, planes, rows,
                       m, layout, packed, nw);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint32_t* packed, int32_t planes, int64_t rows, int64_t m, int32_t layout,
                         uint8_t* codes, hipStream_t s)
{
    const int64_t nw = packed_words(rows, m, planes, layout);
    hipLaunchKernelGGL(k_unpack, dim3(grid_for(nw, kThreads, 8192)), dim3(kThreads), 0, s, packed, planes,
                       rows, m, layout, codes, nw);
    return hipGetLastError();
}

}  // namespace fairy
