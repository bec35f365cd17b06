// fairy_attention.hip -- complex attention forward on the gfx950 matrix cores.
//
// [iFairy press article §三; Fairy2i article §2.2; iFairy talk §2.1.4]: the
// score of query q and key k is the real part of their Hermitian inner
// product, Re(sum_d q_d conj(k_d)) = q_re.k_re + q_im.k_im, i.e. the real dot
// product of the concatenated [re | im] vectors; a softmax over the keys
// gives real weights, and the values' real and imaginary parts are averaged
// with them separately.
//
// One pass, online softmax (FlashAttention style).  A block is 8 waves over
// 128 queries of one head (each staged key chunk serves 128 queries); each
// wave owns 16 queries and walks the keys in chunks (128 keys for d <= 64,
// 64 for d = 128, whose rows fill the registers and LDS), staged in LDS
// through two buffers (keys as [key][re | im], values as [re/im][key][d],
// both copied as they are in memory) and software-pipelined: the score
// MFMAs of chunk i+1 are issued among the softmax arithmetic of chunk i.
//  * Scores are computed transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16,
//    K-dim = 2d): lane l then holds query l % 16 and keys 4(l/16) + v of each
//    16-key tile, so the running maximum of a query lives in the four lanes
//    l % 16 and combines with two row swaps (v_permlane16/32_swap); each
//    lane sums its own weights and the four partial sums meet once, at the
//    end.  The running maximum is raised lazily (only when a chunk exceeds
//    it by 2^8), so the output is rarely rescaled.
//  * The weights P^T are the B operand of O^T = V^T P^T directly: in K-step s
//    of a chunk, lane group g = l/16 supplies keys 32s + 4g + 0..3 and
//    32s + 16 + 4g + 0..3, and the A fragments of V^T are read from the
//    natural-order values in the same key order by LDS transpose reads
//    (ds_read_b64_tr_b16, two per fragment).  P is split into bf16 hi + lo
//    (two MFMAs), so the weights keep ~2^-17 relative precision instead of
//    bf16's 2^-9; the scores are exact products of the bf16 inputs summed in
//    fp32.
//  * O^T accumulates in fp32: lane l holds query l % 16 and four consecutive
//    d, so the rescaling by the running maximum is per lane and the store is
//    a float4 per lane.
// Measured on MI355X (32 heads x 2048 tokens, d = 64, bf16): 0.079 ms causal,
// 0.141 ms full.
#include <type_traits>

#include "fairy_internal.h"

namespace fairy {
namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kQBlock = 16 * kWaves;  // queries per block

struct Args {
    const uint16_t *q_re, *q_im, *k_re, *k_im, *v_re, *v_im;
    float *o_re, *o_im;
    int64_t sq, sk;
    float scale;
    int32_t causal;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));

// (x0, x1) -> the packed bf16 pair nearest to them (ties to even), one
// v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t bf16x2_rne(float x0, float x1)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2_t{x0, x1}), bf16x2_t));
}

typedef short shortx4_t __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives as element
// k the 16-bit element i % 4 of the 8 bytes that lane 4k + i/4 addresses
__device__ __forceinline__ uint2 ds_read_tr16(const uint8_t* p)
{
    const shortx4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) shortx4_t*)(const_cast<uint8_t*>(p)));
    return __builtin_bit_cast(uint2, v);
}

template <int D>
struct Geometry {
    // keys per chunk: 128 halves the per-chunk costs (barrier, maximum,
    // staging) where two buffers of them fit in LDS
    static constexpr int kKeys = D <= 64 ? 128 : 64;
    static constexpr int D2 = 2 * D;              // length of the concatenated [re | im] vector
    static constexpr int kRowK = D2 * 2 + 16;     // bytes per staged key row (+ pad: conflict-free reads)
    // bytes per staged value row ([key][d], natural order): 32 more than the
    // row's 2D, so the four consecutive keys one transpose read touches
    // start 32 bytes apart modulo 128 (distinct banks)
    static constexpr int kRowV = D * 2 + 32;
    static constexpr int kBytesK = kKeys * kRowK;
    static constexpr int kBytesV = 2 * kKeys * kRowV;
};

// Cross-row combination inside a wave: lanes l, l ^ 16, l ^ 32 and l ^ 48
// (one lane of each 16-lane row) combine with two VALU row swaps.  At each
// step both lanes of a pair combine the same two values in the same order,
// so all four lanes end with the same bits.
__device__ __forceinline__ float rows_max(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows_sum(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// x - (the bf16 value in half h of pair w), to within half an ulp of x: one
// v_dot2_f32_bf16 with the multiplier pair (-1, -0) or (0, -1).  (The pair
// (-1, +0) would be emitted as the inline constant -1.0, which the
// instruction reads as the fp32 bit pattern, i.e. as (+0, -1).)
__device__ __forceinline__ float minus_half(uint32_t w, int h, float x)
{
    const uint32_t m = h ? 0xBF800000u : 0x8000BF80u;
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, m), x,
                                           false);
}

// The running maximum is raised only when a chunk's maximum exceeds it by
// more than this (log2 units), so the weights stay below 2^kLazy and the
// output rescaling is rare; any common shift cancels in the normalisation.
constexpr float kLazy = 8.0f;

// The kQBlock queries of query block qb of head h against every key they see.  All
// threads of the block call it (it synchronises on the shared chunk buffers).
//
// Software pipeline over key chunks, two LDS buffers: step i stores the keys
// of chunk i+1 and the values of chunk i into buffer (i+1) % 2, passes one
// barrier, starts the global loads of keys i+2 and values i+1, and then
// issues the score MFMAs of chunk i+1 among the softmax arithmetic of chunk
// i (its scores came from the step before), followed by the P V MFMAs of
// chunk i.  A buffer is rewritten two steps after it was read, with a
// barrier between.
template <int D>
__device__ __forceinline__ void attend_tile(const Args& a, int64_t h, int64_t qb, uint8_t* s_k, uint8_t* s_v)
{
    constexpr int D2 = Geometry<D>::D2;
    constexpr int KS = D2 / 32;               // K-steps of the score product
    constexpr int DT = D / 16;                // 16-wide d tiles of the output
    constexpr int kRowK = Geometry<D>::kRowK;
    constexpr int kRowV = Geometry<D>::kRowV;
    constexpr int kBytesK = Geometry<D>::kBytesK;
    constexpr int kBytesV = Geometry<D>::kBytesV;
    constexpr int kKeys = Geometry<D>::kKeys;
    constexpr int KT = kKeys / 16, KSP = kKeys / 32;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int64_t qi = qb * kQBlock + wave * 16 + c16;  // this lane's query
    const bool q_ok = qi < a.sq;
    const int64_t diag = a.sk - a.sq;  // causal: query i sees keys j <= i + diag

    // B operand of S^T: query qi, dims 32t + 8g .. +8 of [re | im].  A
    // negative scale is moved onto the queries (negating bf16 is exact), so
    // the scores are scaled by |scale| and their maximum is the scaled maximum.
    const uint32_t qflip = (__float_as_uint(a.scale) >> 31) ? 0x80008000u : 0u;
    bf16x8_t qf[KS];
#pragma unroll
    for (int t = 0; t < KS; ++t) {
        const int dim0 = 32 * t + 8 * g;
        const uint16_t* src = (dim0 < D ? a.q_re : a.q_im) + (h * a.sq + (q_ok ? qi : 0)) * D + (dim0 % D);
        uint4 v = q_ok ? *reinterpret_cast<const uint4*>(src) : make_uint4(0, 0, 0, 0);
        v.x ^= qflip;
        v.y ^= qflip;
        v.z ^= qflip;
        v.w ^= qflip;
        qf[t] = __builtin_bit_cast(bf16x8_t, v);
    }

    floatx4_t o[2][DT];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int t = 0; t < DT; ++t) o[c][t] = floatx4_t{0, 0, 0, 0};
    // scores are kept in log2 units (|scale| * log2 e), so the softmax uses exp2
    const float scale2 = fabsf(a.scale) * 1.4426950408889634f;
    // m_run is the query's (lazy) running maximum; l_run the sum of this
    // lane's own weights, added across the query's four lanes at the end
    float m_run = -INFINITY, l_run = 0.0f;

    int64_t kend = a.sk;   // keys the block's queries see: [0, kend)
    int64_t vis = a.sk;    // keys every query of the block sees
    if (a.causal) {
        const int64_t first_q = qb * kQBlock, last_q = first_q + kQBlock - 1;
        if (last_q + diag + 1 < kend) kend = last_q + diag + 1;
        if (first_q + diag + 1 < vis) vis = first_q + diag + 1;
    }
    const int64_t nch = (kend + kKeys - 1) / kKeys;  // >= 1: key 0 is visible to every query
    const int64_t nfull = vis / kKeys;               // chunks that need no masking

    // Per chunk a thread moves KP 16-byte pieces of keys and VP of values
    // (8 d of one key) through registers.
    constexpr int KP = kKeys * (D2 / 8) / kThreads;
    constexpr int VN = 2 * kKeys * (D / 8);  // value pieces per chunk
    constexpr int VP = VN / kThreads;
    static_assert(KP * kThreads == kKeys * (D2 / 8) && VP * kThreads == VN, "staging split");
    uint4 kreg[KP], vreg[VP];
    // guard = false: the chunk lies inside the keys (every chunk but a
    // ragged last one), so its loads need no bounds checks
    auto load_k_g = [&](int64_t c0, bool guard) {
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            const int p = i * kThreads + threadIdx.x;
            const int key = p / (D2 / 8), dim0 = 8 * (p % (D2 / 8));
            const int64_t kj = c0 + key;
            const uint4* src = reinterpret_cast<const uint4*>((dim0 < D ? a.k_re : a.k_im) + (h * a.sk + kj) * D +
                                                              (dim0 % D));
            kreg[i] = (!guard || kj < a.sk) ? *src : make_uint4(0, 0, 0, 0);
        }
    };
    auto load_v_g = [&](int64_t c0, bool guard) {
#pragma unroll
        for (int i = 0; i < VP; ++i) {
            const int p = i * kThreads + threadIdx.x;
            const int comp = p / (kKeys * (D / 8));
            const int rem = p - comp * kKeys * (D / 8);
            const int key = rem / (D / 8), d0 = 8 * (rem % (D / 8));
            const int64_t kj = c0 + key;
            const uint4* src = reinterpret_cast<const uint4*>((comp ? a.v_im : a.v_re) + (h * a.sk + kj) * D + d0);
            vreg[i] = (!guard || kj < a.sk) ? *src : make_uint4(0, 0, 0, 0);
        }
    };
    auto load_k = [&](int64_t c0) {
        if (c0 + kKeys <= a.sk)
            load_k_g(c0, false);
        else
            load_k_g(c0, true);
    };
    auto load_v = [&](int64_t c0) {
        if (c0 + kKeys <= a.sk)
            load_v_g(c0, false);
        else
            load_v_g(c0, true);
    };
    auto store_k = [&](int buf) {
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            const int p = i * kThreads + threadIdx.x;
            const int key = p / (D2 / 8), dim0 = 8 * (p % (D2 / 8));
            *reinterpret_cast<uint4*>(s_k + buf * kBytesK + key * kRowK + dim0 * 2) = kreg[i];
        }
    };
    auto store_v = [&](int buf) {
#pragma unroll
        for (int i = 0; i < VP; ++i) {
            const int p = i * kThreads + threadIdx.x;
            const int comp = p / (kKeys * (D / 8));
            const int rem = p - comp * kKeys * (D / 8);
            const int key = rem / (D / 8), d0 = 8 * (rem % (D / 8));
            *reinterpret_cast<uint4*>(s_v + buf * kBytesV + (comp * kKeys + key) * kRowV + d0 * 2) = vreg[i];
        }
    };
    // S^T tiles of the chunk in buffer buf: st[kt][v] = unscaled score of
    // (key 16kt + 4g + v of the chunk, query qi)
    auto scores = [&](int buf, floatx4_t(&st)[KT]) {
        const uint8_t* kb = s_k + buf * kBytesK;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) st[kt] = floatx4_t{0, 0, 0, 0};
        // K-step outer, key tile inner: consecutive MFMAs use different
        // accumulators (a dependent MFMA waits for its predecessor's result)
#pragma unroll
        for (int t = 0; t < KS; ++t)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                const bf16x8_t kf =
                    *reinterpret_cast<const bf16x8_t*>(kb + (kt * 16 + c16) * kRowK + (32 * t + 8 * g) * 2);
                st[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[t], st[kt], 0, 0, 0);
            }
    };

    // Scores of the chunk whose softmax comes next: unscaled (masked =
    // false) or scaled with the invisible keys at -inf (masked = true).
    floatx4_t st[KT];
    bool masked = false;
    // Maximum of the chunk in st, after masking it when the chunk runs past
    // the keys or (causal) past the diagonal of the wave's first query.
    auto chunk_max = [&](int64_t k0, auto edge_c) -> float {
        float mx = -INFINITY;
        masked = false;
        if constexpr (decltype(edge_c)::value) {
            const int64_t q_first = qb * kQBlock + wave * 16;
            masked = k0 + kKeys > a.sk || (a.causal && k0 + kKeys - 1 > q_first + diag);
        }
        if (masked) {
            // keys k0 + r with r < lim are visible to this lane's query
            int64_t lim64 = a.sk - k0;
            if (a.causal && qi + diag + 1 - k0 < lim64) lim64 = qi + diag + 1 - k0;
            const int lim = (int)(lim64 < 0 ? 0 : lim64 > kKeys ? kKeys : lim64);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    st[kt][v] = (16 * kt + 4 * g + v < lim) ? scale2 * st[kt][v] : -INFINITY;
                    mx = fmaxf(mx, st[kt][v]);
                }
        } else {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int v = 0; v < 4; ++v) mx = fmaxf(mx, st[kt][v]);
            mx *= scale2;  // scale2 >= 0: the maximum of the scaled scores
        }
        return rows_max(mx);
    };

    // One pipeline step (see above).  EDGE: chunk i or i+1 may need masking;
    // NEXT: chunk i+1 exists.  The running maximum for chunk i was settled
    // at the end of the step before, so the softmax arithmetic here has no
    // branch between it and the MFMAs it runs among.
    auto step = [&](int64_t i, auto edge_c, auto next_c) {
        constexpr bool EDGE = decltype(edge_c)::value, NEXT = decltype(next_c)::value;
        const int buf = (int)((i + 1) & 1);
        const int64_t k0 = i * kKeys;
        if (NEXT) store_k(buf);
        store_v(buf);
        __syncthreads();
        if (i + 2 < nch) load_k(k0 + 2 * kKeys);
        if (NEXT) load_v(k0 + kKeys);

        floatx4_t sn[KT];
        if constexpr (NEXT) scores(buf, sn);

        // weights of chunk i against m_run: at most 2^kLazy
        float p[KT][4], ls = 0.0f;
        if (EDGE && masked) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    p[kt][v] = __builtin_amdgcn_exp2f(st[kt][v] - m_run);  // masked: 2^-inf = 0
                    ls += p[kt][v];
                }
        } else {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    p[kt][v] = __builtin_amdgcn_exp2f(fmaf(st[kt][v], scale2, -m_run));
                    ls += p[kt][v];
                }
        }
        l_run += ls;
        // P^T as bf16 hi + lo pairs, the B operands of the two K-steps
        bf16x8_t ph[KSP], pl[KSP];
#pragma unroll
        for (int ks = 0; ks < KSP; ++ks) {
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x0 = (e < 2) ? p[2 * ks][2 * e] : p[2 * ks + 1][2 * e - 4];
                const float x1 = (e < 2) ? p[2 * ks][2 * e + 1] : p[2 * ks + 1][2 * e - 3];
                hi[e] = bf16x2_rne(x0, x1);
                lo[e] = bf16x2_rne(minus_half(hi[e], 0, x0), minus_half(hi[e], 1, x1));
            }
            ph[ks] = __builtin_bit_cast(bf16x8_t, make_uint4(hi[0], hi[1], hi[2], hi[3]));
            pl[ks] = __builtin_bit_cast(bf16x8_t, make_uint4(lo[0], lo[1], lo[2], lo[3]));
        }

        // O^T += V^T P^T, K-steps of 32 keys
        const uint8_t* vbuf = s_v + buf * kBytesV;
#pragma unroll
        for (int ks = 0; ks < KSP; ++ks) {
            // A operand of O^T: lane l needs V[key][16t + l % 16] for keys
            // 32ks + 4g + 0..3 and 32ks + 16 + 4g + 0..3.  A transpose read
            // gives lane i of a 16-lane group element i % 4 of the 8 bytes
            // lane 4k + i/4 addresses, as its element k; so lane j of the
            // group addresses key kb + j/4, d 16t + 4(j % 4).
            const int key_a = 32 * ks + 4 * g + (c16 >> 2), key_b = key_a + 16;
            const int dq = 4 * (c16 & 3);
            auto v_frag = [&](int c, int t) {
                const uint8_t* base = vbuf + (size_t)(c * kKeys) * kRowV + (16 * t + dq) * 2;
                const uint2 va = ds_read_tr16(base + key_a * kRowV);
                const uint2 vb = ds_read_tr16(base + key_b * kRowV);
                return __builtin_bit_cast(bf16x8_t, make_uint4(va.x, va.y, vb.x, vb.y));
            };
            if constexpr (D <= 64) {
                // all hi products, then all lo products: 2 DT independent
                // accumulators between an MFMA and the one that depends on it
                bf16x8_t vf[2][DT];
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int t = 0; t < DT; ++t) vf[c][t] = v_frag(c, t);
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int t = 0; t < DT; ++t)
                        o[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[c][t], ph[ks], o[c][t], 0, 0, 0);
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int t = 0; t < DT; ++t)
                        o[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[c][t], pl[ks], o[c][t], 0, 0, 0);
            } else {
                // d = 128: one fragment at a time (the registers are full)
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int t = 0; t < DT; ++t) {
                        const bf16x8_t vf = v_frag(c, t);
                        o[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, ph[ks], o[c][t], 0, 0, 0);
                        o[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pl[ks], o[c][t], 0, 0, 0);
                    }
            }
        }

        if constexpr (NEXT) {
            // settle the running maximum for chunk i+1: it is raised only
            // when some query of the wave exceeds it by more than kLazy
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) st[kt] = sn[kt];
            const float mx = chunk_max(k0 + kKeys, edge_c);
            if (__ballot(mx > m_run + kLazy) != 0) {
                const float m_new = fmaxf(m_run, mx);
                const float corr = __builtin_amdgcn_exp2f(m_run - m_new);  // 1 if unchanged
                m_run = m_new;
                l_run *= corr;
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int t = 0; t < DT; ++t) o[c][t] *= corr;
            }
        }
    };

    // prologue: keys of chunk 0 into buffer 0, their scores and maximum
    // (finite: key 0 is visible to every query)
    using F = std::integral_constant<bool, false>;
    using T = std::integral_constant<bool, true>;
    __syncthreads();  // a previous tile of this block is done with both buffers
    load_k(0);
    store_k(0);
    if (nch > 1) load_k(kKeys);
    load_v(0);
    __syncthreads();
    scores(0, st);
    m_run = chunk_max(0, T{});

    // steps whose chunks i and i+1 both need no masking, then the rest
    const int64_t nmain = (nfull < nch ? nfull : nch) - 1;
    int64_t i = 0;
    for (; i < nmain; ++i) step(i, F{}, T{});
    for (; i < nch - 1; ++i) step(i, T{}, T{});
    step(nch - 1, T{}, F{});

    const float l_tot = rows_sum(l_run);
    if (q_ok) {
        const float inv = 1.0f / l_tot;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            float* dst = (c ? a.o_im : a.o_re) + (h * a.sq + qi) * D + 4 * g;
#pragma unroll
            for (int t = 0; t < DT; ++t)
                *reinterpret_cast<float4*>(dst + 16 * t) =
                    make_float4(o[c][t][0] * inv, o[c][t][1] * inv, o[c][t][2] * inv, o[c][t][3] * inv);
        }
    }
}

// Non-causal: block x takes query block x.  Causal: query block i walks
// about i+1 key chunks, so block x takes the pair (n-1-x, x) and every block
// does the same amount of work.
template <int D>
__global__ __launch_bounds__(kThreads) void k_cattention(Args a)
{
    __shared__ __align__(16) uint8_t s_k[2 * Geometry<D>::kBytesK];
    __shared__ __align__(16) uint8_t s_v[2 * Geometry<D>::kBytesV];
    // Blocks are dealt to the 8 XCDs round-robin by linear index.  Renumber
    // them so each XCD takes a contiguous run of (head, query block) pairs:
    // the few heads an XCD works on at a time keep their keys and values in
    // its own L2.
    const uint64_t nx = gridDim.x, total = nx * gridDim.y;
    uint64_t id = blockIdx.y * nx + blockIdx.x;
    if (total % 8 == 0) id = (id % 8) * (total / 8) + id / 8;
    const int64_t h = (int64_t)(id / nx), x = (int64_t)(id % nx);
    if (!a.causal) {
        attend_tile<D>(a, h, x, s_k, s_v);
        return;
    }
    const int64_t nqb = (a.sq + kQBlock - 1) / kQBlock;
    const int64_t heavy = nqb - 1 - x, light = x;
    attend_tile<D>(a, h, heavy, s_k, s_v);
    if (light < heavy) attend_tile<D>(a, h, light, s_k, s_v);
}

template <int D>
hipError_t launch(const Args& a, int32_t heads, hipStream_t s)
{
    const int64_t nqb = (a.sq + kQBlock - 1) / kQBlock;
    const dim3 grid((unsigned)(a.causal ? (nqb + 1) / 2 : nqb), (unsigned)heads);
    hipLaunchKernelGGL((k_cattention<D>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace attn

hipError_t launch_cattention(const void* q_re, const void* q_im, const void* k_re, const void* k_im,
                             const void* v_re, const void* v_im, int32_t heads, int64_t sq, int64_t sk, int32_t d,
                             float scale, int32_t causal, float* o_re, float* o_im, hipStream_t s)
{
    attn::Args a;
    a.q_re = static_cast<const uint16_t*>(q_re);
    a.q_im = static_cast<const uint16_t*>(q_im);
    a.k_re = static_cast<const uint16_t*>(k_re);
    a.k_im = static_cast<const uint16_t*>(k_im);
    a.v_re = static_cast<const uint16_t*>(v_re);
    a.v_im = static_cast<const uint16_t*>(v_im);
    a.o_re = o_re;
    a.o_im = o_im;
    a.sq = sq;
    a.sk = sk;
    a.scale = scale;
    a.causal = causal;
    switch (d) {
    case 32: return attn::launch<32>(a, heads, s);
    case 64: return attn::launch<64>(a, heads, s);
    default: return attn::launch<128>(a, heads, s);
    }
}

}  // namespace fairy
