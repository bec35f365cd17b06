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
// wave owns 16 queries and walks the keys in
// chunks of 64 staged in LDS (keys as [key][re | im], values as
// [re/im][key][d], both copied as they are in memory).
//  * Scores are computed transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16,
//    K-dim = 2d): lane l then holds query l % 16 and keys 4(l/16) + v of each
//    16-key tile, so the running maximum and sum of a query live in the four
//    lanes l % 16 and combine with two xor-shuffles.
//  * The weights P^T are the B operand of O^T = V^T P^T directly: in K-step s
//    of a chunk, lane group g = l/16 supplies keys 32s + 4g + 0..3 and
//    32s + 16 + 4g + 0..3, and the A fragments of V^T are read from the
//    natural-order values in the same key order by LDS transpose reads
//    (ds_read_b64_tr_b16, two per fragment).  P is split into bf16 hi + lo (two MFMAs), so the
//    weights keep ~2^-17 relative precision instead of bf16's 2^-9; the
//    scores are exact products of the bf16 inputs summed in fp32.
//  * O^T accumulates in fp32: lane l holds query l % 16 and four consecutive
//    d, so the rescaling by the running maximum is per lane and the store is
//    a float4 per lane.
#include "fairy_internal.h"

namespace fairy {
namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kQBlock = 16 * kWaves;  // queries per block
constexpr int kKeys = 64;             // keys per chunk

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
    static constexpr int D2 = 2 * D;              // length of the concatenated [re | im] vector
    static constexpr int kRowK = D2 * 2 + 16;     // bytes per staged key row (+ pad: conflict-free reads)
    // bytes per staged value row ([key][d], natural order): 32 more than the
    // row's 2D, so the four consecutive keys one transpose read touches
    // start 32 bytes apart modulo 128 (distinct banks)
    static constexpr int kRowV = D * 2 + 32;
    static constexpr int kBytesK = kKeys * kRowK;
    static constexpr int kBytesV = 2 * kKeys * kRowV;
};

// The 64 queries of query block qb against every key they see.  All threads
// of the block call it (it synchronises on the shared chunk buffers).
template <int D>
__device__ __forceinline__ void attend_tile(const Args& a, int64_t qb, uint8_t* s_k, uint8_t* s_v)
{
    constexpr int D2 = Geometry<D>::D2;
    constexpr int KS = D2 / 32;               // K-steps of the score product
    constexpr int DT = D / 16;                // 16-wide d tiles of the output
    constexpr int kRowK = Geometry<D>::kRowK;
    constexpr int kRowV = Geometry<D>::kRowV;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int64_t h = blockIdx.y;
    const int64_t qi = qb * kQBlock + wave * 16 + c16;  // this lane's query
    const bool q_ok = qi < a.sq;
    const int64_t diag = a.sk - a.sq;  // causal: query i sees keys j <= i + diag

    // B operand of S^T: query qi, dims 32t + 8g .. +8 of [re | im]
    bf16x8_t qf[KS];
#pragma unroll
    for (int t = 0; t < KS; ++t) {
        const int dim0 = 32 * t + 8 * g;
        const uint16_t* src = (dim0 < D ? a.q_re : a.q_im) + (h * a.sq + (q_ok ? qi : 0)) * D + (dim0 % D);
        const uint4 v = q_ok ? *reinterpret_cast<const uint4*>(src) : make_uint4(0, 0, 0, 0);
        qf[t] = __builtin_bit_cast(bf16x8_t, v);
    }

    floatx4_t o[2][DT];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int t = 0; t < DT; ++t) o[c][t] = floatx4_t{0, 0, 0, 0};
    // scores are kept in log2 units (scale * log2 e), so the softmax uses exp2
    const float scale2 = a.scale * 1.4426950408889634f;
    float m_run = -INFINITY, l_run = 0.0f;

    int64_t kend = a.sk;
    if (a.causal) {
        const int64_t last_q = qb * kQBlock + kQBlock - 1;
        if (last_q + diag + 1 < kend) kend = last_q + diag + 1;
    }
    // Per chunk a thread moves KP 16-byte pieces of keys and VP of values
    // (8 d of one key); the next chunk's pieces are loaded into registers
    // while the current chunk is multiplied.
    constexpr int KP = kKeys * (D2 / 8) / kThreads;
    constexpr int VN = 2 * kKeys * (D / 8);  // value pieces per chunk
    constexpr int VP = VN / kThreads;
    static_assert(KP * kThreads == kKeys * (D2 / 8) && VP * kThreads == VN, "staging split");
    uint4 kreg[KP], vreg[VP];
    // guard = false: the chunk lies inside the keys (every chunk but a
    // ragged last one), so its loads need no bounds checks
    auto load_chunk_g = [&](int64_t c0, bool guard) {
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            const int p = i * kThreads + threadIdx.x;
            const int key = p / (D2 / 8), dim0 = 8 * (p % (D2 / 8));
            const int64_t kj = c0 + key;
            const uint4* src = reinterpret_cast<const uint4*>((dim0 < D ? a.k_re : a.k_im) + (h * a.sk + kj) * D +
                                                              (dim0 % D));
            kreg[i] = (!guard || kj < a.sk) ? *src : make_uint4(0, 0, 0, 0);
        }
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
    auto load_chunk = [&](int64_t c0) {
        if (c0 + kKeys <= a.sk)
            load_chunk_g(c0, false);
        else
            load_chunk_g(c0, true);
    };
    auto store_chunk = [&]() {
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            const int p = i * kThreads + threadIdx.x;
            const int key = p / (D2 / 8), dim0 = 8 * (p % (D2 / 8));
            *reinterpret_cast<uint4*>(s_k + key * kRowK + dim0 * 2) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < VP; ++i) {
            const int p = i * kThreads + threadIdx.x;
            const int comp = p / (kKeys * (D / 8));
            const int rem = p - comp * kKeys * (D / 8);
            const int key = rem / (D / 8), d0 = 8 * (rem % (D / 8));
            *reinterpret_cast<uint4*>(s_v + (comp * kKeys + key) * kRowV + d0 * 2) = vreg[i];
        }
    };
    if (kend > 0) load_chunk(0);
    for (int64_t k0 = 0; k0 < kend; k0 += kKeys) {
        __syncthreads();  // every wave is done with the previous chunk
        store_chunk();
        __syncthreads();
        if (k0 + kKeys < kend) load_chunk(k0 + kKeys);

        // S^T tiles: st[kt][v] = score(key k0 + 16kt + 4g + v, query qi)
        floatx4_t st[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            st[kt] = floatx4_t{0, 0, 0, 0};
#pragma unroll
            for (int t = 0; t < KS; ++t) {
                const bf16x8_t kf =
                    *reinterpret_cast<const bf16x8_t*>(s_k + (kt * 16 + c16) * kRowK + (32 * t + 8 * g) * 2);
                st[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[t], st[kt], 0, 0, 0);
            }
        }
        // Masking is needed only where the chunk runs past the keys or,
        // causal, past the diagonal of the wave's first query (wave-uniform).
        const int64_t q_first = qb * kQBlock + wave * 16;
        const bool edge = k0 + kKeys > a.sk || (a.causal && k0 + kKeys - 1 > q_first + diag);
        float s[4][4];
        float mx = -INFINITY;
        if (edge) {
            // keys k0 + r with r < lim are visible to this lane's query
            int64_t lim64 = a.sk - k0;
            if (a.causal && qi + diag + 1 - k0 < lim64) lim64 = qi + diag + 1 - k0;
            const int lim = (int)(lim64 < 0 ? 0 : lim64 > kKeys ? kKeys : lim64);
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    s[kt][v] = (16 * kt + 4 * g + v < lim) ? scale2 * st[kt][v] : -INFINITY;
                    mx = fmaxf(mx, s[kt][v]);
                }
        } else {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    s[kt][v] = scale2 * st[kt][v];
                    mx = fmaxf(mx, s[kt][v]);
                }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // key k0 (<= qi + diag) is unmasked in the first chunk, so m_new is finite
        const float m_new = fmaxf(m_run, mx);
        const float corr = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first chunk
        float p[4][4], ls = 0.0f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                p[kt][v] = __builtin_amdgcn_exp2f(s[kt][v] - m_new);  // masked: 2^-inf = 0
                ls += p[kt][v];
            }
        ls += __shfl_xor(ls, 16);
        ls += __shfl_xor(ls, 32);
        l_run = l_run * corr + ls;
        // the output is rescaled only when some query's maximum moved
        // (corr == 1 exactly otherwise)
        if (__ballot(m_new != m_run)) {
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int t = 0; t < DT; ++t) o[c][t] *= corr;
        }
        m_run = m_new;

        // O^T += V^T P^T, two K-steps of 32 keys, P as bf16 hi + lo
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x0 = (e < 2) ? p[2 * ks][2 * e] : p[2 * ks + 1][2 * e - 4];
                const float x1 = (e < 2) ? p[2 * ks][2 * e + 1] : p[2 * ks + 1][2 * e - 3];
                hi[e] = bf16x2_rne(x0, x1);
                lo[e] = bf16x2_rne(x0 - __uint_as_float(hi[e] << 16), x1 - __uint_as_float(hi[e] & 0xFFFF0000u));
            }
            const bf16x8_t ph = __builtin_bit_cast(bf16x8_t, make_uint4(hi[0], hi[1], hi[2], hi[3]));
            const bf16x8_t pl = __builtin_bit_cast(bf16x8_t, make_uint4(lo[0], lo[1], lo[2], lo[3]));
            // A operand of O^T: lane l needs V[key][16t + l % 16] for keys
            // 32ks + 4g + 0..3 and 32ks + 16 + 4g + 0..3.  A transpose read
            // gives lane i of a 16-lane group element i % 4 of the 8 bytes
            // lane 4k + i/4 addresses, as its element k; so lane j of the
            // group addresses key kb + j/4, d 16t + 4(j % 4).
            const int key_a = 32 * ks + 4 * g + (c16 >> 2), key_b = key_a + 16;
            const int dq = 4 * (c16 & 3);
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int t = 0; t < DT; ++t) {
                    const uint8_t* base = s_v + (size_t)(c * kKeys) * kRowV + (16 * t + dq) * 2;
                    const uint2 va = ds_read_tr16(base + key_a * kRowV);
                    const uint2 vb = ds_read_tr16(base + key_b * kRowV);
                    const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, make_uint4(va.x, va.y, vb.x, vb.y));
                    o[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, ph, o[c][t], 0, 0, 0);
                    o[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pl, o[c][t], 0, 0, 0);
                }
        }
    }

    if (q_ok) {
        const float inv = 1.0f / l_run;
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
    __shared__ __align__(16) uint8_t s_k[Geometry<D>::kBytesK];
    __shared__ __align__(16) uint8_t s_v[Geometry<D>::kBytesV];
    if (!a.causal) {
        attend_tile<D>(a, blockIdx.x, s_k, s_v);
        return;
    }
    const int64_t nqb = (a.sq + kQBlock - 1) / kQBlock;
    const int64_t heavy = nqb - 1 - blockIdx.x, light = blockIdx.x;
    attend_tile<D>(a, heavy, s_k, s_v);
    if (light < heavy) attend_tile<D>(a, light, s_k, s_v);
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
