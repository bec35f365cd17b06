// fairy_gemm_mfma.hip -- prefill complex GEMM on the gfx950 matrix cores.
//
// At M in the thousands the layer is a dense contraction [Fairy2i article
// §4.2]: per plane p the four accumulators are the products of the split
// activation planes with the two ternary planes of the codes,
//   A1 = X_re ReB^T, A4 = X_re ImB^T, A3 = X_im ReB^T, A2 = X_im ImB^T,
// ReB, ImB in {-1, 0, 1} ([iFairy abstract]: one non-zero axis per code).
// The ternary planes never exist in memory: each lane decodes its MFMA
// B-operand fragment from the packed TILED64 words with bit operations
//   bf16: the +-2 / 0 bf16 pair decode (decode_bf16_pair), v_mfma_f32_16x16x32_bf16
//   int8: v_perm ternary bytes (ternary_bytes),          v_mfma_i32_16x16x64_i8
// and the activations are the MFMA A operand, staged in LDS.
//
// Waves are planes.  A block has 8 waves and covers 64 tokens (16 or 32 when
// the whole prompt is no longer: no matrix-core work on padding); wave w works
// on plane plane0 + w % Q and on the 32 output rows of row group w / Q, over
// the whole K range.  A plane's sums are therefore complete in registers
// when the K loop ends (exact int32 for int8): the per-axis scales are
// applied once, and the Q planes of a row group are added across waves in
// LDS in a fixed order.  Q is 4, 2 or 1; a layer with another plane count
// runs as several passes (4s, then a 2, then a 1), each later pass adding
// into y.  All waves of a block share the staged activations.
//
// Staging.  A chunk is 256 bytes of each token row (128 bf16 or 256 int8
// columns), re and im, for the block's 64 tokens: 32 KiB (8 KiB per 16
// tokens), written straight from global memory into LDS by
// global_load_lds_dwordx4 (a wave-instruction fills 64 consecutive 16-byte
// slots, lane l slot l, from any addresses).
// Two chunk buffers alternate: the next chunk streams in while the current
// one is multiplied, one barrier per chunk.  Slot p of token row t holds
// piece p ^ (t % 16) of the row, so the 16 rows a 16-lane phase reads sit on
// distinct banks without padding; slots outside the matrix load 16 zero
// bytes.
//
// K order.  A chunk is 4 K-steps.  bf16 K-step s of a 64-column group and
// lane quarter q = lane/16 cover columns 16q + 8s + 0..7, so a lane reads one
// packed word (word q) per row, group and plane and takes its pairs
// 4s..4s+3; the int8 K-step is a whole group, word q, in natural column
// order (the ternary bytes are permuted once per word after decoding).  The
// A fragments of the next K-step are read while the current one is
// multiplied.
//
// Operand layouts (16x16xK, verified on gfx950): lane l holds A row l%16 and
// B column l%16, K elements [(K/4)*(l/16), +K/4); C lane l holds column l%16,
// rows 4*(l/16) + 0..3.
#include "fairy_gemv_impl.h"

#include <type_traits>

namespace fairy {
namespace mfma {

using gemv::GemvArgs;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef int intx4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRT = 2;                  // 16-row tiles per wave
constexpr int kWaveRows = 16 * kRT;     // output rows per wave
constexpr int kMaxGridY = 65535;
constexpr int kRowBytes = 256;          // one token row of a chunk: 16 slots
constexpr int kSteps = 4;               // K-steps per chunk

template <int Q>
constexpr int block_rows() { return (kWaves / Q) * kWaveRows; }

// TT 16-token tiles per wave (4 for long prompts; 1 or 2 when the whole
// prompt is that short, so no matrix-core work goes to padding tokens)
template <int TT>
struct Tiles {
    static constexpr int tok = 16 * TT;                     // tokens per block
    static constexpr int buf_bytes = 2 * tok * kRowBytes;   // re and im: 8 KiB per token tile
    static constexpr int dma_insts = buf_bytes / (64 * 16); // wave-instructions per chunk
    // cross-wave sums: one component of every wave's partial tiles
    static constexpr int red_bytes = kWaves * TT * kRT * 64 * 16;
    static_assert(dma_insts % kWaves == 0, "staging split");
    static_assert(2 * buf_bytes >= red_bytes, "cross-wave sums reuse the chunk buffers");
};

constexpr int token_tiles(int64_t M) { return M <= 16 ? 1 : M <= 32 ? 2 : 4; }

template <int XT>
struct Geo {
    static constexpr int esize = (XT == FAIRY_BF16) ? 2 : 1;
    static constexpr int slot_cols = 16 / esize;               // columns per 16-byte slot
    static constexpr int groups = kRowBytes / (64 * esize);    // 64-column groups per chunk
    static constexpr int cols = 64 * groups;
    using Frag = typename std::conditional<XT == FAIRY_BF16, bf16x8_t, intx4_t>::type;
    using Acc = typename std::conditional<XT == FAIRY_BF16, floatx4_t, intx4_t>::type;
    static_assert(kSteps == ((XT == FAIRY_BF16) ? 2 : 1) * groups, "K-steps per chunk");
};

// 16 zero bytes: the source of staging slots outside the matrix
__device__ uint4 g_zero16;

template <int XT, int TT>
__device__ __forceinline__ void dma_chunk(const GemvArgs& a, int tok0, int c0, uint8_t* buf, int wave, int lane)
{
    constexpr int es = Geo<XT>::esize;
    constexpr int tok = Tiles<TT>::tok;
#pragma unroll
    for (int i = 0; i < Tiles<TT>::dma_insts / kWaves; ++i) {
        const int wi = i * kWaves + wave;
        const int slot = wi * 64 + lane;
        const int plane = slot / (tok * 16);
        const int t = (slot / 16) % tok;
        const int piece = (slot % 16) ^ (t % 16);
        const int c = c0 + Geo<XT>::slot_cols * piece;
        const int tok = tok0 + t;
        const void* src = &g_zero16;
        if (tok < a.B && c < a.m)
            src = reinterpret_cast<const uint8_t*>(plane ? a.x_im : a.x_re) + ((int64_t)tok * a.ldx + c) * es;
        __builtin_amdgcn_global_load_lds(src, buf + wi * 64 * 16, 16, 0, 0);
    }
}

// byte offset of (re/im plane, token row t, 16-byte piece) in a chunk buffer
template <int TT>
__device__ __forceinline__ int slot_off(int plane, int t, int piece)
{
    return (plane * Tiles<TT>::tok + t) * kRowBytes + 16 * (piece ^ (t % 16));
}

// ternary_bytes order (byte b of register s is column i8_group_col(s, b))
// -> natural column order (byte b of register j is column 4j + b), so the
// decoded codes line up with activations staged as they are in memory.
__device__ __forceinline__ intx4_t to_natural_order(const uint32_t (&t)[4])
{
    return intx4_t{(int)__builtin_amdgcn_perm(t[3], t[2], 0x03010705u), (int)__builtin_amdgcn_perm(t[1], t[0], 0x03010705u),
                   (int)__builtin_amdgcn_perm(t[3], t[2], 0x02000604u), (int)__builtin_amdgcn_perm(t[1], t[0], 0x02000604u)};
}

// A fragments of K-step ks for the lane (token rows 16tt + r16, quarter q)
template <int XT, int TT>
__device__ __forceinline__ void read_frags(const uint8_t* xb, int ks, int q, int r16,
                                           typename Geo<XT>::Frag (&xr)[TT], typename Geo<XT>::Frag (&xi)[TT])
{
    using Frag = typename Geo<XT>::Frag;
    // bf16: columns 64(ks/2) + 16q + 8(ks%2) .. +8; int8: columns 64ks + 16q .. +16
    const int piece = (XT == FAIRY_BF16) ? 8 * (ks / 2) + 2 * q + ks % 2 : 4 * ks + q;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        xr[tt] = *reinterpret_cast<const Frag*>(xb + slot_off<TT>(0, tt * 16 + r16, piece));
        xi[tt] = *reinterpret_cast<const Frag*>(xb + slot_off<TT>(1, tt * 16 + r16, piece));
    }
}

// The lane's code words: word q of (row, group g, plane p) for its kRT rows,
// zero outside the matrix.
struct CodeRows {
    const uint32_t* base[kRT];
    bool ok[kRT];
    int G, gstride, q;
    __device__ __forceinline__ CodeRows(const GemvArgs& a, int row, int p, int q_)
    {
        G = a.G;
        gstride = a.P * 4;
        q = q_;
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
            const int r = row + 16 * rt;
            ok[rt] = r < a.n;
            base[rt] = a.packed + ((int64_t)(ok[rt] ? r : 0) * G * a.P + p) * 4;  // the (row, group 0, plane) unit
        }
    }
    // Raw loads of a chunk's words, taken apart by finish() once they have
    // landed.  The loads are unconditional (no branch for the compiler to
    // wait inside): a word outside the matrix or past this block's chunks
    // (live = false) is read from 16 zero bytes instead.
    template <int NG>
    struct Raw {
        uint32_t v[kRT][4];
    };
    template <int NG>
    __device__ __forceinline__ void load(int g0, Raw<NG>& r, bool live) const
    {
        const uint32_t* zero = reinterpret_cast<const uint32_t*>(&g_zero16);
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
            if constexpr (NG == 4) {
                // Four groups, four lane quarters: quarter q loads the whole
                // 16-byte unit of group g0 + q (one 128-bit load per row tile
                // instead of four 32-bit ones).
                const bool on = live && ok[rt] && g0 + q < G;
                const uint4 u = *reinterpret_cast<const uint4*>(on ? base[rt] + (int64_t)(g0 + q) * gstride : zero);
                r.v[rt][0] = u.x;
                r.v[rt][1] = u.y;
                r.v[rt][2] = u.z;
                r.v[rt][3] = u.w;
            } else {
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    const bool on = live && ok[rt] && g0 + gi < G;
                    r.v[rt][gi] = *(on ? base[rt] + (int64_t)(g0 + gi) * gstride + q : zero);
                }
            }
        }
    }
    // word q of (row, group, plane) for each of the chunk's NG groups
    template <int NG>
    __device__ __forceinline__ static void finish(const Raw<NG>& r, uint32_t (&w)[kRT][NG])
    {
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
            if constexpr (NG == 4) {
                // 4x4 transpose across the quarters, two row-swap stages:
                // quarters q, q ^ 2 (the upper pair takes the lower pair's
                // words 2, 3 in exchange for its words 0, 1), then q, q ^ 1
                const auto a02 = __builtin_amdgcn_permlane32_swap(r.v[rt][0], r.v[rt][2], false, false);
                const auto a13 = __builtin_amdgcn_permlane32_swap(r.v[rt][1], r.v[rt][3], false, false);
                const auto b01 = __builtin_amdgcn_permlane16_swap(a02[0], a13[0], false, false);
                const auto b23 = __builtin_amdgcn_permlane16_swap(a02[1], a13[1], false, false);
                w[rt][0] = b01[0];
                w[rt][1] = b01[1];
                w[rt][2] = b23[0];
                w[rt][3] = b23[1];
            } else {
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) w[rt][gi] = r.v[rt][gi];
            }
        }
    }
    template <int NG>
    __device__ __forceinline__ void chunk(int g0, uint32_t (&w)[kRT][NG], bool live = true) const
    {
        Raw<NG> r;
        load<NG>(g0, r, live);
        finish<NG>(r, w);
    }
};

// Epilogue: this wave's plane contribution from its four sums (int8: also
// the raw sums to acc), the cross-wave sum of the Q planes of each row group
// through LDS (red), and the store (or add) of y.
template <int Q, int TT, typename Acc>
__device__ __forceinline__ void finish_tile(const GemvArgs& a, floatx4_t* red, const Acc (&acc)[4][TT][kRT], int p,
                                            int slot, int rg, int row0, int tok0, int q, int r16, int lane,
                                            int accumulate, float* part)
{
    // This plane's contribution.  U planes: y_re += s_re A1 - s_im A2,
    // y_im += s_re A3 + s_im A4; W planes multiply conj(x): A2 and A3 flip,
    // the sign folded into the scale it multiplies.  The bf16 sums come from
    // +-2 weights: half-scales (exact).
    constexpr float kHalf = std::is_same<Acc, floatx4_t>::value ? 0.5f : 1.0f;
    const float sg = (p < a.S) ? 1.0f : -1.0f;
    const float c_re = kHalf * a.scales[2 * p], c_im = kHalf * a.scales[2 * p + 1];
    const float c_re_sg = sg * c_re, c_im_sg = sg * c_im;
    floatx4_t pr[TT][kRT], pi[TT][kRT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
            const int row = row0 + 16 * rt + r16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float f1, f2, f3, f4;
                if constexpr (std::is_same<Acc, floatx4_t>::value) {
                    f1 = acc[0][tt][rt][v];
                    f2 = acc[1][tt][rt][v];
                    f3 = acc[2][tt][rt][v];
                    f4 = acc[3][tt][rt][v];
                } else {
                    const int t1 = acc[0][tt][rt][v], t2 = acc[1][tt][rt][v];
                    const int t3 = acc[2][tt][rt][v], t4 = acc[3][tt][rt][v];
                    const int tok = tok0 + 16 * tt + 4 * q + v;
                    if (a.acc && row < a.n && tok < a.B) {
                        a.acc[(((int64_t)p * 4 + 0) * a.B + tok) * a.n + row] = t1;
                        a.acc[(((int64_t)p * 4 + 1) * a.B + tok) * a.n + row] = t2;
                        a.acc[(((int64_t)p * 4 + 2) * a.B + tok) * a.n + row] = t3;
                        a.acc[(((int64_t)p * 4 + 3) * a.B + tok) * a.n + row] = t4;
                    }
                    f1 = (float)t1;
                    f2 = (float)t2;
                    f3 = (float)t3;
                    f4 = (float)t4;
                }
                pr[tt][rt][v] = c_re * f1 - c_im_sg * f2;
                pi[tt][rt][v] = c_re_sg * f3 + c_im * f4;
            }
        }

    // Sum the Q planes of each row group.  Token tile tt belongs to the wave
    // of slot tt % Q: every wave writes its partial tiles of the others' to
    // LDS, and each owner adds the Q partials of its tiles in a fixed order,
    // (0 + 2) + (1 + 3), then stores them, so all waves share the stores.
    // One component at a time: the two chunk buffers hold one.
    floatx4_t fr[TT][kRT], fi[TT][kRT];  // this wave's finished tiles (those it owns)
    if constexpr (Q > 1) {
        const int me = __builtin_amdgcn_readfirstlane(slot);
        auto at = [&](int tt, int s, int rt) {
            return red + ((((size_t)rg * TT + tt) * Q + s) * kRT + rt) * 64 + lane;
        };
#pragma unroll
        for (int comp = 0; comp < 2; ++comp) {
            const floatx4_t (&mine)[TT][kRT] = comp ? pi : pr;
            floatx4_t (&fin)[TT][kRT] = comp ? fi : fr;
            __syncthreads();  // the buffers are free: the chunks (or the last component) are read
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                if (tt % Q == me) continue;
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt) *at(tt, me, rt) = mine[tt][rt];
            }
            __syncthreads();
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                if (tt % Q != me) continue;
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt) {
                    floatx4_t v[Q];
#pragma unroll
                    for (int s = 0; s < Q; ++s) {
                        if (s == me) v[s] = mine[tt][rt];
                        else v[s] = *at(tt, s, rt);
                    }
                    if constexpr (Q == 4)
                        fin[tt][rt] = (v[0] + v[2]) + (v[1] + v[3]);
                    else
                        fin[tt][rt] = v[0] + v[1];
                }
            }
        }
    } else {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt) {
                fr[tt][rt] = pr[tt][rt];
                fi[tt][rt] = pi[tt][rt];
            }
    }
    if (part) {
        // split K: this block's share of the sum, [split][re/im][M][n]
        const int64_t mn = (int64_t)a.B * a.n;
        float* pre = part + (int64_t)blockIdx.z * 2 * mn;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            if (tt % Q != slot) continue;
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt) {
                const int row = row0 + 16 * rt + r16;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int tok = tok0 + 16 * tt + 4 * q + v;
                    if (row < a.n && tok < a.B) {
                        pre[(int64_t)tok * a.n + row] = fr[tt][rt][v];
                        pre[mn + (int64_t)tok * a.n + row] = fi[tt][rt][v];
                    }
                }
            }
        }
        return;
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        if (tt % Q != slot) continue;
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
            const int row = row0 + 16 * rt + r16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int tok = tok0 + 16 * tt + 4 * q + v;
                if (row < a.n && tok < a.B) {
                    float* yr = a.y_re + (int64_t)tok * a.ldy + row;
                    float* yi = a.y_im + (int64_t)tok * a.ldy + row;
                    float vr = accumulate ? *yr + fr[tt][rt][v] : fr[tt][rt][v];
                    float vi = accumulate ? *yi + fi[tt][rt][v] : fi[tt][rt][v];
                    gemv::rope_apply(a, row, tok, vr, vi);  // set on the last pass only
                    *yr = vr;
                    *yi = vi;
                }
            }
        }
    }
}

template <int XT, int Q, int TT>
__global__ __launch_bounds__(kThreads) void k_cgemm_mfma(GemvArgs a, int tok_base, int plane0, int accumulate,
                                                         int chunks_per_split, float* part)
{
    using G_ = Geo<XT>;
    using Frag = typename G_::Frag;
    using Acc = typename G_::Acc;
    constexpr int NG = G_::groups;
    constexpr int kBufBytes = Tiles<TT>::buf_bytes;
    __shared__ __align__(16) uint8_t lds[2 * kBufBytes];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int slot = wave % Q, rg = wave / Q;
    const int p = plane0 + slot;
    const int row0 = blockIdx.x * block_rows<Q>() + rg * kWaveRows;
    const int tok0 = tok_base + blockIdx.y * Tiles<TT>::tok;
    const int G = a.G;
    const CodeRows codes(a, row0 + r16, p, q);

    Acc acc[4][TT][kRT];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < TT; ++i)
#pragma unroll
            for (int j = 0; j < kRT; ++j) acc[b][i][j] = Acc{0, 0, 0, 0};

    // this block's chunks of the K range: all of them, or one split's share
    const int nchunk = (G + NG - 1) / NG;
    const int ch0 = blockIdx.z * chunks_per_split;
    const int ch1 = (nchunk < ch0 + chunks_per_split) ? nchunk : ch0 + chunks_per_split;
    // The products of one staged chunk (code words cw).  A group past the
    // end has zero activations and zero code words, so its products are
    // exactly zero: the chunk needs no branch.
    uint32_t cw[kRT][NG], nw[kRT][NG];
    auto products = [&](const uint8_t* xb) {
        Frag xf[2][2][TT];
        read_frags<XT, TT>(xb, 0, q, r16, xf[0][0], xf[0][1]);
#pragma unroll
        for (int ks = 0; ks < kSteps; ++ks) {
            if (ks + 1 < kSteps) read_frags<XT, TT>(xb, ks + 1, q, r16, xf[(ks + 1) & 1][0], xf[(ks + 1) & 1][1]);
            const Frag (&xr)[TT] = xf[ks & 1][0];
            const Frag (&xi)[TT] = xf[ks & 1][1];
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt) {
                if constexpr (XT == FAIRY_BF16) {
                    uint32_t re2[4], im2[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) decode_bf16_pair(cw[rt][ks / 2], 4 * (ks % 2) + i, re2[i], im2[i]);
                    const bf16x8_t re8 = __builtin_bit_cast(bf16x8_t, make_uint4(re2[0], re2[1], re2[2], re2[3]));
                    const bf16x8_t im8 = __builtin_bit_cast(bf16x8_t, make_uint4(im2[0], im2[1], im2[2], im2[3]));
#pragma unroll
                    for (int tt = 0; tt < TT; ++tt) {
                        acc[0][tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xr[tt], re8, acc[0][tt][rt], 0, 0, 0);
                        acc[1][tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xi[tt], im8, acc[1][tt][rt], 0, 0, 0);
                        acc[2][tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xi[tt], re8, acc[2][tt][rt], 0, 0, 0);
                        acc[3][tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xr[tt], im8, acc[3][tt][rt], 0, 0, 0);
                    }
                } else {
                    uint32_t re[4], im[4];
                    gemv::ternary_bytes(cw[rt][ks], re, im);
                    const intx4_t re4 = to_natural_order(re);
                    const intx4_t im4 = to_natural_order(im);
#pragma unroll
                    for (int tt = 0; tt < TT; ++tt) {
                        acc[0][tt][rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xr[tt], re4, acc[0][tt][rt], 0, 0, 0);
                        acc[1][tt][rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xi[tt], im4, acc[1][tt][rt], 0, 0, 0);
                        acc[2][tt][rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xi[tt], re4, acc[2][tt][rt], 0, 0, 0);
                        acc[3][tt][rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xr[tt], im4, acc[3][tt][rt], 0, 0, 0);
                    }
                }
            }
        }
    };
    // The code words issued at the top of a chunk stay there (the scheduler
    // would move them next to their use and wait for them inside the
    // chunk); the int8 transpose of them stays after the products.
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

    if constexpr (XT == FAIRY_BF16 && TT == 4) {
        // bf16, 64-token blocks: one chunk ahead.  Chunk ch + 1 streams into
        // the other buffer, which every wave finished reading before the
        // barrier that ended the previous chunk.  (The loop below measured
        // 3% slower here.)
        dma_chunk<XT, TT>(a, tok0, ch0 * G_::cols, lds, wave, lane);
        codes.chunk(ch0 * NG, cw);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        for (int ch = ch0; ch < ch1; ++ch) {
            const int buf = (ch - ch0) & 1;
            if (ch + 1 < ch1) dma_chunk<XT, TT>(a, tok0, (ch + 1) * G_::cols, lds + (buf ^ 1) * kBufBytes, wave, lane);
            CodeRows::Raw<NG> rn;
            codes.load<NG>((ch + 1) * NG, rn, ch + 1 < ch1);
            fence();
            products(lds + buf * kBufBytes);
            CodeRows::finish<NG>(rn, cw);
            __builtin_amdgcn_s_waitcnt(0);  // this wave's loads into the other buffer have landed
            __syncthreads();
        }
    } else {
        // Short prompts and int8.  A block of one or two chunks (a K split
        // of a short prompt) loads both before its first barrier: one round
        // of loads, not two.  A longer one waits for its first chunk only
        // and streams the second under it.  Code words run two chunks ahead
        // (cw, nw, then the raw words of chunk ch + 2).
        const bool both = ch1 - ch0 <= 2;
        dma_chunk<XT, TT>(a, tok0, ch0 * G_::cols, lds, wave, lane);
        codes.chunk(ch0 * NG, cw);
        codes.chunk((ch0 + 1) * NG, nw, ch0 + 1 < ch1);
        if (both && ch0 + 1 < ch1) dma_chunk<XT, TT>(a, tok0, (ch0 + 1) * G_::cols, lds + kBufBytes, wave, lane);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (!both) dma_chunk<XT, TT>(a, tok0, (ch0 + 1) * G_::cols, lds + kBufBytes, wave, lane);
        for (int ch = ch0; ch < ch1; ++ch) {
            const int buf = (ch - ch0) & 1;
            CodeRows::Raw<NG> rnn;
            codes.load<NG>((ch + 2) * NG, rnn, ch + 2 < ch1);
            fence();
            products(lds + buf * kBufBytes);
            if constexpr (NG == 4) fence();
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) cw[rt][gi] = nw[rt][gi];
            CodeRows::finish<NG>(rnn, nw);
            __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the next chunk have landed
            __syncthreads();                // and every wave is done with this buffer:
            // chunk ch + 2 streams into it while chunk ch + 1 is multiplied
            if (ch + 2 < ch1) dma_chunk<XT, TT>(a, tok0, (ch + 2) * G_::cols, lds + buf * kBufBytes, wave, lane);
        }
    }
    finish_tile<Q, TT>(a, reinterpret_cast<floatx4_t*>(lds), acc, p, slot, rg, row0, tok0, q, r16, lane, accumulate,
                   part);
}

// Split K: y = (accumulate ? y : 0) + the splits' partial sums, added in
// split order (deterministic), then the optional rotation.
__global__ __launch_bounds__(256) void k_split_sum(GemvArgs a, const float* part, int splits, int accumulate)
{
    const int64_t mn = (int64_t)a.B * a.n;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= mn) return;
    const int tok = (int)(idx / a.n), row = (int)(idx % a.n);
    float sr = 0.0f, si = 0.0f;
    // eight splits' loads in flight at once (a split past the end re-reads
    // the last one and is not added)
    for (int z0 = 0; z0 < splits; z0 += 8) {
        float vr[8], vi[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t z = (z0 + j < splits) ? z0 + j : splits - 1;
            vr[j] = part[2 * z * mn + idx];
            vi[j] = part[(2 * z + 1) * mn + idx];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (z0 + j < splits) {
                sr += vr[j];
                si += vi[j];
            }
    }
    float* yr = a.y_re + (int64_t)tok * a.ldy + row;
    float* yi = a.y_im + (int64_t)tok * a.ldy + row;
    float fr = accumulate ? *yr + sr : sr;
    float fi = accumulate ? *yi + si : si;
    gemv::rope_apply(a, row, tok, fr, fi);
    *yr = fr;
    *yi = fi;
}

// Groups per staged chunk and chunks of a row, by activation type
template <int XT>
constexpr int chunk_groups() { return Geo<XT>::groups; }

int split_count(int64_t n, int64_t m, int64_t M, int P, int xdtype)
{
    // A single pass (P planes in one launch) that leaves CUs idle is split
    // along K: each split walks a share of the chunks and the shares are
    // added by a second kernel.
    if (P != 1 && P != 2 && P != 4) return 1;
    const int Q = P;
    const int64_t rows = (kWaves / Q) * kWaveRows;
    const int64_t tok = 16 * token_tiles(M);
    const int64_t blocks = ((n + rows - 1) / rows) * ((M + tok - 1) / tok);
    const int64_t G = m / 64;
    const int ng = xdtype == FAIRY_BF16 ? chunk_groups<FAIRY_BF16>() : chunk_groups<FAIRY_I8>();
    const int64_t nchunk = (G + ng - 1) / ng;
    constexpr int64_t kTargetBlocks = 256;  // one block per CU (two waves per SIMD)
    if (blocks >= kTargetBlocks / 2 || nchunk < 2) return 1;
    int64_t splits = (kTargetBlocks + blocks - 1) / blocks;
    if (splits > nchunk) splits = nchunk;
    const int64_t cps = (nchunk + splits - 1) / splits;
    return (int)((nchunk + cps - 1) / cps);
}

template <int XT, int Q, int TT>
hipError_t launch_pass(const GemvArgs& a, int plane0, int accumulate, float* part, int splits, hipStream_t s)
{
    constexpr int kTok = Tiles<TT>::tok;
    const int64_t row_blocks = (a.n + block_rows<Q>() - 1) / block_rows<Q>();
    const int64_t tok_blocks = ((int64_t)a.B + kTok - 1) / kTok;
    const int nchunk = (a.G + Geo<XT>::groups - 1) / Geo<XT>::groups;
    if (part) {
        const int cps = (nchunk + splits - 1) / splits;
        hipLaunchKernelGGL((k_cgemm_mfma<XT, Q, TT>), dim3((unsigned)row_blocks, (unsigned)tok_blocks, (unsigned)splits),
                           dim3(kThreads), 0, s, a, 0, plane0, 0, cps, part);
        const int64_t mn = (int64_t)a.B * a.n;
        hipLaunchKernelGGL(k_split_sum, dim3((unsigned)((mn + 255) / 256)), dim3(256), 0, s, a, part, splits,
                           accumulate);
        return hipGetLastError();
    }
    for (int64_t tb = 0; tb < tok_blocks; tb += kMaxGridY) {
        const int64_t nb = (tok_blocks - tb < kMaxGridY) ? tok_blocks - tb : kMaxGridY;
        hipLaunchKernelGGL((k_cgemm_mfma<XT, Q, TT>), dim3((unsigned)row_blocks, (unsigned)nb), dim3(kThreads), 0, s, a,
                           (int)(tb * kTok), plane0, accumulate, nchunk, (float*)nullptr);
    }
    return hipGetLastError();
}

template <int XT, int TT>
hipError_t launch_all(const GemvArgs& a, void* workspace, hipStream_t s)
{
    // split K when a workspace is given, no raw accumulators are asked for,
    // and the layer is one pass that would leave CUs idle
    const int splits = split_count(a.n, a.m, a.B, a.P, XT);
    if (workspace && !a.acc && splits > 1) {
        float* part = static_cast<float*>(workspace);
        if (a.P == 4) return launch_pass<XT, 4, TT>(a, 0, 0, part, splits, s);
        if (a.P == 2) return launch_pass<XT, 2, TT>(a, 0, 0, part, splits, s);
        return launch_pass<XT, 1, TT>(a, 0, 0, part, splits, s);
    }
    hipError_t e = hipSuccess;
    for (int p0 = 0; p0 < a.P && e == hipSuccess;) {
        const int rem = a.P - p0;
        const int acc = p0 > 0;
        const int q = rem >= 4 ? 4 : rem >= 2 ? 2 : 1;
        GemvArgs pass = a;
        if (p0 + q < a.P) pass.pos = nullptr;  // the rotation applies to the finished sum
        if (q == 4) e = launch_pass<XT, 4, TT>(pass, p0, acc, nullptr, 1, s);
        else if (q == 2) e = launch_pass<XT, 2, TT>(pass, p0, acc, nullptr, 1, s);
        else e = launch_pass<XT, 1, TT>(pass, p0, acc, nullptr, 1, s);
        p0 += q;
    }
    return e;
}

}  // namespace mfma

hipError_t launch_cgemm_mfma(const gemv::GemvArgs& a, int32_t xdtype, void* workspace, hipStream_t s)
{
    using namespace mfma;
    const int tt = token_tiles(a.B);
    if (xdtype == FAIRY_BF16)
        return tt == 1 ? launch_all<FAIRY_BF16, 1>(a, workspace, s)
             : tt == 2 ? launch_all<FAIRY_BF16, 2>(a, workspace, s)
                       : launch_all<FAIRY_BF16, 4>(a, workspace, s);
    return tt == 1 ? launch_all<FAIRY_I8, 1>(a, workspace, s)
         : tt == 2 ? launch_all<FAIRY_I8, 2>(a, workspace, s)
                   : launch_all<FAIRY_I8, 4>(a, workspace, s);
}

size_t cgemm_mfma_workspace_bytes(int64_t n, int64_t m, int64_t M, int32_t P, int32_t xdtype)
{
    const int splits = mfma::split_count(n, m, M, P, xdtype);
    return splits > 1 ? (size_t)splits * 2 * (size_t)M * (size_t)n * sizeof(float) : 0;
}

}  // namespace fairy
