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
// Waves are planes.  A block has 8 waves and covers 64 tokens; wave w works
// on plane plane0 + w % Q and on the 32 output rows of row group w / Q, over
// the whole K range.  A plane's sums are therefore complete in registers
// when the K loop ends (exact int32 for int8): the per-axis scales are
// applied once, and the Q planes of a row group are added across waves in
// LDS in a fixed order.  Q is 4, 2 or 1; a layer with another plane count
// runs as several passes (4s, then a 2, then a 1), each later pass adding
// into y.  All waves of a block share the staged activations.
//
// K order.  Inside a 64-column group, bf16 K-step s (0, 1) and lane quarter
// q = lane/16 cover columns 16q + 8s + 0..7, so a lane reads exactly one
// packed word (word q) per row, group and plane and takes its pairs 4s..4s+3;
// the int8 K-step is the whole group, word q, in the byte order that
// ternary_bytes produces.  The A fragments are read from LDS in the same
// column order.
//
// Latency.  The activations of the next 128-column chunk are loaded into
// registers while the current chunk is multiplied, and the code words one
// chunk ahead.  Two waves share each SIMD.
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
constexpr int kTT = 4;                  // 16-token tiles per wave
constexpr int kRT = 2;                  // 16-row tiles per wave
constexpr int kTok = 16 * kTT;          // tokens per block
constexpr int kWaveRows = 16 * kRT;     // output rows per wave
constexpr int kChunkG = 2;              // 64-column groups per staged chunk
constexpr int kChunkCols = 64 * kChunkG;
constexpr int kMaxGridY = 65535;

template <int Q>
constexpr int block_rows() { return (kWaves / Q) * kWaveRows; }

// Staged chunk: [re/im][kTok][kChunkCols + pad].  The pad puts the 16 token
// rows that one 16-lane phase reads on distinct banks.
constexpr int kRowBf16 = (kChunkCols + 8) * 2;  // bytes
constexpr int kRowI8 = kChunkCols + 16;         // bytes
// cross-wave sums: up to kWaves/2 writers x one component of a wave's tile
constexpr int kRedBytes = (kWaves / 2) * kTT * kRT * 64 * 16;
constexpr int kLdsBytes = (2 * kTok * kRowBf16 > kRedBytes) ? 2 * kTok * kRowBf16 : kRedBytes;

template <int ESIZE>
struct Stage {
    static constexpr int row_bytes = (ESIZE == 2) ? kRowBf16 : kRowI8;
    static constexpr int per_row = kChunkCols * ESIZE / 16;     // 16-byte pieces per token row
    static constexpr int pieces = 2 * kTok * per_row;
    static constexpr int per_thread = pieces / kThreads;
    static_assert(pieces % kThreads == 0, "staging split");
};

// 16-byte piece idx of a chunk -> (re/im plane, token row, byte offset in the
// row, global column).
template <int ESIZE>
struct Piece {
    int plane, t, byte, col;
    __device__ __forceinline__ Piece(int idx, int c0)
    {
        constexpr int per_row = Stage<ESIZE>::per_row;
        plane = idx / (kTok * per_row);
        const int rem = idx - plane * kTok * per_row;
        t = rem / per_row;
        const int pc = rem - t * per_row;
        byte = pc * 16;
        col = c0 + pc * (16 / ESIZE);
    }
};

// Columns >= m and tokens >= M are zero.
template <int ESIZE>
__device__ __forceinline__ void load_chunk(const GemvArgs& a, int tok0, int c0, uint4 (&v)[Stage<ESIZE>::per_thread])
{
#pragma unroll
    for (int i = 0; i < Stage<ESIZE>::per_thread; ++i) {
        const Piece<ESIZE> pc(i * kThreads + threadIdx.x, c0);
        const int tok = tok0 + pc.t;
        v[i] = make_uint4(0, 0, 0, 0);
        if (tok < a.B && pc.col < a.m) {
            const uint8_t* src = reinterpret_cast<const uint8_t*>(pc.plane ? a.x_im : a.x_re) +
                                 ((int64_t)tok * a.ldx + pc.col) * ESIZE;
            v[i] = *reinterpret_cast<const uint4*>(src);
        }
    }
}

// An int8 piece is one 16-column word; reorder its bytes to the dot4 groups
// of ternary_bytes: output byte 4s + b is column i8_group_col(s, b).
__device__ __forceinline__ uint4 permute_i8_word(uint4 v)
{
    const uint32_t in[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        uint32_t o = 0;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const int tc = i8_group_col(s, bb);
            o |= ((in[tc >> 2] >> (8 * (tc & 3))) & 0xFFu) << (8 * bb);
        }
        out[s] = o;
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

template <int ESIZE>
__device__ __forceinline__ void store_chunk(const uint4 (&v)[Stage<ESIZE>::per_thread], uint8_t* xs)
{
#pragma unroll
    for (int i = 0; i < Stage<ESIZE>::per_thread; ++i) {
        const Piece<ESIZE> pc(i * kThreads + threadIdx.x, 0);
        const uint4 w = (ESIZE == 1) ? permute_i8_word(v[i]) : v[i];
        *reinterpret_cast<uint4*>(xs + ((size_t)pc.plane * kTok + pc.t) * Stage<ESIZE>::row_bytes + pc.byte) = w;
    }
}

// The lane's code words: word q of (row, group g, plane p) for its kRT rows,
// zero outside the matrix.
struct CodeRows {
    const uint32_t* base[kRT];
    bool ok[kRT];
    int G, gstride;
    __device__ __forceinline__ CodeRows(const GemvArgs& a, int row, int p, int q)
    {
        G = a.G;
        gstride = a.P * 4;
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
            const int r = row + 16 * rt;
            ok[rt] = r < a.n;
            base[rt] = a.packed + ((int64_t)(ok[rt] ? r : 0) * G * a.P + p) * 4 + q;
        }
    }
    __device__ __forceinline__ void chunk(int g0, uint32_t (&w)[kRT][kChunkG]) const
    {
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
            for (int gi = 0; gi < kChunkG; ++gi)
                w[rt][gi] = (ok[rt] && g0 + gi < G) ? base[rt][(g0 + gi) * gstride] : 0u;
    }
};

// Epilogue shared by the kernels: this wave's plane contribution from its
// four sums (int8: also the raw sums to acc), the cross-wave sum of the Q
// planes of each row group through LDS (red), and the store (or add) of y.
template <int Q, typename Acc>
__device__ __forceinline__ void finish_tile(const GemvArgs& a, floatx4_t* red, const Acc (&acc)[4][kTT][kRT], int p,
                                            int slot, int rg, int row0, int tok0, int q, int r16, int lane,
                                            int accumulate)
{
    // This plane's contribution.  U planes: y_re += s_re A1 - s_im A2,
    // y_im += s_re A3 + s_im A4; W planes multiply conj(x): A2 and A3 flip.
    const float s_re = a.scales[2 * p], s_im = a.scales[2 * p + 1];
    const float sg = (p < a.S) ? 1.0f : -1.0f;
    floatx4_t pr[kTT][kRT], pi[kTT][kRT];
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
            const int row = row0 + 16 * rt + r16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float f1, f2, f3, f4;
                if constexpr (std::is_same<Acc, floatx4_t>::value) {
                    // decoded weights are +-2: half-scales
                    f1 = 0.5f * acc[0][tt][rt][v];
                    f2 = 0.5f * acc[1][tt][rt][v];
                    f3 = 0.5f * acc[2][tt][rt][v];
                    f4 = 0.5f * acc[3][tt][rt][v];
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
                pr[tt][rt][v] = s_re * f1 - sg * (s_im * f2);
                pi[tt][rt][v] = sg * (s_re * f3) + s_im * f4;
            }
        }

    // Sum the Q planes of each row group: at each halving step the waves of
    // the upper half write, the lower half adds (fixed order, no atomics).
    if constexpr (Q > 1) {
#pragma unroll
        for (int step = Q / 2; step >= 1; step /= 2) {
#pragma unroll
            for (int comp = 0; comp < 2; ++comp) {
                floatx4_t (&part)[kTT][kRT] = comp ? pi : pr;
                __syncthreads();
                if (slot >= step && slot < 2 * step) {
                    floatx4_t* dst = red + (size_t)(rg * step + slot - step) * kTT * kRT * 64;
#pragma unroll
                    for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
                        for (int rt = 0; rt < kRT; ++rt) dst[(tt * kRT + rt) * 64 + lane] = part[tt][rt];
                }
                __syncthreads();
                if (slot < step) {
                    const floatx4_t* src = red + (size_t)(rg * step + slot) * kTT * kRT * 64;
#pragma unroll
                    for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
                        for (int rt = 0; rt < kRT; ++rt) part[tt][rt] += src[(tt * kRT + rt) * 64 + lane];
                }
            }
        }
    }
    if (slot != 0) return;
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
            const int row = row0 + 16 * rt + r16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int tok = tok0 + 16 * tt + 4 * q + v;
                if (row < a.n && tok < a.B) {
                    float* yr = a.y_re + (int64_t)tok * a.ldy + row;
                    float* yi = a.y_im + (int64_t)tok * a.ldy + row;
                    *yr = accumulate ? *yr + pr[tt][rt][v] : pr[tt][rt][v];
                    *yi = accumulate ? *yi + pi[tt][rt][v] : pi[tt][rt][v];
                }
            }
        }
}

// ---------------------------------------------------------------------------
// bf16 staging by direct global -> LDS loads (global_load_lds_dwordx4): a
// wave-instruction writes 64 consecutive 16-byte LDS slots, lane l into slot
// l, from any global addresses.  A chunk of 128 columns is [re/im][64 tokens]
// [16 slots of 8 columns]; slot p of token row t holds the columns of piece
// p ^ (t % 16), so the 16 rows one 16-lane phase reads sit on distinct banks
// without padding, and two chunk buffers fit in 64 KiB.  Slots outside the
// matrix load 16 zero bytes.
// ---------------------------------------------------------------------------
__device__ uint4 g_zero16;

constexpr int kDmaRowBytes = 256;                       // 16 slots per token row
constexpr int kDmaBufBytes = 2 * kTok * kDmaRowBytes;   // re and im: 32 KiB
constexpr int kDmaInsts = kDmaBufBytes / (64 * 16);     // wave-instructions per chunk
static_assert(kDmaInsts % kWaves == 0, "dma split");
static_assert(2 * kDmaBufBytes >= kRedBytes, "cross-wave sums reuse the chunk buffers");

__device__ __forceinline__ void dma_chunk_bf16(const GemvArgs& a, int tok0, int c0, uint8_t* buf, int wave,
                                               int lane)
{
#pragma unroll
    for (int i = 0; i < kDmaInsts / kWaves; ++i) {
        const int wi = i * kWaves + wave;
        const int slot = wi * 64 + lane;
        const int plane = slot / (kTok * 16);
        const int t = (slot / 16) % kTok;
        const int piece = (slot % 16) ^ (t % 16);
        const int c = c0 + 8 * piece;
        const int tok = tok0 + t;
        const void* src = &g_zero16;
        if (tok < a.B && c < a.m)
            src = reinterpret_cast<const uint16_t*>(plane ? a.x_im : a.x_re) + (int64_t)tok * a.ldx + c;
        __builtin_amdgcn_global_load_lds(src, buf + wi * 64 * 16, 16, 0, 0);
    }
}

// byte offset of (re/im plane, token row t, 8-column piece) in a chunk buffer
__device__ __forceinline__ int dma_off(int plane, int t, int piece)
{
    return (plane * kTok + t) * kDmaRowBytes + 16 * (piece ^ (t % 16));
}

template <int Q>
__global__ __launch_bounds__(kThreads) void k_cgemm_mfma_bf16(GemvArgs a, int tok_base, int plane0, int accumulate)
{
    __shared__ __align__(16) uint8_t lds[2 * kDmaBufBytes];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int slot = wave % Q, rg = wave / Q;
    const int p = plane0 + slot;
    const int row0 = blockIdx.x * block_rows<Q>() + rg * kWaveRows;
    const int tok0 = tok_base + blockIdx.y * kTok;
    const int G = a.G;
    const CodeRows codes(a, row0 + r16, p, q);

    floatx4_t acc[4][kTT][kRT];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < kTT; ++i)
#pragma unroll
            for (int j = 0; j < kRT; ++j) acc[b][i][j] = floatx4_t{0, 0, 0, 0};

    const int nchunk = (G + kChunkG - 1) / kChunkG;
    dma_chunk_bf16(a, tok0, 0, lds, wave, lane);
    uint32_t cw[kRT][kChunkG];
    codes.chunk(0, cw);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int ch = 0; ch < nchunk; ++ch) {
        // the next chunk streams into the other buffer, which every wave
        // finished reading before the barrier that ended the previous step
        if (ch + 1 < nchunk) dma_chunk_bf16(a, tok0, (ch + 1) * kChunkCols, lds + ((ch + 1) & 1) * kDmaBufBytes, wave, lane);
        const int g0 = ch * kChunkG;
        uint32_t nw[kRT][kChunkG];
        codes.chunk(g0 + kChunkG, nw);
        const uint8_t* xb = lds + (ch & 1) * kDmaBufBytes;
        // K-step ks covers group ks/2, half ks%2; the A fragments of step
        // ks+1 are read while step ks is multiplied
        constexpr int kSteps = 2 * kChunkG;
        bf16x8_t xf[2][2][kTT];
#pragma unroll
        for (int tt = 0; tt < kTT; ++tt) {
            xf[0][0][tt] = *reinterpret_cast<const bf16x8_t*>(xb + dma_off(0, tt * 16 + r16, 2 * q));
            xf[0][1][tt] = *reinterpret_cast<const bf16x8_t*>(xb + dma_off(1, tt * 16 + r16, 2 * q));
        }
#pragma unroll
        for (int ks = 0; ks < kSteps; ++ks) {
            const int gi = ks / 2, s = ks % 2;
            if (ks + 1 < kSteps) {
                const int piece = 8 * ((ks + 1) / 2) + 2 * q + (ks + 1) % 2;  // columns 64gi + 16q + 8s
#pragma unroll
                for (int tt = 0; tt < kTT; ++tt) {
                    xf[(ks + 1) & 1][0][tt] = *reinterpret_cast<const bf16x8_t*>(xb + dma_off(0, tt * 16 + r16, piece));
                    xf[(ks + 1) & 1][1][tt] = *reinterpret_cast<const bf16x8_t*>(xb + dma_off(1, tt * 16 + r16, piece));
                }
            }
            // (a group past the end has zero activations in LDS and zero
            // code words, so its products are exactly zero: no branch)
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt) {
                uint32_t re2[4], im2[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) decode_bf16_pair(cw[rt][gi], 4 * s + i, re2[i], im2[i]);
                const bf16x8_t re8 = __builtin_bit_cast(bf16x8_t, make_uint4(re2[0], re2[1], re2[2], re2[3]));
                const bf16x8_t im8 = __builtin_bit_cast(bf16x8_t, make_uint4(im2[0], im2[1], im2[2], im2[3]));
                const bf16x8_t (&xr)[kTT] = xf[ks & 1][0];
                const bf16x8_t (&xi)[kTT] = xf[ks & 1][1];
#pragma unroll
                for (int tt = 0; tt < kTT; ++tt) {
                    acc[0][tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xr[tt], re8, acc[0][tt][rt], 0, 0, 0);
                    acc[1][tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xi[tt], im8, acc[1][tt][rt], 0, 0, 0);
                    acc[2][tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xi[tt], re8, acc[2][tt][rt], 0, 0, 0);
                    acc[3][tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xr[tt], im8, acc[3][tt][rt], 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
            for (int gi = 0; gi < kChunkG; ++gi) cw[rt][gi] = nw[rt][gi];
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads into the other buffer have landed
        __syncthreads();
    }
    finish_tile<Q>(a, reinterpret_cast<floatx4_t*>(lds), acc, p, slot, rg, row0, tok0, q, r16, lane, accumulate);
}

template <int XT, int Q>
__global__ __launch_bounds__(kThreads) void k_cgemm_mfma(GemvArgs a, int tok_base, int plane0, int accumulate)
{
    constexpr bool kBf16 = XT == FAIRY_BF16;
    constexpr int ES = kBf16 ? 2 : 1;
    constexpr int kRow = Stage<ES>::row_bytes;
    using Acc = typename std::conditional<kBf16, floatx4_t, intx4_t>::type;

    __shared__ __align__(16) uint8_t lds[kLdsBytes];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int slot = wave % Q, rg = wave / Q;
    const int p = plane0 + slot;
    const int row0 = blockIdx.x * block_rows<Q>() + rg * kWaveRows;
    const int tok0 = tok_base + blockIdx.y * kTok;
    const int G = a.G;
    const CodeRows codes(a, row0 + r16, p, q);

    Acc acc[4][kTT][kRT];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < kTT; ++i)
#pragma unroll
            for (int j = 0; j < kRT; ++j) acc[b][i][j] = Acc{0, 0, 0, 0};

    const int nchunk = (G + kChunkG - 1) / kChunkG;
    uint4 xv[Stage<ES>::per_thread];
    load_chunk<ES>(a, tok0, 0, xv);
    uint32_t cw[kRT][kChunkG];
    codes.chunk(0, cw);

    for (int ch = 0; ch < nchunk; ++ch) {
        __syncthreads();  // every wave is done reading the previous chunk
        store_chunk<ES>(xv, lds);
        __syncthreads();
        if (ch + 1 < nchunk) load_chunk<ES>(a, tok0, (ch + 1) * kChunkCols, xv);
        const int g0 = ch * kChunkG;
        uint32_t nw[kRT][kChunkG];
        codes.chunk(g0 + kChunkG, nw);
#pragma unroll
        for (int gi = 0; gi < kChunkG; ++gi) {
            if (g0 + gi >= G) continue;
            if constexpr (kBf16) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    bf16x8_t xr[kTT], xi[kTT];
#pragma unroll
                    for (int tt = 0; tt < kTT; ++tt) {
                        const int off = (tt * 16 + r16) * kRow + (64 * gi + 16 * q + 8 * s) * 2;
                        xr[tt] = *reinterpret_cast<const bf16x8_t*>(lds + off);
                        xi[tt] = *reinterpret_cast<const bf16x8_t*>(lds + kTok * kRow + off);
                    }
#pragma unroll
                    for (int rt = 0; rt < kRT; ++rt) {
                        uint32_t re2[4], im2[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) decode_bf16_pair(cw[rt][gi], 4 * s + i, re2[i], im2[i]);
                        const bf16x8_t re8 = __builtin_bit_cast(bf16x8_t, make_uint4(re2[0], re2[1], re2[2], re2[3]));
                        const bf16x8_t im8 = __builtin_bit_cast(bf16x8_t, make_uint4(im2[0], im2[1], im2[2], im2[3]));
#pragma unroll
                        for (int tt = 0; tt < kTT; ++tt) {
                            acc[0][tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xr[tt], re8, acc[0][tt][rt], 0, 0, 0);
                            acc[1][tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xi[tt], im8, acc[1][tt][rt], 0, 0, 0);
                            acc[2][tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xi[tt], re8, acc[2][tt][rt], 0, 0, 0);
                            acc[3][tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xr[tt], im8, acc[3][tt][rt], 0, 0, 0);
                        }
                    }
                }
            } else {
                intx4_t xr[kTT], xi[kTT];
#pragma unroll
                for (int tt = 0; tt < kTT; ++tt) {
                    const int off = (tt * 16 + r16) * kRow + 64 * gi + 16 * q;
                    xr[tt] = *reinterpret_cast<const intx4_t*>(lds + off);
                    xi[tt] = *reinterpret_cast<const intx4_t*>(lds + kTok * kRow + off);
                }
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt) {
                    uint32_t re[4], im[4];
                    gemv::ternary_bytes(cw[rt][gi], re, im);
                    const intx4_t re4 = {(int)re[0], (int)re[1], (int)re[2], (int)re[3]};
                    const intx4_t im4 = {(int)im[0], (int)im[1], (int)im[2], (int)im[3]};
#pragma unroll
                    for (int tt = 0; tt < kTT; ++tt) {
                        acc[0][tt][rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xr[tt], re4, acc[0][tt][rt], 0, 0, 0);
                        acc[1][tt][rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xi[tt], im4, acc[1][tt][rt], 0, 0, 0);
                        acc[2][tt][rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xi[tt], re4, acc[2][tt][rt], 0, 0, 0);
                        acc[3][tt][rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xr[tt], im4, acc[3][tt][rt], 0, 0, 0);
                    }
                }
            }
        }
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
            for (int gi = 0; gi < kChunkG; ++gi) cw[rt][gi] = nw[rt][gi];
    }

    finish_tile<Q>(a, reinterpret_cast<floatx4_t*>(lds), acc, p, slot, rg, row0, tok0, q, r16, lane, accumulate);
}

template <int XT, int Q>
hipError_t launch_pass(const GemvArgs& a, int plane0, int accumulate, hipStream_t s)
{
    const int64_t row_blocks = (a.n + block_rows<Q>() - 1) / block_rows<Q>();
    const int64_t tok_blocks = ((int64_t)a.B + kTok - 1) / kTok;
    for (int64_t tb = 0; tb < tok_blocks; tb += kMaxGridY) {
        const int64_t nb = (tok_blocks - tb < kMaxGridY) ? tok_blocks - tb : kMaxGridY;
        if constexpr (XT == FAIRY_BF16)
            hipLaunchKernelGGL((k_cgemm_mfma_bf16<Q>), dim3((unsigned)row_blocks, (unsigned)nb), dim3(kThreads), 0, s,
                               a, (int)(tb * kTok), plane0, accumulate);
        else
            hipLaunchKernelGGL((k_cgemm_mfma<XT, Q>), dim3((unsigned)row_blocks, (unsigned)nb), dim3(kThreads), 0, s,
                               a, (int)(tb * kTok), plane0, accumulate);
    }
    return hipGetLastError();
}

template <int XT>
hipError_t launch_all(const GemvArgs& a, hipStream_t s)
{
    hipError_t e = hipSuccess;
    for (int p0 = 0; p0 < a.P && e == hipSuccess;) {
        const int rem = a.P - p0;
        const int acc = p0 > 0;
        if (rem >= 4) {
            e = launch_pass<XT, 4>(a, p0, acc, s);
            p0 += 4;
        } else if (rem >= 2) {
            e = launch_pass<XT, 2>(a, p0, acc, s);
            p0 += 2;
        } else {
            e = launch_pass<XT, 1>(a, p0, acc, s);
            p0 += 1;
        }
    }
    return e;
}

}  // namespace mfma

hipError_t launch_cgemm_mfma(const gemv::GemvArgs& a, int32_t xdtype, hipStream_t s)
{
    return (xdtype == FAIRY_BF16) ? mfma::launch_all<FAIRY_BF16>(a, s) : mfma::launch_all<FAIRY_I8>(a, s);
}

}  // namespace fairy
