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
// and the activations are the MFMA A operand, staged per 64-column chunk in
// LDS (int8: in the same permuted column order the byte decode produces).
//
// Tiles: a wave owns 32 tokens x 64 output rows (2 x 4 MFMA 16x16 tiles);
// a block of 4 waves covers 32 tokens x 256 rows and shares the staged
// activations.  bf16: planes are the inner loop of each 64-column chunk and
// each plane's scaled partial sums are folded into fp32 outputs right away
// (the scales are linear, so chunked folding is exact up to fp32 rounding).
// int8: planes are the outer loop so every plane's int32 sums are complete
// and exact before the float epilogue (and can be returned raw).
//
// Operand layouts (16x16xK, verified on gfx950): lane l holds A row l%16 and
// B column l%16, K elements [(K/4)*(l/16), +K/4); C lane l holds column l%16,
// rows 4*(l/16) + 0..3.
#include "fairy_gemv_impl.h"

namespace fairy {
namespace mfma {

using gemv::GemvArgs;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef int intx4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kTok = 32;                 // tokens per wave (and per block)
constexpr int kRows = 64;                // output rows per wave
constexpr int kTT = kTok / 16;           // token tiles per wave
constexpr int kRT = kRows / 16;          // row tiles per wave
constexpr int kBlockRows = kWaves * kRows;
// staged activations: [re/im][kTok][64 + pad] elements
constexpr int kPadBf16 = 8, kPadI8 = 16;

template <int XT>
__device__ __forceinline__ void stage_chunk(const GemvArgs& a, int tok0, int g, uint8_t* xs)
{
    // 64 columns of kTok tokens, re and im; 16 bytes per thread-step
    constexpr int esize = (XT == FAIRY_BF16) ? 2 : 1;
    constexpr int per_row = 64 * esize / 16;                 // 16-byte pieces per token row
    constexpr int row_bytes = (64 + (XT == FAIRY_BF16 ? kPadBf16 : kPadI8)) * esize;
    for (int idx = threadIdx.x; idx < 2 * kTok * per_row; idx += blockDim.x) {
        const int plane = idx / (kTok * per_row);
        const int rem = idx - plane * kTok * per_row;
        const int t = rem / per_row;
        const int piece = rem - t * per_row;
        const int c = 64 * g + piece * (16 / esize);
        uint4 v = make_uint4(0, 0, 0, 0);
        const int tok = tok0 + t;
        if (tok < a.B && c < a.m) {
            const uint8_t* src = reinterpret_cast<const uint8_t*>(plane ? a.x_im : a.x_re) +
                                 ((int64_t)tok * a.ldx + c) * esize;
            v = *reinterpret_cast<const uint4*>(src);
        }
        if constexpr (XT == FAIRY_I8) {
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
            v = make_uint4(out[0], out[1], out[2], out[3]);
        }
        *reinterpret_cast<uint4*>(xs + ((size_t)plane * kTok + t) * row_bytes + piece * 16) = v;
    }
}

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kWaves * 64) void k_cgemm_mfma_bf16(GemvArgs a)
{
    __shared__ __align__(16) uint8_t xs[2 * kTok * (64 + kPadBf16) * 2];
    constexpr int row_bytes = (64 + kPadBf16) * 2;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int tok0 = blockIdx.x * kTok;
    const int row_base = blockIdx.y * kBlockRows + wave * kRows;
    const int P = a.P;
    const uint4* packed = reinterpret_cast<const uint4*>(a.packed);

    floatx4_t yr[kTT][kRT], yi[kTT][kRT];
#pragma unroll
    for (int i = 0; i < kTT; ++i)
#pragma unroll
        for (int j = 0; j < kRT; ++j) { yr[i][j] = floatx4_t{0, 0, 0, 0}; yi[i][j] = floatx4_t{0, 0, 0, 0}; }

    for (int g = 0; g < a.G; ++g) {
        if (g) __syncthreads();
        stage_chunk<FAIRY_BF16>(a, tok0, g, xs);
        __syncthreads();
        // A fragments: 2 K-steps of 32, kTT token tiles, re and im
        bf16x8_t xr[2][kTT], xi[2][kTT];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int tt = 0; tt < kTT; ++tt) {
                const int off = (tt * 16 + r16) * row_bytes + (32 * s + 8 * q) * 2;
                xr[s][tt] = *reinterpret_cast<const bf16x8_t*>(xs + off);
                xi[s][tt] = *reinterpret_cast<const bf16x8_t*>(xs + kTok * row_bytes + off);
            }
        for (int p = 0; p < P; ++p) {
            uint4 cw[kRT];
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt) {
                const int row = row_base + 16 * rt + r16;
                cw[rt] = (row < a.n) ? packed[((int64_t)row * a.G + g) * P + p] : make_uint4(0, 0, 0, 0);
            }
            floatx4_t acc[4][kTT][kRT];
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int i = 0; i < kTT; ++i)
#pragma unroll
                    for (int j = 0; j < kRT; ++j) acc[b][i][j] = floatx4_t{0, 0, 0, 0};
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                // lane's 8 columns of this K-step: word 2s + q/2, half q%2 -> pairs 4*(q%2)+i
                bf16x8_t re8[kRT], im8[kRT];
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt) {
                    const uint32_t wv[4] = {cw[rt].x, cw[rt].y, cw[rt].z, cw[rt].w};
                    const uint32_t w = wv[2 * s + (q >> 1)];
                    uint32_t re2[4], im2[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) decode_bf16_pair(w, 4 * (q & 1) + i, re2[i], im2[i]);
                    re8[rt] = __builtin_bit_cast(bf16x8_t, make_uint4(re2[0], re2[1], re2[2], re2[3]));
                    im8[rt] = __builtin_bit_cast(bf16x8_t, make_uint4(im2[0], im2[1], im2[2], im2[3]));
                }
#pragma unroll
                for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
                    for (int rt = 0; rt < kRT; ++rt) {
                        acc[0][tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xr[s][tt], re8[rt], acc[0][tt][rt], 0, 0, 0);
                        acc[1][tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xi[s][tt], im8[rt], acc[1][tt][rt], 0, 0, 0);
                        acc[2][tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xi[s][tt], re8[rt], acc[2][tt][rt], 0, 0, 0);
                        acc[3][tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xr[s][tt], im8[rt], acc[3][tt][rt], 0, 0, 0);
                    }
            }
            // fold this plane's chunk: decoded weights are +-2, so half-scales
            const float hr = 0.5f * a.scales[2 * p], hi = 0.5f * a.scales[2 * p + 1];
            const float sg = (p < a.S) ? 1.0f : -1.0f;
#pragma unroll
            for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        yr[tt][rt][v] += hr * acc[0][tt][rt][v] - sg * (hi * acc[1][tt][rt][v]);
                        yi[tt][rt][v] += sg * (hr * acc[2][tt][rt][v]) + hi * acc[3][tt][rt][v];
                    }
        }
    }
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
            const int row = row_base + 16 * rt + r16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int tok = tok0 + 16 * tt + 4 * q + v;
                if (row < a.n && tok < a.B) {
                    a.y_re[(int64_t)tok * a.ldy + row] = yr[tt][rt][v];
                    a.y_im[(int64_t)tok * a.ldy + row] = yi[tt][rt][v];
                }
            }
        }
}

// ---------------------------------------------------------------------------
// int8
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kWaves * 64) void k_cgemm_mfma_i8(GemvArgs a)
{
    __shared__ __align__(16) uint8_t xs[2 * kTok * (64 + kPadI8)];
    constexpr int row_bytes = 64 + kPadI8;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int tok0 = blockIdx.x * kTok;
    const int row_base = blockIdx.y * kBlockRows + wave * kRows;
    const int P = a.P;
    const uint4* packed = reinterpret_cast<const uint4*>(a.packed);

    floatx4_t yr[kTT][kRT], yi[kTT][kRT];
#pragma unroll
    for (int i = 0; i < kTT; ++i)
#pragma unroll
        for (int j = 0; j < kRT; ++j) { yr[i][j] = floatx4_t{0, 0, 0, 0}; yi[i][j] = floatx4_t{0, 0, 0, 0}; }

    for (int p = 0; p < P; ++p) {
        intx4_t acc[4][kTT][kRT];
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int i = 0; i < kTT; ++i)
#pragma unroll
                for (int j = 0; j < kRT; ++j) acc[b][i][j] = intx4_t{0, 0, 0, 0};
        for (int g = 0; g < a.G; ++g) {
            uint4 cw[kRT];
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt) {
                const int row = row_base + 16 * rt + r16;
                cw[rt] = (row < a.n) ? packed[((int64_t)row * a.G + g) * P + p] : make_uint4(0, 0, 0, 0);
            }
            __syncthreads();
            stage_chunk<FAIRY_I8>(a, tok0, g, xs);
            __syncthreads();
            intx4_t xr[kTT], xi[kTT];
#pragma unroll
            for (int tt = 0; tt < kTT; ++tt) {
                const int off = (tt * 16 + r16) * row_bytes + 16 * q;
                xr[tt] = *reinterpret_cast<const intx4_t*>(xs + off);
                xi[tt] = *reinterpret_cast<const intx4_t*>(xs + kTok * row_bytes + off);
            }
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt) {
                const uint32_t wv[4] = {cw[rt].x, cw[rt].y, cw[rt].z, cw[rt].w};
                uint32_t re[4], im[4];
                gemv::ternary_bytes(wv[q], re, im);  // lane's K range is word q of the group
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
        const float s_re = a.scales[2 * p], s_im = a.scales[2 * p + 1];
        const bool conjp = p >= a.S;
#pragma unroll
        for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt) {
                const int row = row_base + 16 * rt + r16;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int t1 = acc[0][tt][rt][v], t2 = acc[1][tt][rt][v];
                    const int t3 = acc[2][tt][rt][v], t4 = acc[3][tt][rt][v];
                    const int tok = tok0 + 16 * tt + 4 * q + v;
                    if (a.acc && row < a.n && tok < a.B) {
                        a.acc[(((int64_t)p * 4 + 0) * a.B + tok) * a.n + row] = t1;
                        a.acc[(((int64_t)p * 4 + 1) * a.B + tok) * a.n + row] = t2;
                        a.acc[(((int64_t)p * 4 + 2) * a.B + tok) * a.n + row] = t3;
                        a.acc[(((int64_t)p * 4 + 3) * a.B + tok) * a.n + row] = t4;
                    }
                    const float f1 = (float)t1, f2 = (float)t2, f3 = (float)t3, f4 = (float)t4;
                    if (!conjp) {
                        yr[tt][rt][v] += s_re * f1 - s_im * f2;
                        yi[tt][rt][v] += s_re * f3 + s_im * f4;
                    } else {
                        yr[tt][rt][v] += s_re * f1 + s_im * f2;
                        yi[tt][rt][v] += s_im * f4 - s_re * f3;
                    }
                }
            }
    }
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
            const int row = row_base + 16 * rt + r16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int tok = tok0 + 16 * tt + 4 * q + v;
                if (row < a.n && tok < a.B) {
                    a.y_re[(int64_t)tok * a.ldy + row] = yr[tt][rt][v];
                    a.y_im[(int64_t)tok * a.ldy + row] = yi[tt][rt][v];
                }
            }
        }
}

}  // namespace mfma

hipError_t launch_cgemm_mfma(const gemv::GemvArgs& a, int32_t xdtype, hipStream_t s)
{
    const dim3 grid((a.B + mfma::kTok - 1) / mfma::kTok, (a.n + mfma::kBlockRows - 1) / mfma::kBlockRows);
    if (grid.y > 65535) return hipErrorInvalidValue;
    if (xdtype == FAIRY_BF16)
        hipLaunchKernelGGL(mfma::k_cgemm_mfma_bf16, grid, dim3(mfma::kWaves * 64), 0, s, a);
    else
        hipLaunchKernelGGL(mfma::k_cgemm_mfma_i8, grid, dim3(mfma::kWaves * 64), 0, s, a);
    return hipGetLastError();
}

}  // namespace fairy
