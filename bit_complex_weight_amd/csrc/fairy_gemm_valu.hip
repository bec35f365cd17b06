// fairy_gemm_valu.hip -- prefill complex GEMM on the vector ALUs, lanes = tokens.
//
//   Y[t] = sum_k What(U_k) X[t] + sum_k What(W_k) conj(X[t])      [Fairy2i article §4.2, §2.1]
//
// Multiplication-free form as in the decode GEMV (four sums per plane, the
// per-axis scales applied once per row and plane at the end: [iFairy
// abstract] one non-zero axis per code, [iFairy talk §2.3.1] times i is a
// swap and a negation), mapped for many tokens at once [iFairy press
// article §二.2: the matrix product becomes additions, subtractions and
// swaps]:
//
//  * a wave's 64 lanes are 64 tokens; a block is kWaves waves over the same
//    R = 32 / P rows (R x P = NC (row, plane) pairs per lane);
//  * every code word a wave reads is the same for all its lanes, so it comes
//    through the scalar cache into SGPRs and is decoded by the scalar ALU
//    (one shift, one mask and one xor per pair of codes: bits 15:14 and
//    31:30 of the shifted word are the sign and top exponent bit of a bf16
//    pair, +-2 or +-0);
//  * the vector ALU does nothing but v_dot2_f32_bf16 with that SGPR operand
//    and the lane's own activations: 2 instructions per code and token
//    (four sums per pair of codes, half the products on zeros);
//  * a lane holds its token's activations for one 64-column group (32 bf16
//    pairs per plane) and reuses them for all NC pairs;
//  * int8 activations are converted to bf16 exactly (|x| <= 128 has at most
//    8 significant bits); with the +-2 weights every partial sum is an
//    integer of magnitude <= 256 m, exact in fp32 for m <= 65536, so the raw
//    accumulators are the exact integer sums.
//
// Blocks that share a token range are placed on one XCD (consecutive block
// numbers go to consecutive XCDs), so the activations of those tokens stay
// in that XCD's L2 while all row blocks stream past.
#include "fairy_gemv_impl.h"

namespace fairy {
namespace valu {

using gemv::GemvArgs;
using gemv::dot2_bf16;

constexpr int kWaves = 4;
constexpr int kNC = 32;  // (row, plane) pairs per lane

// int8 -> bf16 pair: two signed bytes of a word (b, b+1) as (lo, hi) bf16
__device__ __forceinline__ uint32_t i8pair_bf16(uint32_t w, int b)
{
    const float lo = (float)(int8_t)(w >> (8 * b));
    const float hi = (float)(int8_t)(w >> (8 * b + 8));
    // integers of at most 8 significant bits: the top 16 bits are exact
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

// The lane's activations for columns 64g .. 64g+63 as bf16 pairs, zero for
// columns >= m and for tokens >= M.  nw16 = valid 16-column words (1..4).
template <int XT>
__device__ __forceinline__ void load_x64(const GemvArgs& a, int64_t t, bool tok_ok, int g, int nw16,
                                         uint32_t (&xr)[32], uint32_t (&xi)[32])
{
    const uint4* zero = &gemv::g_zero_unit;
    if constexpr (XT == FAIRY_BF16) {
        const uint4* pr = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.x_re) + t * a.ldx + 64 * g);
        const uint4* pi = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.x_im) + t * a.ldx + 64 * g);
        uint4 vr[8], vi[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {  // 16-byte piece i holds columns 8i .. 8i+7 (word i / 2)
            const bool on = tok_ok && (i >> 1) < nw16;
            vr[i] = *(on ? pr + i : zero);
            vi[i] = *(on ? pi + i : zero);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            xr[4 * i] = vr[i].x; xr[4 * i + 1] = vr[i].y; xr[4 * i + 2] = vr[i].z; xr[4 * i + 3] = vr[i].w;
            xi[4 * i] = vi[i].x; xi[4 * i + 1] = vi[i].y; xi[4 * i + 2] = vi[i].z; xi[4 * i + 3] = vi[i].w;
        }
    } else {
        const uint4* pr = reinterpret_cast<const uint4*>(reinterpret_cast<const int8_t*>(a.x_re) + t * a.ldx + 64 * g);
        const uint4* pi = reinterpret_cast<const uint4*>(reinterpret_cast<const int8_t*>(a.x_im) + t * a.ldx + 64 * g);
        uint4 vr[4], vi[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // 16-byte piece i = 16-column word i
            const bool on = tok_ok && i < nw16;
            vr[i] = *(on ? pr + i : zero);
            vi[i] = *(on ? pi + i : zero);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t wr[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
            const uint32_t wi[4] = {vi[i].x, vi[i].y, vi[i].z, vi[i].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                xr[8 * i + 2 * d] = i8pair_bf16(wr[d], 0);
                xr[8 * i + 2 * d + 1] = i8pair_bf16(wr[d], 2);
                xi[8 * i + 2 * d] = i8pair_bf16(wi[d], 0);
                xi[8 * i + 2 * d + 1] = i8pair_bf16(wi[d], 2);
            }
        }
    }
}

template <int XT, int P>
__global__ __launch_bounds__(kWaves * 64) void k_cgemm_valu(GemvArgs a, int nrb, int ntb)
{
    static_assert(P >= 1 && P <= kNC, "plane count");
    constexpr int R = kNC / P;   // rows per block
    constexpr int NC = R * P;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    // block -> (row block, token block); token blocks spread over the XCDs
    // when their count allows, so each XCD keeps its tokens' activations
    const int L = blockIdx.x;
    int rb, tb;
    if ((ntb & 7) == 0) {
        const int q = L >> 3;
        tb = 8 * (q / nrb) + (L & 7);
        rb = q % nrb;
    } else {
        tb = L / nrb;
        rb = L % nrb;
    }
    const int64_t t = ((int64_t)tb * kWaves + wave) * 64 + lane;
    const bool tok_ok = t < a.B;
    const int row0 = rb * R;
    const int G = a.G;
    const uint4* units = reinterpret_cast<const uint4*>(a.packed);

    float A[NC][4];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) A[c][q] = 0.f;

    // unit (row, g, p) of pair c = (r, p); a row past the end reads the
    // last row's words (its sums are not stored)
    auto unit = [&](int c, int g) -> uint4 {
        const int r = c / P, p = c % P;
        const int row = (row0 + r < a.n) ? row0 + r : a.n - 1;
        const uint4 v = units[((int64_t)row * G + g) * P + p];
        // the words are the same in every lane: keep them in SGPRs (the
        // compiler otherwise splits some loads into vector registers and
        // decodes those on the vector ALU)
        return make_uint4(__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
                          __builtin_amdgcn_readfirstlane(v.z), __builtin_amdgcn_readfirstlane(v.w));
    };
    for (int g = 0; g < G; ++g) {
        const int rem = (a.m - 64 * g) >> 4;
        const int nw16 = rem < 4 ? rem : 4;
        uint32_t xr[32], xi[32];
        load_x64<XT>(a, tok_ok ? t : 0, tok_ok, g, nw16, xr, xi);
        // the next pair's code words are loaded while this pair's are used
        // (scheduling barriers keep the compiler from hoisting every load
        // of the group, which would need more SGPRs than a wave has)
        uint4 wn = unit(0, g);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const uint4 w4 = wn;
            if (c + 1 < NC) wn = unit(c + 1, g);
            __builtin_amdgcn_sched_barrier(0);
            // two words per 64-bit scalar operation: bits shifted out of the
            // low word land in bits 0..13 of the high one, which the mask drops
            const uint64_t w01 = (uint64_t)w4.x | ((uint64_t)w4.y << 32);
            const uint64_t w23 = (uint64_t)w4.z | ((uint64_t)w4.w << 32);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint64_t wv = h ? w23 : w01;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const uint64_t im = (wv << (2 * k)) & 0xC000C000C000C000ull;
                    const uint64_t re = im ^ 0x4000400040004000ull;
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int u = 2 * h + e;
                        const uint32_t im2 = (uint32_t)(im >> (32 * e));
                        const uint32_t re2 = (uint32_t)(re >> (32 * e));
                        const uint32_t xrk = xr[8 * u + k], xik = xi[8 * u + k];
                        A[c][0] = dot2_bf16(re2, xrk, A[c][0]);
                        A[c][2] = dot2_bf16(re2, xik, A[c][2]);
                        A[c][1] = dot2_bf16(im2, xik, A[c][1]);
                        A[c][3] = dot2_bf16(im2, xrk, A[c][3]);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // epilogue: the decoded weights are +-2, so half-scales; W planes multiply conj(x)
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = row0 + r;
        if (row >= a.n) break;
        float yr = 0.f, yi = 0.f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int c = r * P + p;
            const float hr = 0.5f * a.scales[2 * p], hi = 0.5f * a.scales[2 * p + 1];
            const float sg = (p < a.S) ? 1.0f : -1.0f;
            yr += hr * A[c][0] - sg * (hi * A[c][1]);
            yi += sg * (hr * A[c][2]) + hi * A[c][3];
            if (XT == FAIRY_I8 && a.acc && tok_ok) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    a.acc[(((int64_t)p * 4 + q) * a.B + t) * a.n + row] = (int32_t)(0.5f * A[c][q]);
            }
        }
        if (tok_ok) {
            gemv::rope_apply(a, row, t, yr, yi);
            a.y_re[t * a.ldy + row] = yr;
            a.y_im[t * a.ldy + row] = yi;
        }
    }
}

template <int XT, int P>
hipError_t launch_t(const GemvArgs& a, hipStream_t s)
{
    constexpr int R = kNC / P;
    const int nrb = (a.n + R - 1) / R;
    const int64_t ntb = ((int64_t)a.B + kWaves * 64 - 1) / (kWaves * 64);
    const int64_t nb = (int64_t)nrb * ntb;
    if (nb > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_cgemm_valu<XT, P>), dim3((unsigned)nb), dim3(kWaves * 64), 0, s, a, nrb, (int)ntb);
    return hipGetLastError();
}

template <int XT>
hipError_t launch_p(const GemvArgs& a, hipStream_t s)
{
    switch (a.P) {
    case 1: return launch_t<XT, 1>(a, s);
    case 2: return launch_t<XT, 2>(a, s);
    case 3: return launch_t<XT, 3>(a, s);
    case 4: return launch_t<XT, 4>(a, s);
    case 6: return launch_t<XT, 6>(a, s);
    case 8: return launch_t<XT, 8>(a, s);
    case 16: return launch_t<XT, 16>(a, s);
    default: return hipErrorNotSupported;
    }
}

}  // namespace valu

bool cgemm_valu_tokens_supported(int32_t xdtype, int64_t m, int32_t planes)
{
    const bool p_ok = planes == 1 || planes == 2 || planes == 3 || planes == 4 || planes == 6 || planes == 8 ||
                      planes == 16;
    if (!p_ok) return false;
    if (xdtype == FAIRY_BF16) return true;
    // int8 sums stay exact integers in fp32 up to 65536 columns
    return xdtype == FAIRY_I8 && m <= 65536;
}

hipError_t launch_cgemm_valu(const gemv::GemvArgs& a, int32_t xdtype, hipStream_t s)
{
    if (xdtype == FAIRY_BF16) return valu::launch_p<FAIRY_BF16>(a, s);
    if (xdtype == FAIRY_I8) return valu::launch_p<FAIRY_I8>(a, s);
    return hipErrorNotSupported;
}

}  // namespace fairy
