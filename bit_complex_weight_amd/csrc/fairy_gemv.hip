// fairy_gemv.hip -- decode-time complex GEMV on gfx950 (the hot path).
//
//   y[b] = sum_k What(U_k) x[b] + sum_k What(W_k) conj(x[b])     [Fairy2i article §4.2, §2.1]
//
// Multiplication-free form: per plane, row and batch column four fp32 sums
//   A1 = sum ReB x_re,  A2 = sum ImB x_im,  A3 = sum ReB x_im,  A4 = sum ImB x_re
// with ReB, ImB in {-1, 0, 1} ([iFairy abstract]: one non-zero axis per code;
// [iFairy talk §2.3.1]: times i is a swap and a negation), and the per-axis
// scales applied once per plane in the epilogue:
//   U plane: y_re += s_re A1 - s_im A2,  y_im += s_re A3 + s_im A4
//   W plane: y_re += s_re A1 + s_im A2,  y_im += s_im A4 - s_re A3
//
// Work mapping (wave64):
//   * a block of 256 threads owns 256/TROW output rows; TROW consecutive lanes
//     split a row's K dimension, lane j taking 64-column groups j, j+TROW, ...
//   * per group a lane issues one 128-bit load per plane: the TILED64 layout
//     stores the P planes of a (row, group) contiguously, so a wave reads
//     P * 1 KiB of consecutive bytes per step (fully coalesced);
//   * activations (split re/im planes) are staged once per block in LDS and
//     reused by every row of the block;
//   * decode is two bit operations per two codes (see decode_bf16_pair); the
//     bf16 path accumulates with v_dot2_f32_bf16 on the +-2 / 0 bf16 pairs,
//     the int8 path with v_dot4_i32_i8 on v_perm-expanded ternary bytes, the
//     fp32 path with fp32 FMAs on +-2 / 0;
//   * split-K partial sums are combined across the TROW lanes with DPP and
//     ds_swizzle butterflies (deterministic, no atomics).
#include "fairy_internal.h"

namespace fairy {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

struct GemvArgs {
    const uint32_t* packed;
    const float* scales;
    const void* x_re;
    const void* x_im;
    float* y_re;
    float* y_im;
    int32_t* acc;
    int64_t ldx, ldy;
    int32_t n, m, m64, G, S, P, B;
};

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Activation staging into LDS.  Layout per batch column b of the chunk:
//   bf16: re plane [m64] then im plane [m64] (uint16)   -> 4*m64 bytes
//   f32 : re [m64], im [m64] (float)                     -> 8*m64 bytes
//   i8  : re [m64], im [m64] bytes; inside every 16-column word the bytes are
//         reordered to the four dot4 groups (see i8_group_col).
// Columns >= m are zero.
// ---------------------------------------------------------------------------
template <int XT>
__device__ __forceinline__ void stage_x(const GemvArgs& a, int b0, int nb, uint8_t* lds)
{
    if (XT == FAIRY_BF16) {
        // 8 columns (16 bytes) per thread-step
        const int per = a.m64 / 8;
        uint4* dst = reinterpret_cast<uint4*>(lds);
        for (int idx = threadIdx.x; idx < nb * 2 * per; idx += blockDim.x) {
            const int b = idx / (2 * per);
            const int rem = idx - b * 2 * per;
            const int plane = rem / per;
            const int c8 = rem - plane * per;
            const uint16_t* src = reinterpret_cast<const uint16_t*>(plane ? a.x_im : a.x_re) +
                                  (int64_t)(b0 + b) * a.ldx + 8 * c8;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (8 * c8 < a.m) v = *reinterpret_cast<const uint4*>(src);
            dst[idx] = v;
        }
    } else if (XT == FAIRY_F32) {
        const int per = a.m64 / 4;
        float4* dst = reinterpret_cast<float4*>(lds);
        for (int idx = threadIdx.x; idx < nb * 2 * per; idx += blockDim.x) {
            const int b = idx / (2 * per);
            const int rem = idx - b * 2 * per;
            const int plane = rem / per;
            const int c4 = rem - plane * per;
            const float* src = reinterpret_cast<const float*>(plane ? a.x_im : a.x_re) +
                               (int64_t)(b0 + b) * a.ldx + 4 * c4;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (4 * c4 < a.m) v = *reinterpret_cast<const float4*>(src);
            dst[idx] = v;
        }
    } else {
        const int per = a.m64 / 16;
        uint4* dst = reinterpret_cast<uint4*>(lds);
        for (int idx = threadIdx.x; idx < nb * 2 * per; idx += blockDim.x) {
            const int b = idx / (2 * per);
            const int rem = idx - b * 2 * per;
            const int plane = rem / per;
            const int c16 = rem - plane * per;
            const int8_t* src = reinterpret_cast<const int8_t*>(plane ? a.x_im : a.x_re) +
                                (int64_t)(b0 + b) * a.ldx + 16 * c16;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (16 * c16 < a.m) v = *reinterpret_cast<const uint4*>(src);
            const uint32_t in[4] = {v.x, v.y, v.z, v.w};
            uint32_t out[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                uint32_t o = 0;
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const int t = i8_group_col(s, bb);
                    o |= ((in[t >> 2] >> (8 * (t & 3))) & 0xFFu) << (8 * bb);
                }
                out[s] = o;
            }
            dst[idx] = make_uint4(out[0], out[1], out[2], out[3]);
        }
    }
}

// ---------------------------------------------------------------------------
// Float paths (bf16 / fp32 activations)
// ---------------------------------------------------------------------------
template <int XT, int PMAX, int TROW, int BCH>
__global__ __launch_bounds__(kThreads) void k_cgemv_float(GemvArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    const int rows_pb = kThreads / TROW;
    const int lr = threadIdx.x % TROW;
    const int row = blockIdx.x * rows_pb + threadIdx.x / TROW;
    const bool row_ok = row < a.n;
    const int P = a.P;

    float hs_re[PMAX], hs_im[PMAX];  // half scales: decoded weights are +-2
#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
        hs_re[p] = (p < P) ? 0.5f * a.scales[2 * p] : 0.f;
        hs_im[p] = (p < P) ? 0.5f * a.scales[2 * p + 1] : 0.f;
    }

    const uint4* wrow = reinterpret_cast<const uint4*>(a.packed) + (int64_t)row * a.G * P;
    const int xbytes = (XT == FAIRY_BF16) ? 2 : 4;
    const int plane_stride = a.m64 * xbytes;  // bytes between re and im planes of one column b

    for (int b0 = 0; b0 < a.B; b0 += BCH) {
        const int nb = (a.B - b0 < BCH) ? a.B - b0 : BCH;
        if (b0) __syncthreads();
        stage_x<XT>(a, b0, nb, lds);
        __syncthreads();

        float yr[BCH], yi[BCH];
#pragma unroll
        for (int b = 0; b < BCH; ++b) { yr[b] = 0.f; yi[b] = 0.f; }

        for (int g = lr; g < a.G; g += TROW) {
            uint4 cw[PMAX];
#pragma unroll
            for (int p = 0; p < PMAX; ++p)
                cw[p] = (p < P && row_ok) ? wrow[(int64_t)g * P + p] : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int p = 0; p < PMAX; ++p) {
                if (p >= P) continue;
                float A1[BCH], A2[BCH], A3[BCH], A4[BCH];
#pragma unroll
                for (int b = 0; b < BCH; ++b) { A1[b] = A2[b] = A3[b] = A4[b] = 0.f; }
                const uint32_t words[4] = {cw[p].x, cw[p].y, cw[p].z, cw[p].w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t w = words[u];
                    const int col0 = 64 * g + 16 * u;
                    if (XT == FAIRY_BF16) {
                        uint32_t re2[8], im2[8];
#pragma unroll
                        for (int k = 0; k < 8; ++k) decode_bf16_pair(w, k, re2[k], im2[k]);
#pragma unroll
                        for (int b = 0; b < BCH; ++b) {
                            if (b >= nb) continue;
                            const uint8_t* xb = lds + (size_t)b * 2 * plane_stride + (size_t)col0 * 2;
                            const uint4 r0 = *reinterpret_cast<const uint4*>(xb);
                            const uint4 r1 = *reinterpret_cast<const uint4*>(xb + 16);
                            const uint4 i0 = *reinterpret_cast<const uint4*>(xb + plane_stride);
                            const uint4 i1 = *reinterpret_cast<const uint4*>(xb + plane_stride + 16);
                            const uint32_t xr[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
                            const uint32_t xi[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
                            for (int k = 0; k < 8; ++k) {
                                A1[b] = dot2_bf16(re2[k], xr[k], A1[b]);
                                A3[b] = dot2_bf16(re2[k], xi[k], A3[b]);
                                A2[b] = dot2_bf16(im2[k], xi[k], A2[b]);
                                A4[b] = dot2_bf16(im2[k], xr[k], A4[b]);
                            }
                        }
                    } else {
                        float re[16], im[16];
#pragma unroll
                        for (int t = 0; t < 16; ++t) {
                            const uint32_t ws = w << f32_shift(t);
                            im[t] = __uint_as_float(ws & 0xC0000000u);
                            re[t] = __uint_as_float((ws ^ 0x40000000u) & 0xC0000000u);
                        }
#pragma unroll
                        for (int b = 0; b < BCH; ++b) {
                            if (b >= nb) continue;
                            const float* xr = reinterpret_cast<const float*>(lds + (size_t)b * 2 * plane_stride) + col0;
                            const float* xi = reinterpret_cast<const float*>(lds + (size_t)b * 2 * plane_stride + plane_stride) + col0;
#pragma unroll
                            for (int t = 0; t < 16; ++t) {
                                const float vr = xr[t], vi = xi[t];
                                A1[b] = fmaf(re[t], vr, A1[b]);
                                A3[b] = fmaf(re[t], vi, A3[b]);
                                A2[b] = fmaf(im[t], vi, A2[b]);
                                A4[b] = fmaf(im[t], vr, A4[b]);
                            }
                        }
                    }
                }
                const bool conjp = p >= a.S;
#pragma unroll
                for (int b = 0; b < BCH; ++b) {
                    if (!conjp) {
                        yr[b] += hs_re[p] * A1[b] - hs_im[p] * A2[b];
                        yi[b] += hs_re[p] * A3[b] + hs_im[p] * A4[b];
                    } else {
                        yr[b] += hs_re[p] * A1[b] + hs_im[p] * A2[b];
                        yi[b] += hs_im[p] * A4[b] - hs_re[p] * A3[b];
                    }
                }
            }
        }
#pragma unroll
        for (int b = 0; b < BCH; ++b) {
            const float sr = group_sum<TROW>(yr[b]);
            const float si = group_sum<TROW>(yi[b]);
            if (lr == 0 && row_ok && b < nb) {
                a.y_re[(int64_t)(b0 + b) * a.ldy + row] = sr;
                a.y_im[(int64_t)(b0 + b) * a.ldy + row] = si;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// int8 path: exact int32 accumulators per plane, reduced across lanes, then
// the float epilogue from the exact sums.
// v_perm tables (pool bytes 0..3 from the second operand, 4..7 from the first;
// selector 8 replicates bit 15, 9 bit 31, 12 gives 0x00, 13.. give 0xFF):
//   codes at byte bits 1:0 -> selector c:      ReB pool 01 00 FF 00, ImB pool 00 01 00 FF
//   codes at byte bits 3:2 -> selector 4c:     ReB: c=0 byte0=01, c=1 byte4=00,
//                                              c=2 sign(bit15)=FF, c=3 -> 00
//                           selector 4c|1:     ImB: c=0 byte1=00, c=1 byte5=01,
//                                              c=2 sign(bit31)=00, c=3 -> FF
// ---------------------------------------------------------------------------
__device__ __forceinline__ void ternary_bytes(uint32_t w, uint32_t (&re)[4], uint32_t (&im)[4])
{
    const uint32_t w4 = w >> 4;
    const uint32_t s0 = w & 0x03030303u;
    const uint32_t s2 = w4 & 0x03030303u;
    const uint32_t s1r = w & 0x0C0C0C0Cu, s1i = s1r | 0x01010101u;
    const uint32_t s3r = w4 & 0x0C0C0C0Cu, s3i = s3r | 0x01010101u;
    re[0] = __builtin_amdgcn_perm(0u, 0x00FF0001u, s0);
    im[0] = __builtin_amdgcn_perm(0u, 0xFF000100u, s0);
    re[1] = __builtin_amdgcn_perm(0u, 0x00008001u, s1r);
    im[1] = __builtin_amdgcn_perm(0x00000100u, 0u, s1i);
    re[2] = __builtin_amdgcn_perm(0u, 0x00FF0001u, s2);
    im[2] = __builtin_amdgcn_perm(0u, 0xFF000100u, s2);
    re[3] = __builtin_amdgcn_perm(0u, 0x00008001u, s3r);
    im[3] = __builtin_amdgcn_perm(0x00000100u, 0u, s3i);
}

template <int PMAX, int TROW, int BCH>
__global__ __launch_bounds__(kThreads) void k_cgemv_i8(GemvArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    const int rows_pb = kThreads / TROW;
    const int lr = threadIdx.x % TROW;
    const int row = blockIdx.x * rows_pb + threadIdx.x / TROW;
    const bool row_ok = row < a.n;
    const int P = a.P;
    const uint4* wrow = reinterpret_cast<const uint4*>(a.packed) + (int64_t)row * a.G * P;
    const int plane_stride = a.m64;

    for (int b0 = 0; b0 < a.B; b0 += BCH) {
        const int nb = (a.B - b0 < BCH) ? a.B - b0 : BCH;
        if (b0) __syncthreads();
        stage_x<FAIRY_I8>(a, b0, nb, lds);
        __syncthreads();

        int A[PMAX][4][BCH];
#pragma unroll
        for (int p = 0; p < PMAX; ++p)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int b = 0; b < BCH; ++b) A[p][q][b] = 0;

        for (int g = lr; g < a.G; g += TROW) {
            uint4 cw[PMAX];
#pragma unroll
            for (int p = 0; p < PMAX; ++p)
                cw[p] = (p < P && row_ok) ? wrow[(int64_t)g * P + p] : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int col0 = 64 * g + 16 * u;
                uint4 xr4[BCH], xi4[BCH];
#pragma unroll
                for (int b = 0; b < BCH; ++b) {
                    const uint8_t* xb = lds + (size_t)b * 2 * plane_stride + col0;
                    xr4[b] = *reinterpret_cast<const uint4*>(xb);
                    xi4[b] = *reinterpret_cast<const uint4*>(xb + plane_stride);
                }
#pragma unroll
                for (int p = 0; p < PMAX; ++p) {
                    if (p >= P) continue;
                    const uint32_t w = (u == 0) ? cw[p].x : (u == 1) ? cw[p].y : (u == 2) ? cw[p].z : cw[p].w;
                    uint32_t re[4], im[4];
                    ternary_bytes(w, re, im);
#pragma unroll
                    for (int b = 0; b < BCH; ++b) {
                        const uint32_t xr[4] = {xr4[b].x, xr4[b].y, xr4[b].z, xr4[b].w};
                        const uint32_t xi[4] = {xi4[b].x, xi4[b].y, xi4[b].z, xi4[b].w};
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            A[p][0][b] = __builtin_amdgcn_sdot4((int)re[s], (int)xr[s], A[p][0][b], false);
                            A[p][1][b] = __builtin_amdgcn_sdot4((int)im[s], (int)xi[s], A[p][1][b], false);
                            A[p][2][b] = __builtin_amdgcn_sdot4((int)re[s], (int)xi[s], A[p][2][b], false);
                            A[p][3][b] = __builtin_amdgcn_sdot4((int)im[s], (int)xr[s], A[p][3][b], false);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int b = 0; b < BCH; ++b) {
            float yr = 0.f, yi = 0.f;
#pragma unroll
            for (int p = 0; p < PMAX; ++p) {
                if (p >= P) continue;
                int t[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) t[q] = group_sum_i<TROW>(A[p][q][b]);
                if (lr == 0 && row_ok && b < nb) {
                    if (a.acc) {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            a.acc[(((int64_t)p * 4 + q) * a.B + (b0 + b)) * a.n + row] = t[q];
                    }
                    const float s_re = a.scales[2 * p], s_im = a.scales[2 * p + 1];
                    const float f1 = (float)t[0], f2 = (float)t[1], f3 = (float)t[2], f4 = (float)t[3];
                    if (p < a.S) {
                        yr += s_re * f1 - s_im * f2;
                        yi += s_re * f3 + s_im * f4;
                    } else {
                        yr += s_re * f1 + s_im * f2;
                        yi += s_im * f4 - s_re * f3;
                    }
                }
            }
            if (lr == 0 && row_ok && b < nb) {
                a.y_re[(int64_t)(b0 + b) * a.ldy + row] = yr;
                a.y_im[(int64_t)(b0 + b) * a.ldy + row] = yi;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------
constexpr size_t kLdsBudget = 64 * 1024;

size_t lds_per_col(int32_t xdtype, int m64)
{
    return (size_t)m64 * 2 * (xdtype == FAIRY_F32 ? 4 : xdtype == FAIRY_BF16 ? 2 : 1);
}

template <int XT, int PMAX, int TROW>
hipError_t launch_float_t(const GemvArgs& a, int bch, hipStream_t s)
{
    const dim3 grid((a.n + (kThreads / TROW) - 1) / (kThreads / TROW));
    const size_t lds = lds_per_col(XT, a.m64) * bch;
    switch (bch) {
    case 8: hipLaunchKernelGGL((k_cgemv_float<XT, PMAX, TROW, 8>), grid, dim3(kThreads), lds, s, a); break;
    case 4: hipLaunchKernelGGL((k_cgemv_float<XT, PMAX, TROW, 4>), grid, dim3(kThreads), lds, s, a); break;
    default: hipLaunchKernelGGL((k_cgemv_float<XT, PMAX, TROW, 1>), grid, dim3(kThreads), lds, s, a); break;
    }
    return hipGetLastError();
}

template <int PMAX, int TROW>
hipError_t launch_i8_t(const GemvArgs& a, int bch, hipStream_t s)
{
    const dim3 grid((a.n + (kThreads / TROW) - 1) / (kThreads / TROW));
    const size_t lds = lds_per_col(FAIRY_I8, a.m64) * bch;
    if (bch >= 4 && PMAX <= 4)
        hipLaunchKernelGGL((k_cgemv_i8<PMAX, TROW, 4>), grid, dim3(kThreads), lds, s, a);
    else
        hipLaunchKernelGGL((k_cgemv_i8<PMAX, TROW, 1>), grid, dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

template <int XT, int TROW>
hipError_t launch_by_p(const GemvArgs& a, int bch, hipStream_t s)
{
    if constexpr (XT == FAIRY_I8) {
        if (a.P <= 2) return launch_i8_t<2, TROW>(a, bch, s);
        if (a.P <= 4) return launch_i8_t<4, TROW>(a, bch, s);
        if (a.P <= 8) return launch_i8_t<8, TROW>(a, bch, s);
        return launch_i8_t<16, TROW>(a, bch, s);
    } else {
        if (a.P <= 2) return launch_float_t<XT, 2, TROW>(a, bch, s);
        if (a.P <= 4) return launch_float_t<XT, 4, TROW>(a, bch, s);
        if (a.P <= 8) return launch_float_t<XT, 8, TROW>(a, bch, s);
        return launch_float_t<XT, 16, TROW>(a, bch, s);
    }
}

template <int XT>
hipError_t launch_by_trow(const GemvArgs& a, int bch, hipStream_t s)
{
    if (a.G >= 24) return launch_by_p<XT, 32>(a, bch, s);
    return launch_by_p<XT, 8>(a, bch, s);
}

}  // namespace

hipError_t launch_cgemv(const LayerArgs& L, const void* x_re, const void* x_im, int32_t xdtype, int64_t batch,
                        int64_t ldx, float* y_re, float* y_im, int64_t ldy, int32_t* acc, hipStream_t s)
{
    GemvArgs a;
    a.packed = L.packed;
    a.scales = L.scales;
    a.x_re = x_re;
    a.x_im = x_im;
    a.y_re = y_re;
    a.y_im = y_im;
    a.acc = acc;
    a.ldx = ldx;
    a.ldy = ldy;
    a.n = (int32_t)L.n;
    a.m = (int32_t)L.m;
    a.G = (int32_t)((L.m + 63) / 64);
    a.m64 = 64 * a.G;
    a.S = L.stages;
    a.P = L.planes;
    a.B = (int32_t)batch;

    // batch columns per LDS chunk: as many as fit the budget (8, 4 or 1)
    const size_t per = lds_per_col(xdtype, a.m64);
    int bch = batch >= 8 ? 8 : batch >= 2 ? 4 : 1;
    if (xdtype == FAIRY_I8 && bch > 4) bch = 4;
    while (bch > 1 && per * bch > kLdsBudget) bch = (bch == 8) ? 4 : 1;
    if (per * bch > kLdsBudget) return hipErrorInvalidValue;  // m too large for v1 staging

    switch (xdtype) {
    case FAIRY_BF16: return launch_by_trow<FAIRY_BF16>(a, bch, s);
    case FAIRY_F32: return launch_by_trow<FAIRY_F32>(a, bch, s);
    default: return launch_by_trow<FAIRY_I8>(a, bch, s);
    }
}

}  // namespace fairy
