// fairy_gemv_i8.hip -- int8-activation GEMV kernels (v_perm ternary bytes,
// v_dot4_i32_i8, exact int32 accumulators).
#include "fairy_gemv_impl.h"

namespace fairy {
namespace gemv {
namespace {

// ---------------------------------------------------------------------------
// One row per wave for rows of >= 64 units and a power-of-two plane count:
// lane l owns plane l % P and groups l/P + k*(64/P), as on the float path.
// A lane's four int32 sums cover its own plane, so a butterfly over the
// lanes of the same plane (xor distances P..32) gives each of them that
// plane's exact totals (the raw accumulators), and a second one over the
// distances below P adds the scaled planes in float.
// ---------------------------------------------------------------------------
// Distances 4 and 8 inside a 16-lane row are DPP row rotations (lane i
// adds lane i - 4, then i - 8, modulo the row): each lane then holds the sum
// of its residue class, added in a lane-dependent order, which is exact for
// integers.
__device__ __forceinline__ int dpp_ror4(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_ror8(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false); }

template <int P>
__device__ __forceinline__ int plane_total(int v)
{
    if (P <= 1) v += dpp_xor1(v);
    if (P <= 2) v += dpp_xor2(v);
    if (P <= 4) v += dpp_ror4(v);
    if (P <= 8) v += dpp_ror8(v);
    if (P <= 16) v = swap16_add(v);
    if (P <= 32) v = swap32_add(v);
    return v;
}

template <int BCH>
__device__ __forceinline__ void unit_i8(const uint4 cw, int g, const uint8_t* xs, int pbytes, int (&A)[4][BCH])
{
    const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        uint32_t re[4], im[4];
        ternary_bytes(words[u], re, im);
        const int off = x_col_off(FAIRY_I8, 64 * g + 16 * u);
#pragma unroll
        for (int b = 0; b < BCH; ++b) {
            const uint8_t* xb = xs + (size_t)b * 2 * pbytes + off;
            const uint4 xr4 = *reinterpret_cast<const uint4*>(xb);
            const uint4 xi4 = *reinterpret_cast<const uint4*>(xb + pbytes);
            const uint32_t xr[4] = {xr4.x, xr4.y, xr4.z, xr4.w};
            const uint32_t xi[4] = {xi4.x, xi4.y, xi4.z, xi4.w};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                A[0][b] = __builtin_amdgcn_sdot4((int)re[s], (int)xr[s], A[0][b], false);
                A[1][b] = __builtin_amdgcn_sdot4((int)im[s], (int)xi[s], A[1][b], false);
                A[2][b] = __builtin_amdgcn_sdot4((int)re[s], (int)xi[s], A[2][b], false);
                A[3][b] = __builtin_amdgcn_sdot4((int)im[s], (int)xr[s], A[3][b], false);
            }
        }
    }
}

// 4 rows (waves) per block: against 8, 2048^2 S=2 at B = 1 took 4.19 us
// instead of 4.35-4.41 (A/B on one machine); the bf16/fp32 kernel measured the
// same either way and keeps 8
constexpr int kThreadsLpI8 = 256;

template <int P, int BCH>
__device__ __forceinline__ void lp_i8_body(const GemvArgs& a, int blk)
{
    static_assert(P >= 1 && P <= 16 && (P & (P - 1)) == 0, "power-of-two plane count");
    constexpr int GS = 64 / P;  // groups one step of the wave covers
    extern __shared__ __align__(16) uint8_t lds[];
    const int lane = threadIdx.x & 63;
    const int row = blk * (kThreadsLpI8 / 64) + (threadIdx.x >> 6);
    const bool row_ok = row < a.n;
    const int p = lane % P, gl = lane / P;
    const int G = a.G;
    const int b0 = blockIdx.y * BCH;
    const int nb = (a.B - b0 < BCH) ? a.B - b0 : BCH;
    // unit (g, p) of the row is at g*P + p = lane + 64k for g = gl + GS*k.
    // Every load is unconditional: one that is not needed reads 16 zero
    // bytes (a load under a branch makes the compiler wait for it inside the
    // branch), and a store that is not needed goes to a spare LDS slot.
    const uint4* wl = reinterpret_cast<const uint4*>(a.packed) + ((int64_t)(row_ok ? row : 0) * G * P + lane);
    const uint4* zero = &g_zero_unit;
    const int pbytes = x_plane_bytes(FAIRY_I8, a.m64);
    uint4* spare = reinterpret_cast<uint4*>(lds + (size_t)BCH * 2 * pbytes);
    // staged activations: 16-byte pieces, per batch column re then im
    const int per = a.m64 / 16;
    const int pieces = nb * 2 * per;
    auto piece = [&](int idx, const uint4*& src, uint4*& dst) {
        const int b = idx / (2 * per);
        const int rem = idx - b * 2 * per;
        const int plane = rem / per;
        const int c = (rem - plane * per) * 16;
        const bool on = idx < pieces;
        src = (on && c < a.m) ? reinterpret_cast<const uint4*>(reinterpret_cast<const int8_t*>(plane ? a.x_im : a.x_re) +
                                                               (int64_t)(b0 + b) * a.ldx + c)
                              : zero;
        dst = on ? reinterpret_cast<uint4*>(lds + (size_t)(2 * b + plane) * pbytes + x_col_off(FAIRY_I8, c)) : spare;
    };
    // The first activation pieces are loaded, then the code words, then the
    // pieces are stored: the stores wait for the activations (from L2) while
    // the code words (from HBM) are still in flight.
    const uint4* src0;
    uint4* dst0;
    piece(threadIdx.x, src0, dst0);
    const uint4 x0 = *src0;
    __builtin_amdgcn_sched_barrier(0);
    uint4 cur[2], nxt[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) cur[u] = *((row_ok && gl + u * GS < G) ? wl + 64 * u : zero);
    *dst0 = i8_reorder(x0);
    for (int idx = threadIdx.x + kThreadsLpI8; idx < pieces; idx += kThreadsLpI8) {
        const uint4* src;
        uint4* dst;
        piece(idx, src, dst);
        *dst = i8_reorder(*src);
    }
    __syncthreads();

    int A[4][BCH];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int b = 0; b < BCH; ++b) A[q][b] = 0;
    for (int g0 = gl; g0 < G; g0 += 2 * GS) {
        // the next two units are in flight while these two are summed
        const int gn = g0 + 2 * GS;
#pragma unroll
        for (int u = 0; u < 2; ++u) nxt[u] = *((row_ok && gn + u * GS < G) ? wl + (int64_t)(gn - gl) * P + 64 * u : zero);
        __builtin_amdgcn_sched_barrier(0);  // issued before these units' sums, not next to their use
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int g = g0 + u * GS;
            if (g < G) unit_i8<BCH>(cur[u], g, lds, pbytes, A);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) cur[u] = nxt[u];
    }
    const float s_re = a.scales[2 * p], s_im = a.scales[2 * p + 1];
    const float sg = (p < a.S) ? 1.0f : -1.0f;  // W planes multiply conj(x)
#pragma unroll
    for (int b = 0; b < BCH; ++b) {
        int t[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) t[q] = plane_total<P>(A[q][b]);
        if (a.acc && row_ok && b < nb && lane < P) {
#pragma unroll
            for (int q = 0; q < 4; ++q) a.acc[(((int64_t)p * 4 + q) * a.B + (b0 + b)) * a.n + row] = t[q];
        }
        float vr = s_re * (float)t[0] - sg * (s_im * (float)t[1]);
        float vi = sg * (s_re * (float)t[2]) + s_im * (float)t[3];
        if constexpr (P > 1) {
            vr = group_sum<P>(vr);
            vi = group_sum<P>(vi);
        }
        if (lane == 0 && row_ok && b < nb) {
            rope_apply(a, row, b0 + b, vr, vi);
            a.y_re[(int64_t)(b0 + b) * a.ldy + row] = vr;
            a.y_im[(int64_t)(b0 + b) * a.ldy + row] = vi;
        }
    }
}

template <int P, int BCH>
__global__ __launch_bounds__(kThreadsLpI8) void k_cgemv_lp_i8(GemvArgs a)
{
    lp_i8_body<P, BCH>(a, blockIdx.x);
}

template <int P, int BCH>
__global__ __launch_bounds__(kThreadsLpI8) void k_cgemv_lp_i8_group(GemvArgs a, GroupTable gt)
{
    const int blk = group_resolve(gt, a, blockIdx.x);
    lp_i8_body<P, BCH>(a, blk);
}

template <int P, int BCH>
hipError_t launch_lp_i8_group_t(const GemvArgs& a, const GroupTable& gt, hipStream_t s)
{
    const dim3 grid(gt.start[gt.count], (a.B + BCH - 1) / BCH);
    const size_t lds = (size_t)x_bytes_per_col(FAIRY_I8, a.m64) * BCH + 16;  // + the spare slot
    hipLaunchKernelGGL((k_cgemv_lp_i8_group<P, BCH>), grid, dim3(kThreadsLpI8), lds, s, a, gt);
    return hipGetLastError();
}

template <int P>
hipError_t launch_lp_i8_group(const GemvArgs& a, const GroupTable& gt, hipStream_t s)
{
    switch (pick_bch_lp(FAIRY_I8, a.B, a.m64)) {
    case 4: return launch_lp_i8_group_t<P, 4>(a, gt, s);
    case 2: return launch_lp_i8_group_t<P, 2>(a, gt, s);
    default: return launch_lp_i8_group_t<P, 1>(a, gt, s);
    }
}

template <int P, int BCH>
hipError_t launch_lp_i8_t(const GemvArgs& a, hipStream_t s)
{
    const dim3 grid((a.n + (kThreadsLpI8 / 64) - 1) / (kThreadsLpI8 / 64), (a.B + BCH - 1) / BCH);
    const size_t lds = (size_t)x_bytes_per_col(FAIRY_I8, a.m64) * BCH + 16;  // + the spare slot
    hipLaunchKernelGGL((k_cgemv_lp_i8<P, BCH>), grid, dim3(kThreadsLpI8), lds, s, a);
    return hipGetLastError();
}

template <int P>
hipError_t launch_lp_i8(const GemvArgs& a, hipStream_t s)
{
    switch (pick_bch_lp(FAIRY_I8, a.B, a.m64)) {
    case 4: return launch_lp_i8_t<P, 4>(a, s);
    case 2: return launch_lp_i8_t<P, 2>(a, s);
    default: return launch_lp_i8_t<P, 1>(a, s);
    }
}

template <int PMAX, int TROW>
hipError_t launch_i8_t(const GemvArgs& a, int bch, hipStream_t s)
{
    const dim3 grid((a.n + (kThreads / TROW) - 1) / (kThreads / TROW));
    const size_t lds = kScaleBytes + (size_t)x_bytes_per_col(FAIRY_I8, a.m64) * bch;
    if (bch >= 4 && PMAX <= 4)
        hipLaunchKernelGGL((k_cgemv_i8<PMAX, TROW, 4>), grid, dim3(kThreads), lds, s, a);
    else
        hipLaunchKernelGGL((k_cgemv_i8<PMAX, TROW, 1>), grid, dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

template <int TROW>
hipError_t launch_i8_p(const GemvArgs& a, int bch, hipStream_t s)
{
    if (a.P <= 2) return launch_i8_t<2, TROW>(a, bch, s);
    if (a.P <= 4) return launch_i8_t<4, TROW>(a, bch, s);
    if (a.P <= 8) return launch_i8_t<8, TROW>(a, bch, s);
    return launch_i8_t<16, TROW>(a, bch, s);
}

}  // namespace

// grouped launch (no raw accumulators): power-of-two P on rows of >= 64 units
hipError_t launch_i8_group(const GemvArgs& a, const GroupTable& gt, hipStream_t s)
{
    if (!(a.G * a.P >= 64 && a.B <= 64) || a.acc) return hipErrorNotSupported;
    switch (a.P) {
    case 1: return launch_lp_i8_group<1>(a, gt, s);
    case 2: return launch_lp_i8_group<2>(a, gt, s);
    case 4: return launch_lp_i8_group<4>(a, gt, s);
    case 8: return launch_lp_i8_group<8>(a, gt, s);
    case 16: return launch_lp_i8_group<16>(a, gt, s);
    default: return hipErrorNotSupported;
    }
}

hipError_t launch_i8(const GemvArgs& a, hipStream_t s)
{
    if (a.G * a.P >= 64 && a.B <= 64) {
        switch (a.P) {
        case 1: return launch_lp_i8<1>(a, s);
        case 2: return launch_lp_i8<2>(a, s);
        case 4: return launch_lp_i8<4>(a, s);
        case 8: return launch_lp_i8<8>(a, s);
        case 16: return launch_lp_i8<16>(a, s);
        default: break;
        }
    }
    const int bch = pick_bch(FAIRY_I8, a.B, a.m64);
    if (a.G >= 24) return launch_i8_p<32>(a, bch, s);
    return launch_i8_p<8>(a, bch, s);
}

}  // namespace gemv
}  // namespace fairy
