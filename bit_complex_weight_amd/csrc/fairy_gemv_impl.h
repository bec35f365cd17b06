// fairy_gemv_impl.h -- kernels of the decode-time complex GEMV (internal).
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
// Work mapping (wave64).  A row's packed data in TILED64 is G*P contiguous
// 16-byte units (group g of 64 columns, plane p).  TROW consecutive lanes
// own a row; lane l takes units l, l+TROW, ... so every load instruction of
// a wave reads consecutive 16-byte units (fully coalesced, 1 KiB per wave
// when TROW = 64).  The lane's first units are loaded before the block stages
// the activations into LDS, so HBM latency overlaps the staging.  Per unit a
// lane decodes 64 codes with bit operations (decode_bf16_pair), multiplies
// nothing, accumulates A1..A4 with v_dot2_f32_bf16 (bf16) or fp32 FMAs on the
// +-2 / 0 decoded values (fp32), and folds the plane's scales in once.  Row
// partial sums are combined across the TROW lanes with DPP / row-swap
// butterflies: deterministic, no atomics.
//
// When the plane count P divides 64 and a row has at least 64 units, a wave
// owns a row and lane l always sees plane l % P (units l + 64k): its scales
// are per-lane constants, its four sums run over the whole row and are
// scaled once before the cross-lane sum, and no index needs a division.
// Those blocks have 8 waves (8 rows), so one staging of the activations
// serves 8 rows.
#pragma once

#include "fairy_internal.h"

namespace fairy {
namespace gemv {

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
    // optional rotary position encoding of the outputs (pos == nullptr: none)
    const int32_t* pos;
    int32_t rope_d;
    double rope_log2_base;
};

// Several layers that read the same activations, in one launch (the q, k and
// v projections of an attention layer, or gate and up of an MLP: [Fairy2i
// article §2.2, item 1] each projection matrix gets its own widely-linear
// form, all of them applied to the same input).  Blocks [start[l],
// start[l+1]) of the grid belong to layer l; the layers share m, stages and
// the conjugate branch, and keep their own rows, words, scales and outputs.
constexpr int kMaxGroup = 8;
struct GroupTable {
    int32_t count;
    int32_t start[kMaxGroup + 1];
    const uint32_t* packed[kMaxGroup];
    const float* scales[kMaxGroup];
    float* y_re[kMaxGroup];
    float* y_im[kMaxGroup];
    int64_t ldy[kMaxGroup];
    int32_t n[kMaxGroup];
};

// The layer of block `blk` (uniform; at most kMaxGroup - 1 comparisons):
// its view of the arguments and the block number inside it.
__device__ __forceinline__ int group_resolve(const GroupTable& gt, GemvArgs& a, int blk)
{
    int l = 0;
#pragma unroll
    for (int i = 1; i < kMaxGroup; ++i) l += (i < gt.count && blk >= gt.start[i]) ? 1 : 0;
    a.packed = gt.packed[l];
    a.scales = gt.scales[l];
    a.y_re = gt.y_re[l];
    a.y_im = gt.y_im[l];
    a.ldy = gt.ldy[l];
    a.n = gt.n[l];
    return blk - gt.start[l];
}

// Complex rotary position encoding of an output [iFairy press article §三;
// iFairy talk §2.1.3: on the complex plane the rotation is one complex
// multiplication]: complex dimension j = row % rope_d of batch column (or
// token) b is multiplied by exp(i pos[b] theta_j), theta_j = base^(-j/rope_d).
// Angles and the rotation are evaluated in fp64: in fp32, pos * theta would
// already be off by ~1e-4 rad at positions in the thousands.
__device__ __forceinline__ void rope_apply(const GemvArgs& a, int64_t row, int64_t b, float& vr, float& vi)
{
    if (!a.pos) return;
    const int64_t j = row % a.rope_d;
    const double theta = exp2(-((double)j / (double)a.rope_d) * a.rope_log2_base);
    const double ang = (double)a.pos[b] * theta;
    double sn, cs;
    sincos(ang, &sn, &cs);
    const double xr = vr, xi = vi;
    vr = (float)(xr * cs - xi * sn);
    vi = (float)(xr * sn + xi * cs);
}

constexpr int kThreads = 256;
constexpr int kScaleBytes = 128;  // LDS prefix holding up to 16 planes x 2 half-scales

// Staged activations are stored per 64-column group with 16 bytes of padding
// after each group: lanes of a wave read different groups, and without the
// pad all groups would start on the same LDS banks (group stride a multiple
// of 128 B), serialising every 128-bit read.
__host__ __device__ inline int x_esize(int xdtype) { return xdtype == FAIRY_F32 ? 4 : xdtype == FAIRY_BF16 ? 2 : 1; }
__host__ __device__ inline int x_group_bytes(int xdtype) { return 64 * x_esize(xdtype) + 16; }
__host__ __device__ inline int x_plane_bytes(int xdtype, int m64) { return (m64 / 64) * x_group_bytes(xdtype); }
// bytes of LDS one staged batch column occupies (re + im planes)
__host__ __device__ inline int x_bytes_per_col(int xdtype, int m64) { return 2 * x_plane_bytes(xdtype, m64); }
// byte offset of column c inside a staged plane
__device__ __forceinline__ int x_col_off(int xdtype, int c)
{
    return (c >> 6) * x_group_bytes(xdtype) + (c & 63) * x_esize(xdtype);
}

// 16 zero bytes: what a load that is not needed reads instead of its address
static __device__ uint4 g_zero_unit;

// ---------------------------------------------------------------------------
// Activation staging into LDS.  Per batch column b of the chunk:
//   bf16: re plane [m64] then im plane [m64] (uint16)
//   f32 : re [m64], im [m64] (float)
//   i8  : re [m64], im [m64] bytes; inside every 16-column word the bytes are
//         reordered to the four dot4 groups (see i8_group_col).
// Columns >= m are zero.
// ---------------------------------------------------------------------------
// int8 staging: the 16 bytes of a 16-column word reordered to the four dot4
// groups (byte b of register s holds column i8_group_col(s, b))
__device__ __forceinline__ uint4 i8_reorder(uint4 v)
{
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
    return make_uint4(out[0], out[1], out[2], out[3]);
}

template <int XT>
__device__ __forceinline__ void stage_x(const GemvArgs& a, int b0, int nb, uint8_t* lds)
{
    constexpr int per_elems = (XT == FAIRY_BF16) ? 8 : (XT == FAIRY_F32) ? 4 : 16;  // elements per 16 B
    constexpr int esize = 16 / per_elems;
    const int per = a.m64 / per_elems;
    const int pbytes = x_plane_bytes(XT, a.m64);
    for (int idx = threadIdx.x; idx < nb * 2 * per; idx += blockDim.x) {
        const int b = idx / (2 * per);
        const int rem = idx - b * 2 * per;
        const int plane = rem / per;
        const int c = (rem - plane * per) * per_elems;
        uint4* dst = reinterpret_cast<uint4*>(lds + (size_t)(2 * b + plane) * pbytes + x_col_off(XT, c));
        const uint8_t* src = reinterpret_cast<const uint8_t*>(plane ? a.x_im : a.x_re) +
                             ((int64_t)(b0 + b) * a.ldx + c) * esize;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (c < a.m) v = *reinterpret_cast<const uint4*>(src);
        if constexpr (XT == FAIRY_I8) v = i8_reorder(v);
        *dst = v;
    }
}

// ---------------------------------------------------------------------------
// Float paths (bf16 / fp32 activations), one 16-byte unit (64 codes of one
// plane) at a time.
// ---------------------------------------------------------------------------
template <int XT, int BCH>
__device__ __forceinline__ void unit_accumulate(const uint4 cw, int col0, const uint8_t* xs, int col_bytes,
                                                int plane_bytes, int nb, float (&A)[4][BCH])
{
    const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const uint32_t w = words[u];
        const int c0 = col0 + 16 * u;
        if constexpr (XT == FAIRY_BF16) {
            uint32_t re2[8], im2[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) decode_bf16_pair(w, k, re2[k], im2[k]);
#pragma unroll
            for (int b = 0; b < BCH; ++b) {
                if (b >= nb) continue;
                const uint8_t* xb = xs + (size_t)b * col_bytes + x_col_off(FAIRY_BF16, c0);
                const uint4 r0 = *reinterpret_cast<const uint4*>(xb);
                const uint4 r1 = *reinterpret_cast<const uint4*>(xb + 16);
                const uint4 i0 = *reinterpret_cast<const uint4*>(xb + plane_bytes);
                const uint4 i1 = *reinterpret_cast<const uint4*>(xb + plane_bytes + 16);
                const uint32_t xr[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
                const uint32_t xi[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    A[0][b] = dot2_bf16(re2[k], xr[k], A[0][b]);
                    A[2][b] = dot2_bf16(re2[k], xi[k], A[2][b]);
                    A[1][b] = dot2_bf16(im2[k], xi[k], A[1][b]);
                    A[3][b] = dot2_bf16(im2[k], xr[k], A[3][b]);
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
                const float* xr = reinterpret_cast<const float*>(xs + (size_t)b * col_bytes + x_col_off(FAIRY_F32, c0));
                const float* xi = reinterpret_cast<const float*>(xs + (size_t)b * col_bytes + plane_bytes +
                                                                 x_col_off(FAIRY_F32, c0));
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const float vr = xr[t], vi = xi[t];
                    A[0][b] = fmaf(re[t], vr, A[0][b]);
                    A[2][b] = fmaf(re[t], vi, A[2][b]);
                    A[1][b] = fmaf(im[t], vi, A[1][b]);
                    A[3][b] = fmaf(im[t], vr, A[3][b]);
                }
            }
        }
    }
}

template <int XT, int TROW, int BCH, int UB>
__global__ __launch_bounds__(kThreads) void k_cgemv_units(GemvArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    float* s_hs = reinterpret_cast<float*>(lds);        // [P][2] half-scales (decoded weights are +-2)
    uint8_t* xs = lds + kScaleBytes;
    const int lr = threadIdx.x % TROW;
    const int row = blockIdx.x * (kThreads / TROW) + threadIdx.x / TROW;
    const bool row_ok = row < a.n;
    const int P = a.P;
    const int units = a.G * P;
    const int nmine = (row_ok && lr < units) ? (units - lr + TROW - 1) / TROW : 0;
    const uint4* wrow = reinterpret_cast<const uint4*>(a.packed) + (int64_t)(row_ok ? row : 0) * units;
    // unit j = lr + k*TROW -> (group, plane), advanced without divisions
    const int dq = TROW / P, dr = TROW - dq * P;
    const int g_first = lr / P, p_first = lr - g_first * P;

    // issue the first batch of weight loads before anything else
    uint4 cw[UB];
#pragma unroll
    for (int k = 0; k < UB; ++k) cw[k] = (k < nmine) ? wrow[lr + k * TROW] : make_uint4(0, 0, 0, 0);

    if (threadIdx.x < 2 * P) s_hs[threadIdx.x] = 0.5f * a.scales[threadIdx.x];
    const int col_bytes = x_bytes_per_col(XT, a.m64);
    const int plane_bytes = col_bytes / 2;

    // blockIdx.y picks the first chunk of BCH batch columns; chunks run side
    // by side on the grid (a block loops only if the grid has fewer chunks)
    bool first = true;
    for (int b0 = blockIdx.y * BCH; b0 < a.B; b0 += gridDim.y * BCH) {
        const int nb = (a.B - b0 < BCH) ? a.B - b0 : BCH;
        if (!first) {
            __syncthreads();
#pragma unroll
            for (int k = 0; k < UB; ++k) cw[k] = (k < nmine) ? wrow[lr + k * TROW] : make_uint4(0, 0, 0, 0);
        }
        first = false;
        stage_x<XT>(a, b0, nb, xs);
        __syncthreads();

        float yr[BCH], yi[BCH];
#pragma unroll
        for (int b = 0; b < BCH; ++b) { yr[b] = 0.f; yi[b] = 0.f; }

        int g = g_first, p = p_first;
        for (int kb = 0; kb < nmine; kb += UB) {
            if (kb) {
#pragma unroll
                for (int k = 0; k < UB; ++k)
                    cw[k] = (kb + k < nmine) ? wrow[lr + (kb + k) * TROW] : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int k = 0; k < UB; ++k) {
                if (kb + k < nmine) {
                    float A[4][BCH];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int b = 0; b < BCH; ++b) A[q][b] = 0.f;
                    unit_accumulate<XT, BCH>(cw[k], 64 * g, xs, col_bytes, plane_bytes, nb, A);
                    const float hr = s_hs[2 * p], hi = s_hs[2 * p + 1];
                    const float sg = (p < a.S) ? 1.0f : -1.0f;  // W planes multiply conj(x)
#pragma unroll
                    for (int b = 0; b < BCH; ++b) {
                        yr[b] += hr * A[0][b] - sg * (hi * A[1][b]);
                        yi[b] += sg * (hr * A[2][b]) + hi * A[3][b];
                    }
                }
                g += dq;
                p += dr;
                if (p >= P) { p -= P; ++g; }
            }
        }
#pragma unroll
        for (int b = 0; b < BCH; ++b) {
            float sr = group_sum<TROW>(yr[b]);
            float si = group_sum<TROW>(yi[b]);
            if (lr == 0 && row_ok && b < nb) {
                rope_apply(a, row, b0 + b, sr, si);
                a.y_re[(int64_t)(b0 + b) * a.ldy + row] = sr;
                a.y_im[(int64_t)(b0 + b) * a.ldy + row] = si;
            }
        }
    }
}


// ---------------------------------------------------------------------------
// Float paths, rows of >= 64 units: one row per wave.  The first
// NL = (64/P)*P lanes are active (all 64 when P divides 64; 60 for P = 6),
// lane l owns plane l % P and groups l/P + k*(64/P), so each step of the wave
// reads NL consecutive units.
// ---------------------------------------------------------------------------
constexpr int kThreadsLp = 512;

// blockIdx.y picks a chunk of BCH batch columns, so the chunks of a batch
// run side by side (each re-reads the codes, from L2 after the first).
template <int XT, int P, int BCH>
__device__ __forceinline__ void lp_body(const GemvArgs& a, int blk)
{
    static_assert(P >= 1 && P <= 64, "plane count");
    constexpr int GS = 64 / P;  // groups one step of the wave covers
    constexpr int NL = GS * P;  // active lanes
    constexpr int esize = (XT == FAIRY_BF16) ? 2 : 4;
    constexpr int per_elems = 16 / esize;
    extern __shared__ __align__(16) uint8_t lds[];
    const int lane = threadIdx.x & 63;
    const int row = blk * (kThreadsLp / 64) + (threadIdx.x >> 6);
    const bool row_ok = row < a.n;
    const int p = lane % P, gl = lane / P;
    // an idle lane must accumulate nothing (a zero code word decodes to +1)
    const bool active = NL == 64 || lane < NL;
    const int G = a.G;
    const int b0 = blockIdx.y * BCH;
    const int nb = (a.B - b0 < BCH) ? a.B - b0 : BCH;
    // unit (g, p) of the row is at g*P + p = lane + NL*k for g = gl + GS*k.
    // Every load below is unconditional: one that is not needed reads 16
    // zero bytes instead (a load under a branch makes the compiler wait for
    // it inside the branch, before anything else can run).
    const uint4* wl = reinterpret_cast<const uint4*>(a.packed) + ((int64_t)(row_ok ? row : 0) * G * P + lane);
    const uint4* zero = &g_zero_unit;
    const int pbytes = x_plane_bytes(XT, a.m64);
    const int col_bytes = 2 * pbytes;
    auto x_src = [&](int b, int pl, int c) -> const uint4* {
        return (b < nb && c < a.m) ? reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(pl ? a.x_im : a.x_re) +
                                                                    ((int64_t)(b0 + b) * a.ldx + c) * esize)
                                   : zero;
    };
    auto x_dst = [&](int b, int pl, int c) {
        return reinterpret_cast<uint4*>(lds + (size_t)b * col_bytes + pl * pbytes + x_col_off(XT, c));
    };
    // The first activation columns are loaded first, then the code words,
    // then the activations are stored: the stores wait for the activations
    // (from L2) while the code words (from HBM) are still in flight.  The
    // stores are unconditional too (one that is not needed goes to a spare
    // 16-byte slot past the staged columns), so the compiler has no branch
    // to sink the activation loads into.
    const int c0 = threadIdx.x * per_elems;
    uint4* spare = reinterpret_cast<uint4*>(lds + (size_t)BCH * col_bytes);
    // (one vector value, not an array: an array live across the scheduling
    // barrier is kept in scratch memory)
    typedef uint32_t xvec_t __attribute__((ext_vector_type(8 * BCH)));
    xvec_t xv;
#pragma unroll
    for (int i = 0; i < 2 * BCH; ++i) {
        const uint4 v = *x_src(i >> 1, i & 1, c0);
        xv[4 * i] = v.x;
        xv[4 * i + 1] = v.y;
        xv[4 * i + 2] = v.z;
        xv[4 * i + 3] = v.w;
    }
    __builtin_amdgcn_sched_barrier(0);  // the code-word loads after these
    uint4 cur[2], nxt[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) cur[u] = *((row_ok && active && gl + u * GS < G) ? wl + NL * u : zero);
#pragma unroll
    for (int i = 0; i < 2 * BCH; ++i)
        *((c0 < a.m64 && (i >> 1) < nb) ? x_dst(i >> 1, i & 1, c0) : spare) =
            make_uint4(xv[4 * i], xv[4 * i + 1], xv[4 * i + 2], xv[4 * i + 3]);
    // rows longer than one pass of the block: one piece at a time, the
    // store unconditional like the first pass's (an array of pieces behind
    // a per-column branch was kept in scratch memory)
    for (int c = c0 + kThreadsLp * per_elems; c < a.m64; c += kThreadsLp * per_elems) {
#pragma unroll
        for (int i = 0; i < 2 * BCH; ++i) {
            const uint4 v = *x_src(i >> 1, i & 1, c);
            *(((i >> 1) < nb) ? x_dst(i >> 1, i & 1, c) : spare) = v;
        }
    }
    // decoded weights are +-2: half-scales; W planes multiply conj(x)
    const float hr = 0.5f * a.scales[2 * p], hi = 0.5f * a.scales[2 * p + 1];
    const float sg = (p < a.S) ? 1.0f : -1.0f;
    __syncthreads();

    float A[4][BCH];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int b = 0; b < BCH; ++b) A[q][b] = 0.f;
    for (int g0 = gl; g0 < G; g0 += 2 * GS) {
        // the next two units are in flight while these two are summed
        const int gn = g0 + 2 * GS;
#pragma unroll
        for (int u = 0; u < 2; ++u)
            nxt[u] = *((row_ok && active && gn + u * GS < G) ? wl + (int64_t)(gn - gl) * P + NL * u : zero);
        __builtin_amdgcn_sched_barrier(0);  // issued before these units' sums, not next to their use
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int g = g0 + u * GS;
            if (active && g < G) unit_accumulate<XT, BCH>(cur[u], 64 * g, lds, col_bytes, pbytes, nb, A);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) cur[u] = nxt[u];
    }
#pragma unroll
    for (int b = 0; b < BCH; ++b) {
        float vr = group_sum<64>(hr * A[0][b] - sg * (hi * A[1][b]));
        float vi = group_sum<64>(sg * (hr * A[2][b]) + hi * A[3][b]);
        if (lane == 0 && row_ok && b < nb) {
            rope_apply(a, row, b0 + b, vr, vi);
            a.y_re[(int64_t)(b0 + b) * a.ldy + row] = vr;
            a.y_im[(int64_t)(b0 + b) * a.ldy + row] = vi;
        }
    }
}

template <int XT, int P, int BCH>
__global__ __launch_bounds__(kThreadsLp) void k_cgemv_lp(GemvArgs a)
{
    lp_body<XT, P, BCH>(a, blockIdx.x);
}

template <int XT, int P, int BCH>
__global__ __launch_bounds__(kThreadsLp) void k_cgemv_lp_group(GemvArgs a, GroupTable gt)
{
    const int blk = group_resolve(gt, a, blockIdx.x);
    lp_body<XT, P, BCH>(a, blk);
}

// ---------------------------------------------------------------------------
// int8 path: exact int32 accumulators per plane, reduced across lanes, then
// the float epilogue from the exact sums.  A lane owns whole 64-column groups
// (all planes), so its per-plane sums stay in registers.
// v_perm tables (pool bytes 0..3 from the second operand, 4..7 from the first;
// selector 8 replicates bit 15, 9 bit 31, 12 gives 0x00, 13.. give 0xFF):
//   codes at byte bits 1:0 -> selector c:    ReB pool 01 00 FF 00, ImB pool 00 01 00 FF
//   codes at byte bits 3:2 -> selector 4c:   ReB: c=0 byte0=01, c=1 byte4=00,
//                                            c=2 sign(bit15)=FF, c=3 -> 00
//                           selector 4c|1:   ImB: c=0 byte1=00, c=1 byte5=01,
//                                            c=2 sign(bit31)=00, c=3 -> FF
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
    uint8_t* xs = lds + kScaleBytes;
    const int rows_pb = kThreads / TROW;
    const int lr = threadIdx.x % TROW;
    const int row = blockIdx.x * rows_pb + threadIdx.x / TROW;
    const bool row_ok = row < a.n;
    const int P = a.P;
    const uint4* wrow = reinterpret_cast<const uint4*>(a.packed) + (int64_t)(row_ok ? row : 0) * a.G * P;
    const int plane_bytes = x_plane_bytes(FAIRY_I8, a.m64);

    for (int b0 = 0; b0 < a.B; b0 += BCH) {
        const int nb = (a.B - b0 < BCH) ? a.B - b0 : BCH;
        if (b0) __syncthreads();
        stage_x<FAIRY_I8>(a, b0, nb, xs);
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
                    const uint8_t* xb = xs + (size_t)b * 2 * plane_bytes + x_col_off(FAIRY_I8, col0);
                    xr4[b] = *reinterpret_cast<const uint4*>(xb);
                    xi4[b] = *reinterpret_cast<const uint4*>(xb + plane_bytes);
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
                rope_apply(a, row, b0 + b, yr, yi);
                a.y_re[(int64_t)(b0 + b) * a.ldy + row] = yr;
                a.y_im[(int64_t)(b0 + b) * a.ldy + row] = yi;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host-side launch helpers (instantiated per activation type in its own
// translation unit so the kernels compile in parallel)
// ---------------------------------------------------------------------------
int pick_trow(int units);
int pick_bch(int xdtype, int B, int m64);

template <int XT, int TROW, int BCH>
hipError_t launch_units_t(const GemvArgs& a, hipStream_t s)
{
    // batch chunks on grid.y, at most 65535 (the kernel loops over the rest:
    // the token rows of the VALU prefill path take this launcher too)
    const int64_t chunks = ((int64_t)a.B + BCH - 1) / BCH;
    const dim3 grid((a.n + (kThreads / TROW) - 1) / (kThreads / TROW), (unsigned)(chunks < 65535 ? chunks : 65535));
    const size_t lds = kScaleBytes + (size_t)x_bytes_per_col(XT, a.m64) * BCH;
    hipLaunchKernelGGL((k_cgemv_units<XT, TROW, BCH, 2>), grid, dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

template <int XT, int TROW>
hipError_t launch_units_bch(const GemvArgs& a, int bch, hipStream_t s)
{
    switch (bch) {
    case 8: return launch_units_t<XT, TROW, 8>(a, s);
    case 4: return launch_units_t<XT, TROW, 4>(a, s);
    case 2: return launch_units_t<XT, TROW, 2>(a, s);
    default: return launch_units_t<XT, TROW, 1>(a, s);
    }
}

template <int XT, int P, int BCH>
hipError_t launch_lp_t(const GemvArgs& a, hipStream_t s)
{
    const dim3 grid((a.n + (kThreadsLp / 64) - 1) / (kThreadsLp / 64), (a.B + BCH - 1) / BCH);
    const size_t lds = (size_t)x_bytes_per_col(XT, a.m64) * BCH + 16;  // + the spare slot
    hipLaunchKernelGGL((k_cgemv_lp<XT, P, BCH>), grid, dim3(kThreadsLp), lds, s, a);
    return hipGetLastError();
}

template <int XT, int P>
hipError_t launch_lp_bch(const GemvArgs& a, int bch, hipStream_t s)
{
    switch (bch) {
    case 4: return launch_lp_t<XT, P, 4>(a, s);
    case 2: return launch_lp_t<XT, P, 2>(a, s);
    default: return launch_lp_t<XT, P, 1>(a, s);
    }
}

// grouped launch: gt.start[gt.count] blocks along x
template <int XT, int P, int BCH>
hipError_t launch_lp_group_t(const GemvArgs& a, const GroupTable& gt, hipStream_t s)
{
    const dim3 grid(gt.start[gt.count], (a.B + BCH - 1) / BCH);
    const size_t lds = (size_t)x_bytes_per_col(XT, a.m64) * BCH + 16;  // + the spare slot
    hipLaunchKernelGGL((k_cgemv_lp_group<XT, P, BCH>), grid, dim3(kThreadsLp), lds, s, a, gt);
    return hipGetLastError();
}

template <int XT, int P>
hipError_t launch_lp_group_bch(const GemvArgs& a, const GroupTable& gt, int bch, hipStream_t s)
{
    switch (bch) {
    case 4: return launch_lp_group_t<XT, P, 4>(a, gt, s);
    case 2: return launch_lp_group_t<XT, P, 2>(a, gt, s);
    default: return launch_lp_group_t<XT, P, 1>(a, gt, s);
    }
}

// Batch columns per block of the one-row-per-wave kernel: wide enough to
// share each decoded word among a few columns, narrow enough that a small
// layer still has several waves per SIMD (the chunks run side by side).
int pick_bch_lp(int xdtype, int B, int m64);

template <int XT>
hipError_t launch_float(const GemvArgs& a, hipStream_t s)
{
    const int bch = pick_bch(XT, a.B, a.m64);
    if (a.G * a.P >= 64 && a.B <= 64) {
        const int bl = pick_bch_lp(XT, a.B, a.m64);
        switch (a.P) {
        case 1: return launch_lp_bch<XT, 1>(a, bl, s);
        case 2: return launch_lp_bch<XT, 2>(a, bl, s);
        case 3: return launch_lp_bch<XT, 3>(a, bl, s);
        case 4: return launch_lp_bch<XT, 4>(a, bl, s);
        case 6: return launch_lp_bch<XT, 6>(a, bl, s);
        case 8: return launch_lp_bch<XT, 8>(a, bl, s);
        case 16: return launch_lp_bch<XT, 16>(a, bl, s);
        default: break;
        }
    }
    switch (pick_trow(a.G * a.P)) {
    case 64: return launch_units_bch<XT, 64>(a, bch, s);
    case 32: return launch_units_bch<XT, 32>(a, bch, s);
    case 16: return launch_units_bch<XT, 16>(a, bch, s);
    default: return launch_units_bch<XT, 8>(a, bch, s);
    }
}

// One launch over the layers of gt (the one-row-per-wave kernels; P in
// {1, 2, 3, 4, 6, 8, 16} and rows of >= 64 units): hipErrorNotSupported for
// any other shape, which the caller then runs layer by layer.
template <int XT>
hipError_t launch_float_group(const GemvArgs& a, const GroupTable& gt, hipStream_t s)
{
    if (!(a.G * a.P >= 64 && a.B <= 64)) return hipErrorNotSupported;
    const int bl = pick_bch_lp(XT, a.B, a.m64);
    switch (a.P) {
    case 1: return launch_lp_group_bch<XT, 1>(a, gt, bl, s);
    case 2: return launch_lp_group_bch<XT, 2>(a, gt, bl, s);
    case 3: return launch_lp_group_bch<XT, 3>(a, gt, bl, s);
    case 4: return launch_lp_group_bch<XT, 4>(a, gt, bl, s);
    case 6: return launch_lp_group_bch<XT, 6>(a, gt, bl, s);
    case 8: return launch_lp_group_bch<XT, 8>(a, gt, bl, s);
    case 16: return launch_lp_group_bch<XT, 16>(a, gt, bl, s);
    default: return hipErrorNotSupported;
    }
}

hipError_t launch_bf16(const GemvArgs& a, hipStream_t s);
hipError_t launch_f32(const GemvArgs& a, hipStream_t s);
hipError_t launch_i8(const GemvArgs& a, hipStream_t s);
hipError_t launch_bf16_group(const GemvArgs& a, const GroupTable& gt, hipStream_t s);
hipError_t launch_f32_group(const GemvArgs& a, const GroupTable& gt, hipStream_t s);
hipError_t launch_i8_group(const GemvArgs& a, const GroupTable& gt, hipStream_t s);

GemvArgs make_args(const LayerArgs& L, const void* x_re, const void* x_im, int64_t batch, int64_t ldx,
                   float* y_re, float* y_im, int64_t ldy, int32_t* acc);

}  // namespace gemv

// vector-ALU prefill with lanes as tokens (fairy_gemm_valu.hip); a.B is the
// token count.  Supported for bf16 and int8 (m <= 65536) activations and
// P in {1, 2, 3, 4, 6, 8, 16}.
bool cgemm_valu_tokens_supported(int32_t xdtype, int64_t m, int32_t planes);
hipError_t launch_cgemm_valu(const gemv::GemvArgs& a, int32_t xdtype, hipStream_t s);

// matrix-core prefill (fairy_gemm_mfma.hip); a.B is the token count.
// workspace (nullable): fp32 partial sums for the split-K launch, of
// cgemm_mfma_workspace_bytes() bytes (0: no split for this shape).
hipError_t launch_cgemm_mfma(const gemv::GemvArgs& a, int32_t xdtype, void* workspace, hipStream_t s);
size_t cgemm_mfma_workspace_bytes(int64_t n, int64_t m, int64_t M, int32_t P, int32_t xdtype);
}  // namespace fairy
