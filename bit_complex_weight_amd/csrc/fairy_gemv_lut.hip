// fairy_gemv_lut.hip -- table-lookup complex GEMV (batch 1), the LUT inference
// of the iFairy talk (§2.3.2: the results of the 16 input combinations of a
// pair of codes are precomputed), kept beside the direct bit decode of
// fairy_gemv as a measured alternative.
//
// Tables.  Nibble i (bits 4i..4i+3) of a TILED64 word holds two columns of
// the same parity: bits 4i..4i+1 column t_lo = (i < 4 ? 14 - 4i : 31 - 4i),
// bits 4i+2..4i+3 column t_lo - 2.  For the activation vector x, plane p
// (scales s_re, s_im; sigma = +1 for U planes, -1 for W planes, which multiply
// conj(x) [Fairy2i article §2.1]) and a column t, the code c in {0,1,2,3}
// (codeword i^c [Fairy2i article §3.1]) contributes to (y_re, y_im)
//   c = 0: ( s_re x_re[t],        sigma s_re x_im[t])      c = 2: minus c = 0
//   c = 1: (-sigma s_im x_im[t],  s_im x_re[t])            c = 3: minus c = 1
// so the table of a nibble has 16 entries, entry v = c_lo | c_hi << 2 being
// the sum of both columns' contributions: the plane scales are folded in,
// and per pair of codes the kernel does one 8-byte LDS read and two fp32
// adds.  A table is 128 bytes, stored with a 16-byte pad (144-byte stride)
// so that the builders (one thread per table, writing 16 bytes at a time)
// hit distinct banks; all lanes of a wave read the same table at a time.
//
// Work split.  A block owns 64*W rows (lane = row) and a contiguous chunk of
// JB 16-byte units of every row (unit j of a row = group j / P, plane j % P);
// it builds the JB*32 tables of its chunk and sweeps the chunk's units.  The
// address of an entry is one v_perm that isolates the byte holding nibble*8
// (the word is shifted and masked once per 8 nibbles); the table's own
// offset is an immediate of the LDS read, the table array being static.
// Chunk sums go to a workspace and a second kernel adds the chunks in a
// fixed order (one chunk: written to y directly).
//
// Lane = row is what lets a wave share one table per read, but it leaves
// only n/64 waves per column chunk, so a decode-size layer must be split
// into many chunks and pays the second launch; the direct decode (a wave per
// row, lanes across the columns) needs neither.
#include "fairy_gemv_impl.h"

namespace fairy {
namespace lut {

constexpr int kTableStride = 144;                        // 128 B of entries + 16 B pad
constexpr int kUnitTables = 32;                          // 4 words x 8 nibbles per unit
constexpr int kUnitBytes = kUnitTables * kTableStride;   // 4608 B, a multiple of 256

struct LutArgs {
    const uint4* units;  // TILED64 packed words as 16-byte units
    const float* scales;
    const void* x_re;
    const void* x_im;
    float* out_re;  // y (one chunk) or the chunk partials [chunk][n]
    float* out_im;
    int64_t n;
    int32_t m, P, S, JB, UR;  // UR = 16-byte units per row (groups x planes)
};

template <int XT>
__device__ __forceinline__ float load_x(const void* base, int c)
{
    if constexpr (XT == FAIRY_BF16)
        return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[c] << 16);
    else
        return reinterpret_cast<const float*>(base)[c];
}

// 16 zero bytes: what a load that is not needed reads instead
static __device__ uint4 g_lut_zero;

// Inputs of table k of the block (unit j of the row, word u, nibble i): the
// activations at the pair's two columns and the unit's plane scales.  Every
// load is unconditional (a column past m reads zero bytes), so none of them
// sits in a branch for the compiler to wait inside.
struct TableIn {
    float xr_lo, xi_lo, xr_hi, xi_hi, s_re, s_im;
};
template <int XT>
__device__ __forceinline__ TableIn table_inputs(const LutArgs& a, int j, int k)
{
    const int u = (k >> 3) & 3, i = k & 7;
    const int g = j / a.P, p = j - g * a.P;
    const int t_lo = (i < 4) ? 14 - 4 * i : 31 - 4 * i;
    const int c_lo = 64 * g + 16 * u + t_lo, c_hi = c_lo - 2;
    const void* zero = &g_lut_zero;
    const bool on_lo = c_lo < a.m, on_hi = c_hi < a.m;
    TableIn t;
    t.xr_lo = load_x<XT>(on_lo ? a.x_re : zero, on_lo ? c_lo : 0);
    t.xi_lo = load_x<XT>(on_lo ? a.x_im : zero, on_lo ? c_lo : 0);
    t.xr_hi = load_x<XT>(on_hi ? a.x_re : zero, on_hi ? c_hi : 0);
    t.xi_hi = load_x<XT>(on_hi ? a.x_im : zero, on_hi ? c_hi : 0);
    t.s_re = a.scales[2 * p];
    t.s_im = a.scales[2 * p + 1];
    return t;
}

// Table k from its inputs: the 16 sums of the pair's two codes.
__device__ __forceinline__ void table_write(const LutArgs& a, int j, int k, const TableIn& t, uint8_t* lds)
{
    const int p = j % a.P;
    const float sg = (p < a.S) ? 1.0f : -1.0f;
    // contributions of codes 0 and 1 (codes 2, 3 are their negatives)
    const float2 f_lo[2] = {make_float2(t.s_re * t.xr_lo, sg * (t.s_re * t.xi_lo)),
                            make_float2(-sg * (t.s_im * t.xi_lo), t.s_im * t.xr_lo)};
    const float2 f_hi[2] = {make_float2(t.s_re * t.xr_hi, sg * (t.s_re * t.xi_hi)),
                            make_float2(-sg * (t.s_im * t.xi_hi), t.s_im * t.xr_hi)};
    float4* dst = reinterpret_cast<float4*>(lds + (size_t)k * kTableStride);
#pragma unroll
    for (int q = 0; q < 8; ++q) {  // entries 2q, 2q+1: c_hi = q >> 1, c_lo = 2(q & 1) + {0, 1}
        const float hs = (q & 4) ? -1.0f : 1.0f;
        const float2 h = f_hi[(q >> 1) & 1];
        const float ls = (q & 1) ? -1.0f : 1.0f;
        dst[q] = make_float4(hs * h.x + ls * f_lo[0].x, hs * h.y + ls * f_lo[0].y, hs * h.x + ls * f_lo[1].x,
                             hs * h.y + ls * f_lo[1].y);
    }
}

__device__ __forceinline__ uint4 load_unit(const uint4* p) { return *p; }

template <int XT, int W, int JB>
__global__ __launch_bounds__(64 * W) void k_cgemv_lut(LutArgs a)
{
    // static size: the table base is a compile-time 0 and every table
    // offset folds into the ds_read immediate
    __shared__ __align__(16) uint8_t lds[JB * kUnitBytes];
    const int j0 = blockIdx.y * JB;
    const int nj = min(JB, a.UR - j0);
    const int64_t row = (int64_t)blockIdx.x * (64 * W) + threadIdx.x;
    const bool live = row < a.n;
    const uint4* src = a.units + row * a.UR + j0;

    // The first tables' inputs are loaded first, then the lane's units, so
    // the tables are built (waiting for their inputs from L2) while the
    // units come from HBM.  A thread without a first table loads table 0's
    // inputs and writes nothing.
    const int k0 = threadIdx.x;
    const bool first = k0 < nj * kUnitTables;
    const TableIn t0 = table_inputs<XT>(a, j0 + (first ? k0 : 0) / kUnitTables, first ? k0 : 0);
    __builtin_amdgcn_sched_barrier(0);
    const uint4* zero = &g_lut_zero;
    uint4 w4[JB];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) w4[jj] = *((live && jj < nj) ? src + jj : zero);
    if (first) table_write(a, j0 + k0 / kUnitTables, k0, t0, lds);
    for (int k = k0 + 64 * W; k < nj * kUnitTables; k += 64 * W) {
        const int j = j0 + k / kUnitTables;
        table_write(a, j, k, table_inputs<XT>(a, j, k), lds);
    }
    __syncthreads();
    if (!live) return;

    float ar[4] = {0.0f, 0.0f, 0.0f, 0.0f}, ai[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
        if (jj >= nj) break;  // partial last chunk (uniform)
        const uint32_t words[4] = {w4[jj].x, w4[jj].y, w4[jj].z, w4[jj].w};
        // all 32 lookups of the unit are issued before the first add, so
        // their LDS latencies overlap even with one wave per SIMD
        float2 e[32];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            // byte b of ev / od = (nibble 2b / 2b+1) * 8
            const uint32_t ev = (words[u] << 3) & 0x78787878u;
            const uint32_t od = (words[u] >> 1) & 0x78787878u;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t off = __builtin_amdgcn_perm(0u, (i & 1) ? od : ev, 0x0C0C0C00u | (uint32_t)(i >> 1));
                e[u * 8 + i] = *reinterpret_cast<const float2*>(
                    lds + off + (uint32_t)(jj * kUnitBytes + (u * 8 + i) * kTableStride));
            }
        }
#pragma unroll
        for (int q = 0; q < 32; ++q) {
            ar[q & 3] += e[q].x;
            ai[q & 3] += e[q].y;
        }
    }
    const float yr = (ar[0] + ar[1]) + (ar[2] + ar[3]);
    const float yi = (ai[0] + ai[1]) + (ai[2] + ai[3]);
    const int64_t o = (int64_t)blockIdx.y * a.n + row;
    a.out_re[o] = yr;
    a.out_im[o] = yi;
}

// y[row] = sum of the chunk partials: one thread per row (coalesced across
// the wave), eight independent sums over the chunks c = q (mod 8) so that
// sixteen loads (re and im) are in flight at a time, combined in a fixed
// tree order (the result does not depend on timing).
__global__ __launch_bounds__(256) void k_lut_reduce(const float* part_re, const float* part_im, int chunks,
                                                    int64_t n, float* y_re, float* y_im)
{
    const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (row >= n) return;
    float ar[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    float ai[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    int c = 0;
    for (; c + 8 <= chunks; c += 8)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            ar[q] += part_re[(int64_t)(c + q) * n + row];
            ai[q] += part_im[(int64_t)(c + q) * n + row];
        }
    // tail: loads from a clamped (valid) chunk, issued together, then selected
#pragma unroll
    for (int q = 0; q < 7; ++q) {
        const int64_t o = (int64_t)min(c + q, chunks - 1) * n + row;
        const float vr = part_re[o], vi = part_im[o];
        ar[q] += (c + q < chunks) ? vr : 0.0f;
        ai[q] += (c + q < chunks) ? vi : 0.0f;
    }
    y_re[row] = ((ar[0] + ar[1]) + (ar[2] + ar[3])) + ((ar[4] + ar[5]) + (ar[6] + ar[7]));
    y_im[row] = ((ai[0] + ai[1]) + (ai[2] + ai[3])) + ((ai[4] + ai[5]) + (ai[6] + ai[7]));
}

}  // namespace lut

// Block shape: W waves (64*W rows per block, so 64*W rows share each table)
// and JB 16-byte units per block.  Measured on 2048- to 16384-row layers of
// 2048 and 5504 columns with 4 and 6 planes: four waves and four units per
// block are the best or within noise of it everywhere (more units per block
// leave too few blocks; fewer leave too many partial chunks to add); small
// layers use fewer waves.
LutConfig cgemv_lut_config(const LayerArgs& L)
{
    LutConfig c;
    c.W = 4;
    while (c.W > 1 && 64 * (c.W / 2) >= L.n) c.W /= 2;
    c.JB = 4;
    return c;
}

size_t cgemv_lut_workspace_bytes(const LayerArgs& L, const LutConfig& c)
{
    const int64_t UR = ((L.m + 63) / 64) * (int64_t)L.planes;
    const int64_t chunks = (UR + c.JB - 1) / c.JB;
    return chunks > 1 ? (size_t)(2 * chunks * L.n) * sizeof(float) : 0;
}

hipError_t launch_cgemv_lut(const LayerArgs& L, const LutConfig& c, const void* x_re, const void* x_im,
                            int32_t xdtype, float* y_re, float* y_im, void* workspace, hipStream_t s)
{
    if ((c.JB != 2 && c.JB != 4 && c.JB != 8) || (c.W != 1 && c.W != 2 && c.W != 4 && c.W != 8)) return hipErrorInvalidValue;
    lut::LutArgs a;
    a.units = reinterpret_cast<const uint4*>(L.packed);
    a.scales = L.scales;
    a.x_re = x_re;
    a.x_im = x_im;
    a.n = L.n;
    a.m = (int32_t)L.m;
    a.P = L.planes;
    a.S = L.stages;
    a.JB = c.JB;
    a.UR = (int32_t)((L.m + 63) / 64) * a.P;
    const int64_t chunks = (a.UR + c.JB - 1) / c.JB;
    if (chunks > 65535) return hipErrorInvalidValue;
    float* part = static_cast<float*>(workspace);
    a.out_re = chunks > 1 ? part : y_re;
    a.out_im = chunks > 1 ? part + chunks * a.n : y_im;
    const dim3 grid((unsigned)((a.n + 64 * c.W - 1) / (64 * c.W)), (unsigned)chunks);
#define FAIRY_LUT_LAUNCH(XT, W, JB) hipLaunchKernelGGL((lut::k_cgemv_lut<XT, W, JB>), grid, dim3(64 * W), 0, s, a)
#define FAIRY_LUT_JB(XT, W)                                 \
    do {                                                    \
        if (c.JB == 8) FAIRY_LUT_LAUNCH(XT, W, 8);          \
        else if (c.JB == 4) FAIRY_LUT_LAUNCH(XT, W, 4);     \
        else FAIRY_LUT_LAUNCH(XT, W, 2);                    \
    } while (0)
#define FAIRY_LUT_W(XT)                                     \
    do {                                                    \
        if (c.W == 8) FAIRY_LUT_JB(XT, 8);                  \
        else if (c.W == 4) FAIRY_LUT_JB(XT, 4);             \
        else if (c.W == 2) FAIRY_LUT_JB(XT, 2);             \
        else FAIRY_LUT_JB(XT, 1);                           \
    } while (0)
    if (xdtype == FAIRY_BF16) FAIRY_LUT_W(FAIRY_BF16);
    else FAIRY_LUT_W(FAIRY_F32);
#undef FAIRY_LUT_W
#undef FAIRY_LUT_JB
#undef FAIRY_LUT_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || chunks == 1) return e;
    hipLaunchKernelGGL(lut::k_lut_reduce, dim3((unsigned)((a.n + 255) / 256)), dim3(256), 0, s,
                       (const float*)part, (const float*)(part + chunks * a.n), (int)chunks, a.n, y_re, y_im);
    return hipGetLastError();
}

}  // namespace fairy
