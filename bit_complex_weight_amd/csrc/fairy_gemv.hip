// fairy_gemv.hip -- dispatch of the decode-time complex GEMV (kernels in
// fairy_gemv_impl.h, instantiated per activation type in fairy_gemv_*.hip).
#include "fairy_gemv_impl.h"

namespace fairy {
namespace gemv {

// Lanes per row: a full wave once a row has >= 64 units of 64 codes, else the
// smallest power of two >= 8 covering the row.
int pick_trow(int units)
{
    if (units >= 64) return 64;
    if (units >= 32) return 32;
    if (units >= 16) return 16;
    return 8;
}

// Batch columns staged per pass: up to 8 (int8: 4), within 64 KiB of LDS.
int pick_bch(int xdtype, int B, int m64)
{
    int bch = B <= 1 ? 1 : B == 2 ? 2 : B <= 4 ? 4 : 8;
    if (xdtype == FAIRY_I8 && bch > 4) bch = 4;
    while (bch > 1 && kScaleBytes + (size_t)x_bytes_per_col(xdtype, m64) * bch > 64 * 1024) bch /= 2;
    return bch;
}

int pick_bch_lp(int xdtype, int B, int m64)
{
    int bch = B <= 1 ? 1 : B <= 4 ? 2 : 4;
    while (bch > 1 && (size_t)x_bytes_per_col(xdtype, m64) * bch + 16 > 64 * 1024) bch /= 2;  // + spare slot
    return bch;
}

}  // namespace gemv

namespace gemv {
GemvArgs make_args(const LayerArgs& L, const void* x_re, const void* x_im, int64_t batch, int64_t ldx,
                   float* y_re, float* y_im, int64_t ldy, int32_t* acc)
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
    a.pos = L.rope_pos;
    a.rope_d = L.rope_d;
    a.rope_log2_base = L.rope_log2_base;
    return a;
}
}  // namespace gemv

hipError_t launch_cgemv(const LayerArgs& L, const void* x_re, const void* x_im, int32_t xdtype, int64_t batch,
                        int64_t ldx, float* y_re, float* y_im, int64_t ldy, int32_t* acc, hipStream_t s)
{
    const gemv::GemvArgs a = gemv::make_args(L, x_re, x_im, batch, ldx, y_re, y_im, ldy, acc);
    if (gemv::kScaleBytes + (size_t)gemv::x_bytes_per_col(xdtype, a.m64) > 64 * 1024) return hipErrorInvalidValue;
    switch (xdtype) {
    case FAIRY_BF16: return gemv::launch_bf16(a, s);
    case FAIRY_F32: return gemv::launch_f32(a, s);
    default: return gemv::launch_i8(a, s);
    }
}

hipError_t launch_cgemv_group(const LayerArgs* L, const float* const* y_re, const float* const* y_im,
                              const int64_t* ldy, int32_t count, const void* x_re, const void* x_im, int32_t xdtype,
                              int64_t batch, int64_t ldx, hipStream_t s)
{
    // one launch when the shape takes the one-row-per-wave kernels, else
    // one launch per layer
    gemv::GemvArgs a = gemv::make_args(L[0], x_re, x_im, batch, ldx, const_cast<float*>(y_re[0]),
                                       const_cast<float*>(y_im[0]), ldy[0], nullptr);
    if (gemv::kScaleBytes + (size_t)gemv::x_bytes_per_col(xdtype, a.m64) > 64 * 1024) return hipErrorInvalidValue;
    gemv::GroupTable gt{};
    gt.count = count;
    const int rows_pb = (xdtype == FAIRY_I8) ? 4 : 8;  // waves (rows) per block of the kernels below
    int64_t blocks = 0;
    for (int l = 0; l < count; ++l) {
        gt.start[l] = (int32_t)blocks;
        gt.packed[l] = L[l].packed;
        gt.scales[l] = L[l].scales;
        gt.y_re[l] = const_cast<float*>(y_re[l]);
        gt.y_im[l] = const_cast<float*>(y_im[l]);
        gt.ldy[l] = ldy[l];
        gt.n[l] = (int32_t)L[l].n;
        blocks += (L[l].n + rows_pb - 1) / rows_pb;
    }
    gt.start[count] = (int32_t)blocks;
    hipError_t e = hipErrorNotSupported;
    if (blocks < 0x7FFFFFFF) {
        switch (xdtype) {
        case FAIRY_BF16: e = gemv::launch_bf16_group(a, gt, s); break;
        case FAIRY_F32: e = gemv::launch_f32_group(a, gt, s); break;
        default: e = gemv::launch_i8_group(a, gt, s); break;
        }
    }
    if (e != hipErrorNotSupported) return e;
    for (int l = 0; l < count; ++l) {
        e = launch_cgemv(L[l], x_re, x_im, xdtype, batch, ldx, const_cast<float*>(y_re[l]),
                         const_cast<float*>(y_im[l]), ldy[l], nullptr, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace fairy
