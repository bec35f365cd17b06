// fairy_gemv_i8.hip -- int8-activation GEMV kernels (v_perm ternary bytes,
// v_dot4_i32_i8, exact int32 accumulators).
#include "fairy_gemv_impl.h"

namespace fairy {
namespace gemv {
namespace {

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

hipError_t launch_i8(const GemvArgs& a, hipStream_t s)
{
    const int bch = pick_bch(FAIRY_I8, a.B, a.m64);
    if (a.G >= 24) return launch_i8_p<32>(a, bch, s);
    return launch_i8_p<8>(a, bch, s);
}

}  // namespace gemv
}  // namespace fairy
