// fairy_gemv_bf16.hip -- bf16-activation GEMV kernels (v_dot2_f32_bf16).
#include "fairy_gemv_impl.h"

namespace fairy {
namespace gemv {
hipError_t launch_bf16(const GemvArgs& a, hipStream_t s) { return launch_float<FAIRY_BF16>(a, s); }
hipError_t launch_bf16_group(const GemvArgs& a, const GroupTable& gt, hipStream_t s)
{
    return launch_float_group<FAIRY_BF16>(a, gt, s);
}
}  // namespace gemv
}  // namespace fairy
