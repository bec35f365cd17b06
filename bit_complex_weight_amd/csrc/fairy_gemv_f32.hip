// fairy_gemv_f32.hip -- fp32-activation GEMV kernels (fp32 FMA on +-2 / 0).
#include "fairy_gemv_impl.h"

namespace fairy {
namespace gemv {
hipError_t launch_f32(const GemvArgs& a, hipStream_t s) { return launch_float<FAIRY_F32>(a, s); }
hipError_t launch_f32_group(const GemvArgs& a, const GroupTable& gt, hipStream_t s)
{
    return launch_float_group<FAIRY_F32>(a, gt, s);
}
}  // namespace gemv
}  // namespace fairy
