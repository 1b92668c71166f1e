// Expert kernels instantiated for the MXFP4 weight format (E2M1 codes, one E8M0 scale per 32) (see k_expert.inc).
#include "k_expert.inc"

namespace moe {
namespace expert_detail {
template hipError_t launch_up_fmt<MOE_FMT_MXFP4>(const PoolView &, const Items &, int, const uint16_t *,
                                         uint16_t *, const uint16_t *, float *, hipStream_t);
template hipError_t launch_down_to_d_fmt<MOE_FMT_MXFP4>(const PoolView &, const Items &, int,
                                                const uint16_t *, float *, const float *,
                                                hipStream_t);
template hipError_t launch_down_fused_fmt<MOE_FMT_MXFP4>(const PoolView &, const int32_t *, const float *,
                                                 int, int, const uint16_t *, const float *,
                                                 const float *, const int32_t *, uint16_t *,
                                                 hipStream_t);
}  // namespace expert_detail
}  // namespace moe
