// FP8 (OCP E4M3FN) variant of the packed mixed-mask attention forward.
#include "kernel_common.h"

namespace pva {

int launch_fwd_fp8(const void*, const void*, const void*, const float*, const float*, const float*,
                   const int32_t*, const pva_seg_desc*, float, void*, hipStream_t) {
  return PVA_ERR_UNSUPPORTED;
}

}  // namespace pva
