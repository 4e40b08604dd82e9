// Implicit-GEMM instantiations for one dtype (float) with the fused epilogue
// (bias, residual, ReLU) compiled in; the kernel is in igemm_impl.h.  Kept
// apart from the plain instantiations so those carry none of its registers.
#include "igemm_impl.h"

namespace cfwd {

cfwd_status igemm_launch_f32_epi(int cfg, const Prob& p, const ig::Geo& g, const void* x, const void* wp,
                               const float* scale, void* y, const Epi& e, hipStream_t st) {
    return ig::launch_dtype<float, true>(cfg, p, g, x, wp, scale, y, e, st);
}

}  // namespace cfwd
