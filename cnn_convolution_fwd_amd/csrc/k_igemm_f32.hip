// Implicit-GEMM instantiations for one dtype (float); the kernel is in igemm_impl.h.
#include "igemm_impl.h"

namespace cfwd {

cfwd_status igemm_launch_f32(int cfg, const Prob& p, const ig::Geo& g, const void* x, const void* wp,
                             const float* scale, void* y, const Epi& e, hipStream_t st) {
    return ig::launch_dtype<float, false>(cfg, p, g, x, wp, scale, y, e, st);
}

cfwd_status igemm_prepare_f32(int cfg, const Prob& p, const ig::Geo& g, const void* w, void* wp, hipStream_t st) {
    return ig::prepare_dtype<float>(cfg, p, g, w, wp, st);
}

}  // namespace cfwd
