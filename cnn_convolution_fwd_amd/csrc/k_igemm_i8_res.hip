// Implicit GEMM with the resident input, int8 NCHW4 (configs after the
// split reduction; see kResCfgs and the kernel's RES main loop in
// igemm_impl.h).  Plain and fused-epilogue instantiations.
#include "igemm_impl.h"

namespace cfwd {

namespace {

template <bool EPI>
cfwd_status launch_res(int base, const Prob& p, const ig::Geo& g, const void* x, const void* wp, const float* scale,
                       void* y, const Epi& e, hipStream_t st) {
    using namespace ig;
    switch (base) {
#define CFWD_IG_RES(ID)                                                                                            \
    case ID: {                                                                                                     \
        constexpr Cfg c = kCfgs[ID];                                                                               \
        if (p.r * p.s == 9)                                                                                        \
            return launch_one<int8_t, 4, c.wm, c.wn, c.fm, c.fn, 0, c.fr, 9, false, EPI, true>(p, g, x, wp, scale, y, \
                                                                                            e, st);                \
        return launch_one<int8_t, 4, c.wm, c.wn, c.fm, c.fn, 0, c.fr, 1, false, EPI, true>(p, g, x, wp, scale, y, e, \
                                                                                        st);                       \
    }
        CFWD_IG_RES(2)
        CFWD_IG_RES(3)
        CFWD_IG_RES(6)
        CFWD_IG_RES(11)
        CFWD_IG_RES(12)
        CFWD_IG_RES(13)
        CFWD_IG_RES(14)
        CFWD_IG_RES(16)
#undef CFWD_IG_RES
        default:
            return set_error(CFWD_ERR_UNSUPPORTED, "implicit GEMM resident input: no such base config");
    }
}

}  // namespace

cfwd_status igemm_launch_i8_res(int rc, const Prob& p, const ig::Geo& g, const void* x, const void* wp,
                                const float* scale, void* y, const Epi& e, hipStream_t st) {
    const int base = ig::kResCfgs[rc];
    if (e.bias || e.res || e.relu) return launch_res<true>(base, p, g, x, wp, scale, y, e, st);
    return launch_res<false>(base, p, g, x, wp, scale, y, e, st);
}

}  // namespace cfwd
