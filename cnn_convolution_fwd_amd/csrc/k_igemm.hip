// Implicit-GEMM family: config checks, prepared-filter sizing and dispatch.
// The kernel itself is documented in igemm_impl.h.
#include "igemm_impl.h"

namespace cfwd {

// Configs 0 .. kNumCfgs-1: the tiled kernel of igemm_impl.h; the next
// lowc_num_configs(): the gather form for few input channels (k_lowc.hip).
int igemm_num_configs() { return ig::kNumCfgs + lowc_num_configs(); }

bool igemm_supported(const Prob& p, int cfg, std::string* why) {
    if (cfg >= ig::kNumCfgs && cfg < igemm_num_configs()) return lowc_supported(p, cfg - ig::kNumCfgs, why);
    if (cfg < 0 || cfg >= ig::kNumCfgs) {
        if (why) *why = "implicit GEMM: no such config";
        return false;
    }
    ig::Geo g;
    return ig::geometry(p, ig::kCfgs[cfg], &g, why);
}

size_t igemm_filter_bytes(const Prob& p, int cfg) {
    if (cfg >= ig::kNumCfgs) return lowc_filter_bytes(p, cfg - ig::kNumCfgs);
    ig::Geo g;
    if (!ig::geometry(p, ig::kCfgs[cfg], &g, nullptr)) return 0;
    return ig::filter_bytes(p, ig::kCfgs[cfg], g);
}

cfwd_status igemm_prepare(const Prob& p, int cfg, const void* w, void* wp, hipStream_t st) {
    if (cfg >= ig::kNumCfgs) return lowc_prepare(p, cfg - ig::kNumCfgs, w, wp, st);
    ig::Geo g;
    std::string why;
    if (!ig::geometry(p, ig::kCfgs[cfg], &g, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    switch (p.dtype) {
        case CFWD_F32: return igemm_prepare_f32(cfg, p, g, w, wp, st);
        case CFWD_BF16: return igemm_prepare_bf16(cfg, p, g, w, wp, st);
        default: return igemm_prepare_i8(cfg, p, g, w, wp, st);
    }
}

cfwd_status igemm_launch(const Prob& p, int cfg, const void* x, const void* wp, const float* scale, void* y,
                         hipStream_t st) {
    if (cfg >= ig::kNumCfgs) return lowc_launch(p, cfg - ig::kNumCfgs, x, wp, scale, y, st);
    ig::Geo g;
    std::string why;
    if (!ig::geometry(p, ig::kCfgs[cfg], &g, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    switch (p.dtype) {
        case CFWD_F32: return igemm_launch_f32(cfg, p, g, x, wp, scale, y, st);
        case CFWD_BF16: return igemm_launch_bf16(cfg, p, g, x, wp, scale, y, st);
        default: return igemm_launch_i8(cfg, p, g, x, wp, scale, y, st);
    }
}

// Preference without measurement: the config whose tiles waste the least
// work (pixels and channels past the problem's edges), ties to the larger
// tile (fewer re-reads of the weights and the patch halo).
int igemm_default_config(const Prob& p) {
    // image stems (a handful of input channels): the gather form
    if (p.cg <= 4 && lowc_supported(p, 0, nullptr)) return ig::kNumCfgs + (p.k > 32 ? 4 : 3);
    int best = -1;
    double best_score = -1.0;
    for (int c = 0; c < ig::kNumCfgs; ++c) {
        ig::Geo g;
        if (!ig::geometry(p, ig::kCfgs[c], &g, nullptr)) continue;
        const double pix_used = static_cast<double>(p.n) * p.oh * p.ow;
        const double pix_run = static_cast<double>(g.tiles_n * g.TN) * g.tiles_h * g.TH * g.tiles_w * g.TW;
        const double frag_pix = static_cast<double>(g.tiles_n) * g.tiles_h * g.tiles_w * ig::kCfgs[c].pixels();
        const double ch_used = p.kg;
        const double ch_run = static_cast<double>(g.ntk) * ig::kCfgs[c].nt();
        const double eff = (pix_used / std::max(pix_run, frag_pix)) * (ch_used / ch_run);
        const double size = static_cast<double>(ig::kCfgs[c].pixels()) * ig::kCfgs[c].nt();
        const double score = eff * 1e6 + size * 1e-3;
        if (score > best_score) {
            best_score = score;
            best = c;
        }
    }
    return best;
}

}  // namespace cfwd
