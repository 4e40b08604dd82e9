// Implicit-GEMM family: config checks, prepared-filter sizing and dispatch.
// The kernel itself is documented in igemm_impl.h.
#include "igemm_impl.h"

namespace cfwd {

// Configs 0 .. kNumCfgs-1: the tiled kernel of igemm_impl.h; the next
// lowc_num_configs(): the gather form for few input channels (k_lowc.hip);
// the next kNumSplitCfgs: the tiled kernel with a split reduction
// (k_igemm_i8_split.hip), whose partial tiles live in the scratch; the next
// kNumResCfgs: the tiled kernel with the resident input (k_igemm_i8_res.hip);
// the next stream_num_configs(): the persistent single-chunk int8 kernel
// (k_igemm_i8_stream.hip).
namespace {
int split_first() { return ig::kNumCfgs + lowc_num_configs(); }
int res_first() { return split_first() + ig::kNumSplitCfgs; }
bool is_lowc(int cfg) { return cfg >= ig::kNumCfgs && cfg < split_first(); }
bool is_split(int cfg) { return cfg >= split_first() && cfg < res_first(); }
bool is_res(int cfg) { return cfg >= res_first() && cfg < res_first() + ig::kNumResCfgs; }
int stream_first() { return res_first() + ig::kNumResCfgs; }
bool is_stream(int cfg) { return cfg >= stream_first() && cfg < stream_first() + stream_num_configs(); }
// The prepared-filter geometry of a streaming config: its tiled filter
// config's output-channel tiles, one channel chunk.
bool stream_filter_geo(const Prob& p, int cfg, int* fcfg, ig::Geo* g, std::string* why) {
    if (!stream_supported(p, cfg - stream_first(), why)) return false;
    *fcfg = stream_filter_config(cfg - stream_first());
    const ig::Cfg c = ig::kCfgs[*fcfg];
    g->ntk = (p.kg + c.nt() - 1) / c.nt();
    g->nchunks = 1;
    return true;
}
// base tile config of a tiled, split or resident config
int base_of(int cfg) {
    if (is_split(cfg)) return ig::kSplitCfgs[cfg - split_first()].base;
    if (is_res(cfg)) return ig::kResCfgs[cfg - res_first()];
    return cfg;
}
// the tiles of a config (a split config has its base config's)
bool geometry_of(const Prob& p, int cfg, ig::Geo* g, std::string* why) {
    if (is_res(cfg)) return ig::res_geometry(p, cfg - res_first(), g, why);
    return ig::geometry(p, ig::kCfgs[base_of(cfg)], g, why);
}
}  // namespace

int igemm_num_configs() { return stream_first() + stream_num_configs(); }

bool igemm_supported(const Prob& p, int cfg, std::string* why) {
    if (is_lowc(cfg)) return lowc_supported(p, cfg - ig::kNumCfgs, why);
    ig::Geo g;
    if (is_split(cfg)) {
        int cps;
        return ig::split_geometry(p, cfg - split_first(), &g, &cps, why);
    }
    if (is_res(cfg)) return ig::res_geometry(p, cfg - res_first(), &g, why);
    if (is_stream(cfg)) return stream_supported(p, cfg - stream_first(), why);
    if (cfg < 0 || cfg >= ig::kNumCfgs) {
        if (why) *why = "implicit GEMM: no such config";
        return false;
    }
    return ig::geometry(p, ig::kCfgs[cfg], &g, why);
}

size_t igemm_filter_bytes(const Prob& p, int cfg) {
    if (is_lowc(cfg)) return lowc_filter_bytes(p, cfg - ig::kNumCfgs);
    ig::Geo g;
    if (is_stream(cfg)) {
        int fc;
        return stream_filter_geo(p, cfg, &fc, &g, nullptr) ? ig::filter_bytes(p, ig::kCfgs[fc], g) : 0;
    }
    if (!geometry_of(p, cfg, &g, nullptr)) return 0;
    return ig::filter_bytes(p, ig::kCfgs[base_of(cfg)], g);
}

size_t igemm_scratch_bytes(const Prob& p, int cfg) {
    return is_split(cfg) ? ig::split_scratch_bytes(p, cfg - split_first()) : 0;
}

cfwd_status igemm_prepare(const Prob& p, int cfg, const void* w, void* wp, hipStream_t st) {
    if (is_lowc(cfg)) return lowc_prepare(p, cfg - ig::kNumCfgs, w, wp, st);
    // split and resident configs read their base config's prepared filter
    // (its layout depends only on the output-channel tile and the chunks),
    // streaming configs their filter config's
    ig::Geo g;
    std::string why;
    if (is_stream(cfg)) {
        int fc;
        if (!stream_filter_geo(p, cfg, &fc, &g, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
        return igemm_prepare_i8(fc, p, g, w, wp, st);
    }
    if (!geometry_of(p, cfg, &g, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    cfg = base_of(cfg);
    switch (p.dtype) {
        case CFWD_F32: return igemm_prepare_f32(cfg, p, g, w, wp, st);
        case CFWD_BF16: return igemm_prepare_bf16(cfg, p, g, w, wp, st);
        default: return igemm_prepare_i8(cfg, p, g, w, wp, st);
    }
}

cfwd_status igemm_launch(const Prob& p, int cfg, const void* x, const void* wp, const float* scale, void* y,
                         void* scratch, const Epi& e, hipStream_t st) {
    if (is_lowc(cfg)) return lowc_launch(p, cfg - ig::kNumCfgs, x, wp, scale, y, e, st);
    ig::Geo g;
    std::string why;
    if (is_split(cfg)) {
        int cps;
        if (!ig::split_geometry(p, cfg - split_first(), &g, &cps, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
        if (scratch == nullptr) return set_error(CFWD_ERR_WORKSPACE, "implicit GEMM split reduction needs scratch");
        return igemm_launch_i8_split(cfg - split_first(), p, g, cps, x, wp, scale, y, scratch, e, st);
    }
    if (is_res(cfg)) {
        if (!ig::res_geometry(p, cfg - res_first(), &g, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
        return igemm_launch_i8_res(cfg - res_first(), p, g, x, wp, scale, y, e, st);
    }
    if (is_stream(cfg)) return stream_launch(p, cfg - stream_first(), x, wp, scale, y, e, st);
    if (!ig::geometry(p, ig::kCfgs[cfg], &g, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    // the fused epilogue has instantiations of its own (no registers of it
    // in the plain kernels)
    const bool epi = e.bias || e.res || e.relu;
    switch (p.dtype) {
        case CFWD_F32:
            return epi ? igemm_launch_f32_epi(cfg, p, g, x, wp, scale, y, e, st)
                       : igemm_launch_f32(cfg, p, g, x, wp, scale, y, e, st);
        case CFWD_BF16:
            return epi ? igemm_launch_bf16_epi(cfg, p, g, x, wp, scale, y, e, st)
                       : igemm_launch_bf16(cfg, p, g, x, wp, scale, y, e, st);
        default:
            return epi ? igemm_launch_i8_epi(cfg, p, g, x, wp, scale, y, e, st)
                       : igemm_launch_i8(cfg, p, g, x, wp, scale, y, e, st);
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
