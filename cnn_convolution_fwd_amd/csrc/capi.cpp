// C ABI of the cfwd library: validation, algorithm resolution, dispatch and
// the Fast-Run selection / execution phases.
//
// Fast-Run (MegEngine inference article, section "Fast-Run" and its
// engineering subsection): a selection phase times every implemented
// algorithm for the target problem on the target device and records the best
// in a map from problem to implementation; the execution phase dispatches
// from that map.  Here the map is keyed by the full descriptor plus the device
// (architecture name, CU count) and this library's kernel set, lives in host
// memory behind a mutex, and can be saved to / merged from a text file.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <map>
#include <mutex>
#include <sstream>
#include <string>
#include <vector>

#include "internal.h"
#include "winograd_i8.h"
#include "bottleneck.h"
#include "nhwc.h"
#include "lowbit.h"
#include "stem_i8.h"

#define CFWD_VERSION "0.1.0"

namespace cfwd {

namespace {
thread_local std::string g_last_error;
}

// Environment, read once: CFWD_LOG (0 silent, 1 failures, 2 + AUTO choices,
// 3 + every call's resolved algorithm), CFWD_FASTRUN_MODE (off: AUTO ignores
// the map; readonly, the default: map, else the fixed preference; search: a
// map miss with a large enough workspace runs the selection),
// CFWD_FASTRUN_CACHE (a map file loaded at the first AUTO call and, in search
// mode, rewritten after each selection).
struct Env {
    int log = 0;
    enum { OFF, READONLY, SEARCH } mode = READONLY;
    std::string cache;
};
const Env& env() {
    static const Env e = [] {
        Env v;
        if (const char* l = std::getenv("CFWD_LOG")) v.log = std::atoi(l);
        if (const char* m = std::getenv("CFWD_FASTRUN_MODE")) {
            if (std::strcmp(m, "off") == 0) v.mode = Env::OFF;
            else if (std::strcmp(m, "search") == 0) v.mode = Env::SEARCH;
        }
        if (const char* c = std::getenv("CFWD_FASTRUN_CACHE")) v.cache = c;
        return v;
    }();
    return e;
}

cfwd_status set_error(cfwd_status st, const std::string& msg) {
    g_last_error = msg;
    if (st != CFWD_OK && env().log >= 1) std::fprintf(stderr, "cfwd: %s\n", msg.c_str());
    return st;
}

cfwd_status check_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return CFWD_OK;
    return set_error(CFWD_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

namespace {

bool esize_of(int dtype, int* es) {
    switch (dtype) {
        case CFWD_F32: *es = 4; return true;
        case CFWD_BF16: *es = 2; return true;
        case CFWD_I8: *es = 1; return true;
        default: return false;
    }
}

int out_size(int in, int k, int stride, int pad, int dil) {
    const long long span = static_cast<long long>(in) + 2LL * pad - static_cast<long long>(dil) * (k - 1) - 1;
    if (span < 0) return 0;
    return static_cast<int>(span / stride) + 1;
}

}  // namespace

cfwd_status make_prob(const cfwd_conv_desc* d, Prob* p, std::string* why) {
    if (d == nullptr) {
        *why = "descriptor is NULL";
        return CFWD_ERR_INVALID_ARG;
    }
    const int pos[] = {d->n, d->c, d->h, d->w, d->k, d->r, d->s, d->stride_h, d->stride_w, d->dil_h, d->dil_w,
                       d->groups};
    const char* names[] = {"n", "c", "h", "w", "k", "r", "s", "stride_h", "stride_w", "dil_h", "dil_w", "groups"};
    for (int i = 0; i < 12; ++i)
        if (pos[i] <= 0) {
            *why = std::string("descriptor field ") + names[i] + " must be >= 1";
            return CFWD_ERR_INVALID_ARG;
        }
    if (d->pad_h < 0 || d->pad_w < 0) {
        *why = "padding must be >= 0";
        return CFWD_ERR_INVALID_ARG;
    }
    if (d->c % d->groups || d->k % d->groups) {
        *why = "C and K must be divisible by groups";
        return CFWD_ERR_INVALID_ARG;
    }
    int es;
    if (!esize_of(d->dtype, &es)) {
        *why = "unknown dtype";
        return CFWD_ERR_INVALID_ARG;
    }
    int xb;
    if (d->layout == CFWD_LAYOUT_NCHW || d->layout == CFWD_LAYOUT_NHWC) {
        xb = 1;  // element counts as NCHW; only the NHWC configs accept NHWC (supported())
    } else if (d->layout == CFWD_LAYOUT_NCHWX) {
        if (d->x != 4 && d->x != 8) {
            *why = "NCHWX block x must be 4 or 8";
            return CFWD_ERR_INVALID_ARG;
        }
        xb = d->x;
    } else {
        *why = "unknown layout";
        return CFWD_ERR_INVALID_ARG;
    }
    const int oh = out_size(d->h, d->r, d->stride_h, d->pad_h, d->dil_h);
    const int ow = out_size(d->w, d->s, d->stride_w, d->pad_w, d->dil_w);
    if (oh <= 0 || ow <= 0) {
        *why = "the dilated kernel does not fit the padded input";
        return CFWD_ERR_INVALID_ARG;
    }
    p->n = d->n; p->c = d->c; p->h = d->h; p->w = d->w; p->k = d->k; p->r = d->r; p->s = d->s;
    p->sh = d->stride_h; p->sw = d->stride_w; p->ph = d->pad_h; p->pw = d->pad_w;
    p->dh = d->dil_h; p->dw = d->dil_w; p->g = d->groups;
    p->oh = oh; p->ow = ow;
    p->cg = d->c / d->groups; p->kg = d->k / d->groups;
    p->layout = d->layout; p->xb = xb; p->dtype = d->dtype; p->esize = es;
    const long long cpad = (static_cast<long long>(d->c) + xb - 1) / xb * xb;
    const long long kpad = (static_cast<long long>(d->k) + xb - 1) / xb * xb;
    p->x_img = cpad * d->h * d->w;
    p->y_img = kpad * oh * ow;
    if (p->x_img >= (1LL << 31) || p->y_img >= (1LL << 31)) {
        *why = "each image of x and y must hold fewer than 2^31 elements";
        return CFWD_ERR_UNSUPPORTED;
    }
    if (static_cast<long long>(d->k) * p->cg * d->r * d->s >= (1LL << 31)) {
        *why = "weights must hold fewer than 2^31 elements";
        return CFWD_ERR_UNSUPPORTED;
    }
    return CFWD_OK;
}

namespace {

// ------------------------------------------------------------- candidates

int family_rank(cfwd_algo_kind k) {
    switch (k) {
        case CFWD_ALGO_IMPLICIT_GEMM: return 0;
        case CFWD_ALGO_POINTWISE: return 1;
        case CFWD_ALGO_DIRECT: return 2;
        case CFWD_ALGO_WINOGRAD_F2X2_3X3: return 3;
        case CFWD_ALGO_WINOGRAD_F6X6_3X3: return 4;
        default: return 5;
    }
}

// Implicit GEMM configs 0 .. igemm_num_configs() - 1 are the NCHW / NCHWX
// kernels; the next nhwc_num_configs() the NHWC kernel (k_nhwc.hip); the
// next stem_i8_num_configs() the int8 NCHW4 stem kernel (k_stem_i8.hip).
int nhwc_first() { return igemm_num_configs(); }
int stem_first() { return nhwc_first() + nhwc_num_configs(); }
bool is_nhwc_cfg(cfwd_algo_kind k, int cfg) {
    return k == CFWD_ALGO_IMPLICIT_GEMM && cfg >= nhwc_first() && cfg < stem_first();
}
bool is_stem_cfg(cfwd_algo_kind k, int cfg) { return k == CFWD_ALGO_IMPLICIT_GEMM && cfg >= stem_first(); }

int num_configs(cfwd_algo_kind k) {
    switch (k) {
        case CFWD_ALGO_IMPLICIT_GEMM: return igemm_num_configs() + nhwc_num_configs() + stem_i8_num_configs();
        case CFWD_ALGO_POINTWISE: return pointwise_num_configs();
        case CFWD_ALGO_DIRECT: return direct_num_configs();
        case CFWD_ALGO_WINOGRAD_F2X2_3X3: return winograd_num_configs(2);
        case CFWD_ALGO_WINOGRAD_F6X6_3X3: return winograd_num_configs(6);
        default: return 0;
    }
}

bool supported(const Prob& p, cfwd_algo_kind k, int cfg, std::string* why) {
    if (cfg < 0 || cfg >= num_configs(k)) {
        if (why) *why = "no such config for this algorithm";
        return false;
    }
    // NHWC problems run only on the NHWC configs, and those only on NHWC
    if (p.layout == CFWD_LAYOUT_NHWC && !is_nhwc_cfg(k, cfg)) {
        if (why) *why = "NHWC activations run on the NHWC implicit GEMM configs only";
        return false;
    }
    if (is_nhwc_cfg(k, cfg)) return nhwc_supported(p, cfg - nhwc_first(), why);
    if (is_stem_cfg(k, cfg)) return stem_i8_supported(p, cfg - stem_first(), why);
    switch (k) {
        case CFWD_ALGO_IMPLICIT_GEMM: return igemm_supported(p, cfg, why);
        case CFWD_ALGO_POINTWISE: return pointwise_supported(p, cfg, why);
        case CFWD_ALGO_DIRECT: return direct_supported(p, cfg, why);
        case CFWD_ALGO_WINOGRAD_F2X2_3X3: return winograd_supported(p, 2, cfg, why);
        case CFWD_ALGO_WINOGRAD_F6X6_3X3: return winograd_supported(p, 6, cfg, why);
        default:
            if (why) *why = "unknown algorithm";
            return false;
    }
}

const cfwd_algo_kind kFamilies[] = {CFWD_ALGO_IMPLICIT_GEMM, CFWD_ALGO_POINTWISE, CFWD_ALGO_DIRECT,
                                    CFWD_ALGO_WINOGRAD_F2X2_3X3, CFWD_ALGO_WINOGRAD_F6X6_3X3};

// int8 results that are not always the exact integer ones: Winograd F(2x2)
// with its float intermediate.  Such candidates join Fast-Run only when the
// caller allows them (cfwd_fastrun_allow_inexact_int8), and then pass its
// gate if no output is more than 1 away from the exact result.
std::atomic<int> g_allow_inexact_i8{0};

bool inexact_i8(const Prob& p, cfwd_algo_kind k) {
    return p.dtype == CFWD_I8 && k == CFWD_ALGO_WINOGRAD_F2X2_3X3;
}

std::vector<cfwd_algo> candidates(const Prob& p) {
    std::vector<cfwd_algo> out;
    const bool inexact_ok = g_allow_inexact_i8.load() != 0;
    for (cfwd_algo_kind k : kFamilies) {
        if (inexact_i8(p, k) && !inexact_ok) continue;
        for (int c = 0; c < num_configs(k); ++c)
            if (supported(p, k, c, nullptr)) out.push_back(cfwd_algo{k, c, 0.0f});
    }
    return out;
}

size_t filter_bytes(const Prob& p, const cfwd_algo& a) {
    if (is_nhwc_cfg(a.kind, a.config_id)) return nhwc_filter_bytes(p, a.config_id - nhwc_first());
    if (is_stem_cfg(a.kind, a.config_id)) return stem_i8_filter_bytes(p, a.config_id - stem_first());
    switch (a.kind) {
        case CFWD_ALGO_IMPLICIT_GEMM: return igemm_filter_bytes(p, a.config_id);
        case CFWD_ALGO_POINTWISE: return pointwise_filter_bytes(p, a.config_id);
        case CFWD_ALGO_WINOGRAD_F2X2_3X3: return winograd_filter_bytes(p, 2, a.config_id);
        case CFWD_ALGO_WINOGRAD_F6X6_3X3: return winograd_filter_bytes(p, 6, a.config_id);
        default: return 0;
    }
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Device scratch an algorithm needs besides its prepared filter.
size_t scratch_bytes(const Prob& p, const cfwd_algo& a) {
    if (is_nhwc_cfg(a.kind, a.config_id) || is_stem_cfg(a.kind, a.config_id)) return 0;
    switch (a.kind) {
        case CFWD_ALGO_IMPLICIT_GEMM: return igemm_scratch_bytes(p, a.config_id);
        case CFWD_ALGO_WINOGRAD_F2X2_3X3: return winograd_scratch_bytes(p, 2, a.config_id);
        case CFWD_ALGO_WINOGRAD_F6X6_3X3: return winograd_scratch_bytes(p, 6, a.config_id);
        default: return 0;
    }
}

// Workspace when no prepared filter is passed: [filter | scratch].
size_t workspace_bytes(const Prob& p, const cfwd_algo& a) {
    const size_t sb = scratch_bytes(p, a);
    return sb ? round_up(filter_bytes(p, a), 256) + sb : filter_bytes(p, a);
}

// ------------------------------------------------------------- Fast-Run map

struct DeviceId {
    std::string arch;
    int cus = 0;
    bool ok = false;
};

// Identity of the current device.  The properties are read once per device
// index and kept: AUTO dispatch asks for them on every call.
constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
DeviceId g_dev_cache[kMaxDevices];

DeviceId current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return DeviceId{};
    }
    if (dev >= 0 && dev < kMaxDevices) {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        if (g_dev_cache[dev].ok) return g_dev_cache[dev];
    }
    DeviceId d;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return d;
    }
    d.arch = prop.gcnArchName;
    const size_t colon = d.arch.find(':');
    if (colon != std::string::npos) d.arch = d.arch.substr(0, colon);
    d.cus = prop.multiProcessorCount;
    d.ok = true;
    if (dev >= 0 && dev < kMaxDevices) {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        g_dev_cache[dev] = d;
    }
    return d;
}

// Identifies the kernel set: changes whenever a family gains or loses configs.
const std::string& kernel_set_id() {
    static const std::string id = [] {
        std::ostringstream s;
        s << "ig" << igemm_num_configs() << "-pw" << pointwise_num_configs() << "-dr" << direct_num_configs()
          << "-w2" << winograd_num_configs(2) << "-w6" << winograd_num_configs(6) << "-" << CFWD_VERSION;
        return s.str();
    }();
    return id;
}

std::string problem_key(const Prob& p) {
    std::ostringstream s;
    s << p.n << ',' << p.c << ',' << p.h << ',' << p.w << ',' << p.k << ',' << p.r << ',' << p.s << ',' << p.sh << ','
      << p.sw << ',' << p.ph << ',' << p.pw << ',' << p.dh << ',' << p.dw << ',' << p.g << ',' << p.layout << ','
      << p.xb << ',' << p.dtype;
    return s.str();
}

std::string full_key(const Prob& p, const DeviceId& d) {
    return d.arch + "|" + std::to_string(d.cus) + "|" + kernel_set_id() + "|" + problem_key(p);
}

std::mutex g_map_mu;
std::map<std::string, cfwd_algo> g_map;

bool map_lookup(const Prob& p, cfwd_algo* out) {
    const DeviceId d = current_device();
    if (!d.ok) return false;
    std::lock_guard<std::mutex> lk(g_map_mu);
    auto it = g_map.find(full_key(p, d));
    if (it == g_map.end()) return false;
    // A stale entry (config no longer valid for the problem) is ignored.
    if (!supported(p, it->second.kind, it->second.config_id, nullptr)) return false;
    *out = it->second;
    return true;
}

// CFWD_FASTRUN_CACHE: merged into the map once, before the first AUTO lookup
std::once_flag g_cache_once;
void load_cache_once() {
    if (env().cache.empty()) return;
    std::call_once(g_cache_once, [] { (void)cfwd_fastrun_load(env().cache.c_str()); });
}

cfwd_algo heuristic(const Prob& p) {
    if (p.layout == CFWD_LAYOUT_NHWC)
        for (int c = 0; c < nhwc_num_configs(); ++c)
            if (nhwc_supported(p, c, nullptr)) return cfwd_algo{CFWD_ALGO_IMPLICIT_GEMM, nhwc_first() + c, 0.0f};
    // Stands in for the article's hand-written preference table (its figure is
    // not preserved): depthwise -> direct, 1x1 -> pointwise, else implicit GEMM.
    if (p.depthwise()) return cfwd_algo{CFWD_ALGO_DIRECT, direct_default_config(p), 0.0f};
    if (p.pointwise())
        for (int c = 0; c < pointwise_num_configs(); ++c)
            if (pointwise_supported(p, c, nullptr)) return cfwd_algo{CFWD_ALGO_POINTWISE, c, 0.0f};
    const int c = igemm_default_config(p);
    if (c >= 0) return cfwd_algo{CFWD_ALGO_IMPLICIT_GEMM, c, 0.0f};
    return cfwd_algo{CFWD_ALGO_DIRECT, 0, 0.0f};
}

// Default config of a family (config_id -1): the first supported one, except
// implicit GEMM, which uses its own preference.
bool family_default(const Prob& p, cfwd_algo_kind k, int* cfg) {
    if (p.layout == CFWD_LAYOUT_NHWC) {
        for (int c = 0; c < num_configs(k); ++c)
            if (supported(p, k, c, nullptr)) {
                *cfg = c;
                return true;
            }
        return false;
    }
    if (k == CFWD_ALGO_IMPLICIT_GEMM) {
        *cfg = igemm_default_config(p);
        return *cfg >= 0;
    }
    if (k == CFWD_ALGO_DIRECT) {
        *cfg = direct_default_config(p);
        return true;
    }
    for (int c = 0; c < num_configs(k); ++c)
        if (supported(p, k, c, nullptr)) {
            *cfg = c;
            return true;
        }
    return false;
}

cfwd_status resolve(const Prob& p, cfwd_algo in, cfwd_algo* out) {
    if (in.kind == CFWD_ALGO_AUTO) {
        load_cache_once();
        if (env().mode != Env::OFF && map_lookup(p, out)) return CFWD_OK;
        *out = heuristic(p);
        std::string why;
        // NHWC problems outside the NHWC kernel's scope have no algorithm
        if (p.layout == CFWD_LAYOUT_NHWC && !supported(p, out->kind, out->config_id, &why))
            return set_error(CFWD_ERR_UNSUPPORTED, why);
        return CFWD_OK;
    }
    if (family_rank(in.kind) > 4) return set_error(CFWD_ERR_INVALID_ARG, "unknown algorithm kind");
    int cfg = in.config_id;
    if (cfg < 0) {
        if (!family_default(p, in.kind, &cfg))
            return set_error(CFWD_ERR_UNSUPPORTED, std::string(cfwd_algo_name(in)) + " cannot run this problem");
    }
    std::string why;
    if (!supported(p, in.kind, cfg, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    *out = cfwd_algo{in.kind, cfg, in.median_ms};
    return CFWD_OK;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

cfwd_status prepare(const Prob& p, const cfwd_algo& a, const void* w, void* wp, hipStream_t st) {
    if (is_nhwc_cfg(a.kind, a.config_id)) return nhwc_prepare(p, a.config_id - nhwc_first(), w, wp, st);
    if (is_stem_cfg(a.kind, a.config_id)) return stem_i8_prepare(p, a.config_id - stem_first(), w, wp, st);
    switch (a.kind) {
        case CFWD_ALGO_IMPLICIT_GEMM: return igemm_prepare(p, a.config_id, w, wp, st);
        case CFWD_ALGO_POINTWISE: return pointwise_prepare(p, a.config_id, w, wp, st);
        case CFWD_ALGO_WINOGRAD_F2X2_3X3: return winograd_prepare(p, 2, a.config_id, w, wp, st);
        case CFWD_ALGO_WINOGRAD_F6X6_3X3: return winograd_prepare(p, 6, a.config_id, w, wp, st);
        default: return CFWD_OK;
    }
}

cfwd_status run(const Prob& p, const cfwd_algo& a, const void* x, const void* w, const void* wp,
                const float* scale, void* y, void* scratch, const Epi& e, hipStream_t st) {
    cfwd_status s;
    if (is_nhwc_cfg(a.kind, a.config_id)) return nhwc_launch(p, a.config_id - nhwc_first(), x, wp, y, e, st);
    if (is_stem_cfg(a.kind, a.config_id)) {
        s = stem_i8_launch(p, a.config_id - stem_first(), x, wp, scale, y, e, st);
        if (s != CFWD_OK) return s;
        return zero_output_channel_padding(p, y, st);
    }
    switch (a.kind) {
        case CFWD_ALGO_IMPLICIT_GEMM: s = igemm_launch(p, a.config_id, x, wp, scale, y, scratch, e, st); break;
        case CFWD_ALGO_POINTWISE: s = pointwise_launch(p, a.config_id, x, wp, scale, y, e, st); break;
        case CFWD_ALGO_DIRECT: s = direct_launch(p, a.config_id, x, w, scale, y, e, st); break;
        case CFWD_ALGO_WINOGRAD_F2X2_3X3:
            s = (p.dtype == CFWD_I8) ? winograd_i8_launch(p, x, wp, scale, scratch, y, e, st)
                                     : winograd_launch(p, 2, a.config_id, x, wp, scratch, y, e, st);
            break;
        case CFWD_ALGO_WINOGRAD_F6X6_3X3: s = winograd_launch(p, 6, a.config_id, x, wp, scratch, y, e, st); break;
        default: return set_error(CFWD_ERR_INVALID_ARG, "unknown algorithm kind");
    }
    if (s != CFWD_OK) return s;
    return zero_output_channel_padding(p, y, st);
}

// Full conv: validation of pointers and sizes, optional on-the-fly prepare.
cfwd_status conv_impl(const Prob& p, const cfwd_algo& a, const void* x, const void* w, const void* wp,
                      const float* scale, void* y, void* ws, size_t ws_bytes, hipStream_t st, const Epi& e = Epi{}) {
    if (!x || !w || !y) return set_error(CFWD_ERR_INVALID_ARG, "x, w and y must not be NULL");
    if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (wp && !aligned16(wp)) || (ws && !aligned16(ws)))
        return set_error(CFWD_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    if (p.dtype == CFWD_I8 && scale == nullptr)
        return set_error(CFWD_ERR_INVALID_ARG, "int8 needs requant_scale[K]");
    if (p.dtype != CFWD_I8 && scale != nullptr)
        return set_error(CFWD_ERR_INVALID_ARG, "requant_scale is only for int8");
    const size_t fb = filter_bytes(p, a);
    const size_t sb = scratch_bytes(p, a);
    uint8_t* wsb = static_cast<uint8_t*>(ws);
    void* scratch = nullptr;
    if (fb > 0 && wp == nullptr) {
        const size_t need = workspace_bytes(p, a);
        if (ws == nullptr || ws_bytes < need)
            return set_error(CFWD_ERR_WORKSPACE, "workspace of " + std::to_string(need) +
                                                     " bytes needed to prepare the filter of " + cfwd_algo_name(a));
        cfwd_status s = prepare(p, a, w, ws, st);
        if (s != CFWD_OK) return s;
        wp = ws;
        if (sb) scratch = wsb + round_up(fb, 256);
    } else if (sb) {
        if (ws == nullptr || ws_bytes < sb)
            return set_error(CFWD_ERR_WORKSPACE, "workspace of " + std::to_string(sb) + " bytes needed by " +
                                                     cfwd_algo_name(a));
        scratch = ws;
    }
    return run(p, a, x, w, wp, scale, y, scratch, e, st);
}

// Checks a C-ABI epilogue and turns it into an Epi.
cfwd_status make_epi(const Prob& p, const cfwd_epilogue* ep, const void* y, Epi* out) {
    *out = Epi{};
    if (ep == nullptr) return CFWD_OK;
    if (ep->act != CFWD_ACT_NONE && ep->act != CFWD_ACT_RELU) return set_error(CFWD_ERR_INVALID_ARG, "unknown activation");
    if (ep->bias && (reinterpret_cast<uintptr_t>(ep->bias) & 3u))
        return set_error(CFWD_ERR_INVALID_ARG, "bias must be 4-byte aligned");
    if (ep->residual) {
        if (!aligned16(ep->residual)) return set_error(CFWD_ERR_INVALID_ARG, "residual must be 16-byte aligned");
        const uintptr_t r0 = reinterpret_cast<uintptr_t>(ep->residual);
        const uintptr_t y0 = reinterpret_cast<uintptr_t>(y);
        const uintptr_t bytes = static_cast<uintptr_t>(p.y_img) * p.n * p.esize;
        if (r0 < y0 + bytes && y0 < r0 + bytes) return set_error(CFWD_ERR_INVALID_ARG, "residual must not overlap y");
    }
    out->bias = ep->bias;
    out->res = ep->residual;
    out->relu = ep->act == CFWD_ACT_RELU ? 1 : 0;
    return CFWD_OK;
}

// ------------------------------------------------------------- allocation-free entry point

// Scratch of cfwd_conv2d_fwd_noalloc: one array per device, holding what a
// call would otherwise take from the caller's workspace (the prepared filter
// when none is passed, and the algorithm's scratch).  Each device holds its
// own copy until the process ends.  `scratch` names a host-side stand-in;
// kernels get the device address hipGetSymbolAddress returns for the
// current device, cached per device on the first call there.
static __device__ __align__(256) uint8_t scratch[CFWD_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

cfwd_status static_scratch(void** out) {
    int dev = 0;
    cfwd_status s = check_hip(hipGetDevice(&dev), "hipGetDevice");
    if (s != CFWD_OK) return s;
    if (dev < 0 || dev >= kMaxDevices) return set_error(CFWD_ERR_UNSUPPORTED, "device index out of range");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        s = check_hip(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (s != CFWD_OK) return s;
        if (ptr == nullptr) return set_error(CFWD_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return CFWD_OK;
}

// ------------------------------------------------------------- Fast-Run selection

constexpr int kWarmup = 2;
constexpr int kReps = 7;
// Candidates are timed from HBM, as a layer of a network runs on data that
// has streamed through since its last call: before every run, a buffer of
// twice the 256 MB Infinity Cache is overwritten (problems whose input and
// output together exceed that stream past the cache by themselves).
constexpr size_t kEvictBytes = size_t(512) << 20;

// Accuracy bound of a candidate: bf16 1e-2; fp32 Winograd F(6x6) 1e-3 (its
// transforms hold entries up to 32, which magnify rounding); every other fp32
// path, F(2x2) included (its transforms hold only 0, +-1, +-1/2), 1e-5.
float gate_tolerance(const Prob& p, cfwd_algo_kind k) {
    if (p.dtype == CFWD_BF16) return 1e-2f;
    if (k == CFWD_ALGO_WINOGRAD_F6X6_3X3) return 1e-3f;
    return 1e-5f;
}

struct FrLayout {
    size_t ref, den, xabs, wabs, stats, cand, evict, evict_bytes, total;
    size_t xn, yn;  // NHWC problems: x and an output converted to NCHW for the reference
};

FrLayout fastrun_layout(const Prob& p, const std::vector<cfwd_algo>& cands) {
    FrLayout L;
    const size_t ybytes = round_up(static_cast<size_t>(p.y_img) * p.n * p.esize, 256);
    const size_t xbytes = round_up(static_cast<size_t>(p.x_img) * p.n * p.esize, 256);
    const size_t wbytes = round_up(static_cast<size_t>(p.k) * p.cg * p.r * p.s * p.esize, 256);
    size_t cand = 0;
    for (const auto& c : cands) cand = std::max(cand, workspace_bytes(p, c));
    size_t off = 0;
    L.ref = off; off += ybytes;
    if (p.dtype == CFWD_I8) {
        L.den = L.xabs = L.wabs = 0;
    } else {
        L.den = off; off += ybytes;
        L.xabs = off; off += xbytes;
        L.wabs = off; off += wbytes;
    }
    L.xn = L.yn = 0;
    if (p.layout == CFWD_LAYOUT_NHWC) {
        L.xn = off; off += xbytes;
        L.yn = off; off += ybytes;
    }
    L.stats = off; off += 256;
    L.cand = off; off += round_up(cand, 256);
    const size_t footprint = static_cast<size_t>(p.x_img + p.y_img) * p.n * p.esize;
    L.evict = off;
    L.evict_bytes = footprint < kEvictBytes ? kEvictBytes : 0;
    off += L.evict_bytes;
    L.total = off;
    return L;
}

}  // namespace

namespace {

// Median of the samples; deterministic choice per the rule documented in the
// header.  Exposed through cfwd_fastrun_choose for host-only testing.
int choose(const std::vector<cfwd_algo>& cands, const std::vector<float>& med, const std::vector<int>& ok) {
    int best = -1;
    for (size_t i = 0; i < cands.size(); ++i) {
        if (!ok[i]) continue;
        if (best < 0) {
            best = static_cast<int>(i);
            continue;
        }
        // Strictly better only if more than 1% faster; ties keep the earlier.
        if (med[i] < med[best] * 0.99f) best = static_cast<int>(i);
    }
    return best;
}

float median_of(std::vector<float> v) {
    std::sort(v.begin(), v.end());
    const size_t n = v.size();
    if (n == 0) return 0.0f;
    return (n % 2) ? v[n / 2] : 0.5f * (v[n / 2 - 1] + v[n / 2]);
}

}  // namespace

}  // namespace cfwd

using namespace cfwd;

extern "C" {

const char* cfwd_version(void) { return "cfwd " CFWD_VERSION " gfx950"; }

const char* cfwd_status_string(cfwd_status s) {
    switch (s) {
        case CFWD_OK: return "ok";
        case CFWD_ERR_INVALID_ARG: return "invalid argument";
        case CFWD_ERR_UNSUPPORTED: return "unsupported";
        case CFWD_ERR_WORKSPACE: return "workspace too small";
        case CFWD_ERR_NO_CANDIDATE: return "no candidate passed";
        case CFWD_ERR_HIP: return "HIP runtime error";
        case CFWD_ERR_CACHE_IO: return "Fast-Run cache I/O error";
        default: return "unknown status";
    }
}

const char* cfwd_last_error(void) { return g_last_error.c_str(); }

const char* cfwd_algo_name(cfwd_algo a) {
    static thread_local char buf[64];
    const char* fam;
    switch (a.kind) {
        case CFWD_ALGO_AUTO: fam = "auto"; break;
        case CFWD_ALGO_IMPLICIT_GEMM: fam = "implicit_gemm"; break;
        case CFWD_ALGO_WINOGRAD_F2X2_3X3: fam = "winograd_f2x2_3x3"; break;
        case CFWD_ALGO_WINOGRAD_F6X6_3X3: fam = "winograd_f6x6_3x3"; break;
        case CFWD_ALGO_DIRECT: fam = "direct"; break;
        case CFWD_ALGO_POINTWISE: fam = "pointwise"; break;
        default: fam = "unknown"; break;
    }
    if (a.kind == CFWD_ALGO_AUTO)
        std::snprintf(buf, sizeof(buf), "%s", fam);
    else
        std::snprintf(buf, sizeof(buf), "%s/%d", fam, a.config_id);
    return buf;
}

cfwd_status cfwd_output_dims(const cfwd_conv_desc* desc, int* oh, int* ow) {
    Prob p;
    std::string why;
    cfwd_status s = make_prob(desc, &p, &why);
    if (s != CFWD_OK) return set_error(s, why);
    if (!oh || !ow) return set_error(CFWD_ERR_INVALID_ARG, "oh/ow must not be NULL");
    *oh = p.oh;
    *ow = p.ow;
    return CFWD_OK;
}

cfwd_status cfwd_resolve_algo(const cfwd_conv_desc* desc, cfwd_algo algo, cfwd_algo* resolved) {
    Prob p;
    std::string why;
    cfwd_status s = make_prob(desc, &p, &why);
    if (s != CFWD_OK) return set_error(s, why);
    if (!resolved) return set_error(CFWD_ERR_INVALID_ARG, "resolved must not be NULL");
    return resolve(p, algo, resolved);
}

cfwd_status cfwd_list_candidates(const cfwd_conv_desc* desc, cfwd_algo* out, int cap, int* count) {
    Prob p;
    std::string why;
    cfwd_status s = make_prob(desc, &p, &why);
    if (s != CFWD_OK) return set_error(s, why);
    if (!count || cap < 0 || (cap > 0 && !out)) return set_error(CFWD_ERR_INVALID_ARG, "bad output buffer");
    const std::vector<cfwd_algo> c = candidates(p);
    *count = static_cast<int>(c.size());
    for (int i = 0; i < cap && i < static_cast<int>(c.size()); ++i) out[i] = c[i];
    return CFWD_OK;
}

cfwd_status cfwd_filter_size(const cfwd_conv_desc* desc, cfwd_algo algo, size_t* bytes) {
    Prob p;
    std::string why;
    cfwd_status s = make_prob(desc, &p, &why);
    if (s != CFWD_OK) return set_error(s, why);
    if (!bytes) return set_error(CFWD_ERR_INVALID_ARG, "bytes must not be NULL");
    cfwd_algo a;
    s = resolve(p, algo, &a);
    if (s != CFWD_OK) return s;
    *bytes = filter_bytes(p, a);
    return CFWD_OK;
}

cfwd_status cfwd_prepare_filter(const cfwd_conv_desc* desc, cfwd_algo algo, const void* w_kcrs, void* w_prepared,
                                size_t bytes, void* stream) {
    Prob p;
    std::string why;
    cfwd_status s = make_prob(desc, &p, &why);
    if (s != CFWD_OK) return set_error(s, why);
    cfwd_algo a;
    s = resolve(p, algo, &a);
    if (s != CFWD_OK) return s;
    const size_t need = filter_bytes(p, a);
    if (need == 0) return CFWD_OK;
    if (!w_kcrs || !w_prepared) return set_error(CFWD_ERR_INVALID_ARG, "w_kcrs and w_prepared must not be NULL");
    if (!aligned16(w_kcrs) || !aligned16(w_prepared))
        return set_error(CFWD_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    if (bytes < need)
        return set_error(CFWD_ERR_WORKSPACE, "prepared filter needs " + std::to_string(need) + " bytes");
    return prepare(p, a, w_kcrs, w_prepared, static_cast<hipStream_t>(stream));
}

cfwd_status cfwd_workspace_size(const cfwd_conv_desc* desc, cfwd_algo algo, size_t* bytes) {
    Prob p;
    std::string why;
    cfwd_status s = make_prob(desc, &p, &why);
    if (s != CFWD_OK) return set_error(s, why);
    if (!bytes) return set_error(CFWD_ERR_INVALID_ARG, "bytes must not be NULL");
    cfwd_algo a;
    s = resolve(p, algo, &a);
    if (s != CFWD_OK) return s;
    *bytes = workspace_bytes(p, a);
    return CFWD_OK;
}

cfwd_status cfwd_scratch_size(const cfwd_conv_desc* desc, cfwd_algo algo, size_t* bytes) {
    Prob p;
    std::string why;
    cfwd_status s = make_prob(desc, &p, &why);
    if (s != CFWD_OK) return set_error(s, why);
    if (!bytes) return set_error(CFWD_ERR_INVALID_ARG, "bytes must not be NULL");
    cfwd_algo a;
    s = resolve(p, algo, &a);
    if (s != CFWD_OK) return s;
    *bytes = scratch_bytes(p, a);
    return CFWD_OK;
}

cfwd_status cfwd_fastrun_workspace_size(const cfwd_conv_desc* desc, size_t* bytes) {
    Prob p;
    std::string why;
    cfwd_status s = make_prob(desc, &p, &why);
    if (s != CFWD_OK) return set_error(s, why);
    if (!bytes) return set_error(CFWD_ERR_INVALID_ARG, "bytes must not be NULL");
    *bytes = fastrun_layout(p, candidates(p)).total;
    return CFWD_OK;
}

cfwd_status cfwd_fastrun_select(const cfwd_conv_desc* desc, const void* x, const void* w_kcrs,
                                const float* requant_scale, void* y, void* workspace, size_t ws_bytes, void* stream,
                                cfwd_algo* best) {
    Prob p;
    std::string why;
    cfwd_status s = make_prob(desc, &p, &why);
    if (s != CFWD_OK) return set_error(s, why);
    if (!best) return set_error(CFWD_ERR_INVALID_ARG, "best must not be NULL");
    if (!x || !w_kcrs || !y || !workspace) return set_error(CFWD_ERR_INVALID_ARG, "NULL buffer");
    if (!aligned16(x) || !aligned16(w_kcrs) || !aligned16(y) || !aligned16(workspace))
        return set_error(CFWD_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    if ((p.dtype == CFWD_I8) != (requant_scale != nullptr))
        return set_error(CFWD_ERR_INVALID_ARG, "requant_scale is required for int8 and only for int8");
    const std::vector<cfwd_algo> cands = candidates(p);
    const FrLayout L = fastrun_layout(p, cands);
    if (ws_bytes < L.total)
        return set_error(CFWD_ERR_WORKSPACE, "Fast-Run needs " + std::to_string(L.total) + " bytes of workspace");
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    void* ref = ws + L.ref;
    unsigned* stats = reinterpret_cast<unsigned*>(ws + L.stats);
    void* cand_ws = ws + L.cand;

    // Reference output: the generic direct kernel (exact integer arithmetic
    // for int8; fp32 accumulation for float).  For float dtypes the error
    // normaliser den = conv(|x|, |w|) is computed the same way.  NHWC
    // problems run it on x converted to NCHW and convert its outputs back.
    const bool nhwc = p.layout == CFWD_LAYOUT_NHWC;
    Prob pr = p;
    pr.layout = CFWD_LAYOUT_NCHW;
    const void* xr = x;
    if (nhwc) {
        s = layout_convert(p.n, p.c, p.h, p.w, p.esize, CFWD_LAYOUT_NHWC, 0, x, CFWD_LAYOUT_NCHW, 0, ws + L.xn, st);
        if (s != CFWD_OK) return s;
        xr = ws + L.xn;
    }
    auto to_layout = [&](void* out) -> cfwd_status {  // NHWC: out <- the NCHW result in yn
        return layout_convert(p.n, p.k, p.oh, p.ow, p.esize, CFWD_LAYOUT_NCHW, 0, ws + L.yn, CFWD_LAYOUT_NHWC, 0, out,
                              st);
    };
    s = direct_launch(pr, 0, xr, w_kcrs, requant_scale, nhwc ? ws + L.yn : ref, Epi{}, st);
    if (s == CFWD_OK && nhwc) s = to_layout(ref);
    if (s != CFWD_OK) return s;
    s = zero_output_channel_padding(p, ref, st);
    if (s != CFWD_OK) return s;
    if (p.dtype != CFWD_I8) {
        s = abs_copy(p, xr, ws + L.xabs, p.x_img * p.n, st);
        if (s != CFWD_OK) return s;
        s = abs_copy(p, w_kcrs, ws + L.wabs, static_cast<long long>(p.k) * p.cg * p.r * p.s, st);
        if (s != CFWD_OK) return s;
        s = direct_launch(pr, 0, ws + L.xabs, ws + L.wabs, nullptr, nhwc ? ws + L.yn : ws + L.den, Epi{}, st);
        if (s == CFWD_OK && nhwc) s = to_layout(ws + L.den);
        if (s != CFWD_OK) return s;
        // NCHWX channels past K: the direct kernel does not write them; den
        // there must be 0 like the candidate's and the reference's outputs
        s = zero_output_channel_padding(p, ws + L.den, st);
        if (s != CFWD_OK) return s;
    }

    hipEvent_t e0, e1;
    s = check_hip(hipEventCreate(&e0), "hipEventCreate");
    if (s != CFWD_OK) return s;
    s = check_hip(hipEventCreate(&e1), "hipEventCreate");
    if (s != CFWD_OK) {
        (void)hipEventDestroy(e0);
        return s;
    }
    std::vector<float> med(cands.size(), 0.0f);
    std::vector<int> ok(cands.size(), 0);
    for (size_t i = 0; i < cands.size() && s == CFWD_OK; ++i) {
        const cfwd_algo& a = cands[i];
        const size_t fb = filter_bytes(p, a);
        if (fb > 0) {
            s = prepare(p, a, w_kcrs, cand_ws, st);
            if (s != CFWD_OK) break;
        }
        const void* wp = fb > 0 ? cand_ws : nullptr;
        void* scr = scratch_bytes(p, a) ? static_cast<uint8_t*>(cand_ws) + round_up(fb, 256) : nullptr;
        std::vector<float> t;
        for (int rep = 0; rep < kWarmup + kReps && s == CFWD_OK; ++rep) {
            if (L.evict_bytes) s = evict_caches(ws + L.evict, L.evict_bytes, static_cast<unsigned>(rep), st);
            if (s == CFWD_OK) s = check_hip(hipEventRecord(e0, st), "hipEventRecord");
            if (s == CFWD_OK) s = run(p, a, x, w_kcrs, wp, requant_scale, y, scr, Epi{}, st);
            if (s == CFWD_OK) s = check_hip(hipEventRecord(e1, st), "hipEventRecord");
            if (s == CFWD_OK) s = check_hip(hipEventSynchronize(e1), "hipEventSynchronize");
            float ms = 0.0f;
            if (s == CFWD_OK) s = check_hip(hipEventElapsedTime(&ms, e0, e1), "hipEventElapsedTime");
            if (rep >= kWarmup) t.push_back(ms);
        }
        if (s != CFWD_OK) break;
        med[i] = median_of(t);
        // accuracy gate on the last run's output
        s = gate_compare(p, y, ref, p.dtype == CFWD_I8 ? nullptr : ws + L.den, stats, st);
        unsigned h[2] = {0, 0};
        if (s == CFWD_OK) s = check_hip(hipMemcpyAsync(h, stats, 8, hipMemcpyDeviceToHost, st), "hipMemcpyAsync");
        if (s == CFWD_OK) s = check_hip(hipStreamSynchronize(st), "hipStreamSynchronize");
        if (s != CFWD_OK) break;
        float err;
        std::memcpy(&err, &h[0], 4);
        if (p.dtype == CFWD_I8)  // h[0]: largest |difference| of the int8 outputs
            ok[i] = inexact_i8(p, a.kind) ? (h[0] <= 1u) : (h[1] == 0);
        else
            ok[i] = h[1] == 0 && err <= gate_tolerance(p, a.kind);
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (s != CFWD_OK) return s;
    const int b = choose(cands, med, ok);
    if (b < 0) return set_error(CFWD_ERR_NO_CANDIDATE, "no candidate passed the accuracy gate");
    cfwd_algo chosen = cands[b];
    chosen.median_ms = med[b];
    // leave y holding the chosen algorithm's output
    {
        const size_t fb = filter_bytes(p, chosen);
        if (fb > 0) {
            s = prepare(p, chosen, w_kcrs, cand_ws, st);
            if (s != CFWD_OK) return s;
        }
        void* scr = scratch_bytes(p, chosen) ? static_cast<uint8_t*>(cand_ws) + round_up(fb, 256) : nullptr;
        s = run(p, chosen, x, w_kcrs, fb > 0 ? cand_ws : nullptr, requant_scale, y, scr, Epi{}, st);
        if (s != CFWD_OK) return s;
        s = check_hip(hipStreamSynchronize(st), "hipStreamSynchronize");
        if (s != CFWD_OK) return s;
    }
    const DeviceId d = current_device();
    if (d.ok) {
        std::lock_guard<std::mutex> lk(g_map_mu);
        g_map[full_key(p, d)] = chosen;
    }
    *best = chosen;
    return CFWD_OK;
}

cfwd_status cfwd_conv2d_fwd(const cfwd_conv_desc* desc, cfwd_algo algo, const void* x, const void* w_kcrs,
                            const void* w_prepared, const float* requant_scale, void* y, void* workspace,
                            size_t ws_bytes, void* stream) {
    return cfwd_conv2d_fwd_ex(desc, algo, x, w_kcrs, w_prepared, requant_scale, nullptr, y, workspace, ws_bytes,
                              stream);
}

cfwd_status cfwd_conv2d_fwd_ex(const cfwd_conv_desc* desc, cfwd_algo algo, const void* x, const void* w_kcrs,
                               const void* w_prepared, const float* requant_scale, const cfwd_epilogue* epilogue,
                               void* y, void* workspace, size_t ws_bytes, void* stream) {
    Prob p;
    std::string why;
    cfwd_status s = make_prob(desc, &p, &why);
    if (s != CFWD_OK) return set_error(s, why);
    Epi e;
    s = make_epi(p, epilogue, y, &e);
    if (s != CFWD_OK) return s;
    const bool has_epi = e.bias || e.res || e.relu;
    hipStream_t st = static_cast<hipStream_t>(stream);
    cfwd_algo a;
    const Env& ev = env();
    if (algo.kind == CFWD_ALGO_AUTO) {
        load_cache_once();
        const char* how = "map";
        if (ev.mode == Env::OFF || !map_lookup(p, &a)) {
            if (ev.mode == Env::SEARCH && workspace && !has_epi) {
                size_t need = fastrun_layout(p, candidates(p)).total;
                if (ws_bytes >= need) {
                    s = cfwd_fastrun_select(desc, x, w_kcrs, requant_scale, y, workspace, ws_bytes, stream, &a);
                    if (s == CFWD_OK && !ev.cache.empty()) s = cfwd_fastrun_save(ev.cache.c_str());
                    if (ev.log >= 2)
                        std::fprintf(stderr, "cfwd: AUTO %s -> %s (search)\n", problem_key(p).c_str(),
                                     cfwd_algo_name(a));
                    return s;
                }
            }
            a = heuristic(p);
            how = "fixed preference";
            // NHWC problems outside the NHWC kernel's scope have no algorithm
            if (p.layout == CFWD_LAYOUT_NHWC && !supported(p, a.kind, a.config_id, &why))
                return set_error(CFWD_ERR_UNSUPPORTED, why);
        }
        if (ev.log >= 2) std::fprintf(stderr, "cfwd: AUTO %s -> %s (%s)\n", problem_key(p).c_str(), cfwd_algo_name(a), how);
    } else {
        s = resolve(p, algo, &a);
        if (s != CFWD_OK) return s;
    }
    if (ev.log >= 3) std::fprintf(stderr, "cfwd: conv %s with %s\n", problem_key(p).c_str(), cfwd_algo_name(a));
    return conv_impl(p, a, x, w_kcrs, w_prepared, requant_scale, y, workspace, ws_bytes, st, e);
}

cfwd_status cfwd_conv2d_fwd_noalloc(const cfwd_conv_desc* desc, cfwd_algo algo, const void* x, const void* w_kcrs,
                                    const void* w_prepared, const float* requant_scale, void* y, void* stream) {
    Prob p;
    std::string why;
    cfwd_status s = make_prob(desc, &p, &why);
    if (s != CFWD_OK) return set_error(s, why);
    cfwd_algo a;
    s = resolve(p, algo, &a);  // AUTO: the Fast-Run map, else the fixed preference (never a search)
    if (s != CFWD_OK) return s;
    const size_t need = w_prepared ? scratch_bytes(p, a) : workspace_bytes(p, a);
    if (need > CFWD_NOALLOC_SCRATCH_BYTES)
        return set_error(CFWD_ERR_WORKSPACE, std::string(cfwd_algo_name(a)) + " needs " + std::to_string(need) +
                                                 " bytes of scratch; the allocation-free entry point has " +
                                                 std::to_string(static_cast<size_t>(CFWD_NOALLOC_SCRATCH_BYTES)) +
                                                 (w_prepared ? "" : " (pass a prepared filter to need less)"));
    void* ws = nullptr;
    if (need > 0) {
        s = static_scratch(&ws);
        if (s != CFWD_OK) return s;
    }
    return conv_impl(p, a, x, w_kcrs, w_prepared, requant_scale, y, ws, ws ? CFWD_NOALLOC_SCRATCH_BYTES : 0,
                     static_cast<hipStream_t>(stream));
}

cfwd_status cfwd_fastrun_lookup(const cfwd_conv_desc* desc, cfwd_algo* algo) {
    Prob p;
    std::string why;
    cfwd_status s = make_prob(desc, &p, &why);
    if (s != CFWD_OK) return set_error(s, why);
    if (!algo) return set_error(CFWD_ERR_INVALID_ARG, "algo must not be NULL");
    if (!map_lookup(p, algo)) return set_error(CFWD_ERR_UNSUPPORTED, "no Fast-Run entry for this problem");
    return CFWD_OK;
}

cfwd_status cfwd_fastrun_clear(void) {
    std::lock_guard<std::mutex> lk(g_map_mu);
    g_map.clear();
    return CFWD_OK;
}

// File format: a first line "cfwd-fastrun 1", then one record per line:
//   <arch>|<cus>|<kernel set>|<problem>\t<kind>\t<config>\t<median ms>
cfwd_status cfwd_fastrun_save(const char* path) {
    if (!path) return set_error(CFWD_ERR_INVALID_ARG, "path must not be NULL");
    std::ofstream f(path, std::ios::trunc);
    if (!f) return set_error(CFWD_ERR_CACHE_IO, std::string("cannot open ") + path + " for writing");
    f << "cfwd-fastrun 1\n";
    std::lock_guard<std::mutex> lk(g_map_mu);
    for (const auto& kv : g_map)
        f << kv.first << '\t' << static_cast<int>(kv.second.kind) << '\t' << kv.second.config_id << '\t'
          << kv.second.median_ms << '\n';
    f.flush();
    if (!f) return set_error(CFWD_ERR_CACHE_IO, std::string("write to ") + path + " failed");
    return CFWD_OK;
}

cfwd_status cfwd_fastrun_load(const char* path) {
    if (!path) return set_error(CFWD_ERR_INVALID_ARG, "path must not be NULL");
    std::ifstream f(path);
    if (!f) {
        set_error(CFWD_OK, std::string("Fast-Run map ") + path + " not found; ignored");
        return CFWD_OK;
    }
    std::string line;
    if (!std::getline(f, line) || line != "cfwd-fastrun 1") {
        set_error(CFWD_OK, std::string("Fast-Run map ") + path + " has no valid header; ignored");
        return CFWD_OK;
    }
    const std::string kset = kernel_set_id();
    std::map<std::string, cfwd_algo> add;
    while (std::getline(f, line)) {
        std::istringstream ls(line);
        std::string key, kind_s, cfg_s, ms_s;
        if (!std::getline(ls, key, '\t') || !std::getline(ls, kind_s, '\t') || !std::getline(ls, cfg_s, '\t') ||
            !std::getline(ls, ms_s))
            continue;  // malformed record
        char* end = nullptr;
        const long kind = std::strtol(kind_s.c_str(), &end, 10);
        if (*end || kind < 1 || kind > 5) continue;
        const long cfg = std::strtol(cfg_s.c_str(), &end, 10);
        if (*end || cfg < 0 || cfg > 1000) continue;
        const float ms = std::strtof(ms_s.c_str(), &end);
        if (*end) continue;
        // key = arch|cus|kset|problem: drop records of another kernel set
        const size_t p1 = key.find('|');
        const size_t p2 = p1 == std::string::npos ? p1 : key.find('|', p1 + 1);
        const size_t p3 = p2 == std::string::npos ? p2 : key.find('|', p2 + 1);
        if (p3 == std::string::npos) continue;
        if (key.substr(p2 + 1, p3 - p2 - 1) != kset) continue;
        add[key] = cfwd_algo{static_cast<cfwd_algo_kind>(kind), static_cast<int>(cfg), ms};
    }
    std::lock_guard<std::mutex> lk(g_map_mu);
    for (const auto& kv : add) g_map[kv.first] = kv.second;
    return CFWD_OK;
}

// Host-only piece of the Fast-Run selection rule, exported for testing:
// given n candidates in Fast-Run order with reps timings each (row-major) and
// a pass/fail flag per candidate, writes the index that would be chosen (or
// -1) to *chosen.
cfwd_status cfwd_bottleneck_check(const cfwd_bottleneck_desc* desc) {
    std::string why;
    const cfwd_status s = bottleneck_check(desc, &why);
    return s == CFWD_OK ? s : set_error(s, why);
}

cfwd_status cfwd_bottleneck_filter_size(const cfwd_bottleneck_desc* desc, size_t* bytes) {
    cfwd_status s = cfwd_bottleneck_check(desc);
    if (s != CFWD_OK) return s;
    if (!bytes) return set_error(CFWD_ERR_INVALID_ARG, "bytes must not be NULL");
    *bytes = bottleneck_filter_bytes();
    return CFWD_OK;
}

cfwd_status cfwd_bottleneck_prepare(const cfwd_bottleneck_desc* desc, const void* w2, void* w2_prepared, size_t bytes,
                                    void* stream) {
    cfwd_status s = cfwd_bottleneck_check(desc);
    if (s != CFWD_OK) return s;
    if (!w2 || !w2_prepared) return set_error(CFWD_ERR_INVALID_ARG, "w2 and w2_prepared must not be NULL");
    if (!aligned16(w2_prepared)) return set_error(CFWD_ERR_INVALID_ARG, "w2_prepared must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(w2) & 1u) != 0) return set_error(CFWD_ERR_INVALID_ARG, "w2 must be 2-byte aligned");
    if (bytes < bottleneck_filter_bytes())
        return set_error(CFWD_ERR_WORKSPACE,
                         "prepared 3x3 weights need " + std::to_string(bottleneck_filter_bytes()) + " bytes");
    return bottleneck_prepare(w2, w2_prepared, static_cast<hipStream_t>(stream));
}

cfwd_status cfwd_bottleneck_fwd(const cfwd_bottleneck_desc* desc, const void* x, const void* w1,
                                const void* w2_prepared, const void* w3, const cfwd_bottleneck_epilogue* epilogue,
                                void* y, void* stream) {
    cfwd_status s = cfwd_bottleneck_check(desc);
    if (s != CFWD_OK) return s;
    if (!x || !w1 || !w2_prepared || !w3 || !y) return set_error(CFWD_ERR_INVALID_ARG, "NULL buffer");
    if (!aligned16(x) || !aligned16(w1) || !aligned16(w2_prepared) || !aligned16(w3) || !aligned16(y))
        return set_error(CFWD_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    const size_t xb = static_cast<size_t>(desc->n) * desc->c * desc->h * desc->w * 2;
    const size_t yb = static_cast<size_t>(desc->n) * desc->k * desc->h * desc->w * 2;
    auto overlaps = [](const void* p, size_t pb, const void* q, size_t qb) {
        const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
        return a < b + qb && b < a + pb;
    };
    if (overlaps(x, xb, y, yb)) return set_error(CFWD_ERR_INVALID_ARG, "y must not overlap x");
    if (epilogue) {
        for (const void* bptr : {epilogue->b1, epilogue->b2, epilogue->b3})
            if (bptr && (reinterpret_cast<uintptr_t>(bptr) & 3u) != 0)
                return set_error(CFWD_ERR_INVALID_ARG, "biases must be 4-byte aligned");
        if (epilogue->residual) {
            if (!aligned16(epilogue->residual))
                return set_error(CFWD_ERR_INVALID_ARG, "residual must be 16-byte aligned");
            if (overlaps(epilogue->residual, yb, y, yb))
                return set_error(CFWD_ERR_INVALID_ARG, "residual must not overlap y");
        }
    }
    return bottleneck_launch(desc, x, w1, w2_prepared, w3, epilogue, y, static_cast<hipStream_t>(stream));
}

cfwd_status cfwd_convert_layout(int n, int c, int h, int w, cfwd_dtype dtype, cfwd_layout src_layout, int src_x,
                                const void* src, cfwd_layout dst_layout, int dst_x, void* dst, void* stream) {
    if (n < 1 || c < 1 || h < 1 || w < 1) return set_error(CFWD_ERR_INVALID_ARG, "n, c, h, w must be >= 1");
    int es;
    if (!esize_of(dtype, &es)) return set_error(CFWD_ERR_INVALID_ARG, "unknown dtype");
    auto lay_ok = [](cfwd_layout l, int xb) {
        return l == CFWD_LAYOUT_NCHW || l == CFWD_LAYOUT_NHWC || (l == CFWD_LAYOUT_NCHWX && (xb == 4 || xb == 8));
    };
    if (!lay_ok(src_layout, src_x) || !lay_ok(dst_layout, dst_x))
        return set_error(CFWD_ERR_INVALID_ARG, "layouts must be NCHW, NHWC or NCHWX with x = 4 or 8");
    if (!src || !dst) return set_error(CFWD_ERR_INVALID_ARG, "src and dst must not be NULL");
    if ((reinterpret_cast<uintptr_t>(src) % es) != 0 || (reinterpret_cast<uintptr_t>(dst) % es) != 0)
        return set_error(CFWD_ERR_INVALID_ARG, "src and dst must be aligned to the element size");
    auto bytes = [&](cfwd_layout l, int xb) {
        const long long cp = (l == CFWD_LAYOUT_NCHWX) ? (c + xb - 1) / xb * xb : c;
        return static_cast<size_t>(n) * cp * h * w * es;
    };
    const size_t sb = bytes(src_layout, src_x), db = bytes(dst_layout, dst_x);
    if (sb / es / n >= (1ULL << 31) || db / es / n >= (1ULL << 31))
        return set_error(CFWD_ERR_UNSUPPORTED, "each image must hold fewer than 2^31 elements");
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    if (a < b + db && b < a + sb) return set_error(CFWD_ERR_INVALID_ARG, "src and dst must not overlap");
    return layout_convert(n, c, h, w, es, src_layout, src_x, src, dst_layout, dst_x, dst, static_cast<hipStream_t>(stream));
}

cfwd_status cfwd_unpack_int4(const void* packed, void* out_int8, long long count, void* stream) {
    if (count < 1) return set_error(CFWD_ERR_INVALID_ARG, "count must be >= 1");
    if (!packed || !out_int8) return set_error(CFWD_ERR_INVALID_ARG, "packed and out_int8 must not be NULL");
    if (!aligned16(packed) || !aligned16(out_int8))
        return set_error(CFWD_ERR_INVALID_ARG, "packed and out_int8 must be 16-byte aligned");
    const uintptr_t a = reinterpret_cast<uintptr_t>(packed), b = reinterpret_cast<uintptr_t>(out_int8);
    const uintptr_t pb = static_cast<uintptr_t>((count + 1) / 2), ob = static_cast<uintptr_t>(count);
    if (a < b + ob && b < a + pb) return set_error(CFWD_ERR_INVALID_ARG, "packed and out_int8 must not overlap");
    return unpack_int4(packed, out_int8, count, static_cast<hipStream_t>(stream));
}

cfwd_status cfwd_fastrun_allow_inexact_int8(int allow) {
    g_allow_inexact_i8.store(allow ? 1 : 0);
    return CFWD_OK;
}

cfwd_status cfwd_fastrun_choose(const cfwd_algo* cands, const float* times, int n, int reps, const int* gate_ok,
                                int* chosen) {
    if (!cands || !times || !gate_ok || !chosen || n < 0 || reps <= 0)
        return set_error(CFWD_ERR_INVALID_ARG, "bad arguments");
    std::vector<cfwd_algo> c(cands, cands + n);
    std::vector<float> med(n);
    std::vector<int> ok(gate_ok, gate_ok + n);
    for (int i = 0; i < n; ++i) med[i] = median_of(std::vector<float>(times + i * reps, times + (i + 1) * reps));
    *chosen = choose(c, med, ok);
    return CFWD_OK;
}

}  // extern "C"
