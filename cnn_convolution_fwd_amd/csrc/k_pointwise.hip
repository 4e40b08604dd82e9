// Pointwise (1x1, stride 1, pad 0, groups 1) convolution on the matrix cores,
// shaped for HBM bandwidth (gfx950).
//
// Momenta talk, section "優化2：Depthwise卷積": a 1x1 layer does one multiply
// per loaded input per output channel, against R*S for a 3x3, so its
// arithmetic intensity is low and the layer is bound by memory traffic, not by
// compute.  ConvSummary ("卷积总结"), conv -> GEMM: a 1x1 convolution is exactly
// the matrix product Y_n[K, H*W] = W[K, C] X_n[C, H*W] per image.
//
// The kernel therefore streams X and Y once, at full width, and lets the
// matrix cores absorb the arithmetic:
//   * MFMA rows = output channels (A = prepared weights, a few KB, from L1/L2),
//     MFMA columns = pixels (B = activations, straight from HBM, no LDS);
//   * each lane loads PPL = 4 consecutive pixels of one channel with one
//     vector load (8 bytes bf16, 16 bytes fp32); the four pixel phases become
//     four MFMAs whose columns are pixels 4j + phase, so every activation byte
//     is loaded once, coalesced, and the lane's 4 outputs of one channel are
//     again 4 consecutive pixels, written with one vector store;
//   * the channel reduction is software-pipelined two steps deep, with no
//     branches in the loop (the last pair is peeled); outputs are written with
//     streaming (non-temporal) stores.
// bf16: step = 16 channels, one v_mfma_f32_32x32x16_bf16 per phase and
// 32-channel block; fp32: step = 8 channels, four v_mfma_f32_32x32x2f32.
#include "internal.h"

namespace cfwd {

namespace {

using f32x16_t = float __attribute__((ext_vector_type(16)));

constexpr int kPPL = 4;      // pixels per lane
constexpr int kWavePix = 128;  // pixels per wave (32 lanes x 4)

template <typename T> struct PwT;
template <> struct PwT<bf16_t> {
    static constexpr int STEP = 16;  // channels per reduction step
    using XV = uint2;                // 4 bf16 pixels of one channel
    // B operand of phase ph from the 8 channel loads of this lane's half
    static __device__ __forceinline__ void mma(f32x16_t& acc, const uint4& a, const XV* xv, int ph) {
        uint32_t r[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t lo = (ph >> 1) ? xv[2 * m].y : xv[2 * m].x;
            const uint32_t hi = (ph >> 1) ? xv[2 * m + 1].y : xv[2 * m + 1].x;
            r[m] = (ph & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        const uint4 b = make_uint4(r[0], r[1], r[2], r[3]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                      acc, 0, 0, 0);
    }
    static constexpr int NLOAD = 8;  // channel loads per step per lane
    // channel of load i for lane half h within a step
    static __device__ __forceinline__ int chan(int i, int h) { return 8 * h + i; }
    static __device__ __forceinline__ void store4(bf16_t* p, const float* v) {
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t q = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        __builtin_nontemporal_store(q, reinterpret_cast<u32x2_t*>(p));
    }
    static __device__ __forceinline__ void unpack4(const XV& q, float* r) {
        r[0] = __uint_as_float(q.x << 16);
        r[1] = __uint_as_float(q.x & 0xffff0000u);
        r[2] = __uint_as_float(q.y << 16);
        r[3] = __uint_as_float(q.y & 0xffff0000u);
    }
};
template <> struct PwT<float> {
    static constexpr int STEP = 8;
    using XV = uint4;  // 4 fp32 pixels of one channel
    // sub-step i of 4 (two channels each); callers interleave the phases and
    // blocks between dependent sub-steps, so no MFMA waits on its predecessor
    static __device__ __forceinline__ void mma_sub(f32x16_t& acc, const uint4& a, const XV* xv, int ph, int i) {
        const uint32_t av[4] = {a.x, a.y, a.z, a.w};
        const uint32_t xw[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(av[i]), __uint_as_float(xw[ph]), acc, 0, 0, 0);
    }
    static constexpr int NLOAD = 4;
    static __device__ __forceinline__ int chan(int i, int h) { return 2 * i + h; }
    static __device__ __forceinline__ void store4(float* p, const float* v) {
        typedef float f32x4_t __attribute__((ext_vector_type(4)));
        const f32x4_t q = {v[0], v[1], v[2], v[3]};
        __builtin_nontemporal_store(q, reinterpret_cast<f32x4_t*>(p));
    }
    static __device__ __forceinline__ void unpack4(const XV& q, float* r) {
        r[0] = __uint_as_float(q.x);
        r[1] = __uint_as_float(q.y);
        r[2] = __uint_as_float(q.z);
        r[3] = __uint_as_float(q.w);
    }
};

// Prepared weights: [k-block of 32][step][lane 64][16 bytes]; lane (row, h)
// holds W[kb*32 + row][step*STEP + chan(i, h)] for its 16 bytes' elements i.
template <typename T>
__global__ __launch_bounds__(256) void pw_prepare_kernel(const T* __restrict__ w, T* __restrict__ out, int K, int C,
                                                         int nkb, int nsteps) {
    using P = PwT<T>;
    constexpr int E = 16 / static_cast<int>(sizeof(T));  // elements per lane
    const long long total = static_cast<long long>(nkb) * nsteps * 64 * E;
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < total; i += static_cast<long long>(gridDim.x) * 256) {
        const int e = static_cast<int>(i % E);
        long long t = i / E;
        const int lane = static_cast<int>(t % 64);
        t /= 64;
        const int s = static_cast<int>(t % nsteps);
        const int kb = static_cast<int>(t / nsteps);
        const int k = kb * 32 + (lane & 31);
        const int c = s * P::STEP + P::chan(e, lane >> 5);
        out[i] = (k < K && c < C) ? w[static_cast<long long>(k) * C + c] : T{};
    }
}

// Workgroup: 4 waves = (4 / KW) pixel blocks x KW k groups; a wave owns 128
// pixels x KBW blocks of 32 output channels.  Grid: pixel groups x k groups.
// EPI: the fused epilogue compiled in (a separate instantiation, so the
// plain kernels carry none of its registers).
template <typename T, int KBW, bool EPI>
__global__ __launch_bounds__(256) void pw_kernel(const T* __restrict__ x, const uint8_t* __restrict__ wp,
                                                 T* __restrict__ y, int C, int K, int HW, long long x_img,
                                                 long long y_img, long long npix, int nsteps, int nkb, int KW,
                                                 int ngk, Epi ep) {
    using P = PwT<T>;
    using XV = typename P::XV;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lrow = lane & 31, h = lane >> 5;
    const int wk = wave % KW, wpx = wave / KW;
    const int kg = static_cast<int>(blockIdx.x) % ngk;
    const long long pg = static_cast<long long>(blockIdx.x) / ngk;
    const int kb0 = (kg * KW + wk) * KBW;
    if (kb0 >= nkb) return;  // no barrier in this kernel: idle waves may leave
    const long long P0 = (pg * (4 / KW) + wpx) * kWavePix;
    // pixel indices fit in 31 bits (checked on the host): a 32-bit division
    const unsigned G = static_cast<unsigned>(P0) + kPPL * lrow;  // this lane's first pixel (npix % 4 == 0)
    const bool pix_ok = G < static_cast<unsigned>(npix);
    const unsigned Gc = pix_ok ? G : static_cast<unsigned>(npix) - kPPL;
    const long long n = Gc / static_cast<unsigned>(HW);
    const int p = static_cast<int>(Gc - static_cast<unsigned>(n) * HW);
    const T* xb = x + n * x_img + p;
    T* yb = y + n * y_img + p;

    f32x16_t acc[KBW][kPPL];
#pragma unroll
    for (int b = 0; b < KBW; ++b)
#pragma unroll
        for (int ph = 0; ph < kPPL; ++ph) acc[b][ph] = f32x16_t{};

    auto load = [&](int s, XV* xv, uint4* wv) {
#pragma unroll
        for (int i = 0; i < P::NLOAD; ++i) {
            const int c = s * P::STEP + P::chan(i, h);
            const int cc = min(c, C - 1);
            XV v = *reinterpret_cast<const XV*>(xb + static_cast<long long>(cc) * HW);
            if (c >= C) v = XV{};
            xv[i] = v;
        }
#pragma unroll
        for (int b = 0; b < KBW; ++b)
            wv[b] = *reinterpret_cast<const uint4*>(wp + ((static_cast<long long>(kb0 + b) * nsteps + s) * 64 + lane) * 16);
    };
    auto compute = [&](const XV* xv, const uint4* wv) {
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int b = 0; b < KBW; ++b)
#pragma unroll
                    for (int ph = 0; ph < kPPL; ++ph) P::mma_sub(acc[b][ph], wv[b], xv, ph, i);
        } else {
#pragma unroll
            for (int b = 0; b < KBW; ++b)
#pragma unroll
                for (int ph = 0; ph < kPPL; ++ph) P::mma(acc[b][ph], wv[b], xv, ph);
        }
    };

    // two-deep pipeline over the (even) number of steps; the last pair is peeled
    XV xa[P::NLOAD], xb2[P::NLOAD];
    uint4 wa[KBW], wb[KBW];
    load(0, xa, wa);
    int s = 0;
    for (; s + 2 < nsteps; s += 2) {
        load(s + 1, xb2, wb);
        compute(xa, wa);
        load(s + 2, xa, wa);
        compute(xb2, wb);
    }
    load(s + 1, xb2, wb);
    compute(xa, wa);
    compute(xb2, wb);

    if (!pix_ok) return;
    // D[row = channel][col = pixel]: lane (j, hh), element v -> channel
    // 8 (v / 4) + 4 hh + v % 4 of the block, pixels 4j .. 4j + 3 over the phases
#pragma unroll
    for (int b = 0; b < KBW; ++b) {
        // fused epilogue: every bias and residual vector of this block is
        // requested before the first is used (the residual vector of a
        // channel is the same 4 pixels the lane stores)
        float bv[16];
        XV rv[16];
        if constexpr (EPI) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int kc = min((kb0 + b) * 32 + 8 * (v / 4) + 4 * h + (v % 4), K - 1);
                bv[v] = ep.bias ? static_cast<const float*>(ep.bias)[kc] : 0.0f;
                if (ep.res)
                    rv[v] = *reinterpret_cast<const XV*>(static_cast<const T*>(ep.res) + (yb - y) +
                                                         static_cast<long long>(kc) * HW);
            }
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int k = (kb0 + b) * 32 + 8 * (v / 4) + 4 * h + (v % 4);
            if (k < K) {
                float o[4] = {acc[b][0][v], acc[b][1][v], acc[b][2][v], acc[b][3][v]};
                if constexpr (EPI) {
                    float r[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                    if (ep.res) P::unpack4(rv[v], r);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float t = o[i] + bv[v] + r[i];
                        o[i] = ep.relu ? fmaxf(t, 0.0f) : t;
                    }
                }
                P::store4(yb + static_cast<long long>(k) * HW, o);
            }
        }
    }
}

struct PwGeo {
    int nkb, nkb_alloc, nsteps, KW, ngk;  // nkb_alloc: k blocks rounded up to a wave's KBW
    long long npix, pgroups;
};

constexpr int kKBW[2] = {2, 1};  // 32-channel blocks per wave, per config

bool geometry(const Prob& p, int cfg, PwGeo* g, std::string* why) {
    auto fail = [&](const char* m) {
        if (why) *why = m;
        return false;
    };
    if (cfg < 0 || cfg > 1) return fail("pointwise: no such config");
    if (!p.pointwise() || p.sh != 1 || p.sw != 1 || p.g != 1)
        return fail("pointwise: needs a 1x1 filter, stride 1, pad 0, groups 1");
    if (p.layout != CFWD_LAYOUT_NCHW || p.dtype == CFWD_I8) return fail("pointwise: needs NCHW fp32 or bf16");
    const long long hw = static_cast<long long>(p.h) * p.w;
    if (hw % kPPL != 0) return fail("pointwise: needs H*W a multiple of 4");
    if (hw * p.c >= (1LL << 31) || hw * p.k >= (1LL << 31)) return fail("pointwise: image too large");
    const int step = (p.dtype == CFWD_F32) ? PwT<float>::STEP : PwT<bf16_t>::STEP;
    g->nsteps = (p.c + step - 1) / step;
    g->nsteps += g->nsteps & 1;  // even, for the two-deep pipeline
    g->nkb = (p.k + 31) / 32;
    const int kbw = kKBW[cfg];
    const int kwaves = (g->nkb + kbw - 1) / kbw;  // waves needed along K
    g->nkb_alloc = kwaves * kbw;  // a wave's last block may be all padding (zeros)
    g->KW = kwaves >= 4 ? 4 : (kwaves >= 2 ? 2 : 1);
    g->ngk = (kwaves + g->KW - 1) / g->KW;
    g->npix = hw * p.n;
    if (g->npix + 1024 >= (1LL << 31)) return fail("pointwise: more than 2^31 pixels");
    const long long pix_per_wg = static_cast<long long>(4 / g->KW) * kWavePix;
    g->pgroups = (g->npix + pix_per_wg - 1) / pix_per_wg;
    if (g->pgroups * g->ngk >= (1LL << 31)) return fail("pointwise: grid too large");
    return true;
}

template <typename T>
cfwd_status launch_t(const Prob& p, int cfg, const PwGeo& g, const void* x, const void* wp, void* y, const Epi& e,
                     hipStream_t st) {
    const unsigned blocks = static_cast<unsigned>(g.pgroups * g.ngk);
    const long long hw = static_cast<long long>(p.h) * p.w;
    const bool epi = e.bias || e.res || e.relu;
    auto kern = (kKBW[cfg] == 2) ? (epi ? pw_kernel<T, 2, true> : pw_kernel<T, 2, false>)
                                 : (epi ? pw_kernel<T, 1, true> : pw_kernel<T, 1, false>);
    kern<<<blocks, 256, 0, st>>>(static_cast<const T*>(x), static_cast<const uint8_t*>(wp), static_cast<T*>(y), p.c,
                                 p.k, static_cast<int>(hw), p.x_img, p.y_img, g.npix, g.nsteps, g.nkb, g.KW, g.ngk,
                                 e);
    return check_hip(hipGetLastError(), "pointwise launch");
}

}  // namespace

int pointwise_num_configs() { return 2; }

bool pointwise_supported(const Prob& p, int cfg, std::string* why) {
    PwGeo g;
    return geometry(p, cfg, &g, why);
}

size_t pointwise_filter_bytes(const Prob& p, int cfg) {
    PwGeo g;
    if (!geometry(p, cfg, &g, nullptr)) return 0;
    return static_cast<size_t>(g.nkb_alloc) * g.nsteps * 64 * 16;
}

cfwd_status pointwise_prepare(const Prob& p, int cfg, const void* w, void* wp, hipStream_t st) {
    PwGeo g;
    std::string why;
    if (!geometry(p, cfg, &g, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    const long long total = static_cast<long long>(g.nkb_alloc) * g.nsteps * 64 * (p.dtype == CFWD_F32 ? 4 : 8);
    const unsigned blocks = static_cast<unsigned>(std::min<long long>((total + 255) / 256, 65536));
    if (p.dtype == CFWD_F32)
        pw_prepare_kernel<float><<<blocks, 256, 0, st>>>(static_cast<const float*>(w), static_cast<float*>(wp), p.k,
                                                         p.c, g.nkb_alloc, g.nsteps);
    else
        pw_prepare_kernel<bf16_t><<<blocks, 256, 0, st>>>(static_cast<const bf16_t*>(w), static_cast<bf16_t*>(wp),
                                                          p.k, p.c, g.nkb_alloc, g.nsteps);
    return check_hip(hipGetLastError(), "pointwise filter prepare launch");
}

cfwd_status pointwise_launch(const Prob& p, int cfg, const void* x, const void* wp, const float*, void* y,
                             const Epi& e, hipStream_t st) {
    PwGeo g;
    std::string why;
    if (!geometry(p, cfg, &g, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    if (wp == nullptr) return set_error(CFWD_ERR_WORKSPACE, "pointwise: prepared filter required");
    if (p.dtype == CFWD_F32) return launch_t<float>(p, cfg, g, x, wp, y, e, st);
    return launch_t<bf16_t>(p, cfg, g, x, wp, y, e, st);
}

}  // namespace cfwd
