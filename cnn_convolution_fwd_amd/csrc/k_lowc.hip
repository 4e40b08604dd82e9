// Implicit GEMM for layers with few input channels (the stem of a CNN: 3
// image channels, 3x3 or 7x7 filters, stride 2), gfx950.
//
// MegEngine inference article, section "Im2col+MatMul": the convolution is a
// matrix product of the weights with the im2col matrix.  When C*R*S is small
// the tiled implicit GEMM of igemm_impl.h wastes most of each 64-byte channel
// chunk (3 real channels of 32 or 64), so this variant gathers the reduction
// dimension directly instead of staging channel chunks:
//   * MFMA rows = output channels (A = prepared weights, 16 bytes per lane
//     per step, from L1/L2), MFMA columns = output pixels (B = gathered
//     input, one column per lane);
//   * the reduction index u runs over (c, r, s) for fp32/bf16 (one element
//     per unit), or over taps (r, s) for int8 NCHW4 with C <= 4, where one
//     unit is the aligned dword holding a pixel's four channels;
//   * a per-workgroup LDS table maps u to (row delta, column delta, channel
//     offset); each lane adds its own pixel's origin, tests the bounds (zero
//     padding) and loads with a clamped, always-valid address -- no branches;
//   * gathers of the next step are in flight while the current one is on the
//     matrix cores (two-deep pipeline, last pair peeled);
//   * the epilogue writes D[k][pixel] in the caller's layout; for int8 NCHW4
//     a lane's four consecutive channels of one pixel leave as one dword.
// Step (units per MFMA step): fp32 8 (four v_mfma_f32_32x32x2f32), bf16 16
// (one v_mfma_f32_32x32x16_bf16), int8 8 dwords = 32 bytes (one
// v_mfma_i32_32x32x32_i8).
#include "internal.h"

namespace cfwd {

namespace {

using f32x16_t = float __attribute__((ext_vector_type(16)));
using i32x16_t = int __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMaxUnits = 1024;  // LDS table entries (12 KB)

struct LcArgs {
    int N, C, H, W, K, OH, OW, R, S, sh, sw, ph, pw, dh, dw;
    long long x_img, y_img;  // elements (bytes for int8)
    int units, nss, nkb, KW, ngk;
    long long npix;
};

struct Tap {
    int dr, ds, off;
};

template <typename T> struct Lc;
template <> struct Lc<float> {
    static constexpr int SSU = 8;   // units per step
    static constexpr int NG = 4;    // gathers per lane per step
    using G = float;
    using Acc = f32x16_t;
    static __device__ __forceinline__ int unit(int g, int h) { return 2 * g + h; }
    static __device__ __forceinline__ void mma(Acc& acc, const uint4& a, const G* v, int i) {
        const uint32_t av[4] = {a.x, a.y, a.z, a.w};
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(av[i]), v[i], acc, 0, 0, 0);
    }
    static constexpr int SUB = 4;  // MFMAs per step
};
template <> struct Lc<bf16_t> {
    static constexpr int SSU = 16;
    static constexpr int NG = 8;
    using G = uint16_t;
    using Acc = f32x16_t;
    static __device__ __forceinline__ int unit(int g, int h) { return 8 * h + g; }
    static __device__ __forceinline__ void mma(Acc& acc, const uint4& a, const G* v, int) {
        const uint4 b = make_uint4(v[0] | (static_cast<uint32_t>(v[1]) << 16), v[2] | (static_cast<uint32_t>(v[3]) << 16),
                                   v[4] | (static_cast<uint32_t>(v[5]) << 16), v[6] | (static_cast<uint32_t>(v[7]) << 16));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                      0, 0, 0);
    }
    static constexpr int SUB = 1;
};
template <> struct Lc<int8_t> {
    static constexpr int SSU = 8;  // dwords (32 bytes)
    static constexpr int NG = 4;
    using G = uint32_t;
    using Acc = i32x16_t;
    static __device__ __forceinline__ int unit(int g, int h) { return 4 * h + g; }
    static __device__ __forceinline__ void mma(Acc& acc, const uint4& a, const G* v, int) {
        const i32x4_t av = {static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z), static_cast<int>(a.w)};
        const i32x4_t bv = {static_cast<int>(v[0]), static_cast<int>(v[1]), static_cast<int>(v[2]), static_cast<int>(v[3])};
        acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, acc, 0, 0, 0);
    }
    static constexpr int SUB = 1;
};

// Prepared weights: [k block of 32][step][lane 64][16 bytes].
template <typename T>
__global__ __launch_bounds__(256) void lc_prepare_kernel(const T* __restrict__ w, uint8_t* __restrict__ out, int K,
                                                         int C, int RS, int units, int nkb, int nss) {
    const long long total = static_cast<long long>(nkb) * nss * 64 * 16;  // bytes
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < total; i += static_cast<long long>(gridDim.x) * 256) {
        const int byte = static_cast<int>(i % 16);
        long long t = i / 16;
        const int lane = static_cast<int>(t % 64);
        t /= 64;
        const int ss = static_cast<int>(t % nss);
        const int kb = static_cast<int>(t / nss);
        const int k = kb * 32 + (lane & 31), h = lane >> 5;
        if constexpr (sizeof(T) == 1) {
            const int u = ss * Lc<int8_t>::SSU + Lc<int8_t>::unit(byte / 4, h);  // tap
            const int c = byte % 4;
            int8_t v = 0;
            if (k < K && u < RS && c < C) v = w[(static_cast<long long>(k) * C + c) * RS + u];
            out[i] = static_cast<uint8_t>(v);
        } else {
            constexpr int E = 16 / static_cast<int>(sizeof(T));
            if (byte % sizeof(T) != 0) continue;
            const int e = byte / static_cast<int>(sizeof(T));
            // fp32: element e of the 16 bytes feeds sub-step e; bf16: element e
            const int u = ss * Lc<T>::SSU + Lc<T>::unit(e, h);
            T v{};
            if (k < K && u < units) v = w[static_cast<long long>(k) * units + u];
            *reinterpret_cast<T*>(out + i) = v;
            (void)E;
        }
    }
}

// Workgroup: 4 waves = (4 / KW) pixel groups x KW k groups; a wave owns NCB
// columns blocks of 32 pixels x KBW blocks of 32 output channels.
template <typename T, int XB, int NCB, int KBW>
__global__ __launch_bounds__(256) void lc_kernel(const T* __restrict__ x, const uint8_t* __restrict__ wp,
                                                 const float* __restrict__ scale, T* __restrict__ y, LcArgs a) {
    using L = Lc<T>;
    using G = typename L::G;
    __shared__ Tap tab[kMaxUnits];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 31, h = lane >> 5;

    // reduction unit -> (row delta, column delta, channel offset)
    const int RS = a.R * a.S;
    const int ntab = a.nss * L::SSU;
    for (int u = tid; u < ntab; u += 256) {
        Tap t;
        t.dr = -(1 << 28);  // padding unit: always out of range -> 0
        t.ds = 0;
        t.off = 0;
        const int nu = (sizeof(T) == 1) ? RS : a.units;
        if (u < nu) {
            const int c = (sizeof(T) == 1) ? 0 : u / RS;
            const int tap = (sizeof(T) == 1) ? u : u % RS;
            const int r = tap / a.S, s = tap % a.S;
            t.dr = r * a.dh;
            t.ds = s * a.dw;
            if (sizeof(T) != 1) t.off = (XB == 1) ? c * a.H * a.W : (c / XB) * a.H * a.W * XB + c % XB;
        }
        tab[u] = t;
    }
    __syncthreads();

    const int wk = wave % a.KW, wpx = wave / a.KW;
    const int kg = static_cast<int>(blockIdx.x) % a.ngk;
    const long long pg = static_cast<long long>(blockIdx.x) / a.ngk;
    const int kb0 = (kg * a.KW + wk) * KBW;
    if (kb0 >= a.nkb) return;  // after the only barrier
    const long long P0 = (pg * (4 / a.KW) + wpx) * (NCB * 32);

    // this lane's pixel in each column block
    const int ohw = a.OH * a.OW;
    long long xbase[NCB];
    int ih0[NCB], iw0[NCB];
    bool pok[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const long long G0 = P0 + cb * 32 + j;
        pok[cb] = G0 < a.npix;
        const long long Gc = pok[cb] ? G0 : 0;
        const int n = static_cast<int>(Gc / ohw);
        const int pix = static_cast<int>(Gc - static_cast<long long>(n) * ohw);
        const int oh = pix / a.OW, ow = pix - (pix / a.OW) * a.OW;
        ih0[cb] = oh * a.sh - a.ph;
        iw0[cb] = ow * a.sw - a.pw;
        xbase[cb] = (sizeof(T) == 1) ? n * (a.x_img / 4) : n * a.x_img;
    }

    typename L::Acc acc[KBW][NCB];
#pragma unroll
    for (int b = 0; b < KBW; ++b)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[b][cb] = typename L::Acc{};

    const G* xg = reinterpret_cast<const G*>(x);
    auto gather = [&](int ss, G (*v)[L::NG], uint4* wv) {
#pragma unroll
        for (int g = 0; g < L::NG; ++g) {
            const Tap t = tab[ss * L::SSU + L::unit(g, h)];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const int ih = ih0[cb] + t.dr, iw = iw0[cb] + t.ds;
                const bool ok = static_cast<unsigned>(ih) < static_cast<unsigned>(a.H) &&
                                static_cast<unsigned>(iw) < static_cast<unsigned>(a.W);
                const long long pix = static_cast<long long>(ih) * a.W + iw;
                const long long o = xbase[cb] + t.off + ((sizeof(T) == 1) ? pix : pix * XB);
                const G val = xg[ok ? o : 0];
                v[cb][g] = ok ? val : G{};
            }
        }
#pragma unroll
        for (int b = 0; b < KBW; ++b)
            wv[b] = *reinterpret_cast<const uint4*>(wp + ((static_cast<long long>(kb0 + b) * a.nss + ss) * 64 + lane) * 16);
    };
    auto compute = [&](G (*v)[L::NG], const uint4* wv) {
#pragma unroll
        for (int i = 0; i < L::SUB; ++i)
#pragma unroll
            for (int b = 0; b < KBW; ++b)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) L::mma(acc[b][cb], wv[b], v[cb], i);
    };

    G va[NCB][L::NG], vb[NCB][L::NG];
    uint4 wa[KBW], wb[KBW];
    gather(0, va, wa);
    int ss = 0;
    for (; ss + 2 < a.nss; ss += 2) {
        gather(ss + 1, vb, wb);
        compute(va, wa);
        gather(ss + 2, va, wa);
        compute(vb, wb);
    }
    gather(ss + 1, vb, wb);
    compute(va, wa);
    compute(vb, wb);

    // D[row = channel][col = pixel]: lane (j, hh), element v -> channel
    // 8 (v / 4) + 4 hh + v % 4 of the block
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        if (!pok[cb]) continue;
        const long long G0 = P0 + cb * 32 + j;
        const int n = static_cast<int>(G0 / ohw);
        const int pix = static_cast<int>(G0 - static_cast<long long>(n) * ohw);
        const int oh = pix / a.OW, ow = pix - (pix / a.OW) * a.OW;
#pragma unroll
        for (int b = 0; b < KBW; ++b) {
            if constexpr (sizeof(T) == 1) {
                // four consecutive channels of one pixel -> one NCHW4 dword
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int k0 = (kb0 + b) * 32 + 8 * q + 4 * h;
                    if (k0 >= a.K) continue;
                    uint32_t word = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int k = k0 + e;
                        const int8_t r8 = (k < a.K) ? requant_i8(acc[b][cb][4 * q + e], scale[k]) : int8_t(0);
                        word |= static_cast<uint32_t>(static_cast<uint8_t>(r8)) << (8 * e);
                    }
                    uint8_t* yb = reinterpret_cast<uint8_t*>(y) + n * a.y_img;
                    *reinterpret_cast<uint32_t*>(yb + (static_cast<long long>(k0 / 4) * ohw + pix) * 4) = word;
                }
            } else {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int k = (kb0 + b) * 32 + 8 * (v / 4) + 4 * h + (v % 4);
                    if (k >= a.K) continue;
                    T* dst = y + n * a.y_img + act_off<XB>(k, oh, ow, a.OH, a.OW);
                    if constexpr (sizeof(T) == 4)
                        *dst = acc[b][cb][v];
                    else
                        dst->bits = float_to_bf16(acc[b][cb][v]);
                }
            }
        }
    }
}

struct LcCfg {
    int ncb, kbw;
};
constexpr LcCfg kLc[6] = {{4, 1}, {2, 2}, {4, 2}, {1, 1}, {1, 2}, {2, 1}};
constexpr int kLcN = 6;

bool lc_geometry(const Prob& p, int cfg, LcArgs* a, std::string* why) {
    auto fail = [&](const char* m) {
        if (why) *why = m;
        return false;
    };
    if (cfg < 0 || cfg >= kLcN) return fail("implicit GEMM (gather): no such config");
    if (p.g != 1) return fail("implicit GEMM (gather): groups must be 1");
    int units, ssu;
    if (p.dtype == CFWD_I8) {
        if (p.layout != CFWD_LAYOUT_NCHWX || p.xb != 4 || p.c > 4)
            return fail("implicit GEMM (gather): int8 needs NCHW4 with C <= 4");
        units = p.r * p.s;
        ssu = Lc<int8_t>::SSU;
    } else {
        units = p.c * p.r * p.s;
        ssu = (p.dtype == CFWD_F32) ? Lc<float>::SSU : Lc<bf16_t>::SSU;
    }
    int nss = (units + ssu - 1) / ssu;
    nss += nss & 1;
    if (nss * ssu > kMaxUnits) return fail("implicit GEMM (gather): C*R*S too large");
    if (static_cast<long long>(p.h) * p.w * p.c >= (1LL << 31) || static_cast<long long>(p.oh) * p.ow >= (1LL << 31))
        return fail("implicit GEMM (gather): image too large");
    a->N = p.n; a->C = p.c; a->H = p.h; a->W = p.w; a->K = p.k; a->OH = p.oh; a->OW = p.ow;
    a->R = p.r; a->S = p.s; a->sh = p.sh; a->sw = p.sw; a->ph = p.ph; a->pw = p.pw; a->dh = p.dh; a->dw = p.dw;
    a->x_img = p.x_img; a->y_img = p.y_img;
    a->units = units;
    a->nss = nss;
    const int kbw = kLc[cfg].kbw;
    const int kwaves = ((p.k + 31) / 32 + kbw - 1) / kbw;
    a->nkb = kwaves * kbw;
    a->KW = kwaves >= 4 ? 4 : (kwaves >= 2 ? 2 : 1);
    a->ngk = (kwaves + a->KW - 1) / a->KW;
    a->npix = static_cast<long long>(p.n) * p.oh * p.ow;
    const long long per_wg = static_cast<long long>(4 / a->KW) * kLc[cfg].ncb * 32;
    const long long pgroups = (a->npix + per_wg - 1) / per_wg;
    if (pgroups * a->ngk >= (1LL << 31)) return fail("implicit GEMM (gather): grid too large");
    return true;
}

template <typename T, int XB>
cfwd_status lc_launch_t(int cfg, const LcArgs& a, const void* x, const void* wp, const float* scale, void* y,
                        hipStream_t st) {
    const long long per_wg = static_cast<long long>(4 / a.KW) * kLc[cfg].ncb * 32;
    const unsigned blocks = static_cast<unsigned>((a.npix + per_wg - 1) / per_wg * a.ngk);
    const T* xt = static_cast<const T*>(x);
    const uint8_t* w8 = static_cast<const uint8_t*>(wp);
    T* yt = static_cast<T*>(y);
    switch (cfg) {
        case 0: lc_kernel<T, XB, 4, 1><<<blocks, 256, 0, st>>>(xt, w8, scale, yt, a); break;
        case 1: lc_kernel<T, XB, 2, 2><<<blocks, 256, 0, st>>>(xt, w8, scale, yt, a); break;
        case 2: lc_kernel<T, XB, 4, 2><<<blocks, 256, 0, st>>>(xt, w8, scale, yt, a); break;
        case 3: lc_kernel<T, XB, 1, 1><<<blocks, 256, 0, st>>>(xt, w8, scale, yt, a); break;
        case 4: lc_kernel<T, XB, 1, 2><<<blocks, 256, 0, st>>>(xt, w8, scale, yt, a); break;
        default: lc_kernel<T, XB, 2, 1><<<blocks, 256, 0, st>>>(xt, w8, scale, yt, a); break;
    }
    return check_hip(hipGetLastError(), "implicit GEMM (gather) launch");
}

template <typename T>
cfwd_status lc_launch_layout(const Prob& p, int cfg, const LcArgs& a, const void* x, const void* wp,
                             const float* scale, void* y, hipStream_t st) {
    switch (p.xb) {
        case 1: return lc_launch_t<T, 1>(cfg, a, x, wp, scale, y, st);
        case 4: return lc_launch_t<T, 4>(cfg, a, x, wp, scale, y, st);
        case 8: return lc_launch_t<T, 8>(cfg, a, x, wp, scale, y, st);
        default: return set_error(CFWD_ERR_UNSUPPORTED, "implicit GEMM (gather): bad channel block");
    }
}

}  // namespace

int lowc_num_configs() { return kLcN; }

bool lowc_supported(const Prob& p, int cfg, std::string* why) {
    LcArgs a;
    return lc_geometry(p, cfg, &a, why);
}

size_t lowc_filter_bytes(const Prob& p, int cfg) {
    LcArgs a;
    if (!lc_geometry(p, cfg, &a, nullptr)) return 0;
    return static_cast<size_t>(a.nkb) * a.nss * 64 * 16;
}

cfwd_status lowc_prepare(const Prob& p, int cfg, const void* w, void* wp, hipStream_t st) {
    LcArgs a;
    std::string why;
    if (!lc_geometry(p, cfg, &a, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    const long long total = static_cast<long long>(a.nkb) * a.nss * 64 * 16;
    const unsigned blocks = static_cast<unsigned>(std::min<long long>((total + 255) / 256, 65536));
    uint8_t* out = static_cast<uint8_t*>(wp);
    const int RS = p.r * p.s;
    if (p.dtype == CFWD_F32)
        lc_prepare_kernel<float><<<blocks, 256, 0, st>>>(static_cast<const float*>(w), out, p.k, p.c, RS, a.units,
                                                         a.nkb, a.nss);
    else if (p.dtype == CFWD_BF16)
        lc_prepare_kernel<bf16_t><<<blocks, 256, 0, st>>>(static_cast<const bf16_t*>(w), out, p.k, p.c, RS, a.units,
                                                          a.nkb, a.nss);
    else
        lc_prepare_kernel<int8_t><<<blocks, 256, 0, st>>>(static_cast<const int8_t*>(w), out, p.k, p.c, RS, a.units,
                                                          a.nkb, a.nss);
    return check_hip(hipGetLastError(), "implicit GEMM (gather) filter prepare launch");
}

cfwd_status lowc_launch(const Prob& p, int cfg, const void* x, const void* wp, const float* scale, void* y,
                        hipStream_t st) {
    LcArgs a;
    std::string why;
    if (!lc_geometry(p, cfg, &a, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    if (wp == nullptr) return set_error(CFWD_ERR_WORKSPACE, "implicit GEMM (gather): prepared filter required");
    if (p.dtype == CFWD_F32) return lc_launch_layout<float>(p, cfg, a, x, wp, scale, y, st);
    if (p.dtype == CFWD_BF16) return lc_launch_layout<bf16_t>(p, cfg, a, x, wp, scale, y, st);
    return lc_launch_t<int8_t, 4>(cfg, a, x, wp, scale, y, st);
}

}  // namespace cfwd
