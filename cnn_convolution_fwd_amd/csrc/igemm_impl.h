// Implicit-GEMM convolution on the gfx950 matrix cores (template; included by
// the per-dtype translation units k_igemm_{f32,bf16,i8}.hip).
//
// The MegEngine inference article (section "Im2col+MatMul") rewrites the
// convolution as a matrix product of the weights with the im2col matrix
// [n, fh*fw*ic, oh*ow], then fixes its two costs: the im2col data is several
// to tens of times the input and overflows the cache, so it is blocked along
// oh*ow ("分块操作"); and the matmul re-packs it, so the pack is fused into
// im2col ("融合 PACK").  On the GPU the same two ideas become:
//   * the im2col matrix is never built: a workgroup owns a block of output
//     pixels (TN images x TH rows x TW columns) and stages only the input patch
//     those pixels read -- (TH-1)*sh + (R-1)*dh + 1 rows by
//     (TW-1)*sw + (S-1)*dw + 1 columns, one 64-byte chunk of channels at a
//     time -- in LDS.  Every filter tap (r, s) then reads its A operand from the
//     same patch at a shifted address, so each input byte comes from HBM once
//     per chunk instead of R*S times;
//   * the patch is written to LDS already in the matrix-core operand order
//     (channel-innermost, 16 bytes per lane), which is the fused pack: the
//     transpose from NCHW happens in the staging copy itself.
//
// GEMM view: M = output pixels (rows of A = the patch), N = output channels
// (columns of B = the prepared weights), K = (channel chunk, r, s).
// Matrix-core instruction per 64-byte K slice and 16x16 output fragment:
//   bf16: one v_mfma_f32_16x16x32_bf16    (fp32 accumulate)
//   int8: one v_mfma_i32_16x16x64_i8      (int32 accumulate)
//   fp32: four v_mfma_f32_16x16x4_f32     (fp32 accumulate)
// Each lane feeds 16 bytes of K (lane / 16 selects which 16 bytes) for the
// A row (lane % 16) and the B column (lane % 16); the hardware pairs equal
// register slots of A and B, so A and B only need the same K order.
// Fragment D[i][j] comes back as lane (j + 16*(i/4)), element i % 4.
//
// Workgroup: WM x WN waves; wave (wm, wn) owns FM x FN fragments.  Tile =
// (WM*FM*16 pixels) x (WN*FN*16 channels).  The LDS patch is double-buffered:
// chunk c+1 is loaded into registers while chunk c is multiplied, then stored.
// Weights (prepared: [g][ntile][chunk][r*s][NT][64 B]) are read straight from
// L2 into registers, one tap ahead.
#pragma once

#include "internal.h"

namespace cfwd {
namespace ig {

struct Args {
    const void* x;
    const void* wp;
    const float* scale;
    void* y;
    int N, C, H, W, K, OH, OW, Cg, Kg, R, S, sh, sw, ph, pw, dh, dw;
    long long x_img, y_img;
    int TN, TH, TW, PH, PW, npix;  // output tile and its input patch
    int tiles_w, tiles_h;
    int nchunks, ntk;              // channel chunks, output-channel tiles
};

template <typename T> struct Mma;
template <> struct Mma<bf16_t> {
    using acc_t = f32x4;
    static __device__ __forceinline__ void run(acc_t& c, const uint4& a, const uint4& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                    0, 0);
    }
};
template <> struct Mma<int8_t> {
    using acc_t = i32x4;
    static __device__ __forceinline__ void run(acc_t& c, const uint4& a, const uint4& b) {
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0,
                                                  0);
    }
};
template <> struct Mma<float> {
    using acc_t = f32x4;
    static __device__ __forceinline__ void run(acc_t& c, const uint4& a, const uint4& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    }
};

// Raw storage element of each dtype.
template <typename T> struct Raw;
template <> struct Raw<float> { using type = uint32_t; };
template <> struct Raw<bf16_t> { using type = uint16_t; };
template <> struct Raw<int8_t> { using type = uint8_t; };

// Pack E16 raw elements into 16 bytes.
template <typename R>
__device__ __forceinline__ uint4 pack16(const R* v) {
    uint32_t w[4];
    constexpr int per = 4 / sizeof(R);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t acc = 0;
#pragma unroll
        for (int j = 0; j < per; ++j) acc |= static_cast<uint32_t>(v[i * per + j]) << (8 * sizeof(R) * j);
        w[i] = acc;
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// 16 bytes of activations: channels c0 .. c0+E16-1 of one pixel, zeros where
// the channel is past the group (nval) or the pixel is outside the image.
// `sp` is the spatial offset (ih*W + iw) inside the image.
template <typename T, int XB>
__device__ __forceinline__ uint4 load_unit(const T* __restrict__ xn, int H, int W, int c0, int nval, int sp) {
    using R = typename Raw<T>::type;
    constexpr int E16 = 16 / static_cast<int>(sizeof(T));
    const R* xr = reinterpret_cast<const R*>(xn);
    const long long HW = static_cast<long long>(H) * W;
    if (XB > 1 && nval >= E16 && (c0 % E16) == 0) {
        if (E16 <= XB) {
            const R* p = xr + (static_cast<long long>(c0 / XB) * HW + sp) * XB + (c0 % XB);
            return *reinterpret_cast<const uint4*>(p);
        }
        // E16 > XB: E16/XB channel blocks, XB elements each.
        constexpr int NB = E16 / (XB > 1 ? XB : 1);
        R v[E16];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const R* p = xr + (static_cast<long long>(c0 / XB + b) * HW + sp) * XB;
#pragma unroll
            for (int e = 0; e < XB; ++e) v[b * XB + e] = p[e];
        }
        return pack16<R>(v);
    }
    R v[E16];
#pragma unroll
    for (int e = 0; e < E16; ++e) {
        R val = 0;
        if (e < nval) {
            const int c = c0 + e;
            if (XB == 1)
                val = xr[static_cast<long long>(c) * HW + sp];
            else
                val = xr[(static_cast<long long>(c / XB) * HW + sp) * XB + (c % XB)];
        }
        v[e] = val;
    }
    return pack16<R>(v);
}

template <typename T> __device__ __forceinline__ void store_out(T* y, long long off, typename Mma<T>::acc_t acc,
                                                               int v, float scale);
template <> __device__ __forceinline__ void store_out<float>(float* y, long long off, f32x4 acc, int v, float) {
    y[off] = acc[v];
}
template <> __device__ __forceinline__ void store_out<bf16_t>(bf16_t* y, long long off, f32x4 acc, int v, float) {
    y[off].bits = float_to_bf16(acc[v]);
}
template <> __device__ __forceinline__ void store_out<int8_t>(int8_t* y, long long off, i32x4 acc, int v,
                                                              float scale) {
    y[off] = requant_i8(acc[v], scale);
}

constexpr int kMaxUnitsPerThread = 8;

// LDS byte offset of 16-byte slot j of patch pixel q.  The XOR with bits 1..2
// of q spreads the 8 lanes of one ds_read_b128 phase (consecutive pixels,
// same j) over all 32 banks.
__device__ __forceinline__ int lds_slot(int q, int j) { return q * 64 + ((j ^ ((q >> 1) & 3)) << 4); }

template <typename T, int XB, int WM, int WN, int FM, int FN>
__global__ __launch_bounds__(WM* WN * 64) void igemm_kernel(Args a) {
    constexpr int NTHR = WM * WN * 64;
    constexpr int NT = WN * FN * 16;
    constexpr int E16 = 16 / static_cast<int>(sizeof(T));
    constexpr int CK = 4 * E16;
    constexpr int MAXU = kMaxUnitsPerThread;
    using acc_t = typename Mma<T>::acc_t;

    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WM;
    const int wn = wave / WM;
    const int jl = lane >> 4;

    int mt = blockIdx.x;
    const int tw_i = mt % a.tiles_w;
    mt /= a.tiles_w;
    const int th_i = mt % a.tiles_h;
    mt /= a.tiles_h;
    const int n0 = mt * a.TN;
    const int oh0 = th_i * a.TH;
    const int ow0 = tw_i * a.TW;
    const int kt = blockIdx.y;
    const int g = blockIdx.z;
    const int RS = a.R * a.S;
    const int PHW = a.PH * a.PW;
    const int thw = a.TH * a.TW;
    const int tile_pix = a.TN * thw;
    const int patch_bytes = a.npix * 64;
    const int ih0 = oh0 * a.sh - a.ph;
    const int iw0 = ow0 * a.sw - a.pw;
    const T* __restrict__ x = static_cast<const T*>(a.x);

    // ---- staging units owned by this thread (chunk-invariant parts)
    const int nunits = 4 * a.npix;
    int u_lds[MAXU];     // LDS byte offset (swizzled), -1 if no unit
    int u_j[MAXU];       // 16-byte slot within the 64-byte channel chunk
    int u_sp[MAXU];      // spatial offset ih*W+iw, -1 if outside the image
    int u_n[MAXU];       // image
#pragma unroll
    for (int i = 0; i < MAXU; ++i) {
        const int u = tid + i * NTHR;
        u_lds[i] = -1;
        u_j[i] = 0;
        u_sp[i] = -1;
        u_n[i] = 0;
        if (u < nunits) {
            const int j = u / a.npix;
            const int q = u - j * a.npix;
            const int tn = q / PHW;
            const int rem = q - tn * PHW;
            const int prow = rem / a.PW;
            const int pcol = rem - prow * a.PW;
            const int n = n0 + tn;
            const int ih = ih0 + prow;
            const int iw = iw0 + pcol;
            u_lds[i] = lds_slot(q, j);
            u_j[i] = j;
            u_n[i] = n;
            if (n < a.N && static_cast<unsigned>(ih) < static_cast<unsigned>(a.H) &&
                static_cast<unsigned>(iw) < static_cast<unsigned>(a.W))
                u_sp[i] = ih * a.W + iw;
        }
    }

    uint4 stg[MAXU];
    auto stage_load = [&](int chunk) {
#pragma unroll
        for (int i = 0; i < MAXU; ++i) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (u_sp[i] >= 0) {
                const int cl = chunk * CK + u_j[i] * E16;
                const int nval = a.Cg - cl;
                if (nval > 0)
                    v = load_unit<T, XB>(x + u_n[i] * a.x_img, a.H, a.W, g * a.Cg + cl, nval, u_sp[i]);
            }
            stg[i] = v;
        }
    };
    auto stage_store = [&](int buf) {
        uint8_t* base = lds + buf * patch_bytes;
#pragma unroll
        for (int i = 0; i < MAXU; ++i)
            if (u_lds[i] >= 0) *reinterpret_cast<uint4*>(base + u_lds[i]) = stg[i];
    };

    // ---- per-lane A fragment bases (pixel index inside the patch)
    int qbase[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f) {
        const int p = (wm * FM + f) * 16 + (lane & 15);
        int qb = 0;
        if (p < tile_pix) {
            const int tn = p / thw;
            const int rem = p - tn * thw;
            const int ohl = rem / a.TW;
            const int owl = rem - ohl * a.TW;
            qb = tn * PHW + ohl * a.sh * a.PW + owl * a.sw;
        }
        qbase[f] = qb;
    }

    // ---- B (prepared weights) addressing
    const uint8_t* __restrict__ wtile =
        static_cast<const uint8_t*>(a.wp) +
        static_cast<long long>(g * a.ntk + kt) * a.nchunks * RS * NT * 64 +
        static_cast<long long>(wn * FN * 16 + (lane & 15)) * 64 + jl * 16;
    auto load_b = [&](uint4* b, int it) {
        const uint8_t* p = wtile + static_cast<long long>(it) * NT * 64;
#pragma unroll
        for (int nf = 0; nf < FN; ++nf) b[nf] = *reinterpret_cast<const uint4*>(p + nf * 16 * 64);
    };

    acc_t acc[FM][FN];
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int nf = 0; nf < FN; ++nf) acc[f][nf] = acc_t{0, 0, 0, 0};

    stage_load(0);
    stage_store(0);
    __syncthreads();

    uint4 bcur[FN], bnxt[FN];
    load_b(bcur, 0);
    const int total_it = a.nchunks * RS;
    int it = 0;
    for (int chunk = 0; chunk < a.nchunks; ++chunk) {
        const int buf = chunk & 1;
        const bool more = chunk + 1 < a.nchunks;
        if (more) stage_load(chunk + 1);
        const uint8_t* pb = lds + buf * patch_bytes;
        int r = 0, s = 0;
        for (int rs = 0; rs < RS; ++rs, ++it) {
            if (it + 1 < total_it) load_b(bnxt, it + 1);
            const int toff = r * a.dh * a.PW + s * a.dw;
            uint4 afr[FM];
#pragma unroll
            for (int f = 0; f < FM; ++f) {
                const int q = qbase[f] + toff;
                afr[f] = *reinterpret_cast<const uint4*>(pb + lds_slot(q, jl));
            }
#pragma unroll
            for (int f = 0; f < FM; ++f)
#pragma unroll
                for (int nf = 0; nf < FN; ++nf) Mma<T>::run(acc[f][nf], afr[f], bcur[nf]);
#pragma unroll
            for (int nf = 0; nf < FN; ++nf) bcur[nf] = bnxt[nf];
            if (++s == a.S) {
                s = 0;
                ++r;
            }
        }
        if (more) stage_store(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: convert and store in the caller's layout
    T* __restrict__ y = static_cast<T*>(a.y);
#pragma unroll
    for (int nf = 0; nf < FN; ++nf) {
        const int kl = kt * NT + (wn * FN + nf) * 16 + (lane & 15);
        if (kl >= a.Kg) continue;
        const int k = g * a.Kg + kl;
        const float sc = (a.scale != nullptr) ? a.scale[k] : 1.0f;
#pragma unroll
        for (int f = 0; f < FM; ++f) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int p = (wm * FM + f) * 16 + 4 * jl + v;
                if (p >= tile_pix) continue;
                const int tn = p / thw;
                const int rem = p - tn * thw;
                const int ohl = rem / a.TW;
                const int owl = rem - ohl * a.TW;
                const int n = n0 + tn;
                const int oh = oh0 + ohl;
                const int ow = ow0 + owl;
                if (n >= a.N || oh >= a.OH || ow >= a.OW) continue;
                store_out<T>(y, n * a.y_img + act_off<XB>(k, oh, ow, a.OH, a.OW), acc[f][nf], v, sc);
            }
        }
    }
}

// Weight preparation: KCRS -> [g][ntile][chunk][r*s][NT][CK], zero padded.
template <typename T, int NT>
__global__ __launch_bounds__(256) void igemm_prepare_kernel(const T* __restrict__ w, T* __restrict__ wp, int G,
                                                            int Kg, int Cg, int RS, int ntk, int nchunks) {
    constexpr int CK = 64 / static_cast<int>(sizeof(T));
    using R = typename Raw<T>::type;
    const long long total = static_cast<long long>(G) * ntk * nchunks * RS * NT * CK;
    const R* wr = reinterpret_cast<const R*>(w);
    R* out = reinterpret_cast<R*>(wp);
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < total; i += static_cast<long long>(gridDim.x) * 256) {
        long long t = i;
        const int cc = static_cast<int>(t % CK); t /= CK;
        const int kk = static_cast<int>(t % NT); t /= NT;
        const int rs = static_cast<int>(t % RS); t /= RS;
        const int chunk = static_cast<int>(t % nchunks); t /= nchunks;
        const int kt = static_cast<int>(t % ntk); t /= ntk;
        const int g = static_cast<int>(t);
        const int kl = kt * NT + kk;
        const int cl = chunk * CK + cc;
        R v = 0;
        if (kl < Kg && cl < Cg) v = wr[(static_cast<long long>(g * Kg + kl) * Cg + cl) * RS + rs];
        out[i] = v;
    }
}

// ---------------------------------------------------------------- host side

struct Cfg {
    int wm, wn, fm, fn;
    int threads() const { return wm * wn * 64; }
    int pixels() const { return wm * fm * 16; }
    int nt() const { return wn * fn * 16; }
};

// Tile configurations, in config-id order.
constexpr Cfg kCfgs[] = {
    {2, 2, 4, 4},  // 0: 128 px x 128 ch
    {2, 2, 7, 4},  // 1: 224 px x 128 ch
    {2, 2, 4, 2},  // 2: 128 px x  64 ch
    {2, 2, 2, 2},  // 3:  64 px x  64 ch
    {4, 1, 2, 4},  // 4: 128 px x  64 ch
    {2, 2, 7, 2},  // 5: 224 px x  64 ch
    {2, 2, 2, 4},  // 6:  64 px x 128 ch
};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

struct Geo {
    int TN, TH, TW, PH, PW, npix, tiles_n, tiles_h, tiles_w, nchunks, ntk;
    size_t lds_bytes;
};

inline bool geometry(const Prob& p, const Cfg& c, Geo* g, std::string* why) {
    const int P = c.pixels();
    const int CK = 64 / p.esize;
    int TN, TH, TW;
    if (p.oh * p.ow <= P) {
        TN = std::min(p.n, P / (p.oh * p.ow));
        TH = p.oh;
        TW = p.ow;
    } else if (p.ow <= P) {
        TN = 1;
        TW = p.ow;
        TH = std::min(p.oh, P / p.ow);
    } else {
        TN = 1;
        TH = 1;
        TW = P;
    }
    const int maxpix = kMaxUnitsPerThread * c.threads() / 4;
    for (;;) {
        const int PH = (TH - 1) * p.sh + (p.r - 1) * p.dh + 1;
        const int PW = (TW - 1) * p.sw + (p.s - 1) * p.dw + 1;
        const long long npix = static_cast<long long>(TN) * PH * PW;
        if (npix <= maxpix) {
            g->TN = TN;
            g->TH = TH;
            g->TW = TW;
            g->PH = PH;
            g->PW = PW;
            g->npix = static_cast<int>(npix);
            break;
        }
        if (TN > 1)
            --TN;
        else if (TH > 1)
            --TH;
        else if (TW > 16)
            TW = (TW + 1) / 2;
        else {
            if (why) *why = "implicit GEMM: the input patch of one output row does not fit this tile config";
            return false;
        }
    }
    g->tiles_n = (p.n + g->TN - 1) / g->TN;
    g->tiles_h = (p.oh + g->TH - 1) / g->TH;
    g->tiles_w = (p.ow + g->TW - 1) / g->TW;
    g->nchunks = (p.cg + CK - 1) / CK;
    g->ntk = (p.kg + c.nt() - 1) / c.nt();
    g->lds_bytes = 2 * static_cast<size_t>(g->npix) * 64;
    if (static_cast<long long>(g->tiles_n) * g->tiles_h * g->tiles_w > 0x7fffffffLL || g->ntk > 65535 ||
        p.g > 65535) {
        if (why) *why = "implicit GEMM: grid too large";
        return false;
    }
    return true;
}

inline size_t filter_bytes(const Prob& p, const Cfg& c, const Geo& g) {
    return static_cast<size_t>(p.g) * g.ntk * g.nchunks * p.r * p.s * c.nt() * 64;
}

template <typename T, int XB, int WM, int WN, int FM, int FN>
cfwd_status launch_one(const Prob& p, const Geo& g, const void* x, const void* wp, const float* scale, void* y,
                       hipStream_t st) {
    Args a;
    a.x = x;
    a.wp = wp;
    a.scale = scale;
    a.y = y;
    a.N = p.n; a.C = p.c; a.H = p.h; a.W = p.w; a.K = p.k; a.OH = p.oh; a.OW = p.ow;
    a.Cg = p.cg; a.Kg = p.kg; a.R = p.r; a.S = p.s;
    a.sh = p.sh; a.sw = p.sw; a.ph = p.ph; a.pw = p.pw; a.dh = p.dh; a.dw = p.dw;
    a.x_img = p.x_img; a.y_img = p.y_img;
    a.TN = g.TN; a.TH = g.TH; a.TW = g.TW; a.PH = g.PH; a.PW = g.PW; a.npix = g.npix;
    a.tiles_w = g.tiles_w; a.tiles_h = g.tiles_h;
    a.nchunks = g.nchunks; a.ntk = g.ntk;
    auto kern = igemm_kernel<T, XB, WM, WN, FM, FN>;
    static bool attr_done = false;
    if (g.lds_bytes > 65536 && !attr_done) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return check_hip(e, "hipFuncSetAttribute(igemm)");
        attr_done = true;
    }
    const dim3 grid(static_cast<unsigned>(g.tiles_n * g.tiles_h * g.tiles_w), static_cast<unsigned>(g.ntk),
                    static_cast<unsigned>(p.g));
    kern<<<grid, WM * WN * 64, g.lds_bytes, st>>>(a);
    return check_hip(hipGetLastError(), "igemm_kernel launch");
}

template <typename T, int XB>
cfwd_status launch_cfg(int cfg, const Prob& p, const Geo& g, const void* x, const void* wp, const float* scale,
                       void* y, hipStream_t st) {
    switch (cfg) {
#define CFWD_IG_CFG(ID)                                                                                     \
    case ID:                                                                                                \
        return launch_one<T, XB, kCfgs[ID].wm, kCfgs[ID].wn, kCfgs[ID].fm, kCfgs[ID].fn>(p, g, x, wp, scale, y, \
                                                                                          st);
        CFWD_IG_CFG(0)
        CFWD_IG_CFG(1)
        CFWD_IG_CFG(2)
        CFWD_IG_CFG(3)
        CFWD_IG_CFG(4)
        CFWD_IG_CFG(5)
        CFWD_IG_CFG(6)
#undef CFWD_IG_CFG
        default:
            return set_error(CFWD_ERR_UNSUPPORTED, "implicit GEMM: no such config");
    }
}

template <typename T>
cfwd_status launch_dtype(int cfg, const Prob& p, const Geo& g, const void* x, const void* wp, const float* scale,
                         void* y, hipStream_t st) {
    switch (p.xb) {
        case 1: return launch_cfg<T, 1>(cfg, p, g, x, wp, scale, y, st);
        case 4: return launch_cfg<T, 4>(cfg, p, g, x, wp, scale, y, st);
        case 8: return launch_cfg<T, 8>(cfg, p, g, x, wp, scale, y, st);
        default: return set_error(CFWD_ERR_UNSUPPORTED, "implicit GEMM: channel block must be 1, 4 or 8");
    }
}

template <typename T>
cfwd_status prepare_dtype(int cfg, const Prob& p, const Geo& g, const void* w, void* wp, hipStream_t st) {
    const long long total = static_cast<long long>(p.g) * g.ntk * g.nchunks * p.r * p.s * kCfgs[cfg].nt() *
                            (64 / static_cast<int>(sizeof(T)));
    long long blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    const int nt = kCfgs[cfg].nt();
    if (nt == 128)
        igemm_prepare_kernel<T, 128><<<static_cast<unsigned>(blocks), 256, 0, st>>>(
            static_cast<const T*>(w), static_cast<T*>(wp), p.g, p.kg, p.cg, p.r * p.s, g.ntk, g.nchunks);
    else if (nt == 64)
        igemm_prepare_kernel<T, 64><<<static_cast<unsigned>(blocks), 256, 0, st>>>(
            static_cast<const T*>(w), static_cast<T*>(wp), p.g, p.kg, p.cg, p.r * p.s, g.ntk, g.nchunks);
    else
        return set_error(CFWD_ERR_UNSUPPORTED, "implicit GEMM: unexpected N tile");
    return check_hip(hipGetLastError(), "igemm_prepare launch");
}

}  // namespace ig

// Per-dtype entry points (defined in k_igemm_{f32,bf16,i8}.hip).
cfwd_status igemm_launch_f32(int cfg, const Prob& p, const ig::Geo& g, const void* x, const void* wp,
                             const float* scale, void* y, hipStream_t st);
cfwd_status igemm_launch_bf16(int cfg, const Prob& p, const ig::Geo& g, const void* x, const void* wp,
                              const float* scale, void* y, hipStream_t st);
cfwd_status igemm_launch_i8(int cfg, const Prob& p, const ig::Geo& g, const void* x, const void* wp,
                            const float* scale, void* y, hipStream_t st);
cfwd_status igemm_prepare_f32(int cfg, const Prob& p, const ig::Geo& g, const void* w, void* wp, hipStream_t st);
cfwd_status igemm_prepare_bf16(int cfg, const Prob& p, const ig::Geo& g, const void* w, void* wp, hipStream_t st);
cfwd_status igemm_prepare_i8(int cfg, const Prob& p, const ig::Geo& g, const void* w, void* wp, hipStream_t st);

}  // namespace cfwd
