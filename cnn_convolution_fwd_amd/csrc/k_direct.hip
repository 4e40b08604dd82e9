// Direct-summation convolution on the vector ALUs (gfx950).
//
// The MegEngine inference article (section "Fast-Run") lists direct
// convolution as one of the implementations Fast-Run chooses between; the
// Momenta talk (section "優化2：Depthwise卷積") explains why depthwise layers are
// memory-bound: each loaded input feeds one output channel only, so the kernel
// is shaped for HBM bandwidth (wide coalesced loads, every input byte read
// from HBM once), not for the matrix cores.
//
// config 0: generic -- one thread per output element, any shape / layout /
//           dtype / groups.  The correctness fallback.
// config 1: depthwise 3x3, stride 1, dilation 1, NCHW, W a multiple of the
//           vector width -- each thread owns a strip of VEC columns and walks
//           ROWS output rows down it, keeping the three input rows it needs in
//           registers (a register-blocked sliding window).
#include "internal.h"

namespace cfwd {

namespace {

struct DirectArgs {
    int N, C, H, W, K, OH, OW, Cg, Kg, R, S, sh, sw, ph, pw, dh, dw;
    long long x_img, y_img;
};

template <typename T> __device__ __forceinline__ T store_cast(float v);
template <> __device__ __forceinline__ float store_cast<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t store_cast<bf16_t>(float v) { return bf16_t{float_to_bf16(v)}; }

// ------------------------------------------------------------ config 0

template <typename T, int XB>
__global__ __launch_bounds__(256) void direct_generic(const T* __restrict__ x, const T* __restrict__ w,
                                                      T* __restrict__ y, DirectArgs a) {
    const long long total = static_cast<long long>(a.N) * a.K * a.OH * a.OW;
    for (long long idx = blockIdx.x * 256LL + threadIdx.x; idx < total;
         idx += static_cast<long long>(gridDim.x) * 256) {
        long long t = idx;
        const int ow = static_cast<int>(t % a.OW); t /= a.OW;
        const int oh = static_cast<int>(t % a.OH); t /= a.OH;
        const int k = static_cast<int>(t % a.K); t /= a.K;
        const int n = static_cast<int>(t);
        const int g = k / a.Kg;
        const T* xn = x + n * a.x_img;
        float acc = 0.0f;
        for (int cl = 0; cl < a.Cg; ++cl) {
            const int c = g * a.Cg + cl;
            for (int r = 0; r < a.R; ++r) {
                const int ih = oh * a.sh - a.ph + r * a.dh;
                if (ih < 0 || ih >= a.H) continue;
                for (int s = 0; s < a.S; ++s) {
                    const int iw = ow * a.sw - a.pw + s * a.dw;
                    if (iw < 0 || iw >= a.W) continue;
                    const float xv = Elem<T>::to_f(xn[act_off<XB>(c, ih, iw, a.H, a.W)]);
                    const float wv = Elem<T>::to_f(w[((static_cast<long long>(k) * a.Cg + cl) * a.R + r) * a.S + s]);
                    acc = fmaf(xv, wv, acc);
                }
            }
        }
        y[n * a.y_img + act_off<XB>(k, oh, ow, a.OH, a.OW)] = store_cast<T>(acc);
    }
}

template <int XB>
__global__ __launch_bounds__(256) void direct_generic_i8(const int8_t* __restrict__ x, const int8_t* __restrict__ w,
                                                         const float* __restrict__ scale, int8_t* __restrict__ y,
                                                         DirectArgs a) {
    const long long total = static_cast<long long>(a.N) * a.K * a.OH * a.OW;
    for (long long idx = blockIdx.x * 256LL + threadIdx.x; idx < total;
         idx += static_cast<long long>(gridDim.x) * 256) {
        long long t = idx;
        const int ow = static_cast<int>(t % a.OW); t /= a.OW;
        const int oh = static_cast<int>(t % a.OH); t /= a.OH;
        const int k = static_cast<int>(t % a.K); t /= a.K;
        const int n = static_cast<int>(t);
        const int g = k / a.Kg;
        const int8_t* xn = x + n * a.x_img;
        int acc = 0;
        for (int cl = 0; cl < a.Cg; ++cl) {
            const int c = g * a.Cg + cl;
            for (int r = 0; r < a.R; ++r) {
                const int ih = oh * a.sh - a.ph + r * a.dh;
                if (ih < 0 || ih >= a.H) continue;
                for (int s = 0; s < a.S; ++s) {
                    const int iw = ow * a.sw - a.pw + s * a.dw;
                    if (iw < 0 || iw >= a.W) continue;
                    acc += static_cast<int>(xn[act_off<XB>(c, ih, iw, a.H, a.W)]) *
                           static_cast<int>(w[((static_cast<long long>(k) * a.Cg + cl) * a.R + r) * a.S + s]);
                }
            }
        }
        y[n * a.y_img + act_off<XB>(k, oh, ow, a.OH, a.OW)] = requant_i8(acc, scale[k]);
    }
}

// ------------------------------------------------------------ config 1
// Depthwise 3x3, stride 1, dilation 1, NCHW.  VEC output columns per thread
// (16 bytes of input per row), ROWS output rows per thread.

template <typename T> struct Vec16;
template <> struct Vec16<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void load(const float* p, float* v) {
        const float4 q = *reinterpret_cast<const float4*>(p);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
    static __device__ __forceinline__ void store(float* p, const float* v) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
};
template <> struct Vec16<bf16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void load(const bf16_t* p, float* v) {
        const uint4 q = *reinterpret_cast<const uint4*>(p);
        const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(u[i] << 16);
            v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void store(bf16_t* p, const float* v) {
        uint32_t u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            u[i] = static_cast<uint32_t>(float_to_bf16(v[2 * i])) |
                   (static_cast<uint32_t>(float_to_bf16(v[2 * i + 1])) << 16);
        *reinterpret_cast<uint4*>(p) = make_uint4(u[0], u[1], u[2], u[3]);
    }
};

template <typename T, int ROWS>
__global__ __launch_bounds__(256) void depthwise3x3_s1(const T* __restrict__ x, const T* __restrict__ w,
                                                       T* __restrict__ y, DirectArgs a, int col_groups,
                                                       int row_bands, long long total) {
    constexpr int V = Vec16<T>::N;
    const long long idx = blockIdx.x * 256LL + threadIdx.x;
    if (idx >= total) return;
    const int cgp = static_cast<int>(idx % col_groups);
    long long t = idx / col_groups;
    const int band = static_cast<int>(t % row_bands);
    const long long plane = t / row_bands;  // n * C + c
    const int c = static_cast<int>(plane % a.C);
    const int n = static_cast<int>(plane / a.C);
    const T* xp = x + n * a.x_img + static_cast<long long>(c) * a.H * a.W;
    T* yp = y + n * a.y_img + static_cast<long long>(c) * a.OH * a.OW;
    float wk[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) wk[i] = Elem<T>::to_f(w[c * 9 + i]);
    const int ow0 = cgp * V;
    const int oh0 = band * ROWS;
    // rows[j][0..V+1] holds input columns ow0-1 .. ow0+V of input row (oh0 - 1 + j)
    float rows[3][V + 2];
    auto load_row = [&](int ih, float* dst) {
        if (ih < 0 || ih >= a.H) {
#pragma unroll
            for (int i = 0; i < V + 2; ++i) dst[i] = 0.0f;
            return;
        }
        const T* rp = xp + static_cast<long long>(ih) * a.W;
        Vec16<T>::load(rp + ow0, dst + 1);
        dst[0] = (ow0 > 0) ? Elem<T>::to_f(rp[ow0 - 1]) : 0.0f;
        dst[V + 1] = (ow0 + V < a.W) ? Elem<T>::to_f(rp[ow0 + V]) : 0.0f;
    };
    load_row(oh0 - 1, rows[0]);
    load_row(oh0, rows[1]);
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int oh = oh0 + i;
        if (oh >= a.OH) break;
        load_row(oh + 1, rows[(i + 2) % 3]);
        const float* r0 = rows[i % 3];
        const float* r1 = rows[(i + 1) % 3];
        const float* r2 = rows[(i + 2) % 3];
        float out[V];
#pragma unroll
        for (int j = 0; j < V; ++j) {
            float acc = 0.0f;
            acc = fmaf(r0[j], wk[0], acc);
            acc = fmaf(r0[j + 1], wk[1], acc);
            acc = fmaf(r0[j + 2], wk[2], acc);
            acc = fmaf(r1[j], wk[3], acc);
            acc = fmaf(r1[j + 1], wk[4], acc);
            acc = fmaf(r1[j + 2], wk[5], acc);
            acc = fmaf(r2[j], wk[6], acc);
            acc = fmaf(r2[j + 1], wk[7], acc);
            acc = fmaf(r2[j + 2], wk[8], acc);
            out[j] = acc;
        }
        Vec16<T>::store(yp + static_cast<long long>(oh) * a.OW + ow0, out);
    }
}

DirectArgs make_args(const Prob& p) {
    DirectArgs a;
    a.N = p.n; a.C = p.c; a.H = p.h; a.W = p.w; a.K = p.k; a.OH = p.oh; a.OW = p.ow;
    a.Cg = p.cg; a.Kg = p.kg; a.R = p.r; a.S = p.s;
    a.sh = p.sh; a.sw = p.sw; a.ph = p.ph; a.pw = p.pw; a.dh = p.dh; a.dw = p.dw;
    a.x_img = p.x_img; a.y_img = p.y_img;
    return a;
}

unsigned grid_for(long long total) {
    long long blocks = (total + 255) / 256;
    if (blocks > 65535LL * 64) blocks = 65535LL * 64;  // grid-stride beyond this
    return static_cast<unsigned>(blocks);
}

constexpr int kDwRows = 8;

bool depthwise_fast_ok(const Prob& p, std::string* why) {
    const int V = (p.dtype == CFWD_F32) ? 4 : 8;
    if (!p.depthwise() || p.r != 3 || p.s != 3 || p.sh != 1 || p.sw != 1 || p.dh != 1 || p.dw != 1 ||
        p.ph != 1 || p.pw != 1) {
        if (why) *why = "depthwise fast path needs G=C=K, 3x3, stride 1, pad 1, dilation 1";
        return false;
    }
    if (p.layout != CFWD_LAYOUT_NCHW || p.dtype == CFWD_I8) {
        if (why) *why = "depthwise fast path needs NCHW fp32 or bf16";
        return false;
    }
    if (p.w % V != 0) {
        if (why) *why = "depthwise fast path needs W divisible by the vector width";
        return false;
    }
    return true;
}

}  // namespace

int direct_num_configs() { return 2; }

bool direct_supported(const Prob& p, int cfg, std::string* why) {
    if (cfg == 0) return true;
    if (cfg == 1) return depthwise_fast_ok(p, why);
    if (why) *why = "no such direct config";
    return false;
}

cfwd_status direct_launch(const Prob& p, int cfg, const void* x, const void* w, const float* scale, void* y,
                          hipStream_t st) {
    const DirectArgs a = make_args(p);
    if (cfg == 1) {
        const int V = (p.dtype == CFWD_F32) ? 4 : 8;
        const int col_groups = p.w / V;
        const int row_bands = (p.oh + kDwRows - 1) / kDwRows;
        const long long total = static_cast<long long>(p.n) * p.c * row_bands * col_groups;
        const unsigned blocks = static_cast<unsigned>((total + 255) / 256);
        if (p.dtype == CFWD_F32)
            depthwise3x3_s1<float, kDwRows><<<blocks, 256, 0, st>>>(
                static_cast<const float*>(x), static_cast<const float*>(w), static_cast<float*>(y), a, col_groups,
                row_bands, total);
        else
            depthwise3x3_s1<bf16_t, kDwRows><<<blocks, 256, 0, st>>>(
                static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w), static_cast<bf16_t*>(y), a,
                col_groups, row_bands, total);
        return check_hip(hipGetLastError(), "depthwise3x3_s1 launch");
    }
    const long long total = static_cast<long long>(p.n) * p.k * p.oh * p.ow;
    const unsigned blocks = grid_for(total);
#define CFWD_DIRECT_CASE(XBV)                                                                                   \
    case XBV:                                                                                                   \
        if (p.dtype == CFWD_F32)                                                                                \
            direct_generic<float, XBV><<<blocks, 256, 0, st>>>(static_cast<const float*>(x),                   \
                                                                static_cast<const float*>(w),                   \
                                                                static_cast<float*>(y), a);                     \
        else if (p.dtype == CFWD_BF16)                                                                          \
            direct_generic<bf16_t, XBV><<<blocks, 256, 0, st>>>(static_cast<const bf16_t*>(x),                 \
                                                                 static_cast<const bf16_t*>(w),                 \
                                                                 static_cast<bf16_t*>(y), a);                   \
        else                                                                                                    \
            direct_generic_i8<XBV><<<blocks, 256, 0, st>>>(static_cast<const int8_t*>(x),                      \
                                                            static_cast<const int8_t*>(w), scale,               \
                                                            static_cast<int8_t*>(y), a);                        \
        break;
    switch (p.xb) {
        CFWD_DIRECT_CASE(1)
        CFWD_DIRECT_CASE(4)
        CFWD_DIRECT_CASE(8)
        default:
            return set_error(CFWD_ERR_UNSUPPORTED, "direct: unsupported channel block");
    }
#undef CFWD_DIRECT_CASE
    return check_hip(hipGetLastError(), "direct_generic launch");
}

// ------------------------------------------------------------ utilities

namespace {

template <typename T>
__global__ __launch_bounds__(256) void zero_pad_channels(T* __restrict__ y, int N, int K, int XB, int CB, int HW,
                                                         long long y_img) {
    // Padded channels live in the last channel block: lanes K%XB .. XB-1.
    const int first = K % XB;
    const int npad = XB - first;
    const long long total = static_cast<long long>(N) * HW * npad;
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < total; i += static_cast<long long>(gridDim.x) * 256) {
        const int lane = first + static_cast<int>(i % npad);
        long long t = i / npad;
        const int pix = static_cast<int>(t % HW);
        const int n = static_cast<int>(t / HW);
        T* p = y + n * y_img + (static_cast<long long>(CB - 1) * HW + pix) * XB + lane;
        *p = T{};
    }
}

}  // namespace

cfwd_status zero_output_channel_padding(const Prob& p, void* y, hipStream_t st) {
    if (p.layout != CFWD_LAYOUT_NCHWX || p.k % p.xb == 0) return CFWD_OK;
    const int CB = (p.k + p.xb - 1) / p.xb;
    const int HW = p.oh * p.ow;
    const long long total = static_cast<long long>(p.n) * HW * (p.xb - p.k % p.xb);
    const unsigned blocks = grid_for(total);
    if (p.esize == 4)
        zero_pad_channels<float><<<blocks, 256, 0, st>>>(static_cast<float*>(y), p.n, p.k, p.xb, CB, HW, p.y_img);
    else if (p.esize == 2)
        zero_pad_channels<bf16_t><<<blocks, 256, 0, st>>>(static_cast<bf16_t*>(y), p.n, p.k, p.xb, CB, HW, p.y_img);
    else
        zero_pad_channels<int8_t><<<blocks, 256, 0, st>>>(static_cast<int8_t*>(y), p.n, p.k, p.xb, CB, HW, p.y_img);
    return check_hip(hipGetLastError(), "zero_pad_channels launch");
}

}  // namespace cfwd
