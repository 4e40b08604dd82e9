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
// configs 1-6: depthwise 3x3, stride 1, pad 1, dilation 1, NCHW, W a
//           multiple of the vector -- each thread owns a strip of one 16-byte
//           (configs 1-4) or 8-byte (configs 5-6) vector of columns and RB
//           output rows (RB = 1, 2, 4, 8, 2, 4).  It
//           issues all RB + 2 input-row loads before computing (many bytes in
//           flight per thread, which is what an HBM-bound kernel needs), takes
//           the left / right neighbour columns from the adjacent lanes with a
//           cross-lane shuffle instead of extra loads, and writes the outputs
//           with streaming (non-temporal) stores.  Every input byte comes from
//           HBM once: the halo rows of a strip are the rows adjacent lanes load.
#include "internal.h"

namespace cfwd {

namespace {

struct DirectArgs {
    int N, C, H, W, K, OH, OW, Cg, Kg, R, S, sh, sw, ph, pw, dh, dw;
    long long x_img, y_img;
    Epi e;  // fused epilogue
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
        const long long o = n * a.y_img + act_off<XB>(k, oh, ow, a.OH, a.OW);
        y[o] = store_cast<T>(epi_float<T>(acc, a.e, k, o));
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
        const long long o = n * a.y_img + act_off<XB>(k, oh, ow, a.OH, a.OW);
        y[o] = static_cast<int8_t>(requant_i8_epi_bits(acc, scale[k], a.e, k, o));
    }
}

// ------------------------------------------------------------ configs 1-6
// Each thread holds NW 32-bit words of every input row it needs (NW = 4: a
// 16-byte vector, NW = 2: 8 bytes): VPT = NW (fp32) or 2 NW (bf16) columns.

template <typename T> struct Words;
template <> struct Words<float> {
    static constexpr int PER_WORD = 1;
    static __device__ __forceinline__ float elem(const uint32_t* wd, int e) { return __uint_as_float(wd[e]); }
    static __device__ __forceinline__ float first(uint32_t word) { return __uint_as_float(word); }
    static __device__ __forceinline__ float last(uint32_t word) { return __uint_as_float(word); }
    static __device__ __forceinline__ uint32_t pack(const float* v, int i) { return __float_as_uint(v[i]); }
};
template <> struct Words<bf16_t> {
    static constexpr int PER_WORD = 2;
    static __device__ __forceinline__ float elem(const uint32_t* wd, int e) {
        const uint32_t w = wd[e >> 1];
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    // a word's first element sits in its low half, its last in the high half
    static __device__ __forceinline__ float first(uint32_t word) { return __uint_as_float(word << 16); }
    static __device__ __forceinline__ float last(uint32_t word) { return __uint_as_float(word & 0xffff0000u); }
    static __device__ __forceinline__ uint32_t pack(const float* v, int i) { return pack_bf16x2(v[2 * i], v[2 * i + 1]); }
};

template <int NW> struct RawVec;
template <> struct RawVec<4> {
    static __device__ __forceinline__ void load(const void* p, uint32_t* d) {
        const uint4 q = *reinterpret_cast<const uint4*>(p);
        d[0] = q.x; d[1] = q.y; d[2] = q.z; d[3] = q.w;
    }
    static __device__ __forceinline__ void store_nt(void* p, const uint32_t* d) {
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        const u32x4_t v = {d[0], d[1], d[2], d[3]};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
    }
};
template <> struct RawVec<2> {
    static __device__ __forceinline__ void load(const void* p, uint32_t* d) {
        const uint2 q = *reinterpret_cast<const uint2*>(p);
        d[0] = q.x; d[1] = q.y;
    }
    static __device__ __forceinline__ void store_nt(void* p, const uint32_t* d) {
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t v = {d[0], d[1]};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(p));
    }
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Division of numerators below 2^31 by a divisor d >= 1 fixed at launch, as
// a multiply-high and a shift (Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994, theorem 4.2 with N = 31):
// with l = ceil(log2 d) and m = ceil(2^(31 + l) / d), which is below 2^32,
// n / d = (n * m) >> (31 + l).  m = 0 stands for d = 1.
struct FastDiv {
    uint32_t m;
    int sh;  // l - 1, the shift applied to the high word of n * m
};
FastDiv make_fastdiv(uint32_t d) {
    if (d <= 1) return FastDiv{0u, 0};
    int l = 0;
    while ((1ull << l) < d) ++l;
    const unsigned long long m = ((1ull << (31 + l)) + d - 1) / d;
    return FastDiv{static_cast<uint32_t>(m), l - 1};
}
__device__ __forceinline__ int fast_div(int n, FastDiv f) {
    return f.m ? static_cast<int>(__umulhi(static_cast<uint32_t>(n), f.m) >> f.sh) : n;
}

template <typename T, int NW> constexpr int dw_vpt() { return NW * Words<T>::PER_WORD; }

// Workgroup = SPB whole strips (a strip = one plane n*C + c and one band of
// RB output rows, all `cols` column vectors of it), SPB = floor(256 / cols),
// so a thread's left and right neighbour columns always belong to threads
// of the same workgroup: they are exchanged through LDS.  Every load is
// issued up front and nothing branches: rows outside the image are read
// clamped (in bounds) and zeroed with selects; threads past the last strip
// work on a clamped strip and store nothing.  Outputs are written with
// streaming (non-temporal) stores.
// EPI: the fused epilogue compiled in (a separate instantiation, so the
// plain kernels carry none of its registers).
template <typename T, int RB, int NW, bool EPI>
__global__ __launch_bounds__(256) void depthwise3x3_s1(const T* __restrict__ x, const T* __restrict__ w,
                                                       T* __restrict__ y, int C, int H, int W, long long x_img,
                                                       long long y_img, int cols, int bands, int strips, int spb,
                                                       FastDiv fd_cols, FastDiv fd_bands, FastDiv fd_c, Epi ep) {
    using WD = Words<T>;
    constexpr int V = dw_vpt<T, NW>();
    __shared__ uint32_t first_w[RB + 2][256], last_w[RB + 2][256];
    const int tid = threadIdx.x;
    // spb = 256 / cols whole strips per workgroup; the divisions by cols,
    // bands and C are multiply-high reciprocals computed on the host
    const int sl = fast_div(tid, fd_cols);
    const int cg = tid - sl * cols;
    // plain dispatch order: at any moment the chip streams one contiguous
    // region of the input (measured faster here than an XCD-aware order; the
    // second read of a halo row between workgroups hits the Infinity Cache)
    const int strip_raw = static_cast<int>(blockIdx.x) * spb + sl;
    const bool valid = sl < spb && strip_raw < strips;
    const int strip = min(strip_raw, strips - 1);
    const int plane = fast_div(strip, fd_bands);
    const int band = strip - plane * bands;
    const int n = fast_div(plane, fd_c);
    const int c = plane - n * C;
    const long long plane_off = static_cast<long long>(c) * H * W;
    const T* xp = x + n * x_img + plane_off;
    T* yp = y + n * y_img + plane_off;
    const int ow0 = cg * V;
    const int oh0 = band * RB;

    float wk[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) wk[i] = Elem<T>::to_f(w[c * 9 + i]);
    // input rows oh0 - 1 .. oh0 + RB, this thread's NW words of columns
    uint32_t raw[RB + 2][NW];
#pragma unroll
    for (int j = 0; j < RB + 2; ++j) {
        const int ih = min(max(oh0 - 1 + j, 0), H - 1);
        RawVec<NW>::load(xp + (ih * W + ow0), raw[j]);
    }
#pragma unroll
    for (int j = 0; j < RB + 2; ++j) {
        const int ih = oh0 - 1 + j;
        const bool in = ih >= 0 && ih < H;
#pragma unroll
        for (int q = 0; q < NW; ++q) raw[j][q] = in ? raw[j][q] : 0u;
        first_w[j][tid] = raw[j][0];
        last_w[j][tid] = raw[j][NW - 1];
    }
    __syncthreads();
    // neighbour columns ow0 - 1 and ow0 + V (zero at the image border)
    const int tl = max(tid - 1, 0), tr = min(tid + 1, 255);
    float left[RB + 2], right[RB + 2];
#pragma unroll
    for (int j = 0; j < RB + 2; ++j) {
        const float l = WD::last(last_w[j][tl]);
        const float r = WD::first(first_w[j][tr]);
        left[j] = (cg > 0) ? l : 0.0f;
        right[j] = (cg < cols - 1) ? r : 0.0f;
    }
    // fused epilogue: the RB residual row vectors this thread stores, all
    // requested here, before any computation (rows past the image clamped)
    uint32_t rres[EPI ? RB : 1][NW];
    float ebias = 0.0f;
    if constexpr (EPI) {
        if (ep.res) {
            const T* rp = static_cast<const T*>(ep.res) + (yp - y);
#pragma unroll
            for (int i = 0; i < RB; ++i) RawVec<NW>::load(rp + (min(oh0 + i, H - 1) * W + ow0), rres[i]);
        }
        if (ep.bias) ebias = static_cast<const float*>(ep.bias)[c];
    }
    // bf16: weight pairs (w0, w1) and (w1, w2) of each filter row, packed
    bf16x2_t w01[3], w12[3];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            const uint32_t a0 = pack_bf16x2(wk[3 * r], 0.0f), a1 = pack_bf16x2(wk[3 * r + 1], 0.0f),
                           a2 = pack_bf16x2(wk[3 * r + 2], 0.0f);
            w01[r] = __builtin_bit_cast(bf16x2_t, a0 | (a1 << 16));
            w12[r] = __builtin_bit_cast(bf16x2_t, a1 | (a2 << 16));
        }
    }

#pragma unroll
    for (int i = 0; i < RB; ++i) {
        const int oh = oh0 + i;
        float out[V];
        if constexpr (sizeof(T) == 2) {
            // bf16: the pair (e, e + 1) of an even e is one 32-bit word, so
            // each filter row costs one two-wide dot product plus one FMA:
            //   even e = 2m: dot(word m, (w1, w2)) + x[e - 1] * w0
            //   odd  e = 2m + 1: dot(word m, (w0, w1)) + x[e + 1] * w2
#pragma unroll
            for (int m = 0; m < NW; ++m) {
                float ev = 0.0f, od = 0.0f;
#pragma unroll
                for (int r = 0; r < 3; ++r) {
                    const uint32_t* wd = raw[i + r];
                    const float xm1 = (m == 0) ? left[i + r] : __uint_as_float(wd[m - 1] & 0xffff0000u);
                    const float xp2 = (m == NW - 1) ? right[i + r] : __uint_as_float(wd[m + 1] << 16);
                    ev = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wd[m]), w12[r], ev, false);
                    ev = fmaf(xm1, wk[3 * r], ev);
                    od = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wd[m]), w01[r], od, false);
                    od = fmaf(xp2, wk[3 * r + 2], od);
                }
                out[2 * m] = ev;
                out[2 * m + 1] = od;
            }
        } else {
#pragma unroll
            for (int e = 0; e < V; ++e) {
                float acc = 0.0f;
#pragma unroll
                for (int r = 0; r < 3; ++r) {
                    const uint32_t* wd = raw[i + r];
                    const float a0 = (e == 0) ? left[i + r] : WD::elem(wd, e - 1);
                    const float a1 = WD::elem(wd, e);
                    const float a2 = (e == V - 1) ? right[i + r] : WD::elem(wd, e + 1);
                    acc = fmaf(a0, wk[3 * r], acc);
                    acc = fmaf(a1, wk[3 * r + 1], acc);
                    acc = fmaf(a2, wk[3 * r + 2], acc);
                }
                out[e] = acc;
            }
        }
        if (valid && oh < H) {
            // fused epilogue: bias, residual (the same vector of the
            // residual tensor), ReLU, before the one conversion
            if constexpr (EPI) {
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    float v = out[e] + ebias;
                    if (ep.res) v += WD::elem(rres[i], e);
                    out[e] = ep.relu ? fmaxf(v, 0.0f) : v;
                }
            }
            uint32_t o[NW];
#pragma unroll
            for (int q = 0; q < NW; ++q) o[q] = WD::pack(out, q);
            RawVec<NW>::store_nt(yp + (oh * W + ow0), o);
        }
    }
}

DirectArgs make_args(const Prob& p, const Epi& e) {
    DirectArgs a;
    a.e = e;
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

// (RB, NW) of configs 1-6
constexpr int kDwRB[7] = {0, 1, 2, 4, 8, 2, 4};
constexpr int kDwNW[7] = {0, 4, 4, 4, 4, 2, 2};

bool depthwise_fast_ok(const Prob& p, int cfg, std::string* why) {
    if (!p.depthwise() || p.r != 3 || p.s != 3 || p.sh != 1 || p.sw != 1 || p.dh != 1 || p.dw != 1 ||
        p.ph != 1 || p.pw != 1) {
        if (why) *why = "depthwise fast path needs G=C=K, 3x3, stride 1, pad 1, dilation 1";
        return false;
    }
    if (p.layout != CFWD_LAYOUT_NCHW || p.dtype == CFWD_I8) {
        if (why) *why = "depthwise fast path needs NCHW fp32 or bf16";
        return false;
    }
    const int V = kDwNW[cfg] * (p.dtype == CFWD_F32 ? 1 : 2);
    if (p.w % V != 0 || p.w / V > 256) {
        if (why) *why = "depthwise fast path needs W a multiple of the vector width, at most 256 vectors";
        return false;
    }
    if (static_cast<long long>(p.h) * p.w >= (1LL << 31) || static_cast<long long>(p.n) * p.c * p.h >= (1LL << 31)) {
        if (why) *why = "depthwise fast path needs 32-bit plane offsets and strip ids";
        return false;
    }
    return true;
}

template <typename T, int RB, int NW>
cfwd_status launch_dw(const Prob& p, const void* x, const void* w, void* y, const Epi& e, hipStream_t st) {
    const bool epi = e.bias || e.res || e.relu;
    constexpr int V = dw_vpt<T, NW>();
    const int cols = p.w / V;
    const int bands = (p.oh + RB - 1) / RB;
    const long long strips = static_cast<long long>(p.n) * p.c * bands;
    const int spb = 256 / cols;  // whole strips per workgroup (cols <= 256 is checked)
    if (strips >= (1LL << 31)) return set_error(CFWD_ERR_UNSUPPORTED, "depthwise: too many strips");
    const unsigned blocks = static_cast<unsigned>((strips + spb - 1) / spb);
    auto kern = epi ? depthwise3x3_s1<T, RB, NW, true> : depthwise3x3_s1<T, RB, NW, false>;
    kern<<<blocks, 256, 0, st>>>(static_cast<const T*>(x), static_cast<const T*>(w), static_cast<T*>(y), p.c, p.h,
                                 p.w, p.x_img, p.y_img, cols, bands, static_cast<int>(strips), spb,
                                 make_fastdiv(cols), make_fastdiv(bands), make_fastdiv(p.c), e);
    return check_hip(hipGetLastError(), "depthwise3x3_s1 launch");
}

template <typename T>
cfwd_status launch_dw_cfg(const Prob& p, int cfg, const void* x, const void* w, void* y, const Epi& e,
                          hipStream_t st) {
    switch (cfg) {
        case 1: return launch_dw<T, 1, 4>(p, x, w, y, e, st);
        case 2: return launch_dw<T, 2, 4>(p, x, w, y, e, st);
        case 3: return launch_dw<T, 4, 4>(p, x, w, y, e, st);
        case 4: return launch_dw<T, 8, 4>(p, x, w, y, e, st);
        case 5: return launch_dw<T, 2, 2>(p, x, w, y, e, st);
        default: return launch_dw<T, 4, 2>(p, x, w, y, e, st);
    }
}

}  // namespace

int direct_num_configs() { return 7; }

int direct_default_config(const Prob& p) {
    if (depthwise_fast_ok(p, 2, nullptr)) return 2;
    if (depthwise_fast_ok(p, 5, nullptr)) return 5;
    return 0;
}

bool direct_supported(const Prob& p, int cfg, std::string* why) {
    if (cfg == 0) return true;
    if (cfg >= 1 && cfg <= 6) return depthwise_fast_ok(p, cfg, why);
    if (why) *why = "no such direct config";
    return false;
}

cfwd_status direct_launch(const Prob& p, int cfg, const void* x, const void* w, const float* scale, void* y,
                          const Epi& e, hipStream_t st) {
    const DirectArgs a = make_args(p, e);
    if (cfg >= 1 && cfg <= 6) {
        if (p.dtype == CFWD_F32) return launch_dw_cfg<float>(p, cfg, x, w, y, e, st);
        return launch_dw_cfg<bf16_t>(p, cfg, x, w, y, e, st);
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
