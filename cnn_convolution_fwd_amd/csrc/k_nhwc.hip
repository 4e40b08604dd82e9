// NHWC activations (gfx950): an implicit-GEMM convolution for channel-
// contiguous activations, and the layout conversions between NCHW, NCHWX and
// NHWC.
//
// MegEngine CPU-inference article, section "结论": after per-operator
// optimisation the next step named is a network-wide choice of layouts
// (global mixed layout) and lower-precision paths.  A layout per layer needs
// (a) kernels for the layout and (b) conversions where neighbouring layers
// differ; this file gives NHWC both.
//
// Convolution: the matrix product of the im2col view (MegEngine inference
// article, section "Im2col+MatMul") with M = output channels, N = output
// pixels (flattened over N x OH x OW), K = (channel chunk, r, s).  In NHWC a
// pixel's channels are contiguous, so both operands are staged into LDS by
// plain 16-byte copies -- the pack the article fuses into im2col costs
// nothing here -- and each K step is one tap of one 64-byte channel chunk.
// Workgroup: 128 channels x TP = 128 pixels, 4 waves of 64 x 64 (16 x 16
// fragments), LDS double-buffered with one barrier per K step; the next
// step's pieces are loaded into registers while the current step
// multiplies.  (A 256-pixel tile measured slower: its 128 accumulators per
// lane leave one wave per SIMD.)
// The weights are prepared once as [k][r][s][C rounded up to the chunk].
#include "internal.h"
#include "nhwc.h"

namespace cfwd {
namespace nh {

constexpr int TK = 128;   // output channels per workgroup
constexpr int NTHR = 256;
constexpr int kTP[1] = {128};  // output pixels per workgroup, per config

template <typename T> struct Op;
template <> struct Op<bf16_t> {
    static constexpr int E16 = 8, CK = 32;  // elements per 16 bytes, channels per 64-byte chunk
    static __device__ __forceinline__ void mma(f32x4& c, const uint4& a, const uint4& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                    0, 0);
    }
};
template <> struct Op<float> {
    static constexpr int E16 = 4, CK = 16;
    // K = 4 per instruction, one value per lane group: element m of every
    // lane's 16-byte slot feeds instruction m (A and B use the same order)
    static __device__ __forceinline__ void mma(f32x4& c, const uint4& a, const uint4& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    }
};

struct Args {
    const void* x;
    const void* wp;
    void* y;
    int N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, OH, OW;
    int Cp, nch, ntk;
    int npix;
    Epi e;
};

// byte offset of 16-byte slot j of row r in a 64-byte-row tile: slots XOR-
// spread by r / 4, so the 16 rows one lane group reads hit 16 bank groups
__device__ __forceinline__ int slot_off(int r, int j) { return r * 64 + ((j ^ ((r >> 2) & 3)) << 4); }

__device__ __forceinline__ uint4 ld16(const void* p) { return __builtin_bit_cast(uint4, *reinterpret_cast<const i32x4*>(p)); }
__device__ __forceinline__ void st16(void* p, const uint4& v) { *reinterpret_cast<i32x4*>(p) = __builtin_bit_cast(i32x4, v); }

template <typename T, bool EPI, int TP>
__global__ __launch_bounds__(NTHR) void nhwc_kernel(Args a) {
    using O = Op<T>;
    constexpr int E16 = O::E16, CK = O::CK;
    constexpr int BUF = (TK + TP) * 64;  // one LDS buffer: A rows then B rows, 64 bytes each
    constexpr int NB = TP / 64;          // pixel pieces per thread per step
    constexpr int NT = TP / 32;          // pixel fragments per wave
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * BUF];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, i = lane & 15;
    const int wk = wave >> 1, wq = wave & 1;
    const int kt = blockIdx.x % a.ntk;  // channel tiles fastest: neighbours share the pixel tile
    const int m0 = (blockIdx.x / a.ntk) * TP;
    const int k0 = kt * TK;
    const int RS = a.R * a.S;
    const T* __restrict__ x = static_cast<const T*>(a.x);
    const T* __restrict__ wp = static_cast<const T*>(a.wp);

    // staging pieces: u = 0, 1 weights (row k, slot j), then NB pixel pieces
    long long wsrc[2];     // element offset of the piece for tap 0, chunk 0 (-1: zero)
    int ih0[NB], iw0[NB];  // pixel pieces: input origin of the output pixel
    long long xbase[NB];   // element offset of the image (-1: no pixel)
    int lofs[2 + NB];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int q = tid + NTHR * u;
        const int row = q >> 2, j = q & 3;
        const int k = k0 + row;
        wsrc[u] = (k < a.K) ? static_cast<long long>(k) * RS * a.Cp + j * E16 : -1;
        lofs[u] = slot_off(row, j);
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const int q = tid + NTHR * u;
        const int px = q >> 2, j = q & 3;
        const int P = m0 + px;
        xbase[u] = -1;
        ih0[u] = iw0[u] = 0;
        if (P < a.npix) {
            const int ow = P % a.OW;
            const int t = P / a.OW;
            const int oh = t % a.OH;
            const int n = t / a.OH;
            ih0[u] = oh * a.sh - a.ph;
            iw0[u] = ow * a.sw - a.pw;
            xbase[u] = static_cast<long long>(n) * a.H * a.W * a.C + j * E16;
        }
        lofs[2 + u] = TK * 64 + slot_off(px, j);
    }
    const int steps = a.nch * RS;
    // two register sets: the pieces of steps st + 1 and st + 2 are in
    // flight while step st multiplies
    uint4 sa[2 + NB], sb[2 + NB];
    auto load = [&](uint4 (&stg)[2 + NB], int st) __attribute__((always_inline)) {
        const int chunk = st / RS, tap = st - chunk * RS;
        const int r = tap / a.S, s = tap - r * a.S;
        const int c0 = chunk * CK;
#pragma unroll
        for (int u = 0; u < 2; ++u)
            stg[u] = (wsrc[u] >= 0) ? ld16(wp + wsrc[u] + static_cast<long long>(tap) * a.Cp + c0) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int ih = ih0[u] + r * a.dh, iw = iw0[u] + s * a.dw;
            const int c = c0 + (((tid + NTHR * u) & 3) * E16);
            const bool ok = xbase[u] >= 0 && static_cast<unsigned>(ih) < static_cast<unsigned>(a.H) &&
                            static_cast<unsigned>(iw) < static_cast<unsigned>(a.W) && c < a.C;
            stg[2 + u] = ok ? ld16(x + xbase[u] + (static_cast<long long>(ih) * a.W + iw) * a.C + c0)
                            : make_uint4(0, 0, 0, 0);
        }
    };
    auto store = [&](const uint4 (&stg)[2 + NB], int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 2 + NB; ++u) st16(lds + buf * BUF + lofs[u], stg[u]);
    };

    f32x4 acc[4][NT];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // this lane's operand rows: weights 64 wk + 16 mt + i, pixels (TP / 2) wq + 16 nt + i
    int aoff[4], boff[NT];
#pragma unroll
    for (int t = 0; t < 4; ++t) aoff[t] = slot_off(64 * wk + 16 * t + i, g);
#pragma unroll
    for (int t = 0; t < NT; ++t) boff[t] = TK * 64 + slot_off((TP / 2) * wq + 16 * t + i, g);

    auto step_mma = [&](int st) __attribute__((always_inline)) {
        const uint8_t* buf = lds + (st & 1) * BUF;
        uint4 af[4], bf[NT];
#pragma unroll
        for (int t = 0; t < 4; ++t) af[t] = ld16(buf + aoff[t]);
#pragma unroll
        for (int t = 0; t < NT; ++t) bf[t] = ld16(buf + boff[t]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) O::mma(acc[mt][nt], af[mt], bf[nt]);
    };
    // at the top of step st: LDS buffer st & 1 holds step st; the set for
    // step st + 1 (sb when st is even) and the other (step st + 2) are in
    // flight; the loop takes two steps so each set is fixed
    load(sa, 0);
    store(sa, 0);
    if (steps > 1) load(sb, 1);
    if (steps > 2) load(sa, 2);
    __syncthreads();
    for (int st = 0; st < steps; st += 2) {
        step_mma(st);
        if (st + 1 < steps) store(sb, 1);  // buffer 1 was last read before the previous barrier
        if (st + 3 < steps) load(sb, st + 3);
        __syncthreads();
        if (st + 1 < steps) {
            step_mma(st + 1);
            if (st + 2 < steps) store(sa, 0);
            if (st + 4 < steps) load(sa, st + 4);
            __syncthreads();
        }
    }

    // D[channel][pixel]: lane holds pixel (TP / 2) wq + 16 nt + i, channels
    // 64 wk + 16 mt + 4g .. + 3, which are consecutive in NHWC
    T* __restrict__ y = static_cast<T*>(a.y);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int P = m0 + (TP / 2) * wq + 16 * nt + i;
        if (P >= a.npix) continue;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int kb = k0 + 64 * wk + 16 * mt + 4 * g;
            if (kb >= a.K) continue;
            const long long o = static_cast<long long>(P) * a.K + kb;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = acc[mt][nt][e];
                if constexpr (EPI)
                    if (kb + e < a.K) v[e] = epi_float<T>(v[e], a.e, kb + e, o + e);
            }
            if (kb + 3 < a.K && (a.K & 3) == 0) {
                if constexpr (sizeof(T) == 4)
                    *reinterpret_cast<f32x4*>(y + o) = f32x4{v[0], v[1], v[2], v[3]};
                else
                    *reinterpret_cast<uint2*>(y + o) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (kb + e >= a.K) break;
                    if constexpr (sizeof(T) == 4)
                        y[o + e] = v[e];
                    else
                        y[o + e].bits = float_to_bf16(v[e]);
                }
            }
        }
    }
}

// wp[k][r][s][c] = w[k][c][r][s], channels C .. Cp - 1 zero
template <typename T>
__global__ __launch_bounds__(256) void nhwc_prepare_kernel(const T* __restrict__ w, T* __restrict__ wp, int K, int C,
                                                           int RS, int Cp) {
    const long long total = static_cast<long long>(K) * RS * Cp;
    for (long long idx = blockIdx.x * 256LL + threadIdx.x; idx < total; idx += static_cast<long long>(gridDim.x) * 256) {
        const int c = static_cast<int>(idx % Cp);
        const long long t = idx / Cp;
        const int tap = static_cast<int>(t % RS);
        const int k = static_cast<int>(t / RS);
        wp[idx] = (c < C) ? w[(static_cast<long long>(k) * C + c) * RS + tap] : T{};
    }
}

// ------------------------------------------------------------ layout conversion
// Element offset of (c, p) in one image, p = h * W + w:
//   NCHW  c * HW + p;  NCHWX ((c / x) * HW + p) * x + c % x;  NHWC p * C + c.
__device__ __forceinline__ long long lay_off(int lay, int xb, int C, long long HW, int c, long long p) {
    if (lay == CFWD_LAYOUT_NCHW) return c * HW + p;
    if (lay == CFWD_LAYOUT_NHWC) return p * C + c;
    return ((c / xb) * HW + p) * xb + c % xb;
}

// A 32-channel x 64-pixel tile through LDS: read in the source's contiguous
// order, written in the destination's (channel-fastest for NHWC and NCHWX,
// pixel-fastest for NCHW).  Channels past C read as 0, so NCHWX destination
// blocks come out zero-padded.
template <typename U>
__global__ __launch_bounds__(256) void convert_kernel(const U* __restrict__ src, U* __restrict__ dst, int C, long long HW,
                                                      int sl, int sx, long long s_img, int dl, int dx, long long d_img,
                                                      int cdst) {
    __shared__ U tile[32][65];
    const int n = blockIdx.z;
    const int c0 = blockIdx.y * 32;
    const long long p0 = static_cast<long long>(blockIdx.x) * 64;
    const U* s = src + n * s_img;
    U* d = dst + n * d_img;
    const bool s_cfast = sl != CFWD_LAYOUT_NCHW;
    const bool d_cfast = dl != CFWD_LAYOUT_NCHW;
    for (int e = threadIdx.x; e < 32 * 64; e += 256) {
        const int cc = s_cfast ? (e & 31) : (e >> 6);
        const int pp = s_cfast ? (e >> 5) : (e & 63);
        const int c = c0 + cc;
        const long long p = p0 + pp;
        tile[cc][pp] = (c < C && p < HW) ? s[lay_off(sl, sx, C, HW, c, p)] : U{};
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 32 * 64; e += 256) {
        const int cc = d_cfast ? (e & 31) : (e >> 6);
        const int pp = d_cfast ? (e >> 5) : (e & 63);
        const int c = c0 + cc;
        const long long p = p0 + pp;
        if (c < cdst && p < HW) d[lay_off(dl, dx, cdst, HW, c, p)] = tile[cc][pp];
    }
}

struct Plan {
    int Cp, nch, ntk, npix;
};

bool plan(const Prob& p, int cfg, Plan* pl, std::string* why) {
    auto no = [&](const char* m) {
        if (why) *why = m;
        return false;
    };
    if (p.layout != CFWD_LAYOUT_NHWC) return no("implicit GEMM (NHWC): NHWC problems only");
    if (p.dtype != CFWD_BF16 && p.dtype != CFWD_F32) return no("implicit GEMM (NHWC): fp32 or bf16");
    if (p.g != 1) return no("implicit GEMM (NHWC): groups 1 only");
    const int e16 = 16 / p.esize, ck = 64 / p.esize;
    if (p.c % e16 != 0) return no("implicit GEMM (NHWC): C must be a multiple of 8 (bf16) or 4 (fp32)");
    const long long npix = static_cast<long long>(p.n) * p.oh * p.ow;
    if (cfg != 0) return no("implicit GEMM (NHWC): no such config");
    if (npix >= (1LL << 31) - kTP[cfg]) return no("implicit GEMM (NHWC): too many output pixels");
    pl->Cp = (p.c + ck - 1) / ck * ck;
    pl->nch = pl->Cp / ck;
    pl->ntk = (p.k + TK - 1) / TK;
    pl->npix = static_cast<int>(npix);
    if (static_cast<long long>(p.k) * p.r * p.s * pl->Cp >= (1LL << 31))
        return no("implicit GEMM (NHWC): prepared weights too large");
    return true;
}

}  // namespace nh

int nhwc_num_configs() { return 1; }

bool nhwc_supported(const Prob& p, int cfg, std::string* why) {
    nh::Plan pl;
    return nh::plan(p, cfg, &pl, why);
}

size_t nhwc_filter_bytes(const Prob& p, int cfg) {
    nh::Plan pl;
    if (!nh::plan(p, cfg, &pl, nullptr)) return 0;
    return static_cast<size_t>(p.k) * p.r * p.s * pl.Cp * p.esize;
}

cfwd_status nhwc_prepare(const Prob& p, int cfg, const void* w, void* wp, hipStream_t st) {
    nh::Plan pl;
    std::string why;
    if (!nh::plan(p, cfg, &pl, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    const long long total = static_cast<long long>(p.k) * p.r * p.s * pl.Cp;
    const unsigned blocks = static_cast<unsigned>(std::min<long long>((total + 255) / 256, 65536));
    if (p.dtype == CFWD_BF16)
        nh::nhwc_prepare_kernel<bf16_t><<<blocks, 256, 0, st>>>(static_cast<const bf16_t*>(w), static_cast<bf16_t*>(wp),
                                                                p.k, p.c, p.r * p.s, pl.Cp);
    else
        nh::nhwc_prepare_kernel<float><<<blocks, 256, 0, st>>>(static_cast<const float*>(w), static_cast<float*>(wp), p.k,
                                                               p.c, p.r * p.s, pl.Cp);
    return check_hip(hipGetLastError(), "NHWC filter prepare launch");
}

cfwd_status nhwc_launch(const Prob& p, int cfg, const void* x, const void* wp, void* y, const Epi& e, hipStream_t st) {
    nh::Plan pl;
    std::string why;
    if (!nh::plan(p, cfg, &pl, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    if (wp == nullptr) return set_error(CFWD_ERR_WORKSPACE, "implicit GEMM (NHWC): the prepared filter is required");
    nh::Args a;
    a.x = x;
    a.wp = wp;
    a.y = y;
    a.N = p.n; a.C = p.c; a.H = p.h; a.W = p.w; a.K = p.k; a.R = p.r; a.S = p.s;
    a.sh = p.sh; a.sw = p.sw; a.ph = p.ph; a.pw = p.pw; a.dh = p.dh; a.dw = p.dw; a.OH = p.oh; a.OW = p.ow;
    a.Cp = pl.Cp; a.nch = pl.nch; a.ntk = pl.ntk; a.npix = pl.npix;
    a.e = e;
    const int tp = nh::kTP[cfg];
    const long long blocks = static_cast<long long>((pl.npix + tp - 1) / tp) * pl.ntk;
    if (blocks > 0x7fffffffLL) return set_error(CFWD_ERR_UNSUPPORTED, "implicit GEMM (NHWC): too many tiles");
    const bool epi = e.bias || e.res || e.relu;
    const unsigned nb = static_cast<unsigned>(blocks);
    auto go = [&](auto kern) { kern<<<nb, nh::NTHR, 0, st>>>(a); };
    if (p.dtype == CFWD_BF16)
        epi ? go(nh::nhwc_kernel<bf16_t, true, 128>) : go(nh::nhwc_kernel<bf16_t, false, 128>);
    else
        epi ? go(nh::nhwc_kernel<float, true, 128>) : go(nh::nhwc_kernel<float, false, 128>);
    return check_hip(hipGetLastError(), "NHWC implicit GEMM launch");
}

cfwd_status layout_convert(int n, int c, int h, int w, int esize, int sl, int sx, const void* src, int dl, int dx,
                           void* dst, hipStream_t st) {
    const long long HW = static_cast<long long>(h) * w;
    auto cpad = [&](int lay, int xb) { return lay == CFWD_LAYOUT_NCHWX ? (c + xb - 1) / xb * xb : c; };
    const long long s_img = cpad(sl, sx) * HW, d_img = cpad(dl, dx) * HW;
    const int cdst = cpad(dl, dx);  // NCHWX destinations get their padding channels written (as 0)
    const dim3 grid(static_cast<unsigned>((HW + 63) / 64), static_cast<unsigned>((cdst + 31) / 32),
                    static_cast<unsigned>(n));
    switch (esize) {
        case 1:
            nh::convert_kernel<uint8_t><<<grid, 256, 0, st>>>(static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst),
                                                              c, HW, sl, sx, s_img, dl, dx, d_img, cdst);
            break;
        case 2:
            nh::convert_kernel<uint16_t><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(src),
                                                               static_cast<uint16_t*>(dst), c, HW, sl, sx, s_img, dl, dx,
                                                               d_img, cdst);
            break;
        default:
            nh::convert_kernel<uint32_t><<<grid, 256, 0, st>>>(static_cast<const uint32_t*>(src),
                                                               static_cast<uint32_t*>(dst), c, HW, sl, sx, s_img, dl, dx,
                                                               d_img, cdst);
    }
    return check_hip(hipGetLastError(), "layout conversion launch");
}

}  // namespace cfwd
