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
    int tiles_w, tiles_h, tiles_n;
    int nchunks, ntk;              // channel chunks, output-channel tiles
    // split reduction (SPLIT kernels only): workgroup split s of a tile sums
    // channel chunks [s*cps, min((s+1)*cps, nchunks)) and writes its int32
    // partial tile to part + s * N * y_img, in the output's NCHW4 order
    int cps;
    int32_t* part;
    Epi e;  // fused epilogue
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

// 32x32 output fragments: one lane holds output column (lane % 32) and, for
// accumulator element v, row 8*(v/4) + 4*(lane/32) + v%4.  Per 64-byte K
// chunk a lane feeds two 16-byte pieces (P0, P1) of its A row / B column:
//   bf16: piece i -> one v_mfma_f32_32x32x16_bf16 (K = 16 each)
//   int8: piece i -> one v_mfma_i32_32x32x32_i8   (K = 32 each)
//   fp32: eight v_mfma_f32_32x32x2_f32, MFMA m taking element m%4 of piece m/4.
// Which channel slots the pieces are is fixed by piece_slot().
template <typename T> struct Mma32;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
template <> struct Mma32<bf16_t> {
    using acc_t = f32x16;
    static __device__ __forceinline__ void piece(acc_t& c, const uint4& a, const uint4& b, int) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                    0, 0);
    }
    static __device__ __forceinline__ void run(acc_t& c, const uint4& a0, const uint4& a1, const uint4& b0,
                                               const uint4& b1) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a0), __builtin_bit_cast(bf16x8, b0), c,
                                                    0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a1), __builtin_bit_cast(bf16x8, b1), c,
                                                    0, 0, 0);
    }
};
template <> struct Mma32<int8_t> {
    using acc_t = i32x16;
    static __device__ __forceinline__ void piece(acc_t& c, const uint4& a, const uint4& b, int) {
        c = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ void run(acc_t& c, const uint4& a0, const uint4& a1, const uint4& b0,
                                               const uint4& b1) {
        c = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a0), __builtin_bit_cast(i32x4, b0), c, 0,
                                                  0, 0);
        c = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a1), __builtin_bit_cast(i32x4, b1), c, 0,
                                                  0, 0);
    }
};
template <> struct Mma32<float> {
    using acc_t = f32x16;
    static __device__ __forceinline__ void piece(acc_t& c, const uint4& a, const uint4& b, int) {
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    }
    static __device__ __forceinline__ void run(acc_t& c, const uint4& a0, const uint4& a1, const uint4& b0,
                                               const uint4& b1) {
        const uint32_t av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        const uint32_t bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
        for (int m = 0; m < 8; ++m)
            c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(av[m]), __uint_as_float(bv[m]), c, 0, 0, 0);
    }
};

// 16-byte channel slot (0..3 of a 64-byte chunk) that piece i of a lane in
// half h (= lane / 32) holds, for 32x32 fragments.  bf16 / int8: each MFMA
// takes 16 (bf16) or 32 (int8) consecutive K, split over the two halves, so
// piece i is slot 2i + h.  fp32: MFMA m takes K = 2, one value per half, and
// lane half h supplies channels 8h .. 8h+7 over m = 0..7: slots 2h, 2h + 1.
template <typename T>
__device__ __host__ __forceinline__ int piece_slot(int i, int h) {
    return (sizeof(T) == 4) ? 2 * h + i : 2 * i + h;
}

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
    y[off] = static_cast<int8_t>(requant_i8_bits(acc[v], scale));
}

// Four consecutive output pixels of one channel (NCHW, 4-aligned).
template <typename T> __device__ __forceinline__ void store_out4(T* y, long long off, typename Mma<T>::acc_t acc,
                                                                float scale);
template <> __device__ __forceinline__ void store_out4<float>(float* y, long long off, f32x4 acc, float) {
    *reinterpret_cast<float4*>(y + off) = make_float4(acc[0], acc[1], acc[2], acc[3]);
}
template <> __device__ __forceinline__ void store_out4<bf16_t>(bf16_t* y, long long off, f32x4 acc, float) {
    const uint32_t lo = pack_bf16x2(acc[0], acc[1]);
    const uint32_t hi = pack_bf16x2(acc[2], acc[3]);
    *reinterpret_cast<uint2*>(y + off) = make_uint2(lo, hi);
}
template <> __device__ __forceinline__ void store_out4<int8_t>(int8_t* y, long long off, i32x4 acc, float scale) {
    *reinterpret_cast<uint32_t*>(y + off) =
        pack_low_bytes(requant_i8_bits(acc[0], scale), requant_i8_bits(acc[1], scale), requant_i8_bits(acc[2], scale),
                       requant_i8_bits(acc[3], scale));
}

// The same stores with the fused epilogue (bias, residual, ReLU) applied
// first; channel k < K, `off` the output element's offset.
template <typename T, bool EPI>
__device__ __forceinline__ void store_out_epi(T* y, long long off, typename Mma<T>::acc_t acc, int v, float scale,
                                              const Epi& e, int k) {
    if constexpr (!EPI) {
        store_out<T>(y, off, acc, v, scale);
    } else if constexpr (sizeof(T) == 1) {
        y[off] = static_cast<int8_t>(requant_i8_epi_bits(acc[v], scale, e, k, off));
    } else {
        f32x4 q;
        q[v] = epi_float<T>(acc[v], e, k, off);
        store_out<T>(y, off, q, v, scale);
    }
}
template <typename T, bool EPI>
__device__ __forceinline__ void store_out4_epi(T* y, long long off, typename Mma<T>::acc_t acc, float scale,
                                               const Epi& e, int k) {
    if constexpr (!EPI) {
        store_out4<T>(y, off, acc, scale);
    } else if constexpr (sizeof(T) == 1) {
        *reinterpret_cast<uint32_t*>(y + off) =
            pack_low_bytes(requant_i8_epi_bits(acc[0], scale, e, k, off), requant_i8_epi_bits(acc[1], scale, e, k, off + 1),
                           requant_i8_epi_bits(acc[2], scale, e, k, off + 2),
                           requant_i8_epi_bits(acc[3], scale, e, k, off + 3));
    } else {
        f32x4 q;
#pragma unroll
        for (int v = 0; v < 4; ++v) q[v] = epi_float<T>(acc[v], e, k, off + v);
        store_out4<T>(y, off, q, scale);
    }
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMaxUnitsPerThread = 8;

// LDS byte offset of 16-byte slot j of patch pixel q.  The slot is XORed with
// two bits of q so that the lanes of one ds_read_b128 (consecutive pixels,
// same slot) spread over all banks.  Which two bits depends on how many
// consecutive pixels one read covers: measured on gfx950, bits 1..2 are
// conflict-free for 16-pixel fragments and bits 2..3 for 32-pixel ones (the
// q>>1 form costs about 30% of LDS throughput there).
//
// 32-pixel fragments instead pad each pixel to 80 bytes (also measured
// conflict-free), which keeps the address linear in the pixel index: a filter
// tap is then a uniform offset added to a per-fragment base.
// LIN: the linear 80-byte layout, used by 32x32 fragments and by the
// nine-tap 16x16 path, where a tap must be a uniform offset (16x16 fragment
// reads -- 16 consecutive pixels of one slot -- are conflict-free in it too).
template <bool LIN> struct PatchStride { static constexpr int value = LIN ? 80 : 64; };
template <bool LIN>
__device__ __forceinline__ int lds_slot(int q, int j) {
    if constexpr (LIN) return q * 80 + j * 16;
    return q * 64 + ((j ^ ((q >> 1) & 3)) << 4);
}

// ---- wide staging ("row blocks")
// One 16-byte global load along W holds PP pixels of SZ bytes each: one
// channel (NCHW, SZ = element size) or one channel block (NCHWX, SZ = x *
// element size).  PP such loads cover PP pixels x 16 bytes of channels, which
// is a PP x PP transpose of SZ-byte sub-elements into PP LDS slots.
template <typename T, int XB> struct Wide {
    static constexpr int ESZ = static_cast<int>(sizeof(T));
    static constexpr int SZ = (XB == 1) ? ESZ : XB * ESZ;
    static constexpr int PP = 16 / SZ;
    static constexpr bool ok = (SZ == 2 || SZ == 4 || SZ == 8);
    // units each thread may own: keeps the in-flight registers at 32 VGPRs
    static constexpr int MAXU = ok ? (32 / (4 * PP) > 0 ? 32 / (4 * PP) : 1) : 1;
};

// Slot p of the transpose: 16 bytes = sub-element p of each of the PP loads.
template <int SZ>
__device__ __forceinline__ uint4 wide_pick(const uint4* ld, int p);
template <>
__device__ __forceinline__ uint4 wide_pick<2>(const uint4* ld, int p) {
    // 8 loads x 8 16-bit pixels -> pixel p: 8 channels, 2 per dword
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 a = ld[2 * i], b = ld[2 * i + 1];
        const uint32_t wa = (p >> 1) == 0 ? a.x : (p >> 1) == 1 ? a.y : (p >> 1) == 2 ? a.z : a.w;
        const uint32_t wb = (p >> 1) == 0 ? b.x : (p >> 1) == 1 ? b.y : (p >> 1) == 2 ? b.z : b.w;
        w[i] = (p & 1) ? ((wa >> 16) | (wb & 0xffff0000u)) : ((wa & 0xffffu) | (wb << 16));
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}
template <>
__device__ __forceinline__ uint4 wide_pick<4>(const uint4* ld, int p) {
    auto word = [](const uint4& v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; };
    return make_uint4(word(ld[0], p), word(ld[1], p), word(ld[2], p), word(ld[3], p));
}
template <>
__device__ __forceinline__ uint4 wide_pick<8>(const uint4* ld, int p) {
    return p == 0 ? make_uint4(ld[0].x, ld[0].y, ld[1].x, ld[1].y) : make_uint4(ld[0].z, ld[0].w, ld[1].z, ld[1].w);
}

// Accumulator and operand types for one fragment size.
template <typename T, int FR> struct Frag;
template <typename T> struct Frag<T, 16> {
    using acc_t = typename Mma<T>::acc_t;
    static constexpr int NPIECE = 1;  // 16-byte pieces per lane per 64-byte chunk
    static constexpr int NACC = 4;
};
template <typename T> struct Frag<T, 32> {
    using acc_t = typename Mma32<T>::acc_t;
    static constexpr int NPIECE = 2;
    static constexpr int NACC = 16;
};

// EPI: the fused epilogue (bias, residual, ReLU) is applied as outputs are
// converted; a separate instantiation, so the plain kernels carry none of
// its registers.
// RES: resident input (int8 NCHW4, 3x3 or 1x1 filters; see the main loop).
template <typename T, int XB, int WM, int WN, int FM, int FN, int STG, int FR, int RSV, bool SPLIT = false,
          bool EPI = false, bool RES = false>
__global__ __launch_bounds__(WM* WN * 64) void igemm_kernel(Args a) {
    constexpr int NTHR = WM * WN * 64;
    constexpr int NT = WN * FN * FR;
    constexpr bool LIN = (FR == 32) || (RSV == 9);  // patch layout (see lds_slot)
    constexpr int E16 = 16 / static_cast<int>(sizeof(T));
    constexpr int CK = 4 * E16;
    using FT = Frag<T, FR>;
    using acc_t = typename FT::acc_t;
    constexpr int NP = FT::NPIECE;
    using WD = Wide<T, XB>;
    constexpr int MAXU = (STG == 1) ? WD::MAXU : kMaxUnitsPerThread;
    constexpr int PP = (STG == 1) ? WD::PP : 1;

    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WM;
    const int wn = wave / WM;
    const int lrow = lane % FR;  // A row / B column this lane feeds
    const int lgrp = lane / FR;  // K group (FR=16: slot 0..3; FR=32: half 0..1)

    // ---- XCD-aware work order: in the linear tile order the output-channel
    // tiles of one pixel tile are adjacent (they share the input patch in an
    // XCD's L2) and consecutive pixel tiles are spatial neighbours (they share
    // halo rows).
    int lin = xcd_linear(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
    // split reduction: the split index is outermost in the work order, so the
    // workgroups running together on one XCD share a chunk range (and its
    // input channels and weights)
    int cb = 0;             // first channel chunk of this workgroup
    int nch = a.nchunks;    // chunks it sums
    int split = 0;
    if constexpr (SPLIT) {
        const int per = static_cast<int>(gridDim.x) / ((a.nchunks + a.cps - 1) / a.cps);
        split = lin / per;
        lin -= split * per;
        cb = split * a.cps;
        nch = min(a.cps, a.nchunks - cb);
    }
    const int kt = lin % a.ntk;
    lin /= a.ntk;
    const int ntm = a.tiles_w * a.tiles_h * a.tiles_n;
    const int g = lin / ntm;
    int mt = lin - g * ntm;
    const int tw_i = mt % a.tiles_w;
    mt /= a.tiles_w;
    const int th_i = mt % a.tiles_h;
    mt /= a.tiles_h;
    const int n0 = mt * a.TN;
    const int oh0 = th_i * a.TH;
    const int ow0 = tw_i * a.TW;
    const int RS = a.R * a.S;
    const int PHW = a.PH * a.PW;
    const int thw = a.TH * a.TW;
    const int tile_pix = a.TN * thw;
    const int patch_bytes = a.npix * PatchStride<LIN>::value;
    // patch buffers in LDS: three on the nine-tap path of big per-wave tiles
    // (chunk c + 1 is staged while chunk c runs; their registers allow one
    // workgroup per CU anyway, so the LDS costs no occupancy), two otherwise
    constexpr bool TB = (RSV == 9) && (FR == 32) && (FM * FN >= 8);
    constexpr int NBUF = TB ? 3 : 2;
    // buffers actually used: a problem of one or two channel chunks needs no
    // more than that many (its LDS allocation holds only those, so more
    // workgroups share a CU); stores and reads of a next chunk are skipped
    // when there is none
    const int nbuf = min(nch, NBUF);
    const int ih0 = oh0 * a.sh - a.ph;
    const int iw0 = ow0 * a.sw - a.pw;
    const T* __restrict__ x = static_cast<const T*>(a.x);

    // ---- staging units owned by this thread (chunk-invariant parts)
    // STG 0: unit = one pixel x 16 bytes of channels (element gathers).
    // STG 1: unit = PP pixels (one aligned column block) x 16 bytes of channels.
    int u_q[MAXU];   // patch pixel of the unit's first pixel
    int u_j[MAXU];   // 16-byte slot within the 64-byte channel chunk (-1: no unit)
    int u_sp[MAXU];  // spatial offset ih*W + iw of the first pixel, -1 if outside
    int u_n[MAXU];   // image
    int u_pc[MAXU];  // patch column of the unit's first pixel (STG 1; may be < 0)
    int ncb = 1, cb0 = 0;
    if (STG == 1) {
        cb0 = (iw0 >= 0) ? iw0 / PP : -((-iw0 + PP - 1) / PP);
        const int last = iw0 + a.PW - 1;
        const int cb1 = (last >= 0) ? last / PP : -((-last + PP - 1) / PP);
        ncb = cb1 - cb0 + 1;
    }
    const int nrows = a.TN * a.PH;
    const int nunits = (STG == 1) ? 4 * nrows * ncb : 4 * a.npix;
#pragma unroll
    for (int i = 0; i < MAXU; ++i) {
        const int u = tid + i * NTHR;
        u_q[i] = 0;
        u_j[i] = -1;
        u_sp[i] = -1;
        u_n[i] = 0;
        u_pc[i] = 0;
        if (u < nunits) {
            int j, tn, prow, pcol;
            if (STG == 1) {
                j = u & 3;
                const int t = u >> 2;
                const int cb = t % ncb;
                const int row = t / ncb;
                tn = row / a.PH;
                prow = row - tn * a.PH;
                pcol = (cb0 + cb) * PP - iw0;
            } else {
                j = u / a.npix;
                const int q = u - j * a.npix;
                tn = q / PHW;
                const int rem = q - tn * PHW;
                prow = rem / a.PW;
                pcol = rem - prow * a.PW;
            }
            const int n = n0 + tn;
            const int ih = ih0 + prow;
            const int iw = iw0 + pcol;
            u_q[i] = (tn * a.PH + prow) * a.PW + pcol;
            u_pc[i] = pcol;
            u_j[i] = j;
            u_n[i] = n;
            if (n < a.N && static_cast<unsigned>(ih) < static_cast<unsigned>(a.H) &&
                static_cast<unsigned>(iw) < static_cast<unsigned>(a.W))
                u_sp[i] = ih * a.W + iw;
        }
    }

    uint4 stg[MAXU][PP];
    auto stage_load = [&](int chunk, uint4 (&dst)[MAXU][PP]) {
#pragma unroll
        for (int i = 0; i < MAXU; ++i) {
#pragma unroll
            for (int l = 0; l < PP; ++l) dst[i][l] = make_uint4(0, 0, 0, 0);
            if (u_sp[i] < 0) continue;
            const int cl = (chunk + cb) * CK + u_j[i] * E16;
            const int nval = a.Cg - cl;
            if (nval <= 0) continue;
            const int c0 = g * a.Cg + cl;
            const T* xn = x + u_n[i] * a.x_img;
            if (STG == 1) {
                using R = typename Raw<T>::type;
                const R* xr = reinterpret_cast<const R*>(xn);
                const long long HW = static_cast<long long>(a.H) * a.W;
#pragma unroll
                for (int l = 0; l < PP; ++l) {
                    if (XB == 1) {
                        if (l < nval)
                            dst[i][l] = *reinterpret_cast<const uint4*>(xr + (c0 + l) * HW + u_sp[i]);
                    } else {
                        if (l * XB < nval)
                            dst[i][l] = *reinterpret_cast<const uint4*>(xr + ((c0 / XB + l) * HW + u_sp[i]) * XB);
                    }
                }
            } else {
                dst[i][0] = load_unit<T, XB>(xn, a.H, a.W, c0, nval, u_sp[i]);
            }
        }
    };
    auto stage_store = [&](int buf, const uint4 (&src)[MAXU][PP]) {
        uint8_t* base = lds + buf * patch_bytes;
#pragma unroll
        for (int i = 0; i < MAXU; ++i) {
            if (u_j[i] < 0) continue;
            if (STG == 1) {
                // pixels outside this patch row go to a per-thread dummy slot
                // past both patch buffers (no branch per pixel)
                uint8_t* dummy = lds + nbuf * patch_bytes + tid * 16;
#pragma unroll
                for (int p = 0; p < PP; ++p) {
                    const int col = u_pc[i] + p;
                    const bool ok = col >= 0 && col < a.PW;
                    uint8_t* dst = ok ? base + lds_slot<LIN>(u_q[i] + p, u_j[i]) : dummy;
                    *reinterpret_cast<uint4*>(dst) = wide_pick<WD::SZ>(src[i], p);
                }
            } else {
                *reinterpret_cast<uint4*>(base + lds_slot<LIN>(u_q[i], u_j[i])) = src[i][0];
            }
        }
    };

    // Branch-free staging of one 16-byte load, index l = unit * PP + load,
    // for chunk `chunk` (wide staging only).  Invalid pixels or channels load
    // from the tensor base and are zeroed afterwards, so every call issues
    // exactly one load and the compiler can count outstanding loads exactly.
    // The chunk-invariant part of each unit's element offset (image, pixel,
    // 16-byte channel part) is computed once, so a load costs a 64-bit add:
    // channel block (c0 / XB + ld) of pixel sp is element
    // (c0 / XB + ld) * H * W * XB + sp * XB of the image (XB = 1: channel
    // c0 + ld), and a chunk is CK / XB channel blocks (the wide path only runs
    // where C / G and the chunk are whole channel blocks).
    const long long HWX = static_cast<long long>(a.H) * a.W * XB;
    long long u_base[MAXU];
#pragma unroll
    for (int i = 0; i < MAXU; ++i) {
        const int j = u_j[i] < 0 ? 0 : u_j[i];
        u_base[i] = (u_sp[i] >= 0) ? u_n[i] * a.x_img + static_cast<long long>((g * a.Cg + j * E16) / XB) * HWX +
                                         static_cast<long long>(u_sp[i]) * XB
                                   : 0;
    }
    auto stage_piece = [&](int chunk, int l) {
        using R = typename Raw<T>::type;
        const int i = l / PP, ld = l % PP;
        const int cl = (chunk + cb) * CK + (u_j[i] < 0 ? 0 : u_j[i]) * E16;
        const int nval = a.Cg - cl;
        const bool valid = (u_sp[i] >= 0) && (XB == 1 ? ld < nval : ld * XB < nval);
        const long long off = u_base[i] + static_cast<long long>((chunk + cb) * (CK / XB) + ld) * HWX;
        const R* src = reinterpret_cast<const R*>(x) + (valid ? off : 0);
        const uint4 v = *reinterpret_cast<const uint4*>(src);
        stg[i][ld] = valid ? v : make_uint4(0, 0, 0, 0);
    };

    // ---- per-lane A fragment bases (pixel index inside the patch)
    int qbase[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f) {
        const int p = (wm * FM + f) * FR + lrow;
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
    // 16-byte slots this lane reads for its pieces
    int pslot[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) pslot[i] = (FR == 16) ? lgrp : piece_slot<T>(i, lgrp);

    // ---- B (prepared weights).  One tap of one output-channel tile is NT rows
    // of 64 bytes, laid out so that each fragment piece is 1 KB contiguous:
    // FR=16: [NT][64 B] (lane reads row lrow, slot lgrp);
    // FR=32: [NT/32][piece][32 rows][half][16 B].
    const uint8_t* __restrict__ wtile = static_cast<const uint8_t*>(a.wp) +
                                        (static_cast<long long>(g * a.ntk + kt) * a.nchunks + cb) * RS * NT * 64;
    const int boff = (FR == 16) ? (wn * FN * 16 + lrow) * 64 + lgrp * 16 : (wn * FN * 2 * 32 + lrow) * 32 + lgrp * 16;
    auto load_b = [&](uint4 (*b)[NP], int it) {
        const uint8_t* p = wtile + static_cast<long long>(it) * NT * 64 + boff;
#pragma unroll
        for (int nf = 0; nf < FN; ++nf)
#pragma unroll
            for (int i = 0; i < NP; ++i)
                b[nf][i] = *reinterpret_cast<const uint4*>(p + (FR == 16 ? nf * 1024 : (nf * 2 + i) * 1024));
    };
    auto load_a = [&](uint4 (*af)[NP], const uint8_t* pb, int toff) {
#pragma unroll
        for (int f = 0; f < FM; ++f) {
            const int q = qbase[f] + toff;
#pragma unroll
            for (int i = 0; i < NP; ++i) af[f][i] = *reinterpret_cast<const uint4*>(pb + lds_slot<LIN>(q, pslot[i]));
        }
    };

    acc_t acc[FM][FN];
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int nf = 0; nf < FN; ++nf) acc[f][nf] = acc_t{};

    auto mma = [&](uint4 (*af)[NP], uint4 (*bf)[NP]) {
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int nf = 0; nf < FN; ++nf) {
                if constexpr (FR == 16)
                    Mma<T>::run(acc[f][nf], af[f][0], bf[nf][0]);
                else
                    Mma32<T>::run(acc[f][nf], af[f][0], af[f][1], bf[nf][0], bf[nf][1]);
            }
    };

    uint4 bcur[FN][NP], bnxt[FN][NP];
    if constexpr (RSV != 9 && !RES) {
        load_b(bcur, 0);
        stage_load(0, stg);
        stage_store(0, stg);
        __syncthreads();
    }

    const int total_it = nch * RS;
    int it = 0;
    if constexpr (RES) {
        // ---- resident input (deep layers with small images: ResNet's 14x14
        // and 7x7 stages).  A layer with a long reduction and few output
        // pixels has few tiles, so each CU runs one or two workgroups, and
        // staging one channel chunk at a time leaves every chunk's load
        // latency (and barrier) exposed.  Here the input rows the tile reads
        // -- whole rows, every channel chunk -- are requested at once, written
        // to LDS, and after one barrier the taps run from LDS with no further
        // barrier: only the weights stream in, one or two chunks ahead.
        //
        // The rows [r0, r1) of an image are one flat run of pixels in each
        // NCHW4 channel-block plane, so they are staged as 16-byte loads of 4
        // consecutive flat pixels (buffer loads: the run's last group may
        // reach past the tensor, which reads as zero), transposed in
        // registers into 4 pixels x 16 bytes of channels.  No halo is kept:
        // a tap that falls outside the image (or a tile row past the batch)
        // reads a zeroed pixel slot instead.
        //
        // LDS per chunk: image tn's pixel (ih, iw) at slot q = tn * e4 +
        // (ih - r0) * W + iw (e4: the run rounded up to 4 pixels), the zero
        // slot at TN * e4; 64 bytes of channels per slot, its 16-byte part j
        // at position j ^ ((q >> SW) & 3) (the lanes of one fragment read,
        // consecutive pixels of one part, spread over the banks).
        static_assert(sizeof(T) == 1 && XB == 4 && !SPLIT && (RSV == 9 || RSV == 1),
                      "resident input: int8 NCHW4, 3x3 or 1x1");
        constexpr int SW = (FR == 32) ? 2 : 1;
        const int r0 = max(ih0, 0), r1 = min(ih0 + a.PH, a.H);
        const int p0 = r0 * a.W;
        const int e4 = (max(r1 - r0, 0) * a.W + 3) & ~3;
        const int zq = a.TN * e4;
        const int chunk_bytes = (zq + 1) * 64;
        {
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<T*>(x), static_cast<short>(0), static_cast<int>(static_cast<long long>(a.N) * a.x_img),
                0x00020000);
            const unsigned HW = static_cast<unsigned>(a.H * a.W);
            const int g4 = e4 / 4;                   // 4-pixel groups per image
            const int units = nch * a.TN * g4 * 4;   // (chunk, image, group, 16-byte part)
            for (int i = tid; i < nch * 4; i += NTHR)
                *reinterpret_cast<uint4*>(lds + (i >> 2) * chunk_bytes + zq * 64 + (i & 3) * 16) = make_uint4(0, 0, 0, 0);
            constexpr int MB = 4;  // units per thread in flight
            for (int u0 = 0; u0 < units; u0 += MB * NTHR) {
                uint4 ld[MB][4];
                int dc[MB], dq[MB], dj[MB];  // chunk buffer, first slot, 16-byte part (dq < 0: none)
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    const int u = u0 + m * NTHR + tid;
                    const int j = u & 3;
                    int rest = u >> 2;
                    const int g = rest % g4;
                    rest /= g4;
                    const int tn = rest % a.TN;
                    const int c = rest / a.TN;
                    const int n = n0 + tn;
                    const bool ok = u < units && n < a.N;
                    // channel blocks 16 c + 4 j + b, pixels p0 + 4 g .. + 3
                    const unsigned base = static_cast<unsigned>(n * a.x_img) +
                                          ((static_cast<unsigned>(16 * c + 4 * j)) * HW + p0 + 4 * g) * 4u;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        // past the buffer's range (all of x is below 2^31 bytes): reads zero
                        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, ok ? base + b * HW * 4u : 0x80000000u, 0, 0);
                        ld[m][b] = make_uint4(v[0], v[1], v[2], v[3]);
                    }
                    dc[m] = c * chunk_bytes;
                    dq[m] = (u < units) ? tn * e4 + 4 * g : -1;
                    dj[m] = j;
                }
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    if (dq[m] < 0) continue;
#pragma unroll
                    for (int pp = 0; pp < 4; ++pp) {
                        const int q = dq[m] + pp;
                        *reinterpret_cast<uint4*>(lds + dc[m] + (q << 6) + ((dj[m] ^ ((q >> SW) & 3)) << 4)) =
                            wide_pick<4>(ld[m], pp);
                    }
                }
            }
        }
        // weights: a ring of D tap buffers, each refilled right after its
        // use with the tap D ahead -- two chunks (3x3) or sixteen taps (1x1)
        // where a tap's weights are at most two 16-byte pieces per lane, one
        // chunk or eight taps otherwise (an L2 hit takes about a thousand
        // cycles under this load, several taps' worth of matrix-core work)
        constexpr bool DEEP = FN * NP <= 2;
        constexpr int D = (RSV == 9) ? (DEEP ? 18 : 9) : (DEEP ? 16 : 8);
        // taps per loop body: a multiple of the ring (ring slots and taps
        // known at compile time) and even (A double buffer, below)
        constexpr int U = (RSV == 9) ? 18 : 16;
        const int last_it = total_it - 1;
        uint4 wr[D][FN][NP];
#pragma unroll
        for (int d = 0; d < D; ++d) load_b(wr[d], min(d, last_it));
        // A byte offsets inside a chunk buffer, per tap and fragment (piece 1
        // of a 32x32 fragment is slot 2 + h: the address with bit 5 flipped)
        int boff[RSV][FM];
#pragma unroll
        for (int f = 0; f < FM; ++f) {
            // this lane's output pixel of fragment f and the input pixel of tap (0, 0)
            const int p = (wm * FM + f) * FR + lrow;
            const int tn = p / thw;
            const int rem = p - tn * thw;
            const int ohl = rem / a.TW;
            const int owl = rem - ohl * a.TW;
            const bool prow = p < tile_pix && n0 + tn < a.N;
            const int ihb = (oh0 + ohl) * a.sh - a.ph;
            const int iwb = (ow0 + owl) * a.sw - a.pw;
#pragma unroll
            for (int t = 0; t < RSV; ++t) {
                const int ih = ihb + (t / a.S) * a.dh, iw = iwb + (t % a.S) * a.dw;
                const bool ok = prow && static_cast<unsigned>(ih) < static_cast<unsigned>(a.H) &&
                                static_cast<unsigned>(iw) < static_cast<unsigned>(a.W);
                const int q = ok ? tn * e4 + ih * a.W + iw - p0 : zq;
                boff[t][f] = (q << 6) + ((pslot[0] ^ ((q >> SW) & 3)) << 4);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);  // every direct load has landed (and the first weights)
        __syncthreads();
        // A double buffer: the next tap's fragments are requested before
        // this tap's matrix-core instructions, which then cover the LDS latency
        uint4 ra[2][FM][NP];
        auto read_a = [&](uint4 (&dst)[FM][NP], const uint8_t* pb, int t) {
#pragma unroll
            for (int f = 0; f < FM; ++f) {
                const uint8_t* pa = pb + boff[t][f];
                dst[f][0] = *reinterpret_cast<const uint4*>(pa);
                if constexpr (NP == 2)
                    dst[f][1] = *reinterpret_cast<const uint4*>(lds + ((static_cast<int>(pa - lds)) ^ 32));
            }
        };
        // tap it0 + d; it0 is a multiple of U (so of 9 for 3x3 filters)
        auto tap = [&](int it0, int d) {
            const int itd = it0 + d;
            // the tap after this one (at the very end: tap 0 of the last
            // chunk, read and never used)
            const int itn = min(itd + 1, last_it);
            const int cn = (RSV == 9) ? itn / 9 : itn;
            read_a(ra[(d + 1) & 1], lds + cn * chunk_bytes, (RSV == 9) ? (d + 1) % 9 : 0);
            // piece-major (32x32): the two MFMAs into one accumulator are FM * FN
            // instructions apart
#pragma unroll
            for (int i = 0; i < NP; ++i)
#pragma unroll
                for (int f = 0; f < FM; ++f)
#pragma unroll
                    for (int nf = 0; nf < FN; ++nf) {
                        if constexpr (FR == 16)
                            Mma<T>::run(acc[f][nf], ra[d & 1][f][0], wr[d % D][nf][0]);
                        else
                            Mma32<T>::piece(acc[f][nf], ra[d & 1][f][i], wr[d % D][nf][i], i);
                    }
            load_b(wr[d % D], min(itd + D, last_it));
        };
        read_a(ra[0], lds, 0);
        // whole loop bodies without a branch inside (the compiler can then
        // count the loads in flight across iterations), then the remainder
        const int nfull = total_it / U;
        for (int o = 0; o < nfull; ++o) {
#pragma unroll
            for (int d = 0; d < U; ++d) tap(o * U, d);
        }
        const int rem = total_it - nfull * U;
#pragma unroll
        for (int d = 0; d < U; ++d)
            if (d < rem) tap(nfull * U, d);
        it = total_it;
        __syncthreads();  // the epilogue reuses the patch's LDS
    } else if constexpr (RSV == 9 && FR == 32) {
        // 3x3 (nine-tap) filters, 32x32 fragments, wide staging: the nine taps
        // of a chunk are unrolled so that every register buffer is addressed
        // at compile time (a copy between prefetch buffers would make the
        // compiler wait for the load behind it):
        //  * weights: a ring of three tap buffers, tap t+2 requested at tap t;
        //  * activations, big per-wave tiles (TB): three patch buffers, chunk
        //    c in buffer c % 3.  While chunk c runs, chunk c + 1 is already in
        //    LDS and the eight 16-byte loads of chunk c + 2 are issued, one per
        //    tap, each after that tap's weight request (so no weight wait
        //    waits for an activation load); they are written to LDS at the
        //    chunk's end, followed by the chunk's only barrier.  Buffer
        //    (c + 2) % 3 held chunk c - 1, whose last reads were issued and
        //    completed before the barrier that ended chunk c - 1;
        //  * activations, otherwise: two buffers, the loads of chunk c + 1
        //    issued during chunk c and written at its end;
        //  * A: rolling single buffer refilled right after each use; with TB
        //    the last tap's refill already reads the next chunk's first tap,
        //    so the matrix cores do not wait for LDS across a chunk boundary.
        static_assert(FR == 32 && STG == 1 && MAXU * PP == 8, "nine-tap path needs 32x32 tiles and wide staging");
        uint4 ring[3][FN][NP];
        uint4 ra[FM][NP];
        // byte offsets: tap (uniform) and fragment base (per lane); piece i of
        // a fragment is a further i * PSTEP bytes (piece_slot is 2i + h for
        // 16-bit / 8-bit types and 2h + i for fp32)
        constexpr int PS = PatchStride<LIN>::value;
        constexpr int PSTEP = (sizeof(T) == 4) ? 16 : 32;
        int toffs[9];
#pragma unroll
        for (int t = 0; t < 9; ++t) toffs[t] = ((t / a.S) * a.dh * a.PW + (t % a.S) * a.dw) * PS;
        int abase[FM];
#pragma unroll
        for (int f = 0; f < FM; ++f) abase[f] = qbase[f] * PS + pslot[0] * 16;
        const int last_it = total_it - 1;
        // prologue: the weights of the first two taps and the first chunk(s)
        // of activations are all requested before anything is waited for
        load_b(ring[0], 0);
        load_b(ring[1], min(1, last_it));
        if constexpr (TB) {
            uint4 stg1[MAXU][PP];
            stage_load(0, stg);
            stage_load(1, stg1);  // zeros past the last chunk
            stage_store(0, stg);
            if (nch > 1) stage_store(1, stg1);
        } else {
            stage_load(0, stg);
            stage_store(0, stg);
        }
        __syncthreads();
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int i = 0; i < NP; ++i) ra[f][i] = *reinterpret_cast<const uint4*>(lds + abase[f] + i * PSTEP);
        int bc = 0;  // buffer of chunk c
        for (int chunk = 0; chunk < nch; ++chunk) {
            const int bnext = TB ? ((bc == 2) ? 0 : bc + 1) : (bc ^ 1);
            const int bfar = (bnext == 2) ? 0 : bnext + 1;
            const uint8_t* pb = lds + bc * patch_bytes;
            const uint8_t* pn = lds + bnext * patch_bytes;
            const int it0 = chunk * 9;
#pragma unroll
            for (int t = 0; t < 9; ++t) {
                load_b(ring[(t + 2) % 3], min(it0 + t + 2, last_it));
                if (t < 8) stage_piece(chunk + (TB ? 2 : 1), t);
                // (at the last chunk the last tap again: there is no next buffer)
                const uint8_t* pt =
                    (t < 8) ? pb + toffs[t + 1] : ((TB && chunk + 1 < nch) ? pn + toffs[0] : pb + toffs[8]);
#pragma unroll
                for (int i = 0; i < NP; ++i) {
#pragma unroll
                    for (int f = 0; f < FM; ++f) {
#pragma unroll
                        for (int nf = 0; nf < FN; ++nf) Mma32<T>::piece(acc[f][nf], ra[f][i], ring[t % 3][nf][i], i);
                        ra[f][i] = *reinterpret_cast<const uint4*>(pt + abase[f] + i * PSTEP);
                    }
                }
            }
            if constexpr (TB) {
                if (chunk + 2 < nch) stage_store(bfar, stg);
                __syncthreads();
            } else {
                const bool more = chunk + 1 < nch;
                if (more) stage_store(bnext, stg);
                __syncthreads();
                if (more) {
#pragma unroll
                    for (int f = 0; f < FM; ++f)
#pragma unroll
                        for (int i = 0; i < NP; ++i)
                            ra[f][i] = *reinterpret_cast<const uint4*>(pn + abase[f] + i * PSTEP);
                }
            }
            bc = bnext;
        }
        it = total_it;
    } else if constexpr (RSV == 9) {
        // 3x3 filters, 16x16 fragments: thin per-wave tiles (a few MFMAs per
        // tap), chosen for layers with a deep reduction and few pixels, where
        // a weight fetch from L2 outlasts several taps of MFMAs.  The nine
        // taps of a chunk are unrolled with one weight buffer per tap,
        // refilled right after its use with the same tap of the next chunk,
        // so every weight fetch has a whole chunk to land.  Two patch buffers
        // (chunk c + 1 written at the end of chunk c; its loads issued at the
        // start of chunk c, or one per tap with wide staging), A refilled
        // right after each use; the patch uses the linear layout, so a tap is
        // a uniform offset.
        static_assert(FR == 16 && (STG == 0 || MAXU * PP == 8), "nine-tap 16x16 path");
        uint4 wr9[9][FN][NP];
        uint4 ra[FM];
        constexpr int PS = PatchStride<LIN>::value;
        int toffs[9];  // byte offset of each tap (uniform)
#pragma unroll
        for (int t = 0; t < 9; ++t) toffs[t] = ((t / a.S) * a.dh * a.PW + (t % a.S) * a.dw) * PS;
        int abase[FM];
#pragma unroll
        for (int f = 0; f < FM; ++f) abase[f] = lds_slot<LIN>(qbase[f], pslot[0]);
        const int last_it = total_it - 1;
#pragma unroll
        for (int t = 0; t < 9; ++t) load_b(wr9[t], t);
        stage_load(0, stg);
        stage_store(0, stg);
        __syncthreads();
#pragma unroll
        for (int f = 0; f < FM; ++f) ra[f] = *reinterpret_cast<const uint4*>(lds + abase[f]);
        for (int chunk = 0; chunk < nch; ++chunk) {
            const int buf = chunk & 1;
            const bool more = chunk + 1 < nch;
            const uint8_t* pb = lds + buf * patch_bytes;
            const int itn = (chunk + 1) * 9;  // first tap of the next chunk
            if constexpr (STG == 0) {
                if (more) stage_load(chunk + 1, stg);
            }
#pragma unroll
            for (int t = 0; t < 9; ++t) {
                if constexpr (STG == 1) {
                    if (t < 8) stage_piece(chunk + 1, t);
                }
                const uint8_t* pt = pb + toffs[t < 8 ? t + 1 : 8];
#pragma unroll
                for (int f = 0; f < FM; ++f) {
#pragma unroll
                    for (int nf = 0; nf < FN; ++nf) Mma<T>::run(acc[f][nf], ra[f], wr9[t][nf][0]);
                    ra[f] = *reinterpret_cast<const uint4*>(pt + abase[f]);
                }
                load_b(wr9[t], min(itn + t, last_it));
            }
            if (more) stage_store(buf ^ 1, stg);
            __syncthreads();
            if (more) {
                const uint8_t* pn = lds + (buf ^ 1) * patch_bytes;
#pragma unroll
                for (int f = 0; f < FM; ++f) ra[f] = *reinterpret_cast<const uint4*>(pn + abase[f]);
            }
        }
        it = total_it;
    } else if constexpr (FR == 32) {
        // 32x32 fragments run one wave per SIMD and are software-pipelined
        // by hand, with a branch-free tap body:
        //  * A is a rolling single buffer: once fragment f's MFMAs of this
        //    tap are issued, its registers are refilled from LDS with
        //    fragment f of the next tap (at a chunk's last tap, the same tap
        //    again: harmless), which then has FM-1 fragments of MFMAs to land;
        //  * B (weights, from L2) is prefetched two taps ahead, so the next
        //    chunk's staging loads -- issued at the chunk start, behind the
        //    weights of its first two taps -- are not waited for until the
        //    third tap.
        uint4 ra[FM][NP];
        uint4 b2[FN][NP];
        auto read_a = [&](const uint8_t* pb, int toff) {
#pragma unroll
            for (int f = 0; f < FM; ++f) {
                const int q = qbase[f] + toff;
#pragma unroll
                for (int i = 0; i < NP; ++i) ra[f][i] = *reinterpret_cast<const uint4*>(pb + lds_slot<LIN>(q, pslot[i]));
            }
        };
        load_b(bnxt, total_it > 1 ? 1 : 0);
        read_a(lds, 0);
        const int last_it = total_it - 1;
        for (int chunk = 0; chunk < nch; ++chunk) {
            const int buf = chunk & 1;
            const bool more = chunk + 1 < nch;
            const uint8_t* pb = lds + buf * patch_bytes;
            if (more) stage_load(chunk + 1, stg);
            int r = 0, s = 0;
            for (int rs = 0; rs < RS; ++rs, ++it) {
                load_b(b2, min(it + 2, last_it));
                // offset of the next tap within this chunk (this tap at the end)
                int rn = r, sn = s + 1;
                if (sn == a.S) {
                    sn = 0;
                    ++rn;
                }
                const bool has_next = rs + 1 < RS;
                const int toff_next = has_next ? rn * a.dh * a.PW + sn * a.dw : r * a.dh * a.PW + s * a.dw;
                // Piece-major issue order: every fragment's first K piece, then
                // every fragment's second, so the two MFMAs accumulating into
                // one register tile are FM*FN instructions apart (a dependent
                // MFMA issued back to back waits for the previous result).
                // Each piece's registers are refilled with the next tap right
                // after their last use.
#pragma unroll
                for (int i = 0; i < NP; ++i) {
#pragma unroll
                    for (int f = 0; f < FM; ++f) {
#pragma unroll
                        for (int nf = 0; nf < FN; ++nf) Mma32<T>::piece(acc[f][nf], ra[f][i], bcur[nf][i], i);
                        ra[f][i] = *reinterpret_cast<const uint4*>(
                            pb + lds_slot<LIN>(qbase[f] + toff_next, pslot[i]));
                    }
                }
#pragma unroll
                for (int nf = 0; nf < FN; ++nf)
#pragma unroll
                    for (int i = 0; i < NP; ++i) {
                        bcur[nf][i] = bnxt[nf][i];
                        bnxt[nf][i] = b2[nf][i];
                    }
                if (has_next) {
                    r = rn;
                    s = sn;
                }
            }
            if (more) stage_store(buf ^ 1, stg);
            __syncthreads();
            if (more) read_a(lds + (buf ^ 1) * patch_bytes, 0);
        }
    } else {
        for (int chunk = 0; chunk < nch; ++chunk) {
            const int buf = chunk & 1;
            const bool more = chunk + 1 < nch;
            const uint8_t* pb = lds + buf * patch_bytes;
            if (more) stage_load(chunk + 1, stg);
            int r = 0, s = 0;
            for (int rs = 0; rs < RS; ++rs, ++it) {
                if (it + 1 < total_it) load_b(bnxt, it + 1);
                uint4 afr[FM][NP];
                load_a(afr, pb, r * a.dh * a.PW + s * a.dw);
                mma(afr, bcur);
#pragma unroll
                for (int nf = 0; nf < FN; ++nf) bcur[nf][0] = bnxt[nf][0];
                if (++s == a.S) {
                    s = 0;
                    ++r;
                }
            }
            if (more) stage_store(buf ^ 1, stg);
            __syncthreads();
        }
    }

    // ---- split reduction: the int32 partial tile of this workgroup's chunk
    // range goes to its split's partial buffer in the output's NCHW4 order
    // (one pixel's four channels = 16 bytes), where the reduce kernel sums the
    // splits and requantises (int32 addition is exact in any order, so the
    // result is the same bit for bit).  A lane holds one channel of four pixel
    // rows; the tile is transposed through LDS as [channel block][tile
    // pixel][4 channels] so that each lane then stores one pixel's 16 bytes
    // and consecutive lanes store consecutive pixels of a channel block.
    if constexpr (SPLIT) {
        static_assert(sizeof(T) == 1 && XB == 4, "split reduction: int8 NCHW4 only");
        // bytes per channel block in LDS; the 64-byte pad takes the up to three
        // rows past tile_pix of a register tile's last 4-row group
        const int pitch = tile_pix * 16 + 64;
        constexpr int NG = FT::NACC / 4;
#pragma unroll
        for (int nf = 0; nf < FN; ++nf) {
            const int kk = (wn * FN + nf) * FR + lrow;  // channel within the tile
            int32_t* cbase = reinterpret_cast<int32_t*>(lds + (kk >> 2) * pitch) + (kk & 3);
#pragma unroll
            for (int f = 0; f < FM; ++f)
#pragma unroll
                for (int grp = 0; grp < NG; ++grp) {
                    const int p0 = (wm * FM + f) * FR + (FR == 16 ? 4 * lgrp : 8 * grp + 4 * lgrp);
                    if (p0 < tile_pix) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) cbase[(p0 + v) * 4] = acc[f][nf][grp * 4 + v];
                    }
                }
        }
        __syncthreads();
        const int OHW = a.OH * a.OW;
        int32_t* pbase = a.part + static_cast<long long>(split) * a.N * a.y_img;
        const int kb0 = kt * NT / 4;                          // first channel block of the tile
        const int nkb4 = (min(NT, a.Kg - kt * NT) + 3) / 4;   // channel blocks it writes
        const int nimg = min(a.TN, a.N - n0);
        for (int q = tid; q < nkb4 * tile_pix; q += NTHR) {
            const int kb = q / tile_pix, pp = q - (q / tile_pix) * tile_pix;
            const int tn = pp / thw, rem = pp - (pp / thw) * thw;
            const int ohl = rem / a.TW, owl = rem - (rem / a.TW) * a.TW;
            const int oh = oh0 + ohl, ow = ow0 + owl;
            if (tn >= nimg || oh >= a.OH || ow >= a.OW) continue;
            const uint4 v = *reinterpret_cast<const uint4*>(lds + kb * pitch + pp * 16);
            *reinterpret_cast<uint4*>(pbase + (n0 + tn) * a.y_img + ((kb0 + kb) * OHW + oh * a.OW + ow) * 4) = v;
        }
        return;
    }

    // ---- epilogue for int8 NCHW4 outputs of tiles of whole output rows (or
    // whole images): a lane holds four consecutive pixels of one channel,
    // whose bytes lie 4 bytes apart in NCHW4, so storing them directly writes
    // single bytes all over the planes.  Instead the requantised tile is
    // written to LDS in NCHW4 order, [channel block][tile pixel][4 channels]
    // (row pitch padded by 16 bytes); a channel block's pixels of one image
    // are contiguous in the output, so consecutive lanes then write
    // consecutive 16-byte pieces of 4 pixels x 4 channels, or, where pieces
    // would not be aligned, consecutive pixels' dwords.
    if constexpr (sizeof(T) == 1 && XB == 4) {
        const bool rows_ok = a.TW == a.OW && (a.TN == 1 ? oh0 + a.TH <= a.OH : a.TH == a.OH) && (a.Kg % 4) == 0;
        if (rows_ok) {
            const int pitch = tile_pix * 4 + 16;  // bytes per channel block in LDS
            const int kt0 = g * a.Kg + kt * NT;   // first output channel of the tile
            constexpr int NG = FT::NACC / 4;
#pragma unroll
            for (int nf = 0; nf < FN; ++nf) {
                const int kk = (wn * FN + nf) * FR + lrow;  // channel within the tile
                const int k = kt0 + kk;
                const bool kval = kt * NT + kk < a.Kg;
                const float sc0 = a.scale[kval ? k : 0];  // no branch around the load
                const float sc = kval ? sc0 : 0.0f;
                // the quad of lanes kk & ~3 .. + 3 holds one channel block:
                // its bytes are transposed across the quad so that each lane
                // writes one pixel's 4 channels as a dword
                uint8_t* cb_base = lds + (kk >> 2) * pitch;
                // fused epilogue: channels past K (scale 0) take the last real
                // channel's bias; pixels of images past N read image N - 1
                // (their bytes are never stored)
                const int ke = EPI ? min(k, a.K - 1) : 0;
                const long long kofs = EPI ? static_cast<long long>(k >> 2) * a.OH * a.OW * 4 + (k & 3) +
                                                 static_cast<long long>(oh0) * a.OW * 4
                                           : 0;
                const int ebias = (EPI && a.e.bias) ? static_cast<const int32_t*>(a.e.bias)[ke] : 0;
                const float elo = (EPI && a.e.relu) ? 0.0f : -127.0f;
#pragma unroll
                for (int f = 0; f < FM; ++f) {
                    // fused epilogue: this fragment's residual bytes, all
                    // requested before any is used; a 4-pixel group's image
                    // and offset come from one division
                    float eres[NG][4];
                    if constexpr (EPI) {
#pragma unroll
                        for (int grp = 0; grp < NG; ++grp) {
                            const int p0 = (wm * FM + f) * FR + (FR == 16 ? 4 * lgrp : 8 * grp + 4 * lgrp);
                            const int tn0 = p0 / thw, r0 = p0 - tn0 * thw;
#pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                eres[grp][v] = 0.0f;
                                int tn = tn0, rem = r0 + v;
                                while (rem >= thw) {  // images of fewer than 4 pixels wrap more than once
                                    rem -= thw;
                                    ++tn;
                                }
                                if (a.e.res && p0 + v < tile_pix)
                                    eres[grp][v] = static_cast<float>(static_cast<const int8_t*>(
                                        a.e.res)[static_cast<long long>(min(n0 + tn, a.N - 1)) * a.y_img + kofs +
                                                 static_cast<long long>(rem) * 4]);
                            }
                        }
                    }
#pragma unroll
                    for (int grp = 0; grp < NG; ++grp) {
                        const int p0 = (wm * FM + f) * FR + (FR == 16 ? 4 * lgrp : 8 * grp + 4 * lgrp);
                        uint32_t q[4];
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            if constexpr (EPI)
                                q[v] = requant_i8_fused(acc[f][nf][grp * 4 + v], ebias, sc, eres[grp][v], elo);
                            else
                                q[v] = requant_i8_bits(acc[f][nf][grp * 4 + v], sc);
                        }
                        const uint32_t d = quad_transpose_bytes(pack_low_bytes(q[0], q[1], q[2], q[3]), lane);
                        // (pixels past the tile land in the row's 16-byte pad)
                        if (p0 < tile_pix) *reinterpret_cast<uint32_t*>(cb_base + (p0 + (lane & 3)) * 4) = d;
                    }
                }
            }
            __syncthreads();
            const long long OHW = static_cast<long long>(a.OH) * a.OW;
            uint8_t* ybase = static_cast<uint8_t*>(a.y) + static_cast<long long>(n0) * a.y_img +
                             static_cast<long long>(oh0) * a.OW * 4;
            const int nkb4 = min(NT, a.Kg - kt * NT) / 4;  // channel blocks of this tile
            if (a.TN == 1 && (tile_pix % 4) == 0 && (a.OW % 4) == 0) {
                const int pieces = tile_pix / 4;  // 16-byte pieces per channel block
                for (int q = tid; q < nkb4 * pieces; q += NTHR) {
                    const int kb = q / pieces, j = q - (q / pieces) * pieces;
                    const uint4 v = *reinterpret_cast<const uint4*>(lds + kb * pitch + j * 16);
                    const u32x4_t w = {v.x, v.y, v.z, v.w};
                    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(ybase + ((kt0 / 4 + kb) * OHW) * 4 + j * 16));
                }
            } else {
                // one pixel's 4 channels (a dword) per lane; tile pixel p is
                // pixel p % (TH * TW) of image n0 + p / (TH * TW)
                const int nimg = min(a.TN, a.N - n0);
                for (int q = tid; q < nkb4 * tile_pix; q += NTHR) {
                    const int kb = q / tile_pix, pp = q - (q / tile_pix) * tile_pix;
                    const int tn = pp / thw, rem = pp - (pp / thw) * thw;
                    if (tn >= nimg) continue;
                    const uint32_t v = *reinterpret_cast<const uint32_t*>(lds + kb * pitch + pp * 4);
                    *reinterpret_cast<uint32_t*>(ybase + tn * a.y_img + ((kt0 / 4 + kb) * OHW + rem) * 4) = v;
                }
            }
            return;
        }
    }

    // ---- epilogue, transposed through LDS (16-bit outputs, NCHW, tiles of
    // whole output rows): the accumulators hold, per lane, one output channel
    // of several 4-pixel groups, so storing them directly would scatter every
    // store instruction over 64 channel planes.  Instead the tile is written
    // to LDS as [channel][tile pixel] (row pitch padded by 16 bytes) and then
    // stored row by row: a channel's tile pixels are contiguous in NCHW, so
    // consecutive lanes write consecutive 16-byte pieces.
    if constexpr (sizeof(T) == 2 && XB == 1 && FR == 32) {
        const bool rows_ok = a.TN == 1 && a.TW == a.OW && oh0 + a.TH <= a.OH && (tile_pix % 8) == 0 &&
                             (a.OW % 8) == 0;
        if (rows_ok) {
            const int pitch = tile_pix * 2 + 16;  // bytes per channel row in LDS
#pragma unroll
            for (int nf = 0; nf < FN; ++nf) {
                const int kk = (wn * FN + nf) * FR + lrow;  // channel within the tile
                const int kl = kt * NT + kk;
                // fused epilogue (whole output rows of one image): output
                // offset of this channel's first tile pixel
                const long long ko = EPI ? static_cast<long long>(n0) * a.y_img +
                                               static_cast<long long>(g * a.Kg + kl) * a.OH * a.OW +
                                               static_cast<long long>(oh0) * a.OW
                                         : 0;
                const bool kin = kl < a.Kg;
                const float ebias = (EPI && a.e.bias && kin) ? static_cast<const float*>(a.e.bias)[g * a.Kg + kl] : 0.0f;
#pragma unroll
                for (int f = 0; f < FM; ++f) {
                    // fused epilogue: this fragment's residual values, all
                    // requested before any is used
                    constexpr int NGB = FT::NACC / 4;
                    float eres[NGB][4];
                    if constexpr (EPI) {
#pragma unroll
                        for (int grp = 0; grp < NGB; ++grp) {
                            const int p0 = (wm * FM + f) * FR + 8 * grp + 4 * lgrp;
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                eres[grp][v] = (a.e.res && kin && p0 + v < tile_pix)
                                                   ? Elem<T>::to_f(static_cast<const T*>(a.e.res)[ko + p0 + v])
                                                   : 0.0f;
                        }
                    }
#pragma unroll
                    for (int grp = 0; grp < NGB; ++grp) {
                        const int p0 = (wm * FM + f) * FR + 8 * grp + 4 * lgrp;
                        if (p0 < tile_pix) {
                            float v4[4];
#pragma unroll
                            for (int v = 0; v < 4; ++v) v4[v] = acc[f][nf][grp * 4 + v];
                            if constexpr (EPI) {
#pragma unroll
                                for (int v = 0; v < 4; ++v) {
                                    const float t = v4[v] + ebias + eres[grp][v];
                                    v4[v] = a.e.relu ? fmaxf(t, 0.0f) : t;
                                }
                            }
                            const uint2 q = make_uint2(pack_bf16x2(v4[0], v4[1]), pack_bf16x2(v4[2], v4[3]));
                            *reinterpret_cast<uint2*>(lds + kk * pitch + p0 * 2) = q;
                        }
                    }
                }
            }
            __syncthreads();
            const int pieces = tile_pix / 8;  // 16-byte pieces per channel row
            const long long OHW = static_cast<long long>(a.OH) * a.OW;
            uint8_t* ybase = static_cast<uint8_t*>(a.y) +
                             (static_cast<long long>(n0) * a.y_img + static_cast<long long>(oh0) * a.OW) * 2;
            const int kbase = g * a.Kg + kt * NT;
            const int nk = min(NT, a.Kg - kt * NT);  // valid channels of this tile
            for (int q = tid; q < nk * pieces; q += NTHR) {
                const int kk = q / pieces, j = q - (q / pieces) * pieces;
                const uint4 v = *reinterpret_cast<const uint4*>(lds + kk * pitch + j * 16);
                const u32x4_t w = {v.x, v.y, v.z, v.w};
                __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(ybase + (kbase + kk) * OHW * 2 + j * 16));
            }
            return;
        }
    }

    // ---- epilogue: convert and store in the caller's layout.  The patch
    // buffers are free now (the last chunk ended with a barrier); they hold a
    // table of each tile pixel's output offset (without the channel term),
    // -1 for pixels outside the output, so the per-element index arithmetic
    // is one LDS read and an add.
    long long* otab = reinterpret_cast<long long*>(lds);
    constexpr int TP = WM * FM * FR;  // pixel rows of the register tiles
    for (int p = tid; p < TP; p += NTHR) {
        long long o = -1;
        if (p < tile_pix) {
            const int tn = p / thw;
            const int rem = p - tn * thw;
            const int ohl = rem / a.TW;
            const int owl = rem - ohl * a.TW;
            const int n = n0 + tn;
            const int oh = oh0 + ohl;
            const int ow = ow0 + owl;
            if (n < a.N && oh < a.OH && ow < a.OW)
                o = n * a.y_img + static_cast<long long>(oh * a.OW + ow) * XB;
        }
        otab[p] = o;
    }
    __syncthreads();
    T* __restrict__ y = static_cast<T*>(a.y);
    const bool vec4 = (XB == 1) && (a.TW % 4 == 0) && (a.OW % 4 == 0);
    const long long OHW = static_cast<long long>(a.OH) * a.OW;
    constexpr int NG = FT::NACC / 4;  // groups of 4 consecutive rows per accumulator
    // rows of group (f, grp): FR=16: 4*lgrp + v; FR=32: 8*grp + 4*lgrp + v
    auto row0 = [&](int f, int grp) { return (wm * FM + f) * FR + (FR == 16 ? 4 * lgrp : 8 * grp + 4 * lgrp); };
    if (vec4) {
        // four consecutive pixels of one channel per store: read this lane's
        // FM*NG pixel-row offsets in one batch, then issue every store
        long long o[FM][NG];
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int grp = 0; grp < NG; ++grp) o[f][grp] = otab[row0(f, grp)];
#pragma unroll
        for (int nf = 0; nf < FN; ++nf) {
            const int kl = kt * NT + (wn * FN + nf) * FR + lrow;
            if (kl >= a.Kg) continue;
            const int k = g * a.Kg + kl;
            const float sc = (a.scale != nullptr) ? a.scale[k] : 1.0f;
            const long long coff = k * OHW;
#pragma unroll
            for (int f = 0; f < FM; ++f)
#pragma unroll
                for (int grp = 0; grp < NG; ++grp) {
                    typename Mma<T>::acc_t quad;
#pragma unroll
                    for (int v = 0; v < 4; ++v) quad[v] = acc[f][nf][grp * 4 + v];
                    if (o[f][grp] >= 0) store_out4_epi<T, EPI>(y, o[f][grp] + coff, quad, sc, a.e, k);
                }
        }
        return;
    }
#pragma unroll
    for (int nf = 0; nf < FN; ++nf) {
        const int kl = kt * NT + (wn * FN + nf) * FR + lrow;
        if (kl >= a.Kg) continue;
        const int k = g * a.Kg + kl;
        const float sc = (a.scale != nullptr) ? a.scale[k] : 1.0f;
        const long long coff = (XB == 1) ? k * OHW : (k / XB) * OHW * XB + (k % XB);
#pragma unroll
        for (int f = 0; f < FM; ++f) {
#pragma unroll
            for (int grp = 0; grp < NG; ++grp) {
                const int p0 = row0(f, grp);
                typename Mma<T>::acc_t quad;
#pragma unroll
                for (int v = 0; v < 4; ++v) quad[v] = acc[f][nf][grp * 4 + v];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const long long ov = otab[p0 + v];
                    if (ov >= 0) store_out_epi<T, EPI>(y, ov + coff, quad, v, sc, a.e, k);
                }
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

// Weight preparation for 32x32 fragments: per tap of one output-channel tile,
// [NT/32][piece][32 rows][half][16 B], piece/half content = slot
// piece_slot(piece, half) of the row's 64-byte channel chunk, zero padded.
template <typename T, int NT>
__global__ __launch_bounds__(256) void igemm_prepare32_kernel(const T* __restrict__ w, T* __restrict__ wp, int G,
                                                              int Kg, int Cg, int RS, int ntk, int nchunks) {
    constexpr int E16 = 16 / static_cast<int>(sizeof(T));
    constexpr int CK = 4 * E16;
    using R = typename Raw<T>::type;
    const long long total = static_cast<long long>(G) * ntk * nchunks * RS * NT * CK;
    const R* wr = reinterpret_cast<const R*>(w);
    R* out = reinterpret_cast<R*>(wp);
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < total; i += static_cast<long long>(gridDim.x) * 256) {
        long long t = i;
        const int e = static_cast<int>(t % E16); t /= E16;
        const int half = static_cast<int>(t % 2); t /= 2;
        const int row = static_cast<int>(t % 32); t /= 32;
        const int piece = static_cast<int>(t % 2); t /= 2;
        const int nfr = static_cast<int>(t % (NT / 32)); t /= (NT / 32);
        const int rs = static_cast<int>(t % RS); t /= RS;
        const int chunk = static_cast<int>(t % nchunks); t /= nchunks;
        const int kt = static_cast<int>(t % ntk); t /= ntk;
        const int g = static_cast<int>(t);
        const int kl = kt * NT + nfr * 32 + row;
        const int cl = chunk * CK + piece_slot<T>(piece, half) * E16 + e;
        R v = 0;
        if (kl < Kg && cl < Cg) v = wr[(static_cast<long long>(g * Kg + kl) * Cg + cl) * RS + rs];
        out[i] = v;
    }
}

// ---------------------------------------------------------------- host side

struct Cfg {
    int wm, wn, fm, fn, fr;
    int threads() const { return wm * wn * 64; }
    int pixels() const { return wm * fm * fr; }
    int nt() const { return wn * fn * fr; }
};

// Tile configurations, in config-id order.
// fr = 16: 16x16 fragments, two or more waves per SIMD.
// fr = 32: 32x32 fragments, big per-wave register tiles, one wave per SIMD.
constexpr Cfg kCfgs[] = {
    {2, 2, 4, 4, 16},  // 0: 128 px x 128 ch
    {2, 2, 7, 4, 16},  // 1: 224 px x 128 ch
    {2, 2, 4, 2, 16},  // 2: 128 px x  64 ch
    {2, 2, 2, 2, 16},  // 3:  64 px x  64 ch
    {4, 1, 2, 4, 16},  // 4: 128 px x  64 ch
    {2, 2, 7, 2, 16},  // 5: 224 px x  64 ch
    {2, 2, 2, 4, 16},  // 6:  64 px x 128 ch
    {1, 4, 7, 2, 32},  // 7: 224 px x 256 ch
    {2, 2, 7, 2, 32},  // 8: 448 px x 128 ch
    {1, 4, 4, 2, 32},  // 9: 128 px x 256 ch
    {2, 2, 4, 2, 32},  // 10: 256 px x 128 ch
    {2, 2, 2, 2, 32},  // 11: 128 px x 128 ch
    {1, 4, 4, 1, 32},  // 12: 128 px x 128 ch
    {2, 2, 4, 1, 32},  // 13: 256 px x  64 ch
    // eight waves, two per SIMD: for layers whose tiles only just fill the
    // CUs (deep, small-image layers), where one wave per SIMD leaves the
    // operand latencies exposed
    {4, 2, 2, 2, 16},  // 14: 128 px x  64 ch
    {4, 2, 2, 4, 16},  // 15: 128 px x 128 ch
    {4, 2, 4, 2, 16},  // 16: 256 px x  64 ch
};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

constexpr size_t kLdsBytes = 160 * 1024;  // LDS of one CU (gfx950)

// Split reduction (int8 NCHW4, groups 1): the channel-chunk reduction of a
// base tile config is divided among `splits` workgroups per tile, which
// write int32 partial tiles; a second kernel sums them and requantises.  For
// deep layers with few output pixels (ResNet-18's 14x14 and 7x7 stages) the
// base tiles alone are too few to fill the 256 CUs, and each would walk the
// whole reduction (up to 8 chunks x 9 taps) by itself.
struct SplitCfg {
    int base, splits;
};
constexpr SplitCfg kSplitCfgs[] = {
    {10, 2}, {10, 4}, {10, 8},  // 256 px x 128 ch, 32x32 fragments
    {9, 2},  {9, 4},  {9, 8},   // 128 px x 256 ch, 32x32 fragments
    {11, 2}, {11, 4}, {11, 8},  // 128 px x 128 ch, 32x32 fragments
    {13, 2}, {13, 4}, {13, 8},  // 256 px x  64 ch, 32x32 fragments
    {2, 2},  {2, 4},  {2, 8},   // 128 px x  64 ch, 16x16 fragments
    {16, 2}, {16, 4}, {16, 8},  // 256 px x  64 ch, 16x16 fragments, eight waves
};
constexpr int kNumSplitCfgs = sizeof(kSplitCfgs) / sizeof(kSplitCfgs[0]);

struct Geo {
    int TN, TH, TW, PH, PW, npix, tiles_n, tiles_h, tiles_w, nchunks, ntk;
    int stg;  // 0: per-pixel gathers, 1: wide row-block loads
    size_t lds_bytes;
};

// Bytes per pixel sub-element of one 16-byte load along W (see Wide<>).
inline int wide_sz(const Prob& p) { return p.xb == 1 ? p.esize : p.xb * p.esize; }

// Geometry of tiles of TN images x TH x TW output pixels (the tile must
// fit: its input patch within the staging capacity of the config).
inline bool tile_geometry(const Prob& p, const Cfg& c, int TN, int TH, int TW, Geo* g, std::string* why) {
    const int CK = 64 / p.esize;
    const int maxpix = kMaxUnitsPerThread * c.threads() / 4;
    const int PH = (TH - 1) * p.sh + (p.r - 1) * p.dh + 1;
    const int PW = (TW - 1) * p.sw + (p.s - 1) * p.dw + 1;
    const long long npix = static_cast<long long>(TN) * PH * PW;
    if (npix > maxpix) {
        if (why) *why = "implicit GEMM: the input patch of one output row does not fit this tile config";
        return false;
    }
    g->TN = TN;
    g->TH = TH;
    g->TW = TW;
    g->PH = PH;
    g->PW = PW;
    g->npix = static_cast<int>(npix);
    g->tiles_n = (p.n + g->TN - 1) / g->TN;
    g->tiles_h = (p.oh + g->TH - 1) / g->TH;
    g->tiles_w = (p.ow + g->TW - 1) / g->TW;
    g->nchunks = (p.cg + CK - 1) / CK;
    g->ntk = (p.kg + c.nt() - 1) / c.nt();
    g->stg = 0;
    {
        const int sz = wide_sz(p);
        if (sz == 2 || sz == 4 || sz == 8) {
            const int pp = 16 / sz;
            const int maxu = std::max(1, 32 / (4 * pp));
            const long long ncb = (g->PW + pp - 1) / pp + 1;
            const long long units = 4LL * g->TN * g->PH * ncb;
            const bool chan_ok = (p.xb == 1) || (p.cg % p.xb == 0);
            if (p.w % pp == 0 && chan_ok && units <= static_cast<long long>(maxu) * c.threads()) g->stg = 1;
        }
    }
    // patch buffers (three on the nine-tap path of big per-wave tiles, see
    // launch_cfg and the kernel) and one
    // 16-byte dummy slot per thread; the epilogue reuses them for an 8-byte
    // offset per register-tile pixel row
    const size_t nbuf = (c.fr == 32 && g->stg == 1 && p.r * p.s == 9 && c.fm * c.fn >= 8) ? 3 : 2;
    // linear 80-byte pixel slots for 32x32 fragments and the nine-tap 16x16
    // path, swizzled 64-byte slots otherwise
    const size_t pstride = (c.fr == 32 || p.r * p.s == 9) ? 80 : 64;
    // (a problem of fewer chunks than buffers allocates only as many)
    const size_t nb = std::min(nbuf, static_cast<size_t>(g->nchunks));
    g->lds_bytes = std::max(nb * static_cast<size_t>(g->npix) * pstride + static_cast<size_t>(c.threads()) * 16,
                            static_cast<size_t>(c.pixels()) * 8);
    // 16-bit NCHW outputs of whole-row tiles leave through an LDS transpose:
    // [NT channels][tile pixels * 2 + 16 bytes]
    if (c.fr == 32 && p.esize == 2 && p.xb == 1)
        g->lds_bytes = std::max(g->lds_bytes, static_cast<size_t>(c.nt()) * (static_cast<size_t>(g->TN) * g->TH * g->TW * 2 + 16));
    // int8 NCHW4 outputs likewise: [NT / 4 channel blocks][tile pixels * 4 + 16 bytes]
    if (p.esize == 1 && p.xb == 4)
        g->lds_bytes = std::max(g->lds_bytes, static_cast<size_t>(c.nt() / 4) * (static_cast<size_t>(g->TN) * g->TH * g->TW * 4 + 16));
    if (g->lds_bytes > kLdsBytes) {
        if (why) *why = "implicit GEMM: the tile needs more LDS than a CU has";
        return false;
    }
    if (static_cast<long long>(g->tiles_n) * g->tiles_h * g->tiles_w * g->ntk * p.g > 0x7fffffffLL) {
        if (why) *why = "implicit GEMM: grid too large";
        return false;
    }
    return true;
}

inline bool geometry(const Prob& p, const Cfg& c, Geo* g, std::string* why) {
    const int P = c.pixels();
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
    // shrink the tile until its input patch fits: the staging units of the
    // workgroup, and the patch buffers (plus the per-thread dummy slots) in
    // the 160 KiB of LDS of a CU
    const size_t nbuf = (c.fr == 32 && p.r * p.s == 9 && c.fm * c.fn >= 8) ? 3 : 2;
    const size_t pstride = (c.fr == 32 || p.r * p.s == 9) ? 80 : 64;
    const int lds_pix = static_cast<int>((kLdsBytes - static_cast<size_t>(c.threads()) * 16) / (nbuf * pstride));
    const int maxpix = std::min(kMaxUnitsPerThread * c.threads() / 4, lds_pix);
    for (;;) {
        const int PH = (TH - 1) * p.sh + (p.r - 1) * p.dh + 1;
        const int PW = (TW - 1) * p.sw + (p.s - 1) * p.dw + 1;
        if (static_cast<long long>(TN) * PH * PW <= maxpix) break;
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
    return tile_geometry(p, c, TN, TH, TW, g, why);
}

// Geometry of split config `sc`: the base config's tiles, the chunks per
// split (*cps) and the LDS of the partial-tile epilogue.  Rejected when the
// splits would not all be non-empty or distinct from a smaller split count.
inline bool split_geometry(const Prob& p, int sc, Geo* g, int* cps, std::string* why) {
    if (sc < 0 || sc >= kNumSplitCfgs) {
        if (why) *why = "implicit GEMM: no such split config";
        return false;
    }
    const SplitCfg s = kSplitCfgs[sc];
    if (p.dtype != CFWD_I8 || p.layout != CFWD_LAYOUT_NCHWX || p.xb != 4 || p.g != 1) {
        if (why) *why = "implicit GEMM split reduction: int8 NCHW4 with groups 1 only";
        return false;
    }
    if (!geometry(p, kCfgs[s.base], g, why)) return false;
    const int c = (g->nchunks + s.splits - 1) / s.splits;
    if (g->nchunks < s.splits || (g->nchunks + c - 1) / c != s.splits) {
        if (why) *why = "implicit GEMM split reduction: the channel chunks do not divide into that many splits";
        return false;
    }
    *cps = c;
    const size_t tile_pix = static_cast<size_t>(g->TN) * g->TH * g->TW;
    g->lds_bytes = std::max(g->lds_bytes, static_cast<size_t>(kCfgs[s.base].nt() / 4) * (tile_pix * 16 + 64));
    if (g->lds_bytes > kLdsBytes) {
        if (why) *why = "implicit GEMM split reduction: the partial tile needs more LDS than a CU has";
        return false;
    }
    // the reduce kernel indexes pixel-channel-blocks of all images in 32 bits
    if (static_cast<long long>(p.n) * p.y_img / 4 >= (1LL << 31) ||
        static_cast<long long>(g->tiles_n) * g->tiles_h * g->tiles_w * g->ntk * s.splits > 0x7fffffffLL) {
        if (why) *why = "implicit GEMM split reduction: problem too large";
        return false;
    }
    return true;
}

// Partial tiles of every split: splits x N x y_img int32.
inline size_t split_scratch_bytes(const Prob& p, int sc) {
    return static_cast<size_t>(kSplitCfgs[sc].splits) * p.n * static_cast<size_t>(p.y_img) * 4;
}

// Resident-input configs (int8 NCHW4, 3x3 or 1x1): the base tile configs
// whose kernel holds the input rows of every channel chunk in LDS at once
// (RES in the kernel).  For layers with deep reductions and small images.
constexpr int kResCfgs[] = {2, 3, 6, 11, 12, 13, 14, 16};
constexpr int kNumResCfgs = sizeof(kResCfgs) / sizeof(kResCfgs[0]);

// Geometry of resident config `rc`: tiles of whole output rows as geometry()
// picks them, shrunk until the input rows of all channel chunks fit in LDS.
inline bool res_geometry(const Prob& p, int rc, Geo* g, std::string* why) {
    if (rc < 0 || rc >= kNumResCfgs) {
        if (why) *why = "implicit GEMM: no such resident-input config";
        return false;
    }
    const Cfg c = kCfgs[kResCfgs[rc]];
    if (p.dtype != CFWD_I8 || p.layout != CFWD_LAYOUT_NCHWX || p.xb != 4 || p.g != 1) {
        if (why) *why = "implicit GEMM resident input: int8 NCHW4 with groups 1 only";
        return false;
    }
    if (!((p.r == 3 && p.s == 3) || (p.r == 1 && p.s == 1))) {
        if (why) *why = "implicit GEMM resident input: 3x3 or 1x1 filters only";
        return false;
    }
    if (p.cg % 64 != 0) {
        if (why) *why = "implicit GEMM resident input: input channels must be a multiple of 64";
        return false;
    }
    if (static_cast<long long>(p.n) * p.x_img >= (1LL << 31)) {
        if (why) *why = "implicit GEMM resident input: input must be below 2 GiB";
        return false;
    }
    const int nch = p.cg / 64;
    const int P = c.pixels();
    // tiles of whole output rows (TN whole images, or TH rows of one)
    if (p.ow > P) {
        if (why) *why = "implicit GEMM resident input: an output row is wider than the tile";
        return false;
    }
    int TN, TH;
    const int TW = p.ow;
    if (p.oh * p.ow <= P) {
        TN = std::min(p.n, P / (p.oh * p.ow));
        TH = p.oh;
    } else {
        TN = 1;
        TH = std::min(p.oh, P / p.ow);
    }
    // LDS: per chunk, TN runs of the input rows the tile reads (at most
    // min(PH, H) rows of W pixels, rounded up to 4 pixels) and a zero slot,
    // 64 bytes each
    int PH = 0, PW = 0;
    long long slots = 0;
    for (;;) {
        PH = (TH - 1) * p.sh + (p.r - 1) * p.dh + 1;
        PW = (TW - 1) * p.sw + (p.s - 1) * p.dw + 1;
        slots = static_cast<long long>(TN) * ((static_cast<long long>(std::min(PH, p.h)) * p.w + 3) & ~3LL) + 1;
        if (nch * slots * 64 <= static_cast<long long>(kLdsBytes)) break;
        if (TN > 1)
            --TN;
        else if (TH > 1)
            --TH;
        else {
            if (why) *why = "implicit GEMM resident input: the rows of one output row do not fit in LDS";
            return false;
        }
    }
    g->TN = TN;
    g->TH = TH;
    g->TW = TW;
    g->PH = PH;
    g->PW = PW;
    g->npix = TN * PH * PW;
    g->tiles_n = (p.n + TN - 1) / TN;
    g->tiles_h = (p.oh + TH - 1) / TH;
    g->tiles_w = (p.ow + TW - 1) / TW;
    g->nchunks = nch;
    g->ntk = (p.kg + c.nt() - 1) / c.nt();
    g->stg = 0;
    const size_t tile_pix = static_cast<size_t>(TN) * TH * TW;
    g->lds_bytes = std::max({static_cast<size_t>(nch * slots * 64), static_cast<size_t>(c.pixels()) * 8,
                             static_cast<size_t>(c.nt() / 4) * (tile_pix * 4 + 16)});
    if (g->lds_bytes > kLdsBytes) {
        if (why) *why = "implicit GEMM resident input: the tile needs more LDS than a CU has";
        return false;
    }
    if (static_cast<long long>(g->tiles_n) * g->tiles_h * g->tiles_w * g->ntk > 0x7fffffffLL) {
        if (why) *why = "implicit GEMM: grid too large";
        return false;
    }
    return true;
}

inline size_t filter_bytes(const Prob& p, const Cfg& c, const Geo& g) {
    return static_cast<size_t>(p.g) * g.ntk * g.nchunks * p.r * p.s * c.nt() * 64;
}

inline Args make_args(const Prob& p, const Geo& g, const void* x, const void* wp, const float* scale, void* y) {
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
    a.tiles_w = g.tiles_w; a.tiles_h = g.tiles_h; a.tiles_n = g.tiles_n;
    a.nchunks = g.nchunks; a.ntk = g.ntk;
    a.cps = g.nchunks;
    a.part = nullptr;
    return a;
}

inline long long tile_count(const Prob& p, const Geo& g) {
    return static_cast<long long>(g.tiles_n) * g.tiles_h * g.tiles_w * g.ntk * p.g;
}

template <typename K> cfwd_status allow_big_lds(K kern, size_t lds_bytes, bool* done) {
    if (lds_bytes > 65536 && !*done) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return check_hip(e, "hipFuncSetAttribute(igemm)");
        *done = true;
    }
    return CFWD_OK;
}

// One launch of a tile config.  SPLIT: `nsplit` workgroups per tile, each
// summing `cps` channel chunks into its partial tile in `part`.
template <typename T, int XB, int WM, int WN, int FM, int FN, int STG, int FR, int RSV, bool SPLIT = false,
          bool EPI = false, bool RES = false>
cfwd_status launch_one(const Prob& p, const Geo& g, const void* x, const void* wp, const float* scale, void* y,
                       const Epi& e, hipStream_t st, int cps = 0, int nsplit = 1, int32_t* part = nullptr) {
    Args a = make_args(p, g, x, wp, scale, y);
    a.e = e;
    if constexpr (SPLIT) {
        a.cps = cps;
        a.part = part;
    }
    auto kern = igemm_kernel<T, XB, WM, WN, FM, FN, STG, FR, RSV, SPLIT, EPI, RES>;
    static bool attr_done = false;
    const cfwd_status s = allow_big_lds(kern, g.lds_bytes, &attr_done);
    if (s != CFWD_OK) return s;
    const dim3 grid(static_cast<unsigned>(tile_count(p, g) * (SPLIT ? nsplit : 1)));
    kern<<<grid, WM * WN * 64, g.lds_bytes, st>>>(a);
    return check_hip(hipGetLastError(), "igemm_kernel launch");
}

template <typename T, int XB, bool EPI>
cfwd_status launch_cfg(int cfg, const Prob& p, const Geo& g, const void* x, const void* wp, const float* scale,
                       void* y, const Epi& e, hipStream_t st) {
    switch (cfg) {
#define CFWD_IG_CFG(ID)                                                                                    \
    case ID: {                                                                                             \
        constexpr Cfg c = kCfgs[ID];                                                                       \
        if constexpr (Wide<T, XB>::ok) {                                                                   \
            if (g.stg == 1) {                                                                              \
                if (p.r * p.s == 9)                                                                        \
                    return launch_one<T, XB, c.wm, c.wn, c.fm, c.fn, 1, c.fr, 9, false, EPI>(p, g, x, wp, scale, y, e, st);   \
                return launch_one<T, XB, c.wm, c.wn, c.fm, c.fn, 1, c.fr, 0, false, EPI>(p, g, x, wp, scale, y, e, st);   \
            }                                                                                              \
        }                                                                                                  \
        if constexpr (c.fr == 16)                                                                          \
            if (p.r * p.s == 9)                                                                            \
                return launch_one<T, XB, c.wm, c.wn, c.fm, c.fn, 0, c.fr, 9, false, EPI>(p, g, x, wp, scale, y, e, st);   \
        return launch_one<T, XB, c.wm, c.wn, c.fm, c.fn, 0, c.fr, 0, false, EPI>(p, g, x, wp, scale, y, e, st);           \
    }
        CFWD_IG_CFG(0)
        CFWD_IG_CFG(1)
        CFWD_IG_CFG(2)
        CFWD_IG_CFG(3)
        CFWD_IG_CFG(4)
        CFWD_IG_CFG(5)
        CFWD_IG_CFG(6)
        CFWD_IG_CFG(7)
        CFWD_IG_CFG(8)
        CFWD_IG_CFG(9)
        CFWD_IG_CFG(10)
        CFWD_IG_CFG(11)
        CFWD_IG_CFG(12)
        CFWD_IG_CFG(13)
        CFWD_IG_CFG(14)
        CFWD_IG_CFG(15)
        CFWD_IG_CFG(16)
#undef CFWD_IG_CFG
        default:
            return set_error(CFWD_ERR_UNSUPPORTED, "implicit GEMM: no such config");
    }
}

template <typename T, bool EPI>
cfwd_status launch_dtype(int cfg, const Prob& p, const Geo& g, const void* x, const void* wp, const float* scale,
                         void* y, const Epi& e, hipStream_t st) {
    switch (p.xb) {
        case 1: return launch_cfg<T, 1, EPI>(cfg, p, g, x, wp, scale, y, e, st);
        case 4: return launch_cfg<T, 4, EPI>(cfg, p, g, x, wp, scale, y, e, st);
        case 8: return launch_cfg<T, 8, EPI>(cfg, p, g, x, wp, scale, y, e, st);
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
    const unsigned nb = static_cast<unsigned>(blocks);
    const T* wi = static_cast<const T*>(w);
    T* wo = static_cast<T*>(wp);
    const int rs = p.r * p.s;
    if (kCfgs[cfg].fr == 16) {
        if (nt == 128)
            igemm_prepare_kernel<T, 128><<<nb, 256, 0, st>>>(wi, wo, p.g, p.kg, p.cg, rs, g.ntk, g.nchunks);
        else if (nt == 64)
            igemm_prepare_kernel<T, 64><<<nb, 256, 0, st>>>(wi, wo, p.g, p.kg, p.cg, rs, g.ntk, g.nchunks);
        else
            return set_error(CFWD_ERR_UNSUPPORTED, "implicit GEMM: unexpected N tile");
    } else {
        if (nt == 256)
            igemm_prepare32_kernel<T, 256><<<nb, 256, 0, st>>>(wi, wo, p.g, p.kg, p.cg, rs, g.ntk, g.nchunks);
        else if (nt == 128)
            igemm_prepare32_kernel<T, 128><<<nb, 256, 0, st>>>(wi, wo, p.g, p.kg, p.cg, rs, g.ntk, g.nchunks);
        else if (nt == 64)
            igemm_prepare32_kernel<T, 64><<<nb, 256, 0, st>>>(wi, wo, p.g, p.kg, p.cg, rs, g.ntk, g.nchunks);
        else
            return set_error(CFWD_ERR_UNSUPPORTED, "implicit GEMM: unexpected N tile");
    }
    return check_hip(hipGetLastError(), "igemm_prepare launch");
}

}  // namespace ig

// Per-dtype entry points (defined in k_igemm_{f32,bf16,i8}.hip).
cfwd_status igemm_launch_f32(int cfg, const Prob& p, const ig::Geo& g, const void* x, const void* wp,
                             const float* scale, void* y, const Epi& e, hipStream_t st);
cfwd_status igemm_launch_bf16(int cfg, const Prob& p, const ig::Geo& g, const void* x, const void* wp,
                              const float* scale, void* y, const Epi& e, hipStream_t st);
cfwd_status igemm_launch_i8(int cfg, const Prob& p, const ig::Geo& g, const void* x, const void* wp,
                            const float* scale, void* y, const Epi& e, hipStream_t st);
cfwd_status igemm_prepare_f32(int cfg, const Prob& p, const ig::Geo& g, const void* w, void* wp, hipStream_t st);
cfwd_status igemm_prepare_bf16(int cfg, const Prob& p, const ig::Geo& g, const void* w, void* wp, hipStream_t st);
cfwd_status igemm_prepare_i8(int cfg, const Prob& p, const ig::Geo& g, const void* w, void* wp, hipStream_t st);
// The same with the fused epilogue compiled in (k_igemm_{f32,bf16,i8}_epi.hip).
cfwd_status igemm_launch_f32_epi(int cfg, const Prob& p, const ig::Geo& g, const void* x, const void* wp,
                                 const float* scale, void* y, const Epi& e, hipStream_t st);
cfwd_status igemm_launch_bf16_epi(int cfg, const Prob& p, const ig::Geo& g, const void* x, const void* wp,
                                  const float* scale, void* y, const Epi& e, hipStream_t st);
cfwd_status igemm_launch_i8_epi(int cfg, const Prob& p, const ig::Geo& g, const void* x, const void* wp,
                                const float* scale, void* y, const Epi& e, hipStream_t st);
// Persistent single-chunk int8 configs (k_igemm_i8_stream.hip): they read
// the prepared filter of tiled config stream_filter_config(sc).
int stream_num_configs();
bool stream_supported(const Prob& p, int sc, std::string* why);
int stream_filter_config(int sc);
cfwd_status stream_launch(const Prob& p, int sc, const void* x, const void* wp, const float* scale, void* y,
                          const Epi& e, hipStream_t st);
// Resident-input config rc (k_igemm_i8_res.hip).
cfwd_status igemm_launch_i8_res(int rc, const Prob& p, const ig::Geo& g, const void* x, const void* wp,
                                const float* scale, void* y, const Epi& e, hipStream_t st);
// Split config sc (k_igemm_i8_split.hip): the split kernel, then the reduce
// kernel that sums the partial tiles in `part` and requantises into y.
cfwd_status igemm_launch_i8_split(int sc, const Prob& p, const ig::Geo& g, int cps, const void* x, const void* wp,
                                  const float* scale, void* y, void* part, const Epi& e, hipStream_t st);

}  // namespace cfwd
