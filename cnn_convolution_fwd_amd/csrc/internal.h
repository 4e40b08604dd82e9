// Internal declarations of the cfwd GPU library (gfx950).  Not installed and
// not part of the C ABI: the public surface is include/cfwd.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "cfwd.h"

namespace cfwd {

// ------------------------------------------------------------------ problem

// A validated problem, with derived sizes.  Activation element (n, c, h, w) is
// at  n*x_img + c*H*W + h*W + w                      (NCHW, xb == 1)
//     n*x_img + (c/xb)*H*W*xb + (h*W + w)*xb + c%xb  (NCHWX)
struct Prob {
    int n, c, h, w, k, r, s;
    int sh, sw, ph, pw, dh, dw, g;
    int oh, ow, cg, kg;
    int layout;  // cfwd_layout
    int xb;      // channel block: 1 for NCHW, 4 or 8 for NCHWX
    int dtype;   // cfwd_dtype
    int esize;   // bytes per element
    long long x_img, y_img;  // elements per image of x and y (incl. channel padding)
    bool depthwise() const { return g == c && g == k && cg == 1; }
    bool pointwise() const { return r == 1 && s == 1 && ph == 0 && pw == 0; }
};

// Fused epilogue of one call (cfwd_epilogue): a per-output-channel bias
// (fp32 for fp32 / bf16 outputs, int32 added to the accumulator for int8), a
// residual in y's layout and dtype, and ReLU -- applied to each output before
// it is converted and stored.  All null / 0: a plain convolution.
struct Epi {
    const void* bias = nullptr;
    const void* res = nullptr;
    int relu = 0;
};

// Fills *p from a descriptor; returns CFWD_OK or INVALID_ARG/UNSUPPORTED and a
// reason in *why.
cfwd_status make_prob(const cfwd_conv_desc* d, Prob* p, std::string* why);

// ------------------------------------------------------------ error plumbing

cfwd_status set_error(cfwd_status st, const std::string& msg);
cfwd_status check_hip(hipError_t e, const char* what);

// ------------------------------------------------------------ kernel families
// Each family answers: can it run (problem, config)?  How many bytes of
// prepared filter / workspace?  And launches on a stream.  Launchers assume the
// problem is valid and the pointers checked; they return CFWD_ERR_HIP if a
// launch fails.

// Direct summation (generic fallback; depthwise specialisation inside).
int direct_num_configs();
int direct_default_config(const Prob& p);  // fastest expected supported config
bool direct_supported(const Prob& p, int cfg, std::string* why);
cfwd_status direct_launch(const Prob& p, int cfg, const void* x, const void* w,
                          const float* scale, void* y, const Epi& e, hipStream_t st);

// Implicit GEMM on the matrix cores.
int igemm_num_configs();
bool igemm_supported(const Prob& p, int cfg, std::string* why);
size_t igemm_filter_bytes(const Prob& p, int cfg);
cfwd_status igemm_prepare(const Prob& p, int cfg, const void* w, void* wp, hipStream_t st);
size_t igemm_scratch_bytes(const Prob& p, int cfg);  // partial tiles of split configs
cfwd_status igemm_launch(const Prob& p, int cfg, const void* x, const void* wp,
                         const float* scale, void* y, void* scratch, const Epi& e, hipStream_t st);
int igemm_default_config(const Prob& p);
// gather form of implicit GEMM for few input channels (implicit-GEMM configs
// after the tiled ones)
int lowc_num_configs();
bool lowc_supported(const Prob& p, int cfg, std::string* why);
size_t lowc_filter_bytes(const Prob& p, int cfg);
cfwd_status lowc_prepare(const Prob& p, int cfg, const void* w, void* wp, hipStream_t st);
cfwd_status lowc_launch(const Prob& p, int cfg, const void* x, const void* wp, const float* scale, void* y,
                        const Epi& e, hipStream_t st);

// Pointwise (1x1) path.
int pointwise_num_configs();
bool pointwise_supported(const Prob& p, int cfg, std::string* why);
size_t pointwise_filter_bytes(const Prob& p, int cfg);
cfwd_status pointwise_prepare(const Prob& p, int cfg, const void* w, void* wp, hipStream_t st);
cfwd_status pointwise_launch(const Prob& p, int cfg, const void* x, const void* wp,
                             const float* scale, void* y, const Epi& e, hipStream_t st);

// Winograd F(m x m, 3 x 3), m = 2 or 6.
int winograd_num_configs(int m);
bool winograd_supported(const Prob& p, int m, int cfg, std::string* why);
size_t winograd_filter_bytes(const Prob& p, int m, int cfg);
size_t winograd_scratch_bytes(const Prob& p, int m, int cfg);  // transformed input U
cfwd_status winograd_prepare(const Prob& p, int m, int cfg, const void* w, void* wp, hipStream_t st);
cfwd_status winograd_launch(const Prob& p, int m, int cfg, const void* x, const void* wp, void* scratch,
                            void* y, const Epi& e, hipStream_t st);

// Fused Winograd F(2x2,3x3) for bf16 NCHW (configs 1 and 2 of F(2x2)): the
// transformed input stays on chip, no scratch.
bool winograd_fused_supported(const Prob& p, int cfg, std::string* why);
size_t winograd_fused_filter_bytes(const Prob& p, int cfg);
cfwd_status winograd_fused_prepare(const Prob& p, int cfg, const void* w, void* wp, hipStream_t st);
cfwd_status winograd_fused_launch(const Prob& p, int cfg, const void* x, const void* wp, void* scratch, void* y,
                                  const Epi& e, hipStream_t st);

// bf16 Winograd keeps its transformed operands in fp16, whose range is far
// narrower than bf16's.  Input and filter are therefore scaled by powers of
// two that bring their largest magnitude into [2^7, 2^8) -- then every
// transformed operand stays below 65504 (F(6x6) grows an input by at most
// 156.25, a filter by 49) and magnitudes down to 2^-22 of the largest stay
// normal -- and the output is scaled back.  Powers of two are exact.
// bf16_absmax: *out = the largest |x| of n bf16 values, as a bit pattern
// (sign cleared); out points to an 8 KiB area whose words 64.. hold the
// per-workgroup partial maxima.
cfwd_status bf16_absmax(const void* x, long long n, unsigned* out, hipStream_t st);

// Writes 0 to the NCHWX output channels past K (no-op unless K % xb != 0).
cfwd_status zero_output_channel_padding(const Prob& p, void* y, hipStream_t st);

// Overwrites `bytes` of buf (16-byte aligned) with plain stores, so that the
// caches no longer hold what earlier launches touched (k_util.hip).
cfwd_status evict_caches(void* buf, size_t bytes, unsigned salt, hipStream_t st);

// Fast-Run accuracy gate helpers (k_util.hip).
cfwd_status abs_copy(const Prob& p, const void* src, void* dst, long long count, hipStream_t st);
// stats[0] = bit pattern of max |cand - ref| / den (float dtypes), stats[1] =
// count of outputs that fail outright (int8: any difference; float: NaN, or
// den == 0 with cand != 0).
cfwd_status gate_compare(const Prob& p, const void* cand, const void* ref, const void* den, unsigned* stats,
                         hipStream_t st);

// ------------------------------------------------------------ device helpers

#if defined(__HIPCC__)
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// bf16 storage type: raw 16-bit pattern.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_float(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi);

// XCD-aware work order: workgroups are dispatched round-robin over the 8
// XCDs (each with its own L2), so give each XCD a contiguous range of the
// logical work order; logically adjacent work items (which share input rows
// or weights) then run at about the same time on the same L2.
__device__ __forceinline__ int xcd_linear(int bid, int total) {
    const int xcd = bid & 7, local = bid >> 3;
    const int per = total >> 3, rem = total & 7;
    return (xcd < rem) ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.  gfx950's
// packed convert does exactly this (checked against the bit-level rule on all
// 2^32 inputs), so both helpers use it.
__device__ __forceinline__ uint16_t float_to_bf16(float f) {
    return static_cast<uint16_t>(pack_bf16x2(f, 0.0f) & 0xffffu);
}

// Two fp32 values -> one 32-bit word of two bf16 (lo in bits 0-15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// int32 accumulator -> int8: clamp(rne(fp32(acc) * scale), -127, 127).
// One IEEE multiply (nothing follows it that could be contracted with it);
// rintf rounds to nearest even.
__device__ __forceinline__ int8_t requant_i8(int acc, float scale) {
    float q = rintf(__fmul_rn(static_cast<float>(acc), scale));
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    return static_cast<int8_t>(static_cast<int>(q));
}

// The same value as requant_i8, in the low byte of the result (the other
// bytes are not defined), in four branch-free instructions: the clamp comes
// before the rounding, which gives the same result because both bounds are
// integers; adding 1.5 * 2^23 then rounds to the nearest integer (ties to
// even, the default rounding) and leaves it, in two's complement, in the low
// mantissa bits.
__device__ __forceinline__ uint32_t requant_i8_bits(int acc, float scale) {
    const float q = __builtin_amdgcn_fmed3f(__fmul_rn(static_cast<float>(acc), scale), -127.0f, 127.0f);
    return __float_as_uint(__fadd_rn(q, 12582912.0f));
}

// 4 x 4 byte transpose within each quad of lanes (lanes 4m .. 4m + 3): lane
// j of a quad holds bytes b0..b3 and afterwards holds byte j of each of the
// four lanes, lane i's in byte i.  Two cross-lane moves (DPP quad
// permutations: lane ^ 1, then lane ^ 2), each followed by a byte / half-word
// merge.  Every lane of a quad must execute it.
__device__ __forceinline__ uint32_t quad_transpose_bytes(uint32_t d, int lane) {
    const uint32_t t1 = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(d), 0xB1, 0xF, 0xF, false));
    const uint32_t e = (lane & 1) ? (((t1 >> 8) & 0x00FF00FFu) | (d & 0xFF00FF00u))
                                  : ((d & 0x00FF00FFu) | ((t1 & 0x00FF00FFu) << 8));
    const uint32_t t2 = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(e), 0x4E, 0xF, 0xF, false));
    return (lane & 2) ? ((t2 >> 16) | (e & 0xFFFF0000u)) : ((e & 0x0000FFFFu) | (t2 << 16));
}

// Low bytes of four words -> one word, b0 in the lowest byte.
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
    const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// ---- fused epilogue, one output value (see Epi)

// fp32 / bf16 outputs: act(v + bias[k] + residual[off]) in fp32, before the
// single conversion to the output type.  k must be a real channel (< K).
template <typename T>
__device__ __forceinline__ float epi_float(float v, const Epi& e, int k, long long off);

// int8 outputs: clamp(rne(fp32(acc + bias[k]) * scale + fp32(residual[off])),
// lo, 127), lo = 0 under ReLU, else -127; the value in the low byte, as in
// requant_i8_bits (which this equals with no bias, residual or ReLU).  k
// must be a real channel (< K) when there is a bias.
// The same with its operands already loaded: bias (0 when absent), residual
// (0.0 when absent: adding +0 only turns a -0 into +0, which rounds to the
// same byte) and the lower clamp lo (0 under ReLU, else -127).
// The multiply and the add are two roundings by definition: contraction into
// one FMA is switched off here (the __f*_rn helpers are plain operators).
__device__ __forceinline__ uint32_t requant_i8_fused(int acc, int bias, float scale, float res, float lo) {
#pragma clang fp contract(off)
    const float q = static_cast<float>(acc + bias) * scale + res;
    return __float_as_uint(__builtin_amdgcn_fmed3f(q, lo, 127.0f) + 12582912.0f);
}

__device__ __forceinline__ uint32_t requant_i8_epi_bits(int acc, float scale, const Epi& e, int k, long long off) {
    const int b = e.bias ? static_cast<const int32_t*>(e.bias)[k] : 0;
    const float r = e.res ? static_cast<float>(static_cast<const int8_t*>(e.res)[off]) : 0.0f;
    return requant_i8_fused(acc, b, scale, r, e.relu ? 0.0f : -127.0f);
}

// Exponent of the largest magnitude whose bf16 bit pattern is `bits`
// (floored, so an all-zero tensor gives finite factors).
__device__ __forceinline__ int wg_exp(unsigned bits) { return max(static_cast<int>(bits >> 7) - 127, -100); }
// Factor that brings that magnitude into [2^7, 2^8) (1 when no maximum is given).
__device__ __forceinline__ float wg_norm(const unsigned* maxbits) {
    return maxbits ? __builtin_amdgcn_ldexpf(1.0f, 7 - wg_exp(*maxbits)) : 1.0f;
}
// Exponent shift that undoes one operand's factor (0 when none is given);
// read once per workgroup, applied per output with wg_denorm.
__device__ __forceinline__ int wg_shift(const unsigned* maxbits) { return maxbits ? wg_exp(*maxbits) - 7 : 0; }
// Undoes the input's and the filter's factors on an output (two steps, so
// a large and a small shift do not overflow in between).
__device__ __forceinline__ float wg_denorm(float v, int shift_x, int shift_w) {
    return __builtin_amdgcn_ldexpf(__builtin_amdgcn_ldexpf(v, shift_x), shift_w);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float to_f(float v) { return v; }
};
template <> struct Elem<bf16_t> {
    static __device__ __forceinline__ float to_f(bf16_t v) { return bf16_to_float(v.bits); }
};
template <> struct Elem<int8_t> {
    static __device__ __forceinline__ int to_f(int8_t v) { return v; }
};

template <typename T>
__device__ __forceinline__ float epi_float(float v, const Epi& e, int k, long long off) {
    if (e.bias) v += static_cast<const float*>(e.bias)[k];
    if (e.res) v += static_cast<float>(Elem<T>::to_f(static_cast<const T*>(e.res)[off]));
    if (e.relu) v = fmaxf(v, 0.0f);
    return v;
}

// Offset of activation element (c, h, w) inside one image.
template <int XB>
__device__ __forceinline__ long long act_off(int c, int h, int w, int H, int W) {
    if (XB == 1)
        return (static_cast<long long>(c) * H + h) * W + w;
    return ((static_cast<long long>(c / XB) * H + h) * W + w) * XB + (c % XB);
}
#endif

}  // namespace cfwd
