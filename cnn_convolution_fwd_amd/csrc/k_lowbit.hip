// 4-bit weights (gfx950).
//
// MegEngine CPU-inference article, section "结论": lower-precision
// quantisation (4-bit, 1-bit) is named as a next step after int8.  gfx950's
// matrix cores take int8 but no int4 operands, so a 4-bit weight tensor is
// kept at half the bytes at rest and widened once, when the network's
// weights are loaded, to the int8 the implicit GEMM and direct kernels read;
// the convolution is then the int8 one, bit for bit.
//
// Packing: value i sits in byte i / 2, low nibble for even i, high nibble
// for odd i, two's complement (-8 .. 7).
#include "lowbit.h"

namespace cfwd {
namespace lb {

// sign-extend the nibble at bit offset `shift` of w
__device__ __forceinline__ uint32_t nib(uint32_t w, int shift) {
    return static_cast<uint32_t>(static_cast<int32_t>(w << (28 - shift)) >> 28) & 0xffu;
}

// bytes 4 .. 7 of the output from a 16-bit half of a packed word: four int8
__device__ __forceinline__ uint32_t widen4(uint32_t h) {
    return nib(h, 0) | (nib(h, 4) << 8) | (nib(h, 8) << 16) | (nib(h, 12) << 24);
}

// 16 packed bytes -> 32 int8 per thread; the tail (count not a multiple of
// 32) byte by byte
__global__ __launch_bounds__(256) void unpack_int4_kernel(const uint8_t* __restrict__ in, int8_t* __restrict__ out,
                                                          long long count) {
    const long long n32 = count / 32;
    const long long stride = static_cast<long long>(gridDim.x) * 256;
    for (long long t = blockIdx.x * 256LL + threadIdx.x; t < n32; t += stride) {
        const uint4 v = *reinterpret_cast<const uint4*>(in + t * 16);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            o[2 * q] = widen4(w[q] & 0xffffu);
            o[2 * q + 1] = widen4(w[q] >> 16);
        }
        uint4* dst = reinterpret_cast<uint4*>(out + t * 32);
        dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
        dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
    for (long long i = n32 * 32 + blockIdx.x * 256LL + threadIdx.x; i < count; i += stride) {
        const uint32_t b = in[i >> 1];
        out[i] = static_cast<int8_t>(nib(b, (i & 1) ? 4 : 0));
    }
}

}  // namespace lb

cfwd_status unpack_int4(const void* packed, void* out, long long count, hipStream_t st) {
    const long long work = std::max(count / 32, 1LL);
    const unsigned blocks = static_cast<unsigned>(std::min<long long>((work + 255) / 256, 4096));
    lb::unpack_int4_kernel<<<blocks, 256, 0, st>>>(static_cast<const uint8_t*>(packed), static_cast<int8_t*>(out), count);
    return check_hip(hipGetLastError(), "int4 unpack launch");
}

}  // namespace cfwd
