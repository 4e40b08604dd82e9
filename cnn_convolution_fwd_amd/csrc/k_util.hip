// Small device helpers used by the Fast-Run accuracy gate.
//
// The gate checks each candidate against the generic direct kernel's output
// on the caller's own data, with the error metric of the parity tests:
// |candidate - reference| / den per output, den = sum |x|*|w| (computed by
// running the reference kernel on |x| and |w|); int8 outputs must match
// exactly.  The MegEngine inference article's Fast-Run assumes every
// implementation is exact; this gate is what makes that assumption safe for
// the inexact (Winograd, bf16) ones.
#include "internal.h"

namespace cfwd {

namespace {

template <typename T> __device__ __forceinline__ T abs_of(T v);
template <> __device__ __forceinline__ float abs_of<float>(float v) { return fabsf(v); }
template <> __device__ __forceinline__ bf16_t abs_of<bf16_t>(bf16_t v) { return bf16_t{static_cast<uint16_t>(v.bits & 0x7fffu)}; }

template <typename T>
__global__ __launch_bounds__(256) void abs_kernel(const T* __restrict__ src, T* __restrict__ dst, long long n) {
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += static_cast<long long>(gridDim.x) * 256)
        dst[i] = abs_of<T>(src[i]);
}

__global__ void zero_stats(unsigned* stats) {
    if (threadIdx.x < 4) stats[threadIdx.x] = 0;
}

template <typename T>
__global__ __launch_bounds__(256) void gate_float(const T* __restrict__ cand, const T* __restrict__ ref,
                                                  const T* __restrict__ den, long long n, unsigned* stats) {
    unsigned worst = 0, bad = 0;
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += static_cast<long long>(gridDim.x) * 256) {
        const float c = Elem<T>::to_f(cand[i]);
        const float r = Elem<T>::to_f(ref[i]);
        const float d = Elem<T>::to_f(den[i]);
        if (!(fabsf(c) <= 3.402823466e38f)) {
            ++bad;  // NaN or infinity
        } else if (!(d > 0.0f)) {
            // den is a sum of absolute values: 0 means every term is zero, so
            // the output must be exactly 0.  Anything else (negative, NaN) is
            // not a valid normaliser and fails rather than passing silently.
            if (c != 0.0f || d != 0.0f) ++bad;
        } else {
            const float e = fabsf(c - r) / d;
            if (!(e <= 3.402823466e38f))
                ++bad;
            else
                worst = max(worst, __float_as_uint(e));  // non-negative floats order as unsigned ints
        }
    }
    for (int off = 32; off > 0; off >>= 1) {
        worst = max(worst, static_cast<unsigned>(__shfl_down(static_cast<int>(worst), off)));
        bad += static_cast<unsigned>(__shfl_down(static_cast<int>(bad), off));
    }
    if ((threadIdx.x & 63) == 0) {
        atomicMax(stats, worst);
        atomicAdd(stats + 1, bad);
    }
}

// stats[0]: largest |cand - ref|; stats[1]: outputs that differ
__global__ __launch_bounds__(256) void gate_i8(const int8_t* __restrict__ cand, const int8_t* __restrict__ ref,
                                               long long n, unsigned* stats) {
    unsigned worst = 0, bad = 0;
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += static_cast<long long>(gridDim.x) * 256) {
        const int d = static_cast<int>(cand[i]) - static_cast<int>(ref[i]);
        bad += (d != 0) ? 1u : 0u;
        worst = max(worst, static_cast<unsigned>(d < 0 ? -d : d));
    }
    for (int off = 32; off > 0; off >>= 1) {
        worst = max(worst, static_cast<unsigned>(__shfl_down(static_cast<int>(worst), off)));
        bad += static_cast<unsigned>(__shfl_down(static_cast<int>(bad), off));
    }
    if ((threadIdx.x & 63) == 0) {
        atomicMax(stats, worst);
        atomicAdd(stats + 1, bad);
    }
}

// Plain (cache-allocating) 16-byte stores over the whole buffer: afterwards
// the Infinity Cache and every L2 hold this buffer's lines, not the ones a
// previous run left behind.
__global__ __launch_bounds__(256) void evict_kernel(uint4* __restrict__ buf, long long n16, unsigned salt) {
    const uint4 v = make_uint4(salt, salt, salt, salt);
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n16; i += static_cast<long long>(gridDim.x) * 256)
        buf[i] = v;
}

unsigned blocks_for(long long n) {
    long long b = (n + 255) / 256;
    return static_cast<unsigned>(b > 8192 ? 8192 : (b < 1 ? 1 : b));
}

}  // namespace

cfwd_status abs_copy(const Prob& p, const void* src, void* dst, long long count, hipStream_t st) {
    if (p.dtype == CFWD_F32)
        abs_kernel<float><<<blocks_for(count), 256, 0, st>>>(static_cast<const float*>(src), static_cast<float*>(dst),
                                                            count);
    else if (p.dtype == CFWD_BF16)
        abs_kernel<bf16_t><<<blocks_for(count), 256, 0, st>>>(static_cast<const bf16_t*>(src),
                                                             static_cast<bf16_t*>(dst), count);
    else
        return set_error(CFWD_ERR_UNSUPPORTED, "abs_copy: float dtypes only");
    return check_hip(hipGetLastError(), "abs_kernel launch");
}

cfwd_status evict_caches(void* buf, size_t bytes, unsigned salt, hipStream_t st) {
    const long long n16 = static_cast<long long>(bytes / 16);
    if (n16 == 0) return CFWD_OK;
    evict_kernel<<<4096, 256, 0, st>>>(static_cast<uint4*>(buf), n16, salt);
    return check_hip(hipGetLastError(), "evict_kernel launch");
}

cfwd_status gate_compare(const Prob& p, const void* cand, const void* ref, const void* den, unsigned* stats,
                         hipStream_t st) {
    zero_stats<<<1, 64, 0, st>>>(stats);
    cfwd_status s = check_hip(hipGetLastError(), "zero_stats launch");
    if (s != CFWD_OK) return s;
    const long long n = p.y_img * p.n;
    if (p.dtype == CFWD_F32)
        gate_float<float><<<blocks_for(n), 256, 0, st>>>(static_cast<const float*>(cand),
                                                         static_cast<const float*>(ref),
                                                         static_cast<const float*>(den), n, stats);
    else if (p.dtype == CFWD_BF16)
        gate_float<bf16_t><<<blocks_for(n), 256, 0, st>>>(static_cast<const bf16_t*>(cand),
                                                          static_cast<const bf16_t*>(ref),
                                                          static_cast<const bf16_t*>(den), n, stats);
    else
        gate_i8<<<blocks_for(n), 256, 0, st>>>(static_cast<const int8_t*>(cand), static_cast<const int8_t*>(ref), n,
                                               stats);
    return check_hip(hipGetLastError(), "gate kernel launch");
}

}  // namespace cfwd
