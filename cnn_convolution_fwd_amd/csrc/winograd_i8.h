// int8 Winograd F(2x2, 3x3) with a float intermediate (MegEngine Beta
// release article, section "业界领先的原生 ARM 推理性能": for devices without
// dot-product instructions, int8 Winograd that computes its transformed
// values in float, so the weights need no narrowing to 6 bits).  The three-launch form of k_winograd.hip with fp16 transformed
// operands: B^T d B (multiples of 1/4, magnitude <= 512) and G g G^T
// (integers, magnitude <= 1152) are exact in fp16, their products exact in
// fp32; the channel sums and the output transform are fp32 and stay exact
// while every partial sum is below 2^22 in magnitude.  The float result is
// rounded to the nearest integer and requantised like the integer paths, so
// an output differs from the exact one only where an fp32 rounding moved the
// accumulator across a requantisation boundary.
#pragma once

#include "internal.h"

namespace cfwd {

// y = requant(conv(x, w)) for an int8 3x3 / stride 1 / groups 1 problem in
// any int8 activation layout; wp from winograd_prepare(p, 2, 0, ...),
// scratch of winograd_scratch_bytes(p, 2, 0), scale = requant scales [K].
cfwd_status winograd_i8_launch(const Prob& p, const void* x, const void* wp, const float* scale, void* scratch,
                               void* y, const Epi& e, hipStream_t st);

}  // namespace cfwd
