// Fused bottleneck block (k_bottleneck.hip): host-side entry points behind
// the cfwd_bottleneck_* calls of cfwd.h.
#pragma once

#include <string>

#include "internal.h"

namespace cfwd {

// CFWD_OK when the fused kernel runs this block; else the reason in *why.
cfwd_status bottleneck_check(const cfwd_bottleneck_desc* d, std::string* why);
// Bytes of the prepared 3x3 weights ([9 taps][64][64] bf16).
size_t bottleneck_filter_bytes();
cfwd_status bottleneck_prepare(const void* w2, void* w2p, hipStream_t st);
cfwd_status bottleneck_launch(const cfwd_bottleneck_desc* d, const void* x, const void* w1, const void* w2p,
                              const void* w3, const cfwd_bottleneck_epilogue* e, void* y, hipStream_t st);

}  // namespace cfwd
