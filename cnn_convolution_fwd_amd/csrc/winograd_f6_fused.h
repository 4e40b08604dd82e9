// Fused Winograd F(6x6,3x3) for bf16 or fp32 NCHW (config 1 of F(6x6),
// k_winograd_f6_fused.hip): the transformed input stays on chip; scratch only
// for bf16's input maximum.
#pragma once

#include "internal.h"

namespace cfwd {

bool winograd_f6_fused_supported(const Prob& p, std::string* why);
size_t winograd_f6_fused_filter_bytes(const Prob& p);
size_t winograd_f6_fused_scratch_bytes(const Prob& p);
cfwd_status winograd_f6_fused_prepare(const Prob& p, const void* w, void* wp, hipStream_t st);
cfwd_status winograd_f6_fused_launch(const Prob& p, const void* x, const void* wp, void* scratch, void* y,
                                     const Epi& e, hipStream_t st);

}  // namespace cfwd
