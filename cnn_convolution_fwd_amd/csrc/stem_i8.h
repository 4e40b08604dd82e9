// int8 NCHW4 image stems (k_stem_i8.hip): implicit GEMM with operands loaded
// straight from global memory; extra IMPLICIT_GEMM configs after the NHWC
// ones at the C ABI.
#pragma once

#include <string>

#include "internal.h"

namespace cfwd {

int stem_i8_num_configs();
bool stem_i8_supported(const Prob& p, int cfg, std::string* why);
size_t stem_i8_filter_bytes(const Prob& p, int cfg);
cfwd_status stem_i8_prepare(const Prob& p, int cfg, const void* w, void* wp, hipStream_t st);
cfwd_status stem_i8_launch(const Prob& p, int cfg, const void* x, const void* wp, const float* scale, void* y,
                           const Epi& e, hipStream_t st);

}  // namespace cfwd
