// NHWC activations (k_nhwc.hip): the channel-contiguous implicit GEMM (extra
// IMPLICIT_GEMM configs after the NCHW / NCHWX ones) and the layout
// conversion behind cfwd_convert_layout.
#pragma once

#include <string>

#include "internal.h"

namespace cfwd {

int nhwc_num_configs();
bool nhwc_supported(const Prob& p, int cfg, std::string* why);
size_t nhwc_filter_bytes(const Prob& p, int cfg);
cfwd_status nhwc_prepare(const Prob& p, int cfg, const void* w, void* wp, hipStream_t st);
cfwd_status nhwc_launch(const Prob& p, int cfg, const void* x, const void* wp, void* y, const Epi& e, hipStream_t st);

// Copy an n x c x h x w tensor of esize-byte elements from layout sl (block
// sx for NCHWX) to layout dl (block dx); NCHWX destinations get their
// padding channels written as 0.  Arguments checked by the caller.
cfwd_status layout_convert(int n, int c, int h, int w, int esize, int sl, int sx, const void* src, int dl, int dx,
                           void* dst, hipStream_t st);

}  // namespace cfwd
