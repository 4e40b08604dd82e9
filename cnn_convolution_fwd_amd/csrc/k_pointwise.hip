// Pointwise (1x1) family.  No dedicated kernel yet: 1x1 layers run on the
// implicit-GEMM family, whose patch for a 1x1 kernel is the tile itself.
#include "internal.h"

namespace cfwd {

int pointwise_num_configs() { return 0; }
bool pointwise_supported(const Prob&, int, std::string* why) {
    if (why) *why = "pointwise: no dedicated kernel in this build";
    return false;
}
size_t pointwise_filter_bytes(const Prob&, int) { return 0; }
cfwd_status pointwise_prepare(const Prob&, int, const void*, void*, hipStream_t) {
    return set_error(CFWD_ERR_UNSUPPORTED, "pointwise: no dedicated kernel in this build");
}
cfwd_status pointwise_launch(const Prob&, int, const void*, const void*, const float*, void*, hipStream_t) {
    return set_error(CFWD_ERR_UNSUPPORTED, "pointwise: no dedicated kernel in this build");
}

}  // namespace cfwd
