// Winograd F(m x m, 3 x 3) family (not built yet).
#include "internal.h"

namespace cfwd {

int winograd_num_configs(int) { return 0; }
bool winograd_supported(const Prob&, int, int, std::string* why) {
    if (why) *why = "winograd: not available in this build";
    return false;
}
size_t winograd_filter_bytes(const Prob&, int, int) { return 0; }
cfwd_status winograd_prepare(const Prob&, int, int, const void*, void*, hipStream_t) {
    return set_error(CFWD_ERR_UNSUPPORTED, "winograd: not available in this build");
}
cfwd_status winograd_launch(const Prob&, int, int, const void*, const void*, void*, hipStream_t) {
    return set_error(CFWD_ERR_UNSUPPORTED, "winograd: not available in this build");
}

}  // namespace cfwd
