// 4-bit weights (k_lowbit.hip): unpacking of packed signed 4-bit values to
// int8, behind cfwd_unpack_int4 of cfwd.h.
#pragma once

#include "internal.h"

namespace cfwd {

// out[i] = the signed 4-bit value i of `packed` (low nibble of byte i / 2 for
// even i, high nibble for odd i), i < count.  Arguments checked by the caller.
cfwd_status unpack_int4(const void* packed, void* out, long long count, hipStream_t st);

}  // namespace cfwd
