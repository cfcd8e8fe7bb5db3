// kvq_host.hpp -- host-side helpers shared by the C ABI's source files: the thread-local error
// text behind kv_last_error().
#pragma once

#include "kv_quant.h"

namespace kvq {

// records a printf-style detail for kv_last_error() and returns st
kv_status fail(kv_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// clears the detail and returns KV_OK
kv_status ok();
const char* last_error();
// a width the block allocator has pools for
bool alloc_accepts_bits(int bits);

}  // namespace kvq
