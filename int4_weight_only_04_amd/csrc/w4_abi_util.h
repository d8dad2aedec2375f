// Error reporting and argument checks shared by the extern "C" entry points
// (host code only; not part of the public ABI).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "w4.h"
#include "w4_internal.h"

namespace w4i {

// Record a formatted message for w4_last_error() (thread-local) and return code.
w4_status fail(w4_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// W4_EHIP with the HIP error string.
w4_status hip_fail(hipError_t err, const char* what);
const char* last_error();
// Shape, pointer and alignment checks of one GEMV launch (W4_OK or a failure).
w4_status check_gemv(const GemvCall& c, const char* who);
// Shape rules shared by the paged attention and the KV append.
w4_status check_kv_shape(int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t page_size, int32_t max_ctx,
                         int32_t num_pages, const char* who);

inline bool aligned16(const void* p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

inline bool aligned_to(const void* p, uintptr_t bytes)
{
    return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0;
}

}  // namespace w4i
