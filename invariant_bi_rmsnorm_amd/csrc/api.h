// Host-side helpers shared by the entry points of libbi.so.
#pragma once

#include <hip/hip_runtime.h>
#include "bi.h"

namespace bi {

// Record a failure message for bi_last_error() and return `s`.
bi_status fail(bi_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the calling thread's message.
void clear_error();
// After a launch: BI_OK, or BI_ERR_HIP with the runtime's message.
bi_status launched(const char* what);

inline hipStream_t as_stream(bi_stream s) { return reinterpret_cast<hipStream_t>(s); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace bi

#define BI_REQUIRE(cond, code, ...)                 \
  do {                                              \
    if (!(cond)) return ::bi::fail(code, __VA_ARGS__); \
  } while (0)
