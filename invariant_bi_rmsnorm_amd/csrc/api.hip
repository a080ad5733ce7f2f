// Status strings, error messages and host helpers of the C ABI.
#include <cstdarg>
#include <cstdio>
#include <string>

#include "api.h"

namespace bi {

static thread_local std::string g_last_error;

bi_status fail(bi_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

void clear_error() { g_last_error.clear(); }

bi_status launched(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BI_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return BI_OK;
}

}  // namespace bi

extern "C" {

int bi_abi_version(void) { return 3; }

const char* bi_status_string(bi_status s) {
  switch (s) {
    case BI_OK: return "ok";
    case BI_ERR_INVALID: return "invalid argument";
    case BI_ERR_UNSUPPORTED: return "unsupported configuration";
    case BI_ERR_WORKSPACE: return "workspace too small";
    case BI_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* bi_last_error(void) { return bi::g_last_error.c_str(); }

int bi_chunk_offsets(const int32_t* kv_len_host, int B, int kv_chunk, int32_t* chunk_off_host) {
  if (!chunk_off_host || B < 0 || kv_chunk <= 0 || (B > 0 && !kv_len_host)) return -1;
  long total = 0;
  chunk_off_host[0] = 0;
  for (int r = 0; r < B; ++r) {
    const int s = kv_len_host[r];
    total += s > 0 ? (s + kv_chunk - 1) / kv_chunk : 0;
    if (total > 0x7fffffffL) return -1;
    chunk_off_host[r + 1] = (int32_t)total;
  }
  return (int)total;
}

size_t bi_attn_partials_bytes(int total_chunks, int h, int d_h) {
  if (total_chunks < 0 || h <= 0 || d_h <= 0) return 0;
  return (size_t)total_chunks * h * ((size_t)d_h + 2) * sizeof(float);
}

}  // extern "C"
