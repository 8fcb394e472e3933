// kda_validate.h -- host-side checks of the KDA_VALIDATE=1 debug mode.
//
// Plain C++ on host arrays (copies of the device buffers), no HIP: the
// library calls them around a launch when KDA_VALIDATE=1, and a CPU test
// compiles this header alone to check them.  Each returns nullptr when the
// data passes, else a static description; *where receives the first bad
// index.
#pragma once

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstring>

namespace kda {
namespace validate {

// cu_seqlens [n + 1]: cu[0] = 0, non-decreasing, cu[n] = total.
inline const char* cu_seqlens(const int32_t* cu, int n, int64_t total, int64_t* where) {
  *where = 0;
  if (n < 0) return "negative document count";
  if (cu[0] != 0) return "cu_seqlens[0] is not 0";
  for (int i = 0; i < n; ++i) {
    if (cu[i + 1] < cu[i]) {
      *where = i + 1;
      return "cu_seqlens decreases";
    }
  }
  if (cu[n] != total) {
    *where = n;
    return "cu_seqlens[N] is not the token count";
  }
  return nullptr;
}

// log_g: every value <= 0 (-inf allowed), none NaN.
inline const char* log_gates(const float* g, size_t count, int64_t* where) {
  for (size_t i = 0; i < count; ++i) {
    if (!(g[i] <= 0.0f)) {  // NaN or positive
      *where = static_cast<int64_t>(i);
      return g[i] != g[i] ? "log_g is NaN" : "log_g is positive (not a decay)";
    }
  }
  *where = -1;
  return nullptr;
}

// Every fp32 value finite (an element left unwritten keeps the NaN fill).
inline const char* finite_f32(const float* x, size_t count, int64_t* where) {
  for (size_t i = 0; i < count; ++i) {
    if (!std::isfinite(x[i])) {
      *where = static_cast<int64_t>(i);
      return "not finite (unwritten, or an overflow)";
    }
  }
  *where = -1;
  return nullptr;
}

// Every bf16 value (raw bits) finite: exponent field not all ones.
inline const char* finite_bf16(const uint16_t* x, size_t count, int64_t* where) {
  for (size_t i = 0; i < count; ++i) {
    if ((x[i] & 0x7f80u) == 0x7f80u) {
      *where = static_cast<int64_t>(i);
      return "not finite (unwritten, or an overflow)";
    }
  }
  *where = -1;
  return nullptr;
}

}  // namespace validate
}  // namespace kda
