// Host-side error reporting shared by the C ABI's translation units: the thread-local message
// behind pkv_last_error_message and the hipError_t behind pkv_last_hip_error.
#pragma once

#include <hip/hip_runtime.h>
#include <string.h>

#include "pagedkv.h"

namespace pkv {

// Records a printf-style message and returns s.
pkv_status fail(pkv_status s, const char* fmt, ...);
// Records a HIP runtime failure of `what` and returns PKV_ERR_HIP.
pkv_status hip_failure(hipError_t e, const char* what);

// The int a caller passed for a parameter of one of the header's enum types. They are plain C
// enums, so a C caller may pass any int; C++ leaves reading a value outside the enumerators
// through the enum type undefined, so such an argument is read through its bytes, and only a
// value checked this way is used as the enum afterwards.
template <class E>
inline int enum_arg(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}

}  // namespace pkv
