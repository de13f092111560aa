// Host-side error reporting shared by the C ABI's translation units: the thread-local message
// behind pkv_last_error_message and the hipError_t behind pkv_last_hip_error.
#pragma once

#include <hip/hip_runtime.h>

#include "pagedkv.h"

namespace pkv {

// Records a printf-style message and returns s.
pkv_status fail(pkv_status s, const char* fmt, ...);
// Records a HIP runtime failure of `what` and returns PKV_ERR_HIP.
pkv_status hip_failure(hipError_t e, const char* what);

}  // namespace pkv
