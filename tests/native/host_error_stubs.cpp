// Minimal definitions of the library's error recorders, so that the block manager's source can be
// linked on its own into a host-only test program.
#include <hip/hip_runtime.h>

#include "host_errors.hpp"

namespace pkv {
pkv_status fail(pkv_status s, const char*, ...) { return s; }
pkv_status hip_failure(hipError_t, const char*) { return PKV_ERR_HIP; }
}  // namespace pkv
