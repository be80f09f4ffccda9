// api.hip -- status strings and the last HIP error of the CSA2 C ABI.
#include <hip/hip_runtime.h>

#include "../../include/csa2.h"

namespace csa2 {
namespace {
thread_local int g_last_hip_error = 0;   // one slot per thread, for every entry point
}
__attribute__((visibility("hidden"))) void set_last_hip_error(int e) { g_last_hip_error = e; }
}  // namespace csa2

extern "C" const char* csa2_status_string(csa2_status s) {
  switch (s) {
    case CSA2_OK: return "ok";
    case CSA2_E_INVAL: return "invalid argument";
    case CSA2_E_UNSUPPORTED: return "unsupported shape";
    case CSA2_E_WORKSPACE: return "workspace too small";
    case CSA2_E_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

extern "C" int csa2_last_hip_error(void) { return csa2::g_last_hip_error; }
