// api.hip -- status strings and the last HIP error of the CSA2 C ABI.
#include <hip/hip_runtime.h>

#include "../../include/csa2.h"

extern "C" int csa2_internal_last_hip_error_index(void);
extern "C" int csa2_internal_last_hip_error_attn(void);
extern "C" int csa2_internal_last_hip_error_quant(void);
extern "C" int csa2_internal_last_hip_error_blocks(void);
extern "C" int csa2_internal_last_hip_error_window(void);
extern "C" int csa2_internal_last_hip_error_merge(void);

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

extern "C" int csa2_last_hip_error(void) {
  int e = csa2_internal_last_hip_error_index();
  if (!e) e = csa2_internal_last_hip_error_attn();
  if (!e) e = csa2_internal_last_hip_error_quant();
  if (!e) e = csa2_internal_last_hip_error_blocks();
  if (!e) e = csa2_internal_last_hip_error_window();
  if (!e) e = csa2_internal_last_hip_error_merge();
  return e;
}
