// gdr_bwd.hip -- backward kernels (in progress).
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

size_t bwd_workspace_bytes(const gdr_problem* p, const Plan& pl) {
  (void)p;
  (void)pl;
  return 0;
}

gdr_status launch_bwd(const gdr_problem*, const Plan&, const void*, const void*, const void*,
                      const float*, const void*, const void*, const void*, const float*,
                      const float*, void*, void*, void*, void*, void*, float*, void*,
                      hipStream_t) {
  set_error("backward not built yet");
  return GDR_ERR_ARG;
}

}  // namespace gdr
