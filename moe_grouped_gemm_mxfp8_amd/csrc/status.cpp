// Status strings of the C ABI, and the optional host check of the offsets.
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/moe_gg.h"

namespace moe_gg {

// With MOE_GG_VALIDATE=1 in the environment (read at each call), copy
// expert_off to the host, wait for it, and reject offsets that are not
// off[0] = 0, nondecreasing, off[E] = M.  A debugging aid: it synchronises
// the stream.  Without the variable it does nothing.
int check_offsets_if_asked(const int32_t *off, int E, int M, hipStream_t stream) {
  const char *v = std::getenv("MOE_GG_VALIDATE");
  if (!v || std::strcmp(v, "1") != 0) return MOE_GG_OK;
  std::vector<int32_t> h(static_cast<size_t>(E) + 1);
  if (hipMemcpyAsync(h.data(), off, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return MOE_GG_ELAUNCH;
  if (hipStreamSynchronize(stream) != hipSuccess) return MOE_GG_ELAUNCH;
  if (h[0] != 0 || h[static_cast<size_t>(E)] != M) return MOE_GG_EINVAL;
  for (int e = 0; e < E; ++e)
    if (h[static_cast<size_t>(e) + 1] < h[static_cast<size_t>(e)]) return MOE_GG_EINVAL;
  return MOE_GG_OK;
}

}  // namespace moe_gg

extern "C" MOE_GG_API const char *moe_gg_status_string(int status) {
  switch (status) {
    case MOE_GG_OK: return "ok";
    case MOE_GG_EINVAL: return "invalid argument (null pointer, negative or misaligned size)";
    case MOE_GG_EUNSUPPORTED: return "unsupported shape for these kernels";
    case MOE_GG_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}
