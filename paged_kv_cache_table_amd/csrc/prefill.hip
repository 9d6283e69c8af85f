// Windowed prefill (placeholder until the matrix-core kernel lands).
#include "pkv_internal.hpp"

namespace pkv {

size_t prefill_workspace(const AttnArgs&, int, int, int, int, bool* found) {
  *found = false;
  return 0;
}

hipError_t launch_prefill(const AttnArgs&, int, int, int, int, hipStream_t, bool* found) {
  *found = false;
  return hipSuccess;
}

}  // namespace pkv
