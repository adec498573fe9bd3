// Stand-ins for libccl's device-side entry points, linked only into the
// host-only build that the sanitizer test compiles with gcc and
// -fsanitize=address,undefined (argument checks, launch resolution and the
// reshard planner, without any HIP kernel).  The CPU tests never reach a
// launch: every call they make is rejected first or is planner-only, so each
// stand-in stops the process if it is ever called.
#include <cstdio>
#include <cstdlib>

#include "ccl_internal.h"

namespace {
[[noreturn]] void reached(const char *what) {
  std::fprintf(stderr, "host-only build: %s was reached\n", what);
  std::abort();
}
}  // namespace

namespace ccl {
ccl_status_t launch_collective(const CollDesc &, const Launch &, hipStream_t) {
  reached("launch_collective");
}
ccl_status_t launch_ar_rmsnorm(const RmsDesc &, const Launch &, hipStream_t, bool, void *) {
  reached("launch_ar_rmsnorm");
}
ccl_status_t noalloc_scratch(void **) { reached("noalloc_scratch"); }
ccl_status_t reshard_launch(ccl_plan *, const void *const *, void *const *, const Launch &,
                            hipStream_t) {
  reached("reshard_launch");
}
ccl_status_t reshard_fp8_launch(ccl_plan *, const void *const *, void *const *, float *const *,
                                const Launch &, hipStream_t) {
  reached("reshard_fp8_launch");
}
// A plan that never ran a copy has no device tables to release.
void reshard_release(ccl_plan *plan) {
  if (!plan->dev.empty()) reached("reshard_release with device tables");
}
}  // namespace ccl
