// One (kind, element type) slice of the collective kernels.  The build
// compiles this file once per slice with CCL_INST_KIND, CCL_INST_DT and
// CCL_INST_NAME set, so the template instantiations spread over parallel
// compiler jobs.
#include "ccl_coll_kernels.h"

namespace ccl {

hipError_t CCL_INST_NAME(const CollArgs &a, const CollPath &p, hipStream_t st) {
  return dispatch_kind<CCL_INST_KIND, CCL_INST_DT>(a, p, st);
}

}  // namespace ccl
