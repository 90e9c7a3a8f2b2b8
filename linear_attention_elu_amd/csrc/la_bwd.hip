// la_bwd.hip -- cumulative-sum backward of the causal form (placeholder until
// the kernels land: reports "not supported").
#include "la_internal.h"

namespace la {

size_t bwd_workspace_bytes(int, int, int, int, int, int) { return 0; }

hipError_t run_bwd(const BwdDesc &) { return hipErrorNotSupported; }

}  // namespace la
