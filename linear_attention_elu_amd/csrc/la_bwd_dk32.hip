// Backward kernels instantiated for d_k = 32 (every d_v, both input types).
#include "la_bwd_launch.hpp"

namespace la {
hipError_t run_bwd_dk32(const BwdDesc &d) { return run_bwd_dk<32>(d); }
}  // namespace la
