// Backward kernels instantiated for d_k = 16 (every d_v, both input types).
#include "la_bwd_launch.hpp"

namespace la {
hipError_t run_bwd_dk16(const BwdDesc &d) { return run_bwd_dk<16>(d); }
}  // namespace la
