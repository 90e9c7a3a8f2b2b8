// Backward kernels instantiated for d_k = 64 (every d_v, both input types).
#include "la_bwd_launch.hpp"

namespace la {
hipError_t run_bwd_dk64(const BwdDesc &d) { return run_bwd_dk<64>(d); }
}  // namespace la
