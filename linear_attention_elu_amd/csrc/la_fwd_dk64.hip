// Chunked forward kernels instantiated for d_k = 64 (every d_v, both input types).
#include "la_fwd_launch.hpp"

namespace la {
hipError_t run_fwd_dk64(const FwdDesc &d, bool causal) { return run_fwd_dk<64>(d, causal); }
}  // namespace la
