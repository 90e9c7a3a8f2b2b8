// Chunked forward kernels instantiated for d_k = 32 (every d_v, both input types).
#include "la_fwd_launch.hpp"

namespace la {
hipError_t run_fwd_dk32(const FwdDesc &d, bool causal) { return run_fwd_dk<32>(d, causal); }
}  // namespace la
