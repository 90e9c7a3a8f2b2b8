// la_bwd.hip -- dispatch of the cumulative-sum backward by d_k, and its
// workspace size (gh and eps buffers plus the per-segment prefix and suffix
// states; see la_bwd_launch.hpp).
#include "la_bwd_launch.hpp"

namespace la {

hipError_t run_bwd_dk16(const BwdDesc &d);
hipError_t run_bwd_dk32(const BwdDesc &d);
hipError_t run_bwd_dk64(const BwdDesc &d);
hipError_t run_bwd_dk128(const BwdDesc &d);

size_t bwd_workspace_bytes(int B, int H, int N, int DK, int DV, int C) {
    const long BH = (long)B * H;
    int L = 0;
    const int Pmax = plan_segments(BH, N, C, kMaxTargetWg, &L);
    return bwd_layout(BH, N, DK, DV, Pmax).total;
}

hipError_t run_bwd(const BwdDesc &d) {
    switch (d.DK) {
        case 16: return run_bwd_dk16(d);
        case 32: return run_bwd_dk32(d);
        case 64: return run_bwd_dk64(d);
        case 128: return run_bwd_dk128(d);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace la
