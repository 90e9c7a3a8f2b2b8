// la_scan.hip -- prefix sums of per-segment states across the segments of one
// (batch, head).  The causal prefix sums S_i, z_i form a scan, which can be
// evaluated in parallel (blog digest "Theoretical significance / prefix-sum
// parallelism"; itwiki table "Comparison of forms", chunked row): segments
// first reduce their own chunks, this kernel turns the segment totals into the
// state entering each segment, and the segments then run their chunk loops
// independently.
#include <hip/hip_runtime.h>

#include "la_internal.h"

namespace la {

// Pass over segments, per (bh, element), in a fixed order:
//   mode 0: exclusive prefix, the initial state folded in.  Only slots
//           [0, lim) hold aggregates; slots [0, lim] are written (slot lim,
//           when it exists, receives the sum of all of them).
//   mode 1: total of all P slots into slot 0 (lim unused).
//   mode 2: exclusive suffix.  Only slots [lim, P) hold aggregates; slots
//           [max(lim - 1, 0), P) are written.
// Slots outside those ranges are neither read nor written, so a caller
// aggregates only the segments whose sums some later pass reads.
// With a per-head decay (gamma non-null) every segment holds L tokens.  Mode
// 0: an aggregate is taken at its segment's last token, so the state entering
// segment s is gamma^L times the state entering s - 1 plus the aggregate of
// s - 1.  Mode 2: an aggregate is normalised at its segment's first token, so
// the suffix after segment s is the aggregate of s + 1 plus gamma^L times the
// suffix after s + 1.
// add (mode 0): aggregates in ws's layout added to ws's as they are read.
static __global__ void __launch_bounds__(256)
la_seg_scan_kernel(float *ws, const float *S0, const float *z0, int P, int DK, int DV, int mode, int lim,
                   const float *gamma, int H, int L, const float *add) {
    const int SS = DK * DV + DK;
    const long bh = blockIdx.x;
    const int idx = blockIdx.y * 256 + threadIdx.x;
    if (idx >= SS) return;
    float *base = ws + bh * (long)P * SS + idx;
    const float *abase = add ? add + bh * (long)P * SS + idx : nullptr;
    float f = 1.0f;  // gamma^L by repeated squaring
    if (gamma) {
        float b = gamma[bh % H];
        for (int e = L; e > 0; e >>= 1) {
            if (e & 1) f *= b;
            b *= b;
        }
    }
    if (mode == 0) {
        float run = 0.f;
        if (idx < DK * DV) {
            if (S0) run = S0[bh * (long)DK * DV + idx];
        } else if (z0) {
            run = z0[bh * (long)DK + (idx - DK * DV)];
        }
        for (int s = 0; s < lim; ++s) {
            const float a = base[(long)s * SS] + (abase ? abase[(long)s * SS] : 0.0f);
            base[(long)s * SS] = run;
            run = f * run + a;
        }
        if (lim < P) base[(long)lim * SS] = run;
    } else if (mode == 1) {
        float run = 0.f;
        for (int s = 0; s < P; ++s) run += base[(long)s * SS];
        base[0] = run;
    } else {
        float run = 0.f;  // exclusive suffix: the sum over the later segments
        for (int s = P - 1; s >= lim; --s) {
            const float a = base[(long)s * SS];
            base[(long)s * SS] = run;
            run = gamma ? a + f * run : run + a;
        }
        if (lim > 0) base[(long)(lim - 1) * SS] = run;
    }
}

hipError_t launch_seg_scan(float *ws, const float *S0, const float *z0, long BH, int P, int DK, int DV,
                           int mode, int lim, hipStream_t stream, const float *gamma, int H, int L,
                           const float *add) {
    if (lim < 0 || lim > P || (add && mode != 0)) return hipErrorInvalidValue;
    const long SS = state_floats(DK, DV);
    const dim3 grid((unsigned)BH, (unsigned)((SS + 255) / 256));
    la_seg_scan_kernel<<<grid, 256, 0, stream>>>(ws, S0, z0, P, DK, DV, mode, lim, gamma, H, L, add);
    return hipGetLastError();
}

}  // namespace la
