// la_internal.h -- host-side plumbing between the C ABI (la_api.cpp) and the
// kernel launchers (la_fwd_dk*.hip, la_decode.hip, la_bwd*.hip).
#pragma once

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#include <atomic>

#include "la.h"

namespace la {

struct FwdDesc {
    const void *q, *k, *v;
    void *o;
    float *den;
    const float *S0, *z0;
    float *S_out, *z_out;
    int B, H, N, DK, DV, C;
    int in_bf16, out_bf16;
    float *ws;
    hipStream_t stream;
    const float *gamma;  // causal only: per-head decay [H] (device), or null for none
    long ws_states;      // causal only: if > 0, at most this many segment states fit the workspace
};

struct DecodeDesc {
    float *S, *z;
    const void *q, *k, *v;
    void *o;
    int B, H, DK, DV;
    int in_bf16;
    hipStream_t stream;
    const float *gamma;  // per-head decay [H] (device), or null for none
};

struct BwdDesc {
    const void *q, *k, *v;
    const void *dO;
    void *dq, *dk, *dv;
    int B, H, N, DK, DV, C;
    int in_bf16;
    float *ws;
    hipStream_t stream;
    int noncausal;  // gradient of the non-causal form (full sums)
};

// Split of each (batch, head) sequence into P segments of L tokens (L a
// multiple of C), aiming at `target_wg` workgroups in total.  P never
// decreases when target_wg grows, so the workspace queries size for
// kMaxTargetWg and the launchers, which aim at what the GPU holds resident
// at once (never more than kMaxTargetWg), always fit.
constexpr long kMaxTargetWg = 2048;
int plan_segments(long BH, int N, int C, long target_wg, int *L);

// Workgroups of `kernel` (`threads` per workgroup) the current device keeps resident at
// once: occupancy per CU times the CU count, at most kMaxTargetWg.  Cached per
// device in `cache`, which belongs to that one kernel (a function-local static
// of the launcher that names the kernel).
constexpr int kMaxDevices = 64;
struct OccCache {
    std::atomic<long> n[kMaxDevices];
};
long resident_workgroups(const void *kernel, OccCache &cache, int threads = 256);

// Floats per stored state: S (DK x DV) followed by z (DK).
inline long state_floats(int DK, int DV) { return (long)DK * DV + DK; }

// Per-(bh, element) pass over the P segment states stored at ws[bh][P][DK*DV + DK]:
// mode 0 replaces slots [0, lim) by their exclusive prefix (S0, z0 folded in
// when given) and writes the sum of all of them into slot lim (when lim < P);
// mode 1 writes the total of all P slots into slot 0; mode 2 replaces slots
// [lim, P) by their exclusive suffix and writes the sum of all of them into
// slot lim - 1 (when lim > 0).  Other slots are not touched.  Fixed order.
// With gamma non-null (mode 0), the segments hold L tokens each and decay by
// gamma[bh % H] per token: entering(s) = gamma^L entering(s - 1) + aggregate(s - 1).
hipError_t launch_seg_scan(float *ws, const float *S0, const float *z0, long BH, int P, int DK, int DV,
                           int mode, int lim, hipStream_t stream, const float *gamma = nullptr, int H = 1,
                           int L = 0);

// Argument checks of the causal forward entry points (all but the workspace),
// before any HIP call; the status the entry point returns.
la_status check_fwd_causal_args(const void *q, const void *k, const void *v, const void *o, const void *den,
                                const void *S0, const void *z0, const void *S_out, const void *z_out, int B,
                                int H, int N, int d_k, int d_v, int C, int in, int out);
// Dispatch of a checked forward by d_k; launch errors map to LA_ERR_LAUNCH.
la_status run_fwd(const FwdDesc &d, bool causal);

hipError_t run_fwd_dk16(const FwdDesc &d, bool causal);
hipError_t run_fwd_dk32(const FwdDesc &d, bool causal);
hipError_t run_fwd_dk64(const FwdDesc &d, bool causal);
hipError_t run_fwd_dk128(const FwdDesc &d, bool causal);
hipError_t run_decode(const DecodeDesc &d);
size_t bwd_workspace_bytes(int B, int H, int N, int DK, int DV, int C);
hipError_t run_bwd(const BwdDesc &d);

}  // namespace la
