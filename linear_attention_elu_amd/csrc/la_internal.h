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
    int phi_id;          // feature map: 0 = elu + 1, 1 = identity (q, k are already features),
                         // kPhiPrfFused = random features applied in the staging waves (W)
    const void *W;       // kPhiPrfFused: directions [H][DK][DK] in the input type
};

// phi_id of the forward with the random-feature map computed in the chunk
// kernels' staging waves (m = d_k; prf_fused_ok shapes, 64-token chunks).
constexpr int kPhiPrfFused = 2;
template <int DK, int DV, typename TI> constexpr bool prf_fused_ok() {
    return sizeof(TI) == 2 && (DK == 32 || DK == 64) && DV <= 64;
}

struct DecodeDesc {
    float *S, *z;
    const void *q, *k, *v;
    void *o;
    int B, H, DK, DV;
    int in_bf16;
    hipStream_t stream;
    const float *gamma;  // per-head decay [H] (device), or null for none
    int fm;              // feature map: 0 = elu + 1, 1 = identity, 2 = random features (DK = their count)
    const void *W;       // random features: directions [H][DK][din] in the input type
    int din;             // random features: width of q and k
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
    int phi_id;     // feature map: 0 = elu + 1, 1 = identity
    const float *gamma;  // causal only: per-head decay [H] (device), or null for none
    // Sweep products on bf16 value-plus-remainder operands (causal, no decay):
    // q and k as two bf16 planes each (value, remainder: [2][B*H][N][DK]),
    // dq and dk fp32, v, dO and dv bf16.  The prefix aggregate then runs once
    // per plane of k on bf16 operands, the second pass writing its segment
    // sums to agg_lo (the size of the prefix workspace).
    int pair_ops;
    float *agg_lo;
};

// Split of each (batch, head) sequence into P segments of L tokens (L a
// multiple of C), aiming at `target_wg` workgroups in total.  P never
// decreases when target_wg grows, so the workspace queries size for
// kMaxTargetWg and the launchers, which aim at what the GPU holds resident
// at once (never more than kMaxTargetWg), always fit.
constexpr long kMaxTargetWg = 2048;
int plan_segments(long BH, int N, int C, long target_wg, int *L);

// Longest sequence accepted (segment bounds are int arithmetic on N + L).
constexpr int kMaxN = 1 << 30;

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
// With gamma non-null, the segments hold L tokens each and decay by
// gamma[bh % H] per token: mode 0, entering(s) = gamma^L entering(s - 1) +
// aggregate(s - 1); mode 2, after(s) = aggregate(s + 1) + gamma^L after(s + 1).
// add (mode 0, nullable): a second buffer of aggregates in ws's layout, added
// to ws's (the two halves of a split aggregate).
hipError_t launch_seg_scan(float *ws, const float *S0, const float *z0, long BH, int P, int DK, int DV,
                           int mode, int lim, hipStream_t stream, const float *gamma = nullptr, int H = 1,
                           int L = 0, const float *add = nullptr);

// Shared argument predicates and sizes of the entry points (la_api.cpp).
bool dim_ok(int d);
bool chunk_ok(int C);
bool dtype_ok(int t);
bool aligned(const void *p);
bool aligned_or_null(const void *p);
la_status check_shape(int B, int H, int N);
la_status from_hip(hipError_t e);
size_t fwd_ws_bytes(int B, int H, int N, int dk, int dv, int C, bool causal);
// Chunk size the non-causal path tiles its sequence with (not part of its ABI).
constexpr int kNonCausalChunk = 64;

// The random-feature map and its backward (la_prf.hip), x [BH][N][DK] and the
// directions W [H][M][DK] in the input type:
//   PRF_PHI      out = phi(x) [BH][N][M] in the input type;
//   PRF_PHI_F32  out = phi(x) in fp32, or with halves non-null phi(x) as
//                its bf16 value (plane 0) and bf16 remainder (plane 1) at
//                halves, bf16 [2][BH][N][M] (out unused);
//   PRF_VJP      out = dx [BH][N][DK] (input type) from x, f = phi(x) and
//                df = dphi, both fp32;
//   PRF_VJP_U    the same from x and df = u = dphi * phi (fp32; f unused).
enum { PRF_PHI = 0, PRF_PHI_F32 = 1, PRF_VJP = 2, PRF_VJP_U = 3 };
hipError_t launch_prf(bool bf16, int what, const void *x, const void *W, const void *f, const void *df, void *out,
                      long BH, int N, int H, int DK, int M, hipStream_t stream, void *halves = nullptr);

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
