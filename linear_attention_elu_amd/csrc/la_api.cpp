// la_api.cpp -- the C ABI of liblinattn.so: argument checks, workspace sizes
// and dispatch to the launchers.  Every check runs before any HIP call, so an
// invalid call enqueues nothing.
#include <stdint.h>

#include <atomic>

#include "la.h"
#include "la_internal.h"

namespace la {

int plan_segments(long BH, int N, int C, long target_wg, int *L) {
    const long nch = (N + (long)C - 1) / C;
    // Never split a sequence finer than one chunk per segment.
    long want = (target_wg + BH - 1) / BH;
    if (want > nch) want = nch;
    if (want < 1) want = 1;
    const long cps = (nch + want - 1) / want;  // chunks per segment
    const long P = (nch + cps - 1) / cps;
    *L = (int)(cps * C);
    return (int)P;
}

long resident_workgroups(const void *kernel, OccCache &cache, int threads) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
    if (dev >= 0) {
        const long c = cache.n[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu < 1) per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) != hipSuccess ||
        cus < 1)
        cus = 256;
    long n = (long)per_cu * cus;
    if (n > kMaxTargetWg) n = kMaxTargetWg;
    if (dev >= 0) cache.n[dev].store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace la

namespace la {

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool chunk_ok(int C) { return C == 16 || C == 32 || C == 64; }
bool dtype_ok(int t) { return t == LA_F32 || t == LA_BF16; }
bool aligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_or_null(const void *p) { return p == nullptr || aligned(p); }

// B, H, N within what the kernels index with 32-bit grid sizes and 64-bit offsets.
la_status check_shape(int B, int H, int N) {
    if (B < 1 || H < 1 || N < 1 || N > kMaxN) return LA_ERR_BAD_SHAPE;
    if ((long long)B * H > 0x7fffffffLL) return LA_ERR_BAD_SHAPE;
    return LA_OK;
}

size_t fwd_ws_bytes(int B, int H, int N, int dk, int dv, int C, bool causal) {
    if (B < 1 || H < 1 || N < 1 || N > kMaxN || !dim_ok(dk) || !dim_ok(dv) || !chunk_ok(C)) return 0;
    const long BH = (long)B * H;
    int L = 0;
    const int P = plan_segments(BH, N, C, kMaxTargetWg, &L);
    if (causal && P == 1) return 0;
    return (size_t)BH * P * state_floats(dk, dv) * sizeof(float);
}

la_status from_hip(hipError_t e) {
    if (e == hipSuccess) return LA_OK;
    if (e == hipErrorNotSupported) return LA_ERR_UNSUPPORTED;
    return LA_ERR_LAUNCH;
}

la_status check_fwd_causal_args(const void *q, const void *k, const void *v, const void *o, const void *den,
                                const void *S0, const void *z0, const void *S_out, const void *z_out, int B,
                                int H, int N, int d_k, int d_v, int C, int in, int out) {
    if (!q || !k || !v || !o) return LA_ERR_NULL_PTR;
    if ((S0 == nullptr) != (z0 == nullptr)) return LA_ERR_NULL_PTR;
    if ((S_out == nullptr) != (z_out == nullptr)) return LA_ERR_NULL_PTR;
    la_status st = check_shape(B, H, N);
    if (st != LA_OK) return st;
    if (!dim_ok(d_k) || !dim_ok(d_v) || !chunk_ok(C)) return LA_ERR_UNSUPPORTED;
    if (!dtype_ok(in) || !dtype_ok(out)) return LA_ERR_BAD_DTYPE;
    if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(o) || !aligned_or_null(den) ||
        !aligned_or_null(S0) || !aligned_or_null(z0) || !aligned_or_null(S_out) || !aligned_or_null(z_out))
        return LA_ERR_ALIGNMENT;
    return LA_OK;
}

la_status run_fwd(const FwdDesc &d, bool causal) {
    switch (d.DK) {
        case 16: return from_hip(run_fwd_dk16(d, causal));
        case 32: return from_hip(run_fwd_dk32(d, causal));
        case 64: return from_hip(run_fwd_dk64(d, causal));
        case 128: return from_hip(run_fwd_dk128(d, causal));
        default: return LA_ERR_UNSUPPORTED;
    }
}

}  // namespace la

namespace {

using la::aligned;
using la::aligned_or_null;
using la::check_shape;
using la::chunk_ok;
using la::dim_ok;
using la::dtype_ok;
using la::from_hip;
using la::fwd_ws_bytes;
using la::run_fwd;

using la::kNonCausalChunk;

}  // namespace

extern "C" {

const char *la_status_string(la_status s) {
    switch (s) {
        case LA_OK: return "LA_OK: success";
        case LA_ERR_NULL_PTR: return "LA_ERR_NULL_PTR: a required pointer is NULL";
        case LA_ERR_BAD_SHAPE: return "LA_ERR_BAD_SHAPE: B, H and N must be >= 1 (and B*H < 2^31)";
        case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED: d_k, d_v must be in {16,32,64,128} and C in {16,32,64}";
        case LA_ERR_BAD_DTYPE: return "LA_ERR_BAD_DTYPE: dtype must be LA_F32 or LA_BF16";
        case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE: workspace missing or smaller than the size query returns";
        case LA_ERR_LAUNCH: return "LA_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
        case LA_ERR_ALIGNMENT: return "LA_ERR_ALIGNMENT: every pointer must be 16-byte aligned";
    }
    return "unknown la_status";
}

size_t la_fwd_causal_workspace_bytes(int B, int H, int N, int d_k, int d_v, int C) {
    return fwd_ws_bytes(B, H, N, d_k, d_v, C, true);
}

size_t la_fwd_noncausal_workspace_bytes(int B, int H, int N, int d_k, int d_v) {
    return fwd_ws_bytes(B, H, N, d_k, d_v, kNonCausalChunk, false);
}

size_t la_bwd_causal_workspace_bytes(int B, int H, int N, int d_k, int d_v, int C) {
    if (B < 1 || H < 1 || N < 1 || N > la::kMaxN || !dim_ok(d_k) || !dim_ok(d_v) || !chunk_ok(C)) return 0;
    return la::bwd_workspace_bytes(B, H, N, d_k, d_v, C);
}

size_t la_bwd_noncausal_workspace_bytes(int B, int H, int N, int d_k, int d_v) {
    if (B < 1 || H < 1 || N < 1 || N > la::kMaxN || !dim_ok(d_k) || !dim_ok(d_v)) return 0;
    return la::bwd_workspace_bytes(B, H, N, d_k, d_v, kNonCausalChunk);
}

la_status la_fwd_causal_decay(const void *q, const void *k, const void *v, void *o, float *den,
                              const float *S0, const float *z0, float *S_out, float *z_out, const float *gamma,
                              int B, int H, int N, int d_k, int d_v, int C,
                              la_dtype in, la_dtype out,
                              void *ws, size_t ws_bytes, hipStream_t stream) {
    la_status st = la::check_fwd_causal_args(q, k, v, o, den, S0, z0, S_out, z_out, B, H, N, d_k, d_v, C, in, out);
    if (st != LA_OK) return st;
    if (!aligned_or_null(ws)) return LA_ERR_ALIGNMENT;
    const size_t need = fwd_ws_bytes(B, H, N, d_k, d_v, C, true);
    if (need > 0 && (ws == nullptr || ws_bytes < need)) return LA_ERR_WORKSPACE;
    la::FwdDesc d{q, k, v, o, den, S0, z0, S_out, z_out, B, H, N, d_k, d_v, C,
                  in == LA_BF16, out == LA_BF16, static_cast<float *>(ws), stream, gamma};
    return run_fwd(d, true);
}

la_status la_fwd_causal_state(const void *q, const void *k, const void *v, void *o, float *den,
                              const float *S0, const float *z0, float *S_out, float *z_out,
                              int B, int H, int N, int d_k, int d_v, int C,
                              la_dtype in, la_dtype out,
                              void *ws, size_t ws_bytes, hipStream_t stream) {
    return la_fwd_causal_decay(q, k, v, o, den, S0, z0, S_out, z_out, nullptr, B, H, N, d_k, d_v, C, in, out,
                               ws, ws_bytes, stream);
}

la_status la_fwd_causal(const void *q, const void *k, const void *v, void *o, float *den,
                        int B, int H, int N, int d_k, int d_v, int C,
                        la_dtype in, la_dtype out,
                        void *ws, size_t ws_bytes, hipStream_t stream) {
    return la_fwd_causal_state(q, k, v, o, den, nullptr, nullptr, nullptr, nullptr, B, H, N, d_k, d_v, C,
                               in, out, ws, ws_bytes, stream);
}

la_status la_fwd_noncausal(const void *q, const void *k, const void *v, void *o,
                           int B, int H, int N, int d_k, int d_v,
                           la_dtype in, la_dtype out,
                           void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!q || !k || !v || !o) return LA_ERR_NULL_PTR;
    la_status st = check_shape(B, H, N);
    if (st != LA_OK) return st;
    if (!dim_ok(d_k) || !dim_ok(d_v)) return LA_ERR_UNSUPPORTED;
    if (!dtype_ok(in) || !dtype_ok(out)) return LA_ERR_BAD_DTYPE;
    if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(o) || !aligned_or_null(ws)) return LA_ERR_ALIGNMENT;
    const size_t need = fwd_ws_bytes(B, H, N, d_k, d_v, kNonCausalChunk, false);
    if (ws == nullptr || ws_bytes < need) return LA_ERR_WORKSPACE;
    la::FwdDesc d{q, k, v, o, nullptr, nullptr, nullptr, nullptr, nullptr, B, H, N, d_k, d_v, kNonCausalChunk,
                  in == LA_BF16, out == LA_BF16, static_cast<float *>(ws), stream, nullptr};
    return run_fwd(d, false);
}

la_status la_bwd_causal(const void *q, const void *k, const void *v, const void *dO,
                        void *dq, void *dk, void *dv,
                        int B, int H, int N, int d_k, int d_v, int C, la_dtype in,
                        void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!q || !k || !v || !dO || !dq || !dk || !dv) return LA_ERR_NULL_PTR;
    la_status st = check_shape(B, H, N);
    if (st != LA_OK) return st;
    if (!dim_ok(d_k) || !dim_ok(d_v) || !chunk_ok(C)) return LA_ERR_UNSUPPORTED;
    if (!dtype_ok(in)) return LA_ERR_BAD_DTYPE;
    if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(dO) || !aligned(dq) || !aligned(dk) ||
        !aligned(dv) || !aligned_or_null(ws))
        return LA_ERR_ALIGNMENT;
    const size_t need = la::bwd_workspace_bytes(B, H, N, d_k, d_v, C);
    if (ws == nullptr || ws_bytes < need) return LA_ERR_WORKSPACE;
    la::BwdDesc d{q, k, v, dO, dq, dk, dv, B, H, N, d_k, d_v, C, in == LA_BF16, static_cast<float *>(ws), stream};
    return from_hip(la::run_bwd(d));
}

la_status la_bwd_causal_decay(const void *q, const void *k, const void *v, const void *dO,
                              void *dq, void *dk, void *dv, const float *gamma,
                              int B, int H, int N, int d_k, int d_v, int C, la_dtype in,
                              void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!gamma) return LA_ERR_NULL_PTR;
    if ((reinterpret_cast<uintptr_t>(gamma) & 3u) != 0) return LA_ERR_ALIGNMENT;
    if (!q || !k || !v || !dO || !dq || !dk || !dv) return LA_ERR_NULL_PTR;
    la_status st = check_shape(B, H, N);
    if (st != LA_OK) return st;
    if (!dim_ok(d_k) || !dim_ok(d_v) || !chunk_ok(C)) return LA_ERR_UNSUPPORTED;
    if (!dtype_ok(in)) return LA_ERR_BAD_DTYPE;
    if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(dO) || !aligned(dq) || !aligned(dk) ||
        !aligned(dv) || !aligned_or_null(ws))
        return LA_ERR_ALIGNMENT;
    const size_t need = la::bwd_workspace_bytes(B, H, N, d_k, d_v, C);
    if (ws == nullptr || ws_bytes < need) return LA_ERR_WORKSPACE;
    la::BwdDesc d{q, k, v, dO, dq, dk, dv, B, H, N, d_k, d_v, C, in == LA_BF16, static_cast<float *>(ws), stream,
                  0, 0, gamma};
    return from_hip(la::run_bwd(d));
}

la_status la_bwd_noncausal(const void *q, const void *k, const void *v, const void *dO,
                           void *dq, void *dk, void *dv,
                           int B, int H, int N, int d_k, int d_v, la_dtype in,
                           void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!q || !k || !v || !dO || !dq || !dk || !dv) return LA_ERR_NULL_PTR;
    la_status st = check_shape(B, H, N);
    if (st != LA_OK) return st;
    if (!dim_ok(d_k) || !dim_ok(d_v)) return LA_ERR_UNSUPPORTED;
    if (!dtype_ok(in)) return LA_ERR_BAD_DTYPE;
    if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(dO) || !aligned(dq) || !aligned(dk) ||
        !aligned(dv) || !aligned_or_null(ws))
        return LA_ERR_ALIGNMENT;
    const size_t need = la::bwd_workspace_bytes(B, H, N, d_k, d_v, kNonCausalChunk);
    if (ws == nullptr || ws_bytes < need) return LA_ERR_WORKSPACE;
    la::BwdDesc d{q, k, v, dO, dq, dk, dv, B, H, N, d_k, d_v, kNonCausalChunk, in == LA_BF16,
                  static_cast<float *>(ws), stream, 1};
    return from_hip(la::run_bwd(d));
}

la_status la_decode_step(float *S, float *z, const void *q, const void *k, const void *v,
                         void *o, int B, int H, int d_k, int d_v, la_dtype in, hipStream_t stream) {
    if (!S || !z || !q || !k || !v || !o) return LA_ERR_NULL_PTR;
    la_status st = check_shape(B, H, 1);
    if (st != LA_OK) return st;
    if (!dim_ok(d_k) || !dim_ok(d_v)) return LA_ERR_UNSUPPORTED;
    if (!dtype_ok(in)) return LA_ERR_BAD_DTYPE;
    if (!aligned(S) || !aligned(z) || !aligned(q) || !aligned(k) || !aligned(v) || !aligned(o))
        return LA_ERR_ALIGNMENT;
    la::DecodeDesc d{S, z, q, k, v, o, B, H, d_k, d_v, in == LA_BF16, stream, nullptr};
    return from_hip(la::run_decode(d));
}

la_status la_decode_step_decay(float *S, float *z, const void *q, const void *k, const void *v,
                               void *o, const float *gamma, int B, int H, int d_k, int d_v, la_dtype in,
                               hipStream_t stream) {
    if (!S || !z || !q || !k || !v || !o || !gamma) return LA_ERR_NULL_PTR;
    la_status st = check_shape(B, H, 1);
    if (st != LA_OK) return st;
    if (!dim_ok(d_k) || !dim_ok(d_v)) return LA_ERR_UNSUPPORTED;
    if (!dtype_ok(in)) return LA_ERR_BAD_DTYPE;
    if (!aligned(S) || !aligned(z) || !aligned(q) || !aligned(k) || !aligned(v) || !aligned(o))
        return LA_ERR_ALIGNMENT;
    la::DecodeDesc d{S, z, q, k, v, o, B, H, d_k, d_v, in == LA_BF16, stream, gamma};
    return from_hip(la::run_decode(d));
}

}  // extern "C"
