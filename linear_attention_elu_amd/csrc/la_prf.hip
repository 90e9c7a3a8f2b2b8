// la_prf.hip -- the pluggable feature map: positive random features on the
// matrix cores, and the entry points that take a feature map.
//
// Feature maps (itwiki "선형 어텐션", section "특징 사상 선택" (choice of
// feature map): elu + 1, Performer's positive orthogonal random features, and
// the identity; blog digest "Digest", open questions):
//   elu + 1   the default of every other entry point;
//   identity  q and k are the features (the caller keeps the normaliser
//             positive);
//   random    phi(x)_r = exp(w_r . x - |x|^2 / 2) / sqrt(m), r < m, with m
//             directions w_r of dimension d_k per head, W [H][m][d_k]; then
//             phi(q) . phi(k) estimates exp(q . k) without bias when the w_r
//             are drawn from N(0, I) (orthogonal blocks lower the variance).
//
// The random map is a dense contraction (a d_k x m matrix per row), so it runs
// on the matrix cores in its own kernel: la_prf_kernel writes phi(q) and
// phi(k) into the workspace and the chunked kernels read them with the
// identity map; the state then has m rows.  Its backward is a second
// contraction: with u = dphi * phi (elementwise),
//   dx = sum_r u_r (w_r - x) = W^T u - x (sum_r u_r),
// which la_prf_vjp_kernel forms from x, W, phi and the dphi the backward
// sweeps leave (with the identity map they return dphi).
#include <hip/hip_runtime.h>

#include "la.h"
#include "la_device.hpp"
#include "la_internal.h"

namespace la {

namespace {

constexpr int kPrfThreads = 256;        // four waves
constexpr int kPrfTokensPerBlock = 64;  // 16 tokens per wave and step
constexpr int kPrfSteps = 8;            // token blocks per workgroup (W staged once)

// Rows of W (or of W^T) in LDS, padded by 16 bytes against bank conflicts of
// the 16-byte fragment reads (lanes p = 0..15 read rows p at one column).
template <typename TC, int D> constexpr int prf_ld() { return D + 16 / (int)sizeof(TC); }

// W [M][DK] of one head into LDS with 16-byte copies, as rows of length LD
// (TRANS: as W^T, row e holding w_{0..M-1, e}, with element copies).
template <typename TC, int DK, int M, int LD, bool TRANS>
__device__ __forceinline__ void stage_w(TC *sw, const TC *Wh, int tid) {
    if constexpr (TRANS) {
        for (int i = tid; i < M * DK; i += kPrfThreads) sw[(i % DK) * LD + i / DK] = Wh[i];
    } else {
        constexpr int VR = DK * (int)sizeof(TC) / 16;  // 16-byte vectors per row
        for (int i = tid; i < M * VR; i += kPrfThreads)
            *reinterpret_cast<uint4 *>(sw + (i / VR) * LD + (i % VR) * (16 / (int)sizeof(TC))) =
                *reinterpret_cast<const uint4 *>(Wh + (long)i * (16 / (int)sizeof(TC)));
    }
}

// Eight consecutive elements of a global row as an operand fragment (straight
// K assignment: slot t of lane group g is K index 8g + t of the step).
template <typename TC>
__device__ __forceinline__ void frag_global8(Frag<TC> &f, const TC *row) {
    if constexpr (sizeof(TC) == 2) {
        f.v = __builtin_bit_cast(bf16x8, load_stream16(row));
    } else {
        const uint4 a = load_stream16(row), b = load_stream16(row + 4);
        f.v[0] = __uint_as_float(a.x), f.v[1] = __uint_as_float(a.y), f.v[2] = __uint_as_float(a.z);
        f.v[3] = __uint_as_float(a.w), f.v[4] = __uint_as_float(b.x), f.v[5] = __uint_as_float(b.y);
        f.v[6] = __uint_as_float(b.z), f.v[7] = __uint_as_float(b.w);
    }
}

// Four floats to out[0..3] in the storage type.
template <typename TS> __device__ __forceinline__ void store4_to(TS *out, const f32x4 &a) {
    if constexpr (sizeof(TS) == 2) *reinterpret_cast<uint2 *>(out) = pack_bf16x4(a);
    else *reinterpret_cast<f32x4 *>(out) = a;
}

// Four consecutive elements of a row as floats.
template <typename TC> __device__ __forceinline__ f32x4 load4(const TC *p) {
    if constexpr (sizeof(TC) == 2) {
        const uint2 u = *reinterpret_cast<const uint2 *>(p);
        return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u)};
    } else {
        return *reinterpret_cast<const f32x4 *>(p);
    }
}

// phi(x)^T tiles: for a block of 16 tokens per wave and every feature tile F,
// acc = W[16F.., :] x^T, so lane (g, p) ends with features 16F + 4g + r of
// token p -- four consecutive features of one token, stored as one vector.
// ||x||^2 comes from the same x fragments (each lane holds eight elements of
// token p per K step; the four lane groups hold the rest).  Each wave walks
// kPrfSteps blocks 64 tokens apart with two register sets: the rows of block
// i + 1 are in flight while block i is computed, and those of block 0 are
// issued before W is staged.
// HV: phi goes out as two bf16 planes (value, remainder) at halves instead
// of to out.  A lane's four features of one token are 16 apart from one
// feature tile to the next, so the wave first gathers its 16 tokens' rows in
// LDS and then writes whole 16-byte pieces of each row.
template <typename TC, typename TO, int DK, int M, bool HV = false>
__global__ void __launch_bounds__(kPrfThreads) la_prf_kernel(const TC *__restrict__ x, const TC *__restrict__ W,
                                                             TO *__restrict__ out, __bf16 *__restrict__ halves, int N,
                                                             int H) {
    constexpr int LW = prf_ld<TC, DK>();
    constexpr int NF = M / 16, NS = DK / 32;
    constexpr int LR = M + 8;  // row of the gather tile (bf16), 16-byte aligned, banks staggered
    __shared__ __attribute__((aligned(16))) TC sw[M * LW];
    __shared__ __attribute__((aligned(16))) __bf16 srow[HV ? (kPrfThreads / 64) * 2 * 16 * LR : 8];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, pp = lane & 15;
    const long bh = blockIdx.x;
    const int first = blockIdx.y * (kPrfSteps * kPrfTokensPerBlock) + 16 * wave;  // this wave's block 0
    const TC *xb = x + bh * (long)N * DK;
    Frag<TC> fx[2][NS];
    auto load = [&](Frag<TC>(&f)[NS], int step) {
        const int t = min(first + kPrfTokensPerBlock * step + pp, N - 1);
#pragma unroll
        for (int s = 0; s < NS; ++s) frag_global8(f[s], xb + (long)t * DK + 32 * s + 8 * g);
    };
    load(fx[0], 0);
    stage_w<TC, DK, M, LW, false>(sw, W + (bh % H) * (long)M * DK, tid);
    __syncthreads();
    const float scale = __builtin_amdgcn_rsqf((float)M);
#pragma unroll
    for (int step = 0; step < kPrfSteps; ++step) {
        const int t0 = first + kPrfTokensPerBlock * step;
        if (t0 >= N) break;  // uniform per wave; no barrier follows
        if (step + 1 < kPrfSteps && t0 + kPrfTokensPerBlock < N) load(fx[(step + 1) & 1], step + 1);
        const Frag<TC>(&cx)[NS] = fx[step & 1];
        f32x4 acc[NF];
#pragma unroll
        for (int F = 0; F < NF; ++F) acc[F] = f32x4{0.f, 0.f, 0.f, 0.f};
        float nx = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int u = 0; u < 8; ++u) nx += cx[s].get(u) * cx[s].get(u);
#pragma unroll
            for (int F = 0; F < NF; ++F) {
                Frag<TC> fw;
                lds_frag_straight(fw, sw + (16 * F + pp) * LW + 32 * s, g);
                acc[F] = mma(fw, cx[s], acc[F]);
            }
        }
        nx = sum_over_groups(nx);
        if constexpr (HV) {
            // rows of this wave's 16 tokens: plane 0 the bf16 value, plane 1 the bf16 remainder
            __bf16 *rows = srow + wave * (2 * 16 * LR);
#pragma unroll
            for (int F = 0; F < NF; ++F) {
                f32x4 f;
#pragma unroll
                for (int r = 0; r < 4; ++r) f[r] = __expf(acc[F][r] - 0.5f * nx) * scale;
                const uint2 hv = pack_bf16x4(f);
                const f32x4 h = {__uint_as_float(hv.x << 16), __uint_as_float(hv.x & 0xffff0000u),
                                 __uint_as_float(hv.y << 16), __uint_as_float(hv.y & 0xffff0000u)};
                *reinterpret_cast<uint2 *>(rows + pp * LR + 16 * F + 4 * g) = hv;
                *reinterpret_cast<uint2 *>(rows + (16 + pp) * LR + 16 * F + 4 * g) = pack_bf16x4(f - h);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // 16-byte pieces: M / 8 per row, 16 rows per plane
            constexpr int PR = M / 8;
#pragma unroll
            for (int c = lane; c < 2 * 16 * PR; c += 64) {
                const int plane = c / (16 * PR), tok = (c / PR) % 16, col = 8 * (c % PR);
                const uint4 piece = *reinterpret_cast<const uint4 *>(rows + (16 * plane + tok) * LR + col);
                if (t0 + tok < N)
                    *reinterpret_cast<uint4 *>(halves + plane * (long)gridDim.x * N * M + (bh * N + t0 + tok) * (long)M +
                                               col) = piece;
            }
            // the next step's rows overwrite these only after every lane has read them
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        } else if (t0 + pp < N) {
#pragma unroll
            for (int F = 0; F < NF; ++F) {
                f32x4 f;
#pragma unroll
                for (int r = 0; r < 4; ++r) f[r] = __expf(acc[F][r] - 0.5f * nx) * scale;
                store4_to(out + (bh * N + t0 + pp) * (long)M + 16 * F + 4 * g, f);
            }
        }
    }
}

// dx^T tiles: acc = W^T[16E.., :] u^T over the m features (u = dphi * phi,
// both fp32, or u as given: UG), lane (g, p) ending with elements 16E + 4g + r of token p; then
// dx = acc - x * sum_r u_r.  With bf16 operands u enters the matrix cores as
// a bf16 value plus its bf16 remainder, so the product keeps about 16
// significant bits (W is exact in its storage type).  That precision is
// needed: phi(x) spans many orders of magnitude across features, so an error
// of dphi that is small against its row but large against a small entry is
// multiplied by a large phi_r(x).  The token blocks are pipelined as in
// la_prf_kernel (phi and dphi, or u, and the x elements of the epilogue in
// flight).
template <typename TC, int DK, int M, bool UG = false>  // UG: dphi_x holds u = dphi * phi (phi_x unused)
__global__ void __launch_bounds__(kPrfThreads) la_prf_vjp_kernel(const TC *__restrict__ x, const TC *__restrict__ W,
                                                                 const void *__restrict__ phi_x,
                                                                 const float *__restrict__ dphi_x,
                                                                 TC *__restrict__ dx, int N, int H) {
    constexpr int LT = prf_ld<TC, M>();
    constexpr int NE = DK / 16, NS = M / 32;
    constexpr bool LO = sizeof(TC) == 2;
    __shared__ __attribute__((aligned(16))) TC swt[DK * LT];  // W^T: row e holds w_{0..m-1, e}
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, pp = lane & 15;
    const long bh = blockIdx.x;
    const int first = blockIdx.y * (kPrfSteps * kPrfTokensPerBlock) + 16 * wave;
    struct Regs {
        Frag<float> ff[UG ? 1 : NS], fd[NS];
        f32x4 xv[NE];
    } rg[2];
    auto load = [&](Regs &r, int step) {
        const long row = bh * N + min(first + kPrfTokensPerBlock * step + pp, N - 1);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if constexpr (!UG) frag_global8(r.ff[s], static_cast<const float *>(phi_x) + row * M + 32 * s + 8 * g);
            frag_global8(r.fd[s], dphi_x + row * M + 32 * s + 8 * g);
        }
#pragma unroll
        for (int E = 0; E < NE; ++E) r.xv[E] = load4(x + row * DK + 16 * E + 4 * g);
    };
    load(rg[0], 0);
    stage_w<TC, DK, M, LT, true>(swt, W + (bh % H) * (long)M * DK, tid);
    __syncthreads();
#pragma unroll
    for (int step = 0; step < kPrfSteps; ++step) {
        const int t0 = first + kPrfTokensPerBlock * step;
        if (t0 >= N) break;  // uniform per wave; no barrier follows
        if (step + 1 < kPrfSteps && t0 + kPrfTokensPerBlock < N) load(rg[(step + 1) & 1], step + 1);
        const Regs &cr = rg[step & 1];
        f32x4 acc[NE];
#pragma unroll
        for (int E = 0; E < NE; ++E) acc[E] = f32x4{0.f, 0.f, 0.f, 0.f};
        float su = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            Frag<TC> fu, fu_lo;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                float val;
                if constexpr (UG) val = cr.fd[s].get(u);
                else val = cr.ff[s].get(u) * cr.fd[s].get(u);
                su += val;
                fu.set(u, val);
                if constexpr (LO) fu_lo.set(u, val - fu.get(u));
            }
#pragma unroll
            for (int E = 0; E < NE; ++E) {
                Frag<TC> fw;
                lds_frag_straight(fw, swt + (16 * E + pp) * LT + 32 * s, g);
                acc[E] = mma(fw, fu, acc[E]);
                if constexpr (LO) acc[E] = mma(fw, fu_lo, acc[E]);
            }
        }
        su = sum_over_groups(su);
        if (t0 + pp < N) {
            TC *dr = dx + (bh * N + t0 + pp) * DK;
#pragma unroll
            for (int E = 0; E < NE; ++E) store4_to(dr + 16 * E + 4 * g, acc[E] - cr.xv[E] * su);
        }
    }
}

template <typename TC, int DK, int M>
hipError_t launch_prf_t(int what, const void *x, const void *W, const void *f, const void *df, void *out, long BH,
                        int N, int H, hipStream_t stream, void *halves) {
    const int per_wg = kPrfTokensPerBlock * kPrfSteps;
    const dim3 grid((unsigned)BH, (unsigned)((N + per_wg - 1) / per_wg));
    const TC *xc = static_cast<const TC *>(x), *wc = static_cast<const TC *>(W);
    if (what == PRF_VJP)
        la_prf_vjp_kernel<TC, DK, M><<<grid, kPrfThreads, 0, stream>>>(xc, wc, f, static_cast<const float *>(df),
                                                                        static_cast<TC *>(out), N, H);
    else if (what == PRF_VJP_U)
        la_prf_vjp_kernel<TC, DK, M, true><<<grid, kPrfThreads, 0, stream>>>(xc, wc, f, static_cast<const float *>(df),
                                                                              static_cast<TC *>(out), N, H);
    else if (what == PRF_PHI_F32 && halves)
        la_prf_kernel<TC, float, DK, M, true><<<grid, kPrfThreads, 0, stream>>>(xc, wc, nullptr,
                                                                                static_cast<__bf16 *>(halves), N, H);
    else if (what == PRF_PHI_F32)
        la_prf_kernel<TC, float, DK, M><<<grid, kPrfThreads, 0, stream>>>(xc, wc, static_cast<float *>(out), nullptr,
                                                                          N, H);
    else
        la_prf_kernel<TC, TC, DK, M><<<grid, kPrfThreads, 0, stream>>>(xc, wc, static_cast<TC *>(out), nullptr, N, H);
    return hipGetLastError();
}

template <typename TC, int DK>
hipError_t launch_prf_dk(int what, const void *x, const void *W, const void *f, const void *df, void *out, long BH,
                         int N, int H, int M, hipStream_t stream, void *halves) {
    switch (M) {
        case 32: return launch_prf_t<TC, DK, 32>(what, x, W, f, df, out, BH, N, H, stream, halves);
        case 64: return launch_prf_t<TC, DK, 64>(what, x, W, f, df, out, BH, N, H, stream, halves);
        case 128: return launch_prf_t<TC, DK, 128>(what, x, W, f, df, out, BH, N, H, stream, halves);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prf_any(bool bf16, int what, const void *x, const void *W, const void *f, const void *df,
                          void *out, long BH, int N, int H, int DK, int M, hipStream_t stream, void *halves) {
    switch (DK) {
        case 32:
            return bf16 ? launch_prf_dk<__bf16, 32>(what, x, W, f, df, out, BH, N, H, M, stream, halves)
                        : launch_prf_dk<float, 32>(what, x, W, f, df, out, BH, N, H, M, stream, halves);
        case 64:
            return bf16 ? launch_prf_dk<__bf16, 64>(what, x, W, f, df, out, BH, N, H, M, stream, halves)
                        : launch_prf_dk<float, 64>(what, x, W, f, df, out, BH, N, H, M, stream, halves);
        case 128:
            return bf16 ? launch_prf_dk<__bf16, 128>(what, x, W, f, df, out, BH, N, H, M, stream, halves)
                        : launch_prf_dk<float, 128>(what, x, W, f, df, out, BH, N, H, M, stream, halves);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prf(bool bf16, int what, const void *x, const void *W, const void *f, const void *df, void *out,
                      long BH, int N, int H, int DK, int M, hipStream_t stream, void *halves) {
    return launch_prf_any(bf16, what, x, W, f, df, out, BH, N, H, DK, M, stream, halves);
}


}  // namespace la

namespace {

using la::aligned;
using la::aligned_or_null;

bool fm_known(int fm) { return fm == LA_PHI_ELU1 || fm == LA_PHI_IDENTITY || fm == LA_PHI_PRF; }
bool prf_dim_ok(int d) { return d == 32 || d == 64 || d == 128; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace of the random map.  Forward: phi(q), phi(k) as [BH][N][m] in the
// input type, then the inner call's workspace.  Backward: phi(q), phi(k) in
// fp32 (bf16 inputs: as two bf16 planes each, value and remainder, the same
// bytes), dphi(q), dphi(k) in fp32, for bf16 inputs the segment sums of the
// prefix aggregate's remainder pass, then the inner backward's workspace.
struct FmLayout {
    size_t fq, fk, dfq, dfk, agglo, inner, total;
};
// (C: the backward's chunk size, which sizes the prefix aggregate's slots.)
FmLayout fm_layout(bool bwd, int B, int H, int N, int m, int d_v, int C, int in, size_t inner_bytes) {
    const size_t th = (size_t)B * H * N;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t a = off;
        off += align256(bytes);
        return a;
    };
    FmLayout l{};
    const size_t fe = bwd ? 4 : (in == LA_BF16 ? 2 : 4);
    l.fq = take(th * m * fe);
    l.fk = take(th * m * fe);
    if (bwd) {
        l.dfq = take(th * m * 4);
        l.dfk = take(th * m * 4);
        if (in == LA_BF16) {
            int L = 0;
            const long Pmax = la::plan_segments((long)B * H, N, C, la::kMaxTargetWg, &L);
            l.agglo = take((size_t)B * H * Pmax * ((size_t)m * d_v + m) * 4);
        }
    }
    l.inner = off;
    l.total = off + inner_bytes;
    return l;
}

// Checks of the feature-map arguments; the width the state sees in *mf.
la_status check_fm(int fm, const void *W, int m, int d_k, int *mf) {
    if (!fm_known(fm)) return LA_ERR_UNSUPPORTED;
    *mf = d_k;
    if (fm != LA_PHI_PRF) return LA_OK;
    if (!W) return LA_ERR_NULL_PTR;
    if (!prf_dim_ok(m) || !prf_dim_ok(d_k)) return LA_ERR_UNSUPPORTED;
    if (!aligned(W)) return LA_ERR_ALIGNMENT;
    *mf = m;
    return LA_OK;
}

char *at(void *ws, size_t off) { return static_cast<char *>(ws) + off; }

// The forward applies the random features inside the chunk kernels' staging
// waves (no feature tensors in HBM) for bf16 inputs with m = d_k in {32, 64},
// d_v <= 64 and 64-token chunks (the shapes of la::prf_fused_ok); other shapes
// project q and k in la_prf_kernel first.
bool prf_fused(int in, int d_k, int m, int d_v, int C) {
    return in == LA_BF16 && (d_k == 32 || d_k == 64) && m == d_k && d_v <= 64 && C == 64;
}

}  // namespace

extern "C" {

size_t la_fwd_causal_fm_workspace_bytes(int B, int H, int N, int d_k, int d_v, int C, la_feature_map fm, int m,
                                        la_dtype in) {
    int mf = 0;
    if (check_fm(fm, fm == LA_PHI_PRF ? (const void *)16 : nullptr, m, d_k, &mf) != LA_OK) return 0;
    const size_t inner = la::fwd_ws_bytes(B, H, N, mf, d_v, C, true);
    if (fm != LA_PHI_PRF) return inner;
    if (B < 1 || H < 1 || N < 1 || N > la::kMaxN || !la::dim_ok(d_v) || !la::chunk_ok(C) || !la::dtype_ok(in)) return 0;
    if (prf_fused(in, d_k, m, d_v, C)) return inner;
    return fm_layout(false, B, H, N, m, d_v, 0, in, inner).total;
}

size_t la_fwd_noncausal_fm_workspace_bytes(int B, int H, int N, int d_k, int d_v, la_feature_map fm, int m,
                                           la_dtype in) {
    int mf = 0;
    if (check_fm(fm, fm == LA_PHI_PRF ? (const void *)16 : nullptr, m, d_k, &mf) != LA_OK) return 0;
    const size_t inner = la::fwd_ws_bytes(B, H, N, mf, d_v, la::kNonCausalChunk, false);
    if (fm != LA_PHI_PRF) return inner;
    if (inner == 0 || !la::dtype_ok(in)) return 0;
    if (prf_fused(in, d_k, m, d_v, la::kNonCausalChunk)) return inner;
    return fm_layout(false, B, H, N, m, d_v, 0, in, inner).total;
}

size_t la_bwd_causal_fm_workspace_bytes(int B, int H, int N, int d_k, int d_v, int C, la_feature_map fm, int m,
                                        la_dtype in) {
    int mf = 0;
    if (check_fm(fm, fm == LA_PHI_PRF ? (const void *)16 : nullptr, m, d_k, &mf) != LA_OK) return 0;
    if (B < 1 || H < 1 || N < 1 || N > la::kMaxN || !la::dim_ok(mf) || !la::dim_ok(d_v) || !la::chunk_ok(C)) return 0;
    const size_t inner = la::bwd_workspace_bytes(B, H, N, mf, d_v, C);
    if (fm != LA_PHI_PRF) return inner;
    if (!la::dtype_ok(in)) return 0;
    return fm_layout(true, B, H, N, m, d_v, C, in, inner).total;
}

la_status la_fwd_causal_fm(const void *q, const void *k, const void *v, void *o, float *den, la_feature_map fm,
                           const void *W, int m, int B, int H, int N, int d_k, int d_v, int C, la_dtype in,
                           la_dtype out, void *ws, size_t ws_bytes, hipStream_t stream) {
    la_status st = la::check_fwd_causal_args(q, k, v, o, den, nullptr, nullptr, nullptr, nullptr, B, H, N, d_k, d_v,
                                             C, in, out);
    if (st != LA_OK) return st;
    int mf = 0;
    if ((st = check_fm(fm, W, m, d_k, &mf)) != LA_OK) return st;
    if (!aligned_or_null(ws)) return LA_ERR_ALIGNMENT;
    const size_t need = la_fwd_causal_fm_workspace_bytes(B, H, N, d_k, d_v, C, fm, m, in);
    if (need > 0 && (ws == nullptr || ws_bytes < need)) return LA_ERR_WORKSPACE;
    if (fm == LA_PHI_ELU1) return la_fwd_causal(q, k, v, o, den, B, H, N, d_k, d_v, C, in, out, ws, ws_bytes, stream);
    la::FwdDesc d{q, k, v, o, den, nullptr, nullptr, nullptr, nullptr, B, H, N, mf, d_v, C,
                  in == LA_BF16, out == LA_BF16, static_cast<float *>(ws), stream, nullptr, 0, 1};
    if (fm == LA_PHI_PRF && prf_fused(in, d_k, m, d_v, C)) {
        d.phi_id = la::kPhiPrfFused;
        d.W = W;
    } else if (fm == LA_PHI_PRF) {
        const FmLayout l = fm_layout(false, B, H, N, m, d_v, 0, in, 0);
        const long BH = (long)B * H;
        hipError_t e = la::launch_prf(in == LA_BF16, la::PRF_PHI, q, W, nullptr, nullptr, at(ws, l.fq), BH, N, H, d_k,
                                      m, stream);
        if (e == hipSuccess)
            e = la::launch_prf(in == LA_BF16, la::PRF_PHI, k, W, nullptr, nullptr, at(ws, l.fk), BH, N, H, d_k, m,
                               stream);
        if (e != hipSuccess) return la::from_hip(e);
        d.q = at(ws, l.fq);
        d.k = at(ws, l.fk);
        d.ws = reinterpret_cast<float *>(at(ws, l.inner));
    }
    return la::run_fwd(d, true);
}

la_status la_fwd_noncausal_fm(const void *q, const void *k, const void *v, void *o, la_feature_map fm,
                              const void *W, int m, int B, int H, int N, int d_k, int d_v, la_dtype in, la_dtype out,
                              void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!q || !k || !v || !o) return LA_ERR_NULL_PTR;
    la_status st = la::check_shape(B, H, N);
    if (st != LA_OK) return st;
    if (!la::dim_ok(d_k) || !la::dim_ok(d_v)) return LA_ERR_UNSUPPORTED;
    if (!la::dtype_ok(in) || !la::dtype_ok(out)) return LA_ERR_BAD_DTYPE;
    if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(o) || !aligned_or_null(ws)) return LA_ERR_ALIGNMENT;
    int mf = 0;
    if ((st = check_fm(fm, W, m, d_k, &mf)) != LA_OK) return st;
    const size_t need = la_fwd_noncausal_fm_workspace_bytes(B, H, N, d_k, d_v, fm, m, in);
    if (ws == nullptr || ws_bytes < need) return LA_ERR_WORKSPACE;
    if (fm == LA_PHI_ELU1) return la_fwd_noncausal(q, k, v, o, B, H, N, d_k, d_v, in, out, ws, ws_bytes, stream);
    la::FwdDesc d{q, k, v, o, nullptr, nullptr, nullptr, nullptr, nullptr, B, H, N, mf, d_v, la::kNonCausalChunk,
                  in == LA_BF16, out == LA_BF16, static_cast<float *>(ws), stream, nullptr, 0, 1};
    if (fm == LA_PHI_PRF && prf_fused(in, d_k, m, d_v, la::kNonCausalChunk)) {
        d.phi_id = la::kPhiPrfFused;
        d.W = W;
    } else if (fm == LA_PHI_PRF) {
        const FmLayout l = fm_layout(false, B, H, N, m, d_v, 0, in, 0);
        const long BH = (long)B * H;
        hipError_t e = la::launch_prf(in == LA_BF16, la::PRF_PHI, q, W, nullptr, nullptr, at(ws, l.fq), BH, N, H, d_k,
                                      m, stream);
        if (e == hipSuccess)
            e = la::launch_prf(in == LA_BF16, la::PRF_PHI, k, W, nullptr, nullptr, at(ws, l.fk), BH, N, H, d_k, m,
                               stream);
        if (e != hipSuccess) return la::from_hip(e);
        d.q = at(ws, l.fq);
        d.k = at(ws, l.fk);
        d.ws = reinterpret_cast<float *>(at(ws, l.inner));
    }
    return la::run_fwd(d, false);
}

la_status la_bwd_causal_fm(const void *q, const void *k, const void *v, const void *dO, void *dq, void *dk, void *dv,
                           la_feature_map fm, const void *W, int m, int B, int H, int N, int d_k, int d_v, int C,
                           la_dtype in, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!q || !k || !v || !dO || !dq || !dk || !dv) return LA_ERR_NULL_PTR;
    la_status st = la::check_shape(B, H, N);
    if (st != LA_OK) return st;
    if (!la::dim_ok(d_k) || !la::dim_ok(d_v) || !la::chunk_ok(C)) return LA_ERR_UNSUPPORTED;
    if (!la::dtype_ok(in)) return LA_ERR_BAD_DTYPE;
    if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(dO) || !aligned(dq) || !aligned(dk) ||
        !aligned(dv) || !aligned_or_null(ws))
        return LA_ERR_ALIGNMENT;
    int mf = 0;
    if ((st = check_fm(fm, W, m, d_k, &mf)) != LA_OK) return st;
    const size_t need = la_bwd_causal_fm_workspace_bytes(B, H, N, d_k, d_v, C, fm, m, in);
    if (ws == nullptr || ws_bytes < need) return LA_ERR_WORKSPACE;
    if (fm == LA_PHI_ELU1) return la_bwd_causal(q, k, v, dO, dq, dk, dv, B, H, N, d_k, d_v, C, in, ws, ws_bytes, stream);
    la::BwdDesc d{q, k, v, dO, dq, dk, dv, B, H, N, mf, d_v, C, in == LA_BF16, static_cast<float *>(ws), stream, 0, 1};
    if (fm == LA_PHI_IDENTITY) return la::from_hip(la::run_bwd(d));
    // Random features: the sweeps read the features and write dphi in fp32,
    // so that the chain rule gets it far more accurate than a bf16 rounding of
    // the features would leave it.  fp32 inputs: fp32 features and products.
    // bf16 inputs: features as a bf16 value and a bf16 remainder (two planes,
    // about 16 bits), products of such pairs (four bf16 MFMAs each) on the
    // bf16 v and dO as given, dv written in bf16, and the prefix aggregate as
    // two bf16 passes, one per plane of phi(k).
    const FmLayout l = fm_layout(true, B, H, N, m, d_v, C, in, 0);
    const long BH = (long)B * H;
    const bool bf = in == LA_BF16;
    hipError_t e = hipSuccess;
    for (int t = 0; t < 2 && e == hipSuccess; ++t) {
        void *fx = at(ws, t == 0 ? l.fq : l.fk);
        e = la::launch_prf(bf, la::PRF_PHI_F32, t == 0 ? q : k, W, nullptr, nullptr, bf ? nullptr : fx, BH, N, H,
                           d_k, m, stream, bf ? fx : nullptr);
    }
    if (e != hipSuccess) return la::from_hip(e);
    d.q = at(ws, l.fq);
    d.k = at(ws, l.fk);
    d.dq = at(ws, l.dfq);  // the sweeps return dphi(q), dphi(k) (identity map)
    d.dk = at(ws, l.dfk);
    d.in_bf16 = 0;
    if (bf) {
        d.pair_ops = 1;
        d.agg_lo = reinterpret_cast<float *>(at(ws, l.agglo));
    }
    d.ws = reinterpret_cast<float *>(at(ws, l.inner));
    if ((e = la::run_bwd(d)) != hipSuccess) return la::from_hip(e);
    const int vjp = bf ? la::PRF_VJP_U : la::PRF_VJP;  // the pair sweeps write u = dphi * phi
    e = la::launch_prf(bf, vjp, q, W, at(ws, l.fq), at(ws, l.dfq), dq, BH, N, H, d_k, m, stream);
    if (e == hipSuccess) e = la::launch_prf(bf, vjp, k, W, at(ws, l.fk), at(ws, l.dfk), dk, BH, N, H, d_k, m, stream);
    return la::from_hip(e);
}

la_status la_decode_step_fm(float *S, float *z, const void *q, const void *k, const void *v, void *o,
                            la_feature_map fm, const void *W, int m, int B, int H, int d_k, int d_v, la_dtype in,
                            hipStream_t stream) {
    if (!S || !z || !q || !k || !v || !o) return LA_ERR_NULL_PTR;
    la_status st = la::check_shape(B, H, 1);
    if (st != LA_OK) return st;
    if (!la::dim_ok(d_k) || !la::dim_ok(d_v)) return LA_ERR_UNSUPPORTED;
    if (!la::dtype_ok(in)) return LA_ERR_BAD_DTYPE;
    if (!aligned(S) || !aligned(z) || !aligned(q) || !aligned(k) || !aligned(v) || !aligned(o))
        return LA_ERR_ALIGNMENT;
    int mf = 0;
    if ((st = check_fm(fm, W, m, d_k, &mf)) != LA_OK) return st;
    la::DecodeDesc d{S, z, q, k, v, o, B, H, mf, d_v, in == LA_BF16, stream, nullptr, (int)fm,
                     fm == LA_PHI_PRF ? W : nullptr, d_k};
    return la::from_hip(la::run_decode(d));
}

}  // extern "C"
