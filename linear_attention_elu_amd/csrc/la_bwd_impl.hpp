// la_bwd_impl.hpp -- cumulative-sum backward of the causal form for gfx950.
//
// The velog review (section 3.5 "Gradient Computation") states that storing
// every prefix state S_i would cost O(N d_k d_v) memory, so the gradient is
// itself written as cumulative sums, linear in time and memory; the formulas
// are not printed.  What is computed here is the exact gradient of
// out_i = num_i / den_i.  With g_i = dO_i, gh_i = g_i / den_i and
// eps_i = -(g_i . out_i) / den_i, and M_ij = gh_i . v_j + eps_i (i >= j):
//   dphi(q_i) = sum_{j<=i} M_ij phi(k_j)              = S_i gh_i + eps_i z_i
//   dphi(k_j) = sum_{i>=j} M_ij phi(q_i)              = R_j v_j + r_j
//   dv_j      = sum_{i>=j} (phi(q_i).phi(k_j)) gh_i   = R_j^T phi(k_j)
// with the prefix sums S_i, z_i of the forward and the suffix sums
// R_j = sum_{i>=j} phi(q_i) gh_i^T, r_j = sum_{i>=j} phi(q_i) eps_i; then
// dq = dphi(q) * phi'(q), dk = dphi(k) * phi'(k), where phi'(x) = min(phi(x), 1).
//
// Chunked evaluation, as in the forward (itwiki "선형 어텐션", table
// "Comparison of forms", chunked row): inside a chunk the masked products
// M and A_ij = phi(q_i).phi(k_j) are matrix products on MFMA; between chunks
// the dq sweep carries (S, z) forward and the dk/dv sweep carries (R, r)
// backward.  The states entering each segment come from fixed-order scans
// of per-segment aggregates (exclusive prefix for S, z; exclusive suffix for
// R, r).  No per-token state is stored.
//
// The dq sweep does not take out_i or den_i from the forward: with
// X_i = S_i g_i and den_i = phi(q_i) . z_i it forms
//   dphi(q_i) = (X_i - z_i (phi(q_i) . X_i) / den_i) / den_i,
// which is the formula above (g_i . out_i = phi(q_i) . X_i / den_i) written so
// that the cancellation between its two terms happens in fp32 on one
// consistent set of values; it then leaves a_i = 1 / den_i and
// e_i = eps_i den_i = -(phi(q_i) . X_i) / den_i per token for the dk/dv sweep.
// That sweep keeps the same consistency: M_ij = (g_i . v_j + e_i) a_i in fp32,
// and the suffix state is R = sum_i (phi(q_i) a_i) g_i^T, r = sum_i (phi(q_i) a_i) e_i,
// so R v_j + r sums the same brackets g_i . v_j + e_i.
//
// Workgroups have eight waves.  In the dq sweep wave w owns the feature
// blocks eb = w, w + 8, ... of dq and its slice S[eb, :] of the state, held
// as accumulators of S^T so it feeds the matrix cores as an operand over the
// value index.  In the dk/dv sweep wave w owns the feature blocks of dk with
// R[eb, :] in accumulators, and the value blocks of dv; the dv product needs R
// contracted over features, so a bf16 copy of R is kept in LDS and read with
// the transpose read.
#pragma once

#include "la_device.hpp"

namespace la {

constexpr int kBwdThreads = 512;  // eight waves

struct BwdParams {
    const void *q, *k, *v;
    const void *g;           // dO, [BH][N][DV]
    float *inv_den;          // a = 1 / den per token, [BH][N]: written by the dq sweep
    float *eps;              // e = eps * den per token, [BH][N]: written by the dq sweep
    void *dq, *dk, *dv;
    const float *state;      // per (bh, segment) entering states [DK*DV + DK]
    int N, C;                // C: tile chunk (<= the kernel's maximum)
    int L;                   // tokens per segment of this launch
    int state_P;             // segments per bh in the state array
    int state_mult;          // fine segments per segment of this launch
};

template <typename TI, int DK, int DV> constexpr int bwd_cmax() {
    return (sizeof(TI) == 4 && (DK > 64 || DV > 64)) ? 32 : 64;
}

// Row-major tiles of one chunk in LDS (padding keeps 16-byte alignment).
template <typename TC> struct BwdTile {
    static constexpr int PAD = 16 / sizeof(TC);
};

// Stage one chunk of rows [r0, r0 + nrows) of a [N][D] tensor into a tile,
// optionally through phi or times a per-row factor.  Rows past nrows are zero.
template <typename TI, int D, int LD, int NT>
__device__ __forceinline__ void bwd_stage(const void *src, long row_base, int r0, int nrows, int C, TI *tile,
                                          int tid, int how /*0 raw, 1 phi, 3 times row_scale*/,
                                          const float *row_scale = nullptr) {
    constexpr int VEC = Store<TI>::VEC;
    constexpr int VPR = D / VEC;
    for (int idx = tid; idx < C * VPR; idx += NT) {
        const int row = idx / VPR;
        const int col = (idx % VPR) * VEC;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (row < nrows)
            u = *reinterpret_cast<const uint4 *>(static_cast<const char *>(src) +
                                                 ((row_base + r0 + row) * D + col) * (long)sizeof(TI));
        if (how == 0 || row >= nrows) {
            *reinterpret_cast<uint4 *>(tile + row * LD + col) = u;
        } else {
            float x[VEC];
            unpack16(u, x, TI());
            Frag<TI> w;
            const float sc = how == 3 ? row_scale[row] : 1.0f;
#pragma unroll
            for (int t = 0; t < VEC; ++t) w.set(t, how == 1 ? phi(x[t]) : x[t] * sc);
            if constexpr (sizeof(TI) == 2) {
                *reinterpret_cast<uint4 *>(tile + row * LD + col) = __builtin_bit_cast(uint4, w.v);
            } else {
                f32x4 w4 = {w.get(0), w.get(1), w.get(2), w.get(3)};
                *reinterpret_cast<f32x4 *>(tile + row * LD + col) = w4;
            }
        }
    }
}

template <typename TI>
__device__ __forceinline__ void store4(void *dst, long idx, const f32x4 &a) {
    if constexpr (sizeof(TI) == 2) {
        uint2 w;
        w.x = (uint32_t)f32_to_bf16_bits(a[0]) | ((uint32_t)f32_to_bf16_bits(a[1]) << 16);
        w.y = (uint32_t)f32_to_bf16_bits(a[2]) | ((uint32_t)f32_to_bf16_bits(a[3]) << 16);
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(dst) + idx) = w;
    } else {
        *reinterpret_cast<f32x4 *>(static_cast<float *>(dst) + idx) = a;
    }
}

// ---------------------------------------------------------------------------
// dq sweep (forward over chunks, state S, z).
// ---------------------------------------------------------------------------
template <int DK, int DV, typename TI> struct DqSmem {
    static constexpr int CM = bwd_cmax<TI, DK, DV>();
    static constexpr int DKP = DK < 32 ? 32 : DK;
    static constexpr int DVP = DV < 32 ? 32 : DV;
    static constexpr int LK = DKP + BwdTile<TI>::PAD;
    static constexpr int LV = DVP + BwdTile<TI>::PAD;
    TI k[CM * LK];    // phi(K)
    TI q[CM * LK];    // phi(Q)
    TI v[CM * LV];    // V
    TI g[CM * LV];    // dO
    float red[kBwdThreads / 64][64][2];  // per-wave partial phi(q).X and phi(q).z
};

template <int DK, int DV, typename TI>
__global__ void __launch_bounds__(kBwdThreads)
la_bwd_dq_kernel(const BwdParams p) {
    using TC = TI;
    using SM = DqSmem<DK, DV, TI>;
    constexpr int NW = kBwdThreads / 64;
    constexpr int EB = DK / 16, EBW = (EB + NW - 1) / NW;
    constexpr int NWA = EB < NW ? EB : NW;     // waves holding feature blocks
    constexpr int CV = DV / 16;                // value tiles of the state
    constexpr int NSV = (DV + 31) / 32;        // value K steps
    __shared__ alignas(16) SM sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, pp = lane & 15;
    const long bh = blockIdx.x;
    const int seg = blockIdx.y;
    const int C = p.C, N = p.N;
    const int row_begin = seg * p.L;
    const int row_end = min(N, row_begin + p.L);
    const int nch = (row_end - row_begin + C - 1) / C;
    const int nib = C / 16, nts = (C + 31) / 32;
    const bool active = wave < EB;

    {
        uint32_t *w = reinterpret_cast<uint32_t *>(&sm);
        for (int i = tid; i < (int)(sizeof(SM) / 4); i += kBwdThreads) w[i] = 0u;
    }

    const float *Sin = p.state ? p.state + (bh * p.state_P + (long)seg * p.state_mult) * (long)(DK * DV + DK) : nullptr;
    const float *zin = Sin ? Sin + DK * DV : nullptr;
    // S^T(c', eb) tiles: lane (pp, g) holds S[16 eb + pp][16 c' + 4g + r]; z(eb): z[16 eb + 4g + r].
    f32x4 accS[CV][EBW];
    f32x4 accZ[EBW];
#pragma unroll
    for (int es = 0; es < EBW; ++es) {
        const int eb = wave + NW * es;
#pragma unroll
        for (int r = 0; r < 4; ++r) accZ[es][r] = (zin && eb < EB) ? zin[16 * eb + 4 * g + r] : 0.f;
#pragma unroll
        for (int cv = 0; cv < CV; ++cv)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                accS[cv][es][r] = (Sin && eb < EB) ? Sin[(16 * eb + pp) * DV + 16 * cv + 4 * g + r] : 0.f;
    }
    Frag<TC> fragS[EBW][NSV];  // S rows e, split over the value index
    auto refresh = [&]() {
        const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int es = 0; es < EBW; ++es)
#pragma unroll
            for (int s = 0; s < NSV; ++s)
                acc_to_frag(fragS[es][s], accS[2 * s][es], (2 * s + 1 < CV) ? accS[2 * s + 1][es] : zero4);
    };
    refresh();
    Frag<TC> ones;
    frag_ones(ones);

    for (int ch = 0; ch < nch; ++ch) {
        const int r0 = row_begin + ch * C;
        const int nrows = min(C, row_end - r0);
        __syncthreads();
        bwd_stage<TI, DK, SM::LK, kBwdThreads>(p.k, bh * N, r0, nrows, C, sm.k, tid, 1);
        bwd_stage<TI, DK, SM::LK, kBwdThreads>(p.q, bh * N, r0, nrows, C, sm.q, tid, 1);
        bwd_stage<TI, DV, SM::LV, kBwdThreads>(p.v, bh * N, r0, nrows, C, sm.v, tid, 0);
        bwd_stage<TI, DV, SM::LV, kBwdThreads>(p.g, bh * N, r0, nrows, C, sm.g, tid, 0);
        __syncthreads();

        // X(eb, I) = sum_{j<=i} (v_j . g_i) phi(k_j) + S g_i and Z(eb, I) = z_i,
        // both with rows e = 16 eb + 4g + r of query column i = 16 I + pp.
        f32x4 X[4][EBW], Z[4][EBW];
        if (active) {
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                if (I < nib) {
                    Frag<TC> fg[NSV];
                    const TC *grow = &sm.g[(16 * I + pp) * SM::LV];
#pragma unroll
                    for (int s = 0; s < NSV; ++s) lds_frag_split(fg[s], grow + 32 * s, grow + 32 * s + 16, g);
                    f32x4 accM[4];
#pragma unroll
                    for (int J = 0; J < 4; ++J) {
                        accM[J] = f32x4{0.f, 0.f, 0.f, 0.f};
                        if (J <= I) {
                            const TC *vrow = &sm.v[(16 * J + pp) * SM::LV];
#pragma unroll
                            for (int s = 0; s < NSV; ++s) {
                                Frag<TC> fv;
                                lds_frag_split(fv, vrow + 32 * s, vrow + 32 * s + 16, g);
                                accM[J] = mma(fv, fg[s], accM[J]);
                            }
                            if (J == I) {
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    if (4 * g + r > pp) accM[J][r] = 0.f;  // j <= i
                            }
                        }
                    }
                    // masked scores as operand value + remainder, and the causal
                    // all-ones mask over the same tokens
                    Frag<TC> fb[2], fbl[2], ftr[2];
#pragma unroll
                    for (int jp = 0; jp < 2; ++jp) {
                        if (2 * jp <= I) {
                            acc_to_frag(fb[jp], accM[2 * jp], accM[2 * jp + 1]);
#pragma unroll
                            for (int t = 0; t < 4; ++t) {
                                fbl[jp].set(t, accM[2 * jp][t] - fb[jp].get(t));
                                fbl[jp].set(t + 4, accM[2 * jp + 1][t] - fb[jp].get(t + 4));
                                const int j0 = 32 * jp + 4 * g + t, j1 = j0 + 16, i = 16 * I + pp;
                                ftr[jp].set(t, j0 <= i ? 1.f : 0.f);
                                ftr[jp].set(t + 4, j1 <= i ? 1.f : 0.f);
                            }
                        }
                    }
                    float px = 0.f, pz = 0.f;
                    const TC *qrow = &sm.q[(16 * I + pp) * SM::LK];
#pragma unroll
                    for (int es = 0; es < EBW; ++es) {
                        const int eb = wave + NW * es;
                        f32x4 ax = {0.f, 0.f, 0.f, 0.f};
                        f32x4 az = accZ[es];
                        if (eb < EB) {
#pragma unroll
                            for (int jp = 0; jp < 2; ++jp) {
                                if (2 * jp <= I) {
                                    Frag<TC> fkt;
                                    lds_frag_tr(fkt, sm.k, SM::LK, 32 * jp + 4 * g, 32 * jp + 16 + 4 * g, 16 * eb, pp);
                                    ax = mma(fkt, fb[jp], ax);
                                    if (sizeof(TC) == 2) ax = mma(fkt, fbl[jp], ax);
                                    az = mma(fkt, ftr[jp], az);
                                }
                            }
#pragma unroll
                            for (int s = 0; s < NSV; ++s) ax = mma(fragS[es][s], fg[s], ax);
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const float fq = static_cast<float>(qrow[16 * eb + 4 * g + r]);
                                px += fq * ax[r];
                                pz += fq * az[r];
                            }
                        }
                        X[I][es] = ax;
                        Z[I][es] = az;
                    }
                    px = sum_over_groups(px);
                    pz = sum_over_groups(pz);
                    if (g == 0) {
                        sm.red[wave][16 * I + pp][0] = px;
                        sm.red[wave][16 * I + pp][1] = pz;
                    }
                }
            }
        }
        __syncthreads();  // partial dot products of every wave are in LDS
        if (active) {
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                if (I < nib) {
                    const int row_local = 16 * I + pp;
                    float t = 0.f, den = 0.f;
#pragma unroll
                    for (int w = 0; w < NWA; ++w) {
                        t += sm.red[w][row_local][0];
                        den += sm.red[w][row_local][1];
                    }
                    const float inv = 1.0f / den;
                    const float coef = t * inv;
                    const bool valid = row_local < nrows;
                    const long orow = bh * N + r0 + row_local;
                    if (wave == 0 && g == 0 && valid) {
                        p.inv_den[orow] = inv;
                        p.eps[orow] = -coef;
                    }
                    const TC *qrow = &sm.q[row_local * SM::LK];
#pragma unroll
                    for (int es = 0; es < EBW; ++es) {
                        const int eb = wave + NW * es;
                        if (eb < EB) {
                            f32x4 out;
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const float dphi_q = fminf(static_cast<float>(qrow[16 * eb + 4 * g + r]), 1.0f);
                                out[r] = (X[I][es][r] - Z[I][es][r] * coef) * inv * dphi_q;
                            }
                            if (valid) store4<TI>(p.dq, orow * DK + 16 * eb + 4 * g, out);
                        }
                    }
                }
            }
            // state carry: S^T(c', eb) += V^T(c') phi(K)(eb), z(eb) += phi(K)(eb)^T 1
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                if (s < nts) {
                    Frag<TC> fk[EBW];
#pragma unroll
                    for (int es = 0; es < EBW; ++es) {
                        const int eb = wave + NW * es;
                        if (eb < EB) {
                            lds_frag_tr(fk[es], sm.k, SM::LK, 32 * s + 8 * g, 32 * s + 8 * g + 4, 16 * eb, pp);
                            accZ[es] = mma(fk[es], ones, accZ[es]);
                        }
                    }
#pragma unroll
                    for (int cv = 0; cv < CV; ++cv) {
                        Frag<TC> fvt;
                        lds_frag_tr(fvt, sm.v, SM::LV, 32 * s + 8 * g, 32 * s + 8 * g + 4, 16 * cv, pp);
#pragma unroll
                        for (int es = 0; es < EBW; ++es)
                            if (wave + NW * es < EB) accS[cv][es] = mma(fvt, fk[es], accS[cv][es]);
                    }
                }
            }
            refresh();
        }
    }
}

// ---------------------------------------------------------------------------
// dk / dv sweep (backward over chunks, state R, r).
// ---------------------------------------------------------------------------
template <int DK, int DV, typename TI> struct DkvSmem {
    static constexpr int CM = bwd_cmax<TI, DK, DV>();
    static constexpr int DKP = DK < 32 ? 32 : DK;
    static constexpr int DVP = DV < 32 ? 32 : DV;
    static constexpr int LK = DKP + BwdTile<TI>::PAD;
    static constexpr int LV = DVP + BwdTile<TI>::PAD;
    static constexpr int LR = DV + BwdTile<TI>::PAD;
    static constexpr int RROWS = DKP;
    TI q[CM * LK];     // phi(Q)
    TI k[CM * LK];     // phi(K)
    TI v[CM * LV];     // V
    TI g[CM * LV];     // dO
    TI R[RROWS * LR];  // copy of the suffix state R[e][c'] for the dv product
    float e[64];       // e = eps * den
    float a[64];       // a = 1 / den
};

template <int DK, int DV, typename TI>
__global__ void __launch_bounds__(kBwdThreads)
la_bwd_dkdv_kernel(const BwdParams p) {
    using TC = TI;
    using SM = DkvSmem<DK, DV, TI>;
    constexpr int NW = kBwdThreads / 64;
    constexpr int EB = DK / 16, EBW = (EB + NW - 1) / NW;
    constexpr int CB = DV / 16, CBW = (CB + NW - 1) / NW;
    constexpr int CV = DV / 16;
    constexpr int NSV = (DV + 31) / 32;
    constexpr int NSE = (DK + 31) / 32;
    __shared__ alignas(16) SM sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, pp = lane & 15;
    const long bh = blockIdx.x;
    const int seg = blockIdx.y;
    const int C = p.C, N = p.N;
    const int row_begin = seg * p.L;
    const int row_end = min(N, row_begin + p.L);
    const int nch = (row_end - row_begin + C - 1) / C;
    const int nib = C / 16, nts = (C + 31) / 32;

    {
        uint32_t *w = reinterpret_cast<uint32_t *>(&sm);
        for (int i = tid; i < (int)(sizeof(SM) / 4); i += kBwdThreads) w[i] = 0u;
    }
    __syncthreads();

    // Suffix state after this segment: the exclusive suffix of its last fine segment.
    const float *Rin = nullptr;
    if (p.state) {
        const long last = min((long)(seg + 1) * p.state_mult, (long)p.state_P) - 1;
        Rin = p.state + (bh * p.state_P + last) * (long)(DK * DV + DK);
    }
    const float *rin = Rin ? Rin + DK * DV : nullptr;
    // R^T(c', eb) tiles: lane (pp, g) holds R[16 eb + pp][16 c' + 4g + r]; r(eb): r[16 eb + 4g + r].
    f32x4 accR[CV][EBW];
    f32x4 accr[EBW];
#pragma unroll
    for (int es = 0; es < EBW; ++es) {
        const int eb = wave + NW * es;
#pragma unroll
        for (int r = 0; r < 4; ++r) accr[es][r] = (rin && eb < EB) ? rin[16 * eb + 4 * g + r] : 0.f;
#pragma unroll
        for (int cv = 0; cv < CV; ++cv)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                accR[cv][es][r] = (Rin && eb < EB) ? Rin[(16 * eb + pp) * DV + 16 * cv + 4 * g + r] : 0.f;
    }
    Frag<TC> fragR[EBW][NSV];  // R rows e, split over the value index
    auto refresh = [&]() {
        const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int es = 0; es < EBW; ++es) {
            const int eb = wave + NW * es;
#pragma unroll
            for (int s = 0; s < NSV; ++s)
                acc_to_frag(fragR[es][s], accR[2 * s][es], (2 * s + 1 < CV) ? accR[2 * s + 1][es] : zero4);
            if (eb < EB) {
                // bf16 / fp32 copy of R rows 16 eb + pp into LDS (row-major [e][c'])
#pragma unroll
                for (int cv = 0; cv < CV; ++cv) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sm.R[(16 * eb + pp) * SM::LR + 16 * cv + 4 * g + r] = static_cast<TC>(accR[cv][es][r]);
                }
            }
        }
    };
    refresh();
    Frag<TC> ones;
    frag_ones(ones);

    for (int ch = nch - 1; ch >= 0; --ch) {
        const int r0 = row_begin + ch * C;
        const int nrows = min(C, row_end - r0);
        __syncthreads();  // previous chunk's tile reads done; R copy written
        bwd_stage<TI, DK, SM::LK, kBwdThreads>(p.q, bh * N, r0, nrows, C, sm.q, tid, 1);
        bwd_stage<TI, DK, SM::LK, kBwdThreads>(p.k, bh * N, r0, nrows, C, sm.k, tid, 1);
        bwd_stage<TI, DV, SM::LV, kBwdThreads>(p.v, bh * N, r0, nrows, C, sm.v, tid, 0);
        bwd_stage<TI, DV, SM::LV, kBwdThreads>(p.g, bh * N, r0, nrows, C, sm.g, tid, 0);
        if (tid < 64) {
            sm.e[tid] = tid < nrows ? p.eps[bh * N + r0 + tid] : 0.f;
            sm.a[tid] = tid < nrows ? p.inv_den[bh * N + r0 + tid] : 0.f;
        }
        __syncthreads();

        const bool has_e = wave < EB, has_c = wave < CB;
        if (has_e || has_c) {
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                if (J < nib) {
                    Frag<TC> fvj[NSV], fkj[NSE];
                    const TC *vrow = &sm.v[(16 * J + pp) * SM::LV];
                    const TC *krow = &sm.k[(16 * J + pp) * SM::LK];
#pragma unroll
                    for (int s = 0; s < NSV; ++s) lds_frag_split(fvj[s], vrow + 32 * s, vrow + 32 * s + 16, g);
#pragma unroll
                    for (int s = 0; s < NSE; ++s) lds_frag_split(fkj[s], krow + 32 * s, krow + 32 * s + 16, g);
                    f32x4 accM[4], accA[4];
#pragma unroll
                    for (int I = 0; I < 4; ++I) {
                        accM[I] = f32x4{0.f, 0.f, 0.f, 0.f};
                        accA[I] = f32x4{0.f, 0.f, 0.f, 0.f};
                        if (I >= J && I < nib) {
                            const TC *grow = &sm.g[(16 * I + pp) * SM::LV];
                            const TC *qrow = &sm.q[(16 * I + pp) * SM::LK];
                            if (has_e) {
#pragma unroll
                                for (int s = 0; s < NSV; ++s) {
                                    Frag<TC> fg;
                                    lds_frag_split(fg, grow + 32 * s, grow + 32 * s + 16, g);
                                    accM[I] = mma(fg, fvj[s], accM[I]);
                                }
                            }
                            if (has_c) {
#pragma unroll
                                for (int s = 0; s < NSE; ++s) {
                                    Frag<TC> fq;
                                    lds_frag_split(fq, qrow + 32 * s, qrow + 32 * s + 16, g);
                                    accA[I] = mma(fq, fkj[s], accA[I]);
                                }
                            }
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const bool keep = !(I == J && 4 * g + r < pp);  // i >= j
                                const int i = 16 * I + 4 * g + r;
                                const float a = sm.a[i];
                                accM[I][r] = keep ? (accM[I][r] + sm.e[i]) * a : 0.f;
                                accA[I][r] = keep ? accA[I][r] * a : 0.f;
                            }
                        }
                    }
                    const int row_local = 16 * J + pp;
                    const bool valid = row_local < nrows;
                    const long orow = bh * N + r0 + row_local;
                    if (has_e) {
                        Frag<TC> fb[2], fbl[2];  // M as operand value + remainder
#pragma unroll
                        for (int ip = 0; ip < 2; ++ip) {
                            if (2 * ip + 1 >= J) {
                                acc_to_frag(fb[ip], accM[2 * ip], accM[2 * ip + 1]);
#pragma unroll
                                for (int t = 0; t < 4; ++t) {
                                    fbl[ip].set(t, accM[2 * ip][t] - fb[ip].get(t));
                                    fbl[ip].set(t + 4, accM[2 * ip + 1][t] - fb[ip].get(t + 4));
                                }
                            }
                        }
#pragma unroll
                        for (int es = 0; es < EBW; ++es) {
                            const int eb = wave + NW * es;
                            if (eb < EB) {
                                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                                for (int ip = 0; ip < 2; ++ip) {
                                    if (2 * ip + 1 >= J && 2 * ip < nib) {
                                        Frag<TC> fqt;
                                        lds_frag_tr(fqt, sm.q, SM::LK, 32 * ip + 4 * g, 32 * ip + 16 + 4 * g, 16 * eb, pp);
                                        acc = mma(fqt, fb[ip], acc);
                                        if (sizeof(TC) == 2) acc = mma(fqt, fbl[ip], acc);
                                    }
                                }
#pragma unroll
                                for (int s = 0; s < NSV; ++s) acc = mma(fragR[es][s], fvj[s], acc);
                                const TC *kd = &sm.k[row_local * SM::LK + 16 * eb + 4 * g];
                                f32x4 out;
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    out[r] = (acc[r] + accr[es][r]) * fminf(static_cast<float>(kd[r]), 1.0f);
                                if (valid) store4<TI>(p.dk, orow * DK + 16 * eb + 4 * g, out);
                            }
                        }
                    }
                    if (has_c) {
                        Frag<TC> fb[2];
#pragma unroll
                        for (int ip = 0; ip < 2; ++ip)
                            if (2 * ip + 1 >= J) acc_to_frag(fb[ip], accA[2 * ip], accA[2 * ip + 1]);
#pragma unroll
                        for (int cs = 0; cs < CBW; ++cs) {
                            const int cb = wave + NW * cs;
                            if (cb < CB) {
                                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                                for (int ip = 0; ip < 2; ++ip) {
                                    if (2 * ip + 1 >= J && 2 * ip < nib) {
                                        Frag<TC> fgt;
                                        lds_frag_tr(fgt, sm.g, SM::LV, 32 * ip + 4 * g, 32 * ip + 16 + 4 * g, 16 * cb, pp);
                                        acc = mma(fgt, fb[ip], acc);
                                    }
                                }
#pragma unroll
                                for (int s = 0; s < NSE; ++s) {
                                    Frag<TC> frt;  // R^T rows c', split over features
                                    lds_frag_tr(frt, sm.R, SM::LR, 32 * s + 4 * g, 32 * s + 16 + 4 * g, 16 * cb, pp);
                                    acc = mma(frt, fkj[s], acc);
                                }
                                if (valid) store4<TI>(p.dv, orow * DV + 16 * cb + 4 * g, acc);
                            }
                        }
                    }
                }
            }
        }
        __syncthreads();  // every wave is done reading the R copy
        if (has_e) {
            // state carry: R^T(c', eb) += g^T(c') (a phi(Q))(eb), r(eb) += (a phi(Q))(eb)^T e
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                if (s < nts) {
                    // e as a pair of operands (value and rounding remainder) so that
                    // r keeps fp32-level accuracy with bf16 operands
                    Frag<TC> fq[EBW], fe, fe_lo;
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const float e = sm.e[32 * s + 8 * g + t];
                        fe.set(t, e);
                        fe_lo.set(t, e - fe.get(t));
                    }
#pragma unroll
                    for (int es = 0; es < EBW; ++es) {
                        const int eb = wave + NW * es;
                        if (eb < EB) {
                            lds_frag_tr(fq[es], sm.q, SM::LK, 32 * s + 8 * g, 32 * s + 8 * g + 4, 16 * eb, pp);
#pragma unroll
                            for (int t = 0; t < 8; ++t)  // slot t holds token 32s + 8g + t
                                fq[es].set(t, fq[es].get(t) * sm.a[32 * s + 8 * g + t]);
                            accr[es] = mma(fq[es], fe, accr[es]);
                            if (sizeof(TC) == 2) accr[es] = mma(fq[es], fe_lo, accr[es]);
                        }
                    }
#pragma unroll
                    for (int cv = 0; cv < CV; ++cv) {
                        Frag<TC> fgt;
                        lds_frag_tr(fgt, sm.g, SM::LV, 32 * s + 8 * g, 32 * s + 8 * g + 4, 16 * cv, pp);
#pragma unroll
                        for (int es = 0; es < EBW; ++es)
                            if (wave + NW * es < EB) accR[cv][es] = mma(fgt, fq[es], accR[cv][es]);
                    }
                }
            }
            refresh();
        }
    }
}

}  // namespace la
