// la_fwd_impl.hpp -- chunked forward kernels (causal and non-causal) for gfx950.
//
// One kernel template serves three modes over a segment of one (batch, head):
//   MODE_AGG    -- sum phi(K)^T V and sum phi(K) over the segment (no output);
//   MODE_CAUSAL -- the chunk loop of the causal form, starting from the state
//                  carried into the segment;
//   MODE_APPLY  -- the non-causal read-out phi(Q) S / phi(Q) z with a fixed state.
// Chunked causal form (itwiki "선형 어텐션", table "Comparison of forms", chunked
// row, and section "Implementation"): inside a chunk of C tokens the causal
// scores are a masked matrix product, between chunks the state
// S = sum phi(k) v^T, z = sum phi(k) is carried.  The sequence of one
// (batch, head) is cut into P segments of whole chunks; the states entering
// the segments come from an exclusive prefix sum of per-segment aggregates
// (the prefix sum is a scan and can be taken in parallel: blog digest
// "Theoretical significance / prefix-sum parallelism").
//
// Data path of one chunk: the workgroup loads q, k, v rows with 16-byte
// global loads one chunk ahead into registers, applies phi to q and k while
// writing the rows to LDS (row-major, 16-byte writes), and every matrix
// operand is then read from those row-major tiles -- with plain reads where
// the contraction runs over features and with the gfx950 transpose read
// (ds_read_b64_tr_b16) where it runs over tokens.
//
// Work split inside a workgroup of four waves: wave w owns value-column
// blocks cb = w, w + 4, ... (16 columns each).  Its slice S[:, cb] of the
// state lives in accumulator registers for the whole segment and is fed back
// to the matrix cores as an operand through the split K assignment (see
// la_device.hpp), so the carry never leaves the registers; the normaliser z
// is carried the same way, as phi(K)^T times an all-ones operand.  Each wave
// computes the transposed score tiles A^T = phi(K) phi(Q)^T itself and the
// transposed output O^T(cb) = V^T(cb) A^T + S(cb)^T phi(Q)^T, which puts each
// query's normaliser in the lanes that store that query's outputs.
#pragma once

#include "la_device.hpp"

namespace la {

enum { MODE_AGG = 0, MODE_CAUSAL = 1, MODE_APPLY = 2 };

constexpr int kThreads = 256;  // four waves
constexpr int kCMax = 64;      // largest chunk

struct FwdParams {
    const void *q;
    const void *k;
    const void *v;
    void *o;
    float *den;             // nullable, [BH][N]
    const float *seg_state; // per (bh, segment) entering state [DK*DV + DK], or null
    const float *S0;        // per-bh initial state, used only when seg_state is null
    const float *z0;
    float *seg_out;         // MODE_AGG: per (bh, segment) aggregates
    const float *zw;        // MODE_AGG: per-token weights [BH][N] for z (null: all ones)
    const float *kscale;    // MODE_AGG: per-token factors [BH][N] applied to phi(k) rows (null: none)
    float *S_fin;           // final state of the last segment (nullable)
    float *z_fin;
    int N, C;
    int L;                  // tokens per segment of this launch (a multiple of C)
    int state_P;            // segments per (bh) in the state array
    int state_mult;         // segment s of this launch starts at state slot s * state_mult
    int out_bf16;
};

template <int DK, int DV, typename TC> struct alignas(16) FwdSmem {
    static constexpr int DKP = DK < 32 ? 32 : DK;        // feature dim padded to a K step
    static constexpr int PAD = 16 / sizeof(TC);          // 16-byte row padding
    static constexpr int LQ = DKP + PAD;                  // row length of q, k tiles
    static constexpr int LV = DV + PAD;                   // row length of the v tile
    TC q[kCMax * LQ];    // phi(Q) rows
    TC k[kCMax * LQ];    // phi(K) rows
    TC v[kCMax * LV];    // V rows
    float w[kCMax];      // per-token z weights (MODE_AGG with zw)
    float s[kCMax];      // per-token phi(k) factors (MODE_AGG with kscale)
};

// Waves per SIMD the compiler must leave room for (registers are split
// among them): three for the d = 64 bf16 kernels, which are latency-bound.
template <int DK, int DV, typename TI> constexpr int fwd_waves_per_eu() {
    return (sizeof(TI) == 2 && DK <= 64 && DV <= 64) ? 3 : 1;
}

template <int DK, int DV, typename TI, int MODE>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(fwd_waves_per_eu<DK, DV, TI>())))
la_chunk_kernel(const FwdParams p) {
    using TC = TI;  // matrix operands keep the input precision
    using SM = FwdSmem<DK, DV, TC>;
    constexpr int VEC = Store<TI>::VEC;
    constexpr int NE = DK / 16;            // feature tiles
    constexpr int NSE = (DK + 31) / 32;    // feature K steps
    constexpr int CBT = DV / 16;           // value-column blocks in total
    constexpr int CBW = (CBT + 3) / 4;     // per wave (at most)
    constexpr int VQ = DK / VEC;           // 16-byte vectors per q/k row
    constexpr int VV = DV / VEC;           // per v row
    constexpr int NLQ = (kCMax * VQ + kThreads - 1) / kThreads;
    constexpr int NLV = (kCMax * VV + kThreads - 1) / kThreads;
    constexpr bool NEED_Q = MODE != MODE_AGG;
    constexpr bool NEED_K = MODE != MODE_APPLY;

    __shared__ SM sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;
    const int pp = lane & 15;
    const long bh = blockIdx.x;
    const int seg = blockIdx.y;
    const int C = p.C;
    const int N = p.N;
    const int row_begin = seg * p.L;
    const int row_end = min(N, row_begin + p.L);
    const int nch = (row_end - row_begin + C - 1) / C;
    const int nib = C / 16;                 // query/key row blocks per chunk
    const int nts = (C + 31) / 32;          // token K steps per chunk
    const bool has_cols = wave < CBT;       // waves without value columns only stage data

    const char *qg = static_cast<const char *>(p.q) + (bh * N) * (long)DK * sizeof(TI);
    const char *kg = static_cast<const char *>(p.k) + (bh * N) * (long)DK * sizeof(TI);
    const char *vg = static_cast<const char *>(p.v) + (bh * N) * (long)DV * sizeof(TI);

    // ---- zero the whole tile storage once: padding rows/columns stay zero ----
    {
        uint32_t *w = reinterpret_cast<uint32_t *>(&sm);
        for (int i = tid; i < (int)(sizeof(SM) / 4); i += kThreads) w[i] = 0u;
    }

    // ---- state entering this segment ----
    const float *Sin = nullptr;
    const float *zin = nullptr;
    if (MODE == MODE_APPLY || MODE == MODE_CAUSAL) {
        if (p.seg_state) {
            const long slot = (MODE == MODE_APPLY) ? bh * p.state_P : bh * p.state_P + (long)seg * p.state_mult;
            Sin = p.seg_state + slot * (long)(DK * DV + DK);
            zin = Sin + DK * DV;
        } else if (p.S0) {
            Sin = p.S0 + bh * (long)(DK * DV);
            zin = p.z0 + bh * (long)DK;
        }
    }

    // S(cb) slices and z in accumulator layout: lane (pp, g) holds rows
    // 16E + 4g + r; for z every column holds the same value.
    f32x4 accS[CBW][NE];
    f32x4 accZ[NE];
#pragma unroll
    for (int E = 0; E < NE; ++E) {
#pragma unroll
        for (int r = 0; r < 4; ++r) accZ[E][r] = zin ? zin[16 * E + 4 * g + r] : 0.0f;
#pragma unroll
        for (int cs = 0; cs < CBW; ++cs) {
            const int cb = wave + 4 * cs;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                accS[cs][E][r] = (Sin && cb < CBT) ? Sin[(16 * E + 4 * g + r) * DV + 16 * cb + pp] : 0.0f;
        }
    }

    // Operand copies of the state for the inter-chunk read (rounded to TC):
    // S(cb)^T and z as A operands over features in the split assignment (for z
    // all sixteen operand rows are the same vector).
    Frag<TC> fragS[CBW][NSE];
    Frag<TC> fragZ[NSE];
    auto refresh_state_frags = [&]() {
        const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NSE; ++s) {
#pragma unroll
            for (int cs = 0; cs < CBW; ++cs)
                acc_to_frag(fragS[cs][s], accS[cs][2 * s], (2 * s + 1 < NE) ? accS[cs][2 * s + 1] : zero4);
            acc_to_frag(fragZ[s], accZ[2 * s], (2 * s + 1 < NE) ? accZ[2 * s + 1] : zero4);
        }
    };
    if (MODE != MODE_AGG) refresh_state_frags();
    Frag<TC> ones;
    frag_ones(ones);
    bool diag_keep[4];  // causal mask on a diagonal score tile: row 4g + r <= column pp
#pragma unroll
    for (int r = 0; r < 4; ++r) diag_keep[r] = 4 * g + r <= pp;

    // ---- register prefetch of one chunk ----
    uint4 rq[NEED_Q ? NLQ : 1], rk[NEED_K ? NLQ : 1], rv[NEED_K ? NLV : 1];
    float rw = 0.f, rs = 1.f;
    const bool weighted = MODE == MODE_AGG && p.zw != nullptr;
    const bool kscaled = MODE == MODE_AGG && p.kscale != nullptr;
    auto load_chunk = [&](int r0, int nrows) {
        if (weighted) rw = tid < nrows ? p.zw[bh * N + r0 + tid] : 0.f;
        if (kscaled) rs = tid < nrows ? p.kscale[bh * N + r0 + tid] : 0.f;
        if (NEED_Q) {
#pragma unroll
            for (int i = 0; i < NLQ; ++i) {
                const int idx = tid + kThreads * i;
                const int row = idx / VQ;
                rq[i] = make_uint4(0, 0, 0, 0);
                if (row < nrows)
                    rq[i] = *reinterpret_cast<const uint4 *>(qg + ((long)(r0 + row) * DK + (idx % VQ) * VEC) * sizeof(TI));
            }
        }
        if (NEED_K) {
#pragma unroll
            for (int i = 0; i < NLQ; ++i) {
                const int idx = tid + kThreads * i;
                const int row = idx / VQ;
                rk[i] = make_uint4(0, 0, 0, 0);
                if (row < nrows)
                    rk[i] = *reinterpret_cast<const uint4 *>(kg + ((long)(r0 + row) * DK + (idx % VQ) * VEC) * sizeof(TI));
            }
#pragma unroll
            for (int i = 0; i < NLV; ++i) {
                const int idx = tid + kThreads * i;
                const int row = idx / VV;
                rv[i] = make_uint4(0, 0, 0, 0);
                if (row < nrows)
                    rv[i] = *reinterpret_cast<const uint4 *>(vg + ((long)(r0 + row) * DV + (idx % VV) * VEC) * sizeof(TI));
            }
        }
    };

    // Write the prefetched chunk into LDS, applying phi to q and k (rows at
    // or beyond nrows become zeros: they add nothing; rows beyond C are never
    // written and stay zero).  V is copied as loaded.
    auto stage_phi = [&](const uint4 *regs, int nl, int vpr, TC *tile, int ld, int nrows) {
#pragma unroll
        for (int i = 0; i < nl; ++i) {
            const int idx = tid + kThreads * i;
            const int row = idx / vpr;
            const int col = (idx % vpr) * VEC;
            if (row < C) {
                float x[VEC];
                unpack16(regs[i], x, TI());
                Frag<TC> w;  // VEC <= 8 elements, written as one 16-byte store
                if (nrows == C) {
#pragma unroll
                    for (int t = 0; t < VEC; ++t) w.set(t, phi(x[t]));
                } else {
#pragma unroll
                    for (int t = 0; t < VEC; ++t) w.set(t, row < nrows ? phi(x[t]) : 0.0f);
                }
                if constexpr (sizeof(TC) == 2) {
                    *reinterpret_cast<uint4 *>(tile + row * ld + col) = __builtin_bit_cast(uint4, w.v);
                } else {
                    f32x4 w4 = {w.get(0), w.get(1), w.get(2), w.get(3)};
                    *reinterpret_cast<f32x4 *>(tile + row * ld + col) = w4;
                }
            }
        }
    };
    auto stage_phi_scaled = [&](const uint4 *regs, int nl, int vpr, TC *tile, int ld) {
#pragma unroll
        for (int i = 0; i < nl; ++i) {
            const int idx = tid + kThreads * i;
            const int row = idx / vpr;
            const int col = (idx % vpr) * VEC;
            if (row < C) {
                float x[VEC];
                unpack16(regs[i], x, TI());
                const float f = sm.s[row];  // zero past nrows
                Frag<TC> w;
#pragma unroll
                for (int t = 0; t < VEC; ++t) w.set(t, phi(x[t]) * f);
                if constexpr (sizeof(TC) == 2) {
                    *reinterpret_cast<uint4 *>(tile + row * ld + col) = __builtin_bit_cast(uint4, w.v);
                } else {
                    f32x4 w4 = {w.get(0), w.get(1), w.get(2), w.get(3)};
                    *reinterpret_cast<f32x4 *>(tile + row * ld + col) = w4;
                }
            }
        }
    };
    auto stage_raw = [&](const uint4 *regs, int nl, int vpr, TC *tile, int ld) {
#pragma unroll
        for (int i = 0; i < nl; ++i) {
            const int idx = tid + kThreads * i;
            const int row = idx / vpr;
            if (row < C)  // rows past nrows were loaded as zeros
                *reinterpret_cast<uint4 *>(tile + row * ld + (idx % vpr) * VEC) = regs[i];
        }
    };

    if (nch > 0) load_chunk(row_begin, min(C, row_end - row_begin));

    for (int ch = 0; ch < nch; ++ch) {
        const int r0 = row_begin + ch * C;
        const int nrows = min(C, row_end - r0);
        __syncthreads();  // previous chunk's LDS reads are done (and the initial fill)
        if (NEED_Q) stage_phi(rq, NLQ, VQ, sm.q, SM::LQ, nrows);
        if (NEED_K) {
            if (kscaled) {
                if (tid < kCMax) sm.s[tid] = rs;  // rows past nrows load 0
                __syncthreads();
                stage_phi_scaled(rk, NLQ, VQ, sm.k, SM::LQ);
            } else {
                stage_phi(rk, NLQ, VQ, sm.k, SM::LQ, nrows);
            }
            if (weighted && tid < kCMax) sm.w[tid] = rw;  // rows past nrows load 0
            stage_raw(rv, NLV, VV, sm.v, SM::LV);
        }
        if (ch + 1 < nch) {
            const int r1 = r0 + C;
            load_chunk(r1, min(C, row_end - r1));
        }
        __syncthreads();  // chunk tiles ready

        if (NEED_Q && has_cols) {
            // V^T(cb) in the split assignment over tokens (A operand of the intra product)
            Frag<TC> fvt[CBW][2];
            if (MODE == MODE_CAUSAL) {
#pragma unroll
                for (int cs = 0; cs < CBW; ++cs)
#pragma unroll
                    for (int jp = 0; jp < 2; ++jp)
                        if (2 * jp < nib)
                            lds_frag_tr(fvt[cs][jp], sm.v, SM::LV, 32 * jp + 4 * g, 32 * jp + 16 + 4 * g,
                                        16 * (wave + 4 * cs), pp);
            }
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                if (I < nib) {
                    const TC *qrow = &sm.q[(16 * I + pp) * SM::LQ];
                    Frag<TC> fq[NSE];
#pragma unroll
                    for (int s = 0; s < NSE; ++s) lds_frag_split(fq[s], qrow + 32 * s, qrow + 32 * s + 16, g);
                    // den_i = phi(q_i) . z + sum_{j <= i} A_ij, both on the matrix
                    // cores: every accumulator slot of lane (i, g) ends up holding den_i.
                    f32x4 accD = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < NSE; ++s) accD = mma(fragZ[s], fq[s], accD);
                    Frag<TC> fb[2];  // A^T key-block pairs as B operands (split over tokens)
                    if (MODE == MODE_CAUSAL) {
                        f32x4 accA[4];
#pragma unroll
                        for (int J = 0; J < 4; ++J) {
                            accA[J] = f32x4{0.f, 0.f, 0.f, 0.f};
                            if (J <= I) {
#pragma unroll
                                for (int s = 0; s < NSE; ++s) {
                                    // phi(K) rows of key block J, split over features
                                    Frag<TC> fk;
                                    const TC *krow = &sm.k[(16 * J + pp) * SM::LQ + 32 * s];
                                    lds_frag_split(fk, krow, krow + 16, g);
                                    accA[J] = mma(fk, fq[s], accA[J]);
                                }
                            }
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r) accA[I][r] = diag_keep[r] ? accA[I][r] : 0.f;  // j <= i
#pragma unroll
                        for (int jp = 0; jp < 2; ++jp) {
                            if (2 * jp <= I) {
                                acc_to_frag(fb[jp], accA[2 * jp], accA[2 * jp + 1]);
                                accD = mma(ones, fb[jp], accD);
                            }
                        }
                    }
                    const float den = accD[0];
                    const int row_local = 16 * I + pp;
                    const bool valid = row_local < nrows;
                    const long grow = (long)r0 + row_local;
                    if (p.den && wave == 0 && g == 0 && valid) p.den[bh * N + grow] = den;
                    const float inv = __builtin_amdgcn_rcpf(den);
#pragma unroll
                    for (int cs = 0; cs < CBW; ++cs) {
                        const int cb = wave + 4 * cs;
                        if (cb < CBT) {
                            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                            if (MODE == MODE_CAUSAL) {
#pragma unroll
                                for (int jp = 0; jp < 2; ++jp)
                                    if (2 * jp <= I) acc = mma(fvt[cs][jp], fb[jp], acc);
                            }
#pragma unroll
                            for (int s = 0; s < NSE; ++s) acc = mma(fragS[cs][s], fq[s], acc);
                            if (valid) {
                                const long base = (bh * N + grow) * DV + 16 * cb + 4 * g;
                                if (p.out_bf16) {
                                    uint2 w;
                                    w.x = (uint32_t)f32_to_bf16_bits(acc[0] * inv) |
                                          ((uint32_t)f32_to_bf16_bits(acc[1] * inv) << 16);
                                    w.y = (uint32_t)f32_to_bf16_bits(acc[2] * inv) |
                                          ((uint32_t)f32_to_bf16_bits(acc[3] * inv) << 16);
                                    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.o) + base) = w;
                                } else {
                                    f32x4 w = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
                                    *reinterpret_cast<f32x4 *>(static_cast<float *>(p.o) + base) = w;
                                }
                            }
                        }
                    }
                }
            }
        }

        // ---- state carry: S(cb) += phi(K_c)^T V_c(cb), z += phi(K_c)^T 1 ----
        if (NEED_K && has_cols) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                if (s < nts) {
                    Frag<TC> fkt[NE];
                    // z weights over this step's tokens (straight assignment), as a
                    // value and its rounding remainder when the operands are bf16
                    Frag<TC> fw = ones, fw_lo;
                    if (weighted) {
#pragma unroll
                        for (int t = 0; t < 8; ++t) {
                            const float x = sm.w[32 * s + 8 * g + t];
                            fw.set(t, x);
                            fw_lo.set(t, x - fw.get(t));
                        }
                    }
#pragma unroll
                    for (int E = 0; E < NE; ++E) {
                        lds_frag_tr(fkt[E], sm.k, SM::LQ, 32 * s + 8 * g, 32 * s + 8 * g + 4, 16 * E, pp);
                        accZ[E] = mma(fkt[E], fw, accZ[E]);
                        if (weighted && sizeof(TC) == 2) accZ[E] = mma(fkt[E], fw_lo, accZ[E]);
                    }
#pragma unroll
                    for (int cs = 0; cs < CBW; ++cs) {
                        const int cb = wave + 4 * cs;
                        if (cb < CBT) {
                            Frag<TC> fv;
                            lds_frag_tr(fv, sm.v, SM::LV, 32 * s + 8 * g, 32 * s + 8 * g + 4, 16 * cb, pp);
#pragma unroll
                            for (int E = 0; E < NE; ++E) accS[cs][E] = mma(fkt[E], fv, accS[cs][E]);
                        }
                    }
                }
            }
            if (MODE == MODE_CAUSAL) refresh_state_frags();
        }
    }

    // ---- write the segment's resulting state ----
    float *Sdst = nullptr;
    float *zdst = nullptr;
    if (MODE == MODE_AGG) {
        Sdst = p.seg_out + (bh * p.state_P + seg) * (long)(DK * DV + DK);
        zdst = Sdst + DK * DV;
    } else if (MODE == MODE_CAUSAL && seg == (int)gridDim.y - 1 && p.S_fin) {
        Sdst = p.S_fin + bh * (long)(DK * DV);
        zdst = p.z_fin + bh * (long)DK;
    }
    if (Sdst && has_cols) {
#pragma unroll
        for (int cs = 0; cs < CBW; ++cs) {
            const int cb = wave + 4 * cs;
            if (cb < CBT) {
#pragma unroll
                for (int E = 0; E < NE; ++E)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        Sdst[(16 * E + 4 * g + r) * DV + 16 * cb + pp] = accS[cs][E][r];
            }
        }
        if (wave == 0 && pp == 0) {
#pragma unroll
            for (int E = 0; E < NE; ++E)
#pragma unroll
                for (int r = 0; r < 4; ++r) zdst[16 * E + 4 * g + r] = accZ[E][r];
        }
    }
}

}  // namespace la
