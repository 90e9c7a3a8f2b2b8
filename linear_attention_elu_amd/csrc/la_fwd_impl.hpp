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
// Work split inside a workgroup of four waves: wave w owns value-column
// blocks cb = w, w + 4, ... (16 columns each).  Its slice S[:, cb] of the
// state lives in accumulator registers for the whole segment and is fed back
// to the matrix cores as an operand through the split K assignment (see
// la_device.hpp), so the carry never leaves the registers.  Each wave
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
    float *S_fin;           // final state of the last segment (nullable)
    float *z_fin;
    int N, C, L, P;         // L = tokens per segment (a multiple of C)
    int out_bf16;
};

template <int DK, int DV, typename TC> struct alignas(16) FwdSmem {
    static constexpr int DKP = DK < 32 ? 32 : DK;        // feature dim padded to a K step
    static constexpr int PAD = 16 / sizeof(TC);          // 16-byte row padding
    static constexpr int LQ = DKP + PAD;                  // row length of sQ, sK
    static constexpr int LT = kCMax + PAD;                // row length of sKt, sVt
    TC q[kCMax * LQ];    // phi(Q) rows
    TC k[kCMax * LQ];    // phi(K) rows
    TC kt[DK * LT];      // phi(K)^T (feature-major)
    TC vt[DV * LT];      // V^T (value-column-major)
    float z[2][DKP];     // normaliser, ping-pong between chunks
};

template <int DK, int DV, typename TI, int MODE>
__global__ void __launch_bounds__(kThreads)
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

    const char *qg = static_cast<const char *>(p.q) + (bh * N) * (long)DK * sizeof(TI);
    const char *kg = static_cast<const char *>(p.k) + (bh * N) * (long)DK * sizeof(TI);
    const char *vg = static_cast<const char *>(p.v) + (bh * N) * (long)DV * sizeof(TI);

    // ---- zero the whole tile storage once: padding rows/columns stay zero ----
    {
        uint32_t *w = reinterpret_cast<uint32_t *>(&sm);
        for (int i = tid; i < (int)(sizeof(SM) / 4); i += kThreads) w[i] = 0u;
    }
    __syncthreads();

    // ---- state entering this segment ----
    const float *Sin = nullptr;
    const float *zin = nullptr;
    if (MODE == MODE_APPLY || MODE == MODE_CAUSAL) {
        if (p.seg_state) {
            const long slot = (MODE == MODE_APPLY) ? bh * p.P : bh * p.P + seg;
            Sin = p.seg_state + slot * (long)(DK * DV + DK);
            zin = Sin + DK * DV;
        } else if (p.S0) {
            Sin = p.S0 + bh * (long)(DK * DV);
            zin = p.z0 + bh * (long)DK;
        }
    }

    f32x4 accS[CBW][NE];
#pragma unroll
    for (int cs = 0; cs < CBW; ++cs)
#pragma unroll
        for (int E = 0; E < NE; ++E) {
            const int cb = wave + 4 * cs;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                accS[cs][E][r] = (Sin && cb < CBT) ? Sin[(16 * E + 4 * g + r) * DV + 16 * cb + pp] : 0.0f;
        }
    if (zin && tid < DK) sm.z[0][tid] = zin[tid];

    // Operand copy of the state for the inter-chunk read (rounded to TC).
    Frag<TC> fragS[CBW][NSE];
    auto refresh_state_frags = [&]() {
#pragma unroll
        for (int cs = 0; cs < CBW; ++cs)
#pragma unroll
            for (int s = 0; s < NSE; ++s) {
                const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
                acc_to_frag(fragS[cs][s], accS[cs][2 * s], (2 * s + 1 < NE) ? accS[cs][2 * s + 1] : zero4);
            }
    };
    refresh_state_frags();

    // ---- register prefetch of one chunk ----
    uint4 rq[NEED_Q ? NLQ : 1], rk[NEED_K ? NLQ : 1], rv[NEED_K ? NLV : 1];
    auto load_chunk = [&](int r0, int nrows) {
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
    // or beyond nrows, and beyond C, become zeros: they add nothing).
    auto stage_chunk = [&](int nrows) {
        if (NEED_Q) {
#pragma unroll
            for (int i = 0; i < NLQ; ++i) {
                const int idx = tid + kThreads * i;
                const int row = idx / VQ;
                const int col = (idx % VQ) * VEC;
                if (row < C) {
                    float x[VEC];
                    unpack16(rq[i], x, TI());
#pragma unroll
                    for (int t = 0; t < VEC; ++t) {
                        const float y = row < nrows ? to_operand<TC>(phi(x[t])) : 0.0f;
                        sm.q[row * SM::LQ + col + t] = static_cast<TC>(y);
                    }
                }
            }
        }
        if (NEED_K) {
#pragma unroll
            for (int i = 0; i < NLQ; ++i) {
                const int idx = tid + kThreads * i;
                const int row = idx / VQ;
                const int col = (idx % VQ) * VEC;
                if (row < C) {
                    float x[VEC];
                    unpack16(rk[i], x, TI());
#pragma unroll
                    for (int t = 0; t < VEC; ++t) {
                        const TC y = static_cast<TC>(row < nrows ? phi(x[t]) : 0.0f);
                        if (MODE == MODE_CAUSAL) sm.k[row * SM::LQ + col + t] = y;
                        sm.kt[(col + t) * SM::LT + row] = y;
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < NLV; ++i) {
                const int idx = tid + kThreads * i;
                const int row = idx / VV;
                const int col = (idx % VV) * VEC;
                if (row < C) {
                    float x[VEC];
                    unpack16(rv[i], x, TI());
#pragma unroll
                    for (int t = 0; t < VEC; ++t)
                        sm.vt[(col + t) * SM::LT + row] = static_cast<TC>(row < nrows ? x[t] : 0.0f);
                }
            }
        }
    };

    float zreg[2] = {0.f, 0.f};  // wave 0: running z for features lane, lane + 64
    if (wave == 0) {
        if (lane < DK) zreg[0] = zin ? zin[lane] : 0.0f;
        if (lane + 64 < DK) zreg[1] = zin ? zin[lane + 64] : 0.0f;
    }

    if (nch > 0) load_chunk(row_begin, min(C, row_end - row_begin));

    for (int ch = 0; ch < nch; ++ch) {
        const int r0 = row_begin + ch * C;
        const int nrows = min(C, row_end - r0);
        const int zc = (MODE == MODE_APPLY) ? 0 : (ch & 1);
        __syncthreads();  // previous chunk's LDS reads are done
        stage_chunk(nrows);
        if (ch + 1 < nch) {
            const int r1 = r0 + C;
            load_chunk(r1, min(C, row_end - r1));
        }
        __syncthreads();  // chunk tiles ready

        // ---- normaliser carry (wave 0): z_next = z + sum of this chunk's phi(k) ----
        if (NEED_K && wave == 0) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int e = lane + 64 * h;
                if (e < DK) {
                    float s = 0.f;
                    const TC *row = &sm.kt[e * SM::LT];
                    for (int j = 0; j < kCMax; ++j) s += static_cast<float>(row[j]);
                    zreg[h] += s;
                    sm.z[zc ^ 1][e] = zreg[h];
                }
            }
        }

        if (NEED_Q && wave < CBT) {
            const float *zcur = sm.z[zc];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                if (I < nib) {
                    const TC *qrow = &sm.q[(16 * I + pp) * SM::LQ];
                    Frag<TC> fqs[NSE], fqp[NSE];
                    float part = 0.f;
#pragma unroll
                    for (int s = 0; s < NSE; ++s) {
                        lds_frag_straight(fqs[s], qrow + 32 * s, g);
                        lds_frag_split(fqp[s], qrow + 32 * s, qrow + 32 * s + 16, g);
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            part += fqp[s].get(t) * zcur[32 * s + 4 * g + t];
                            part += fqp[s].get(t + 4) * zcur[32 * s + 16 + 4 * g + t];
                        }
                    }
                    f32x4 accA[4];
                    if (MODE == MODE_CAUSAL) {
#pragma unroll
                        for (int J = 0; J < 4; ++J) {
                            accA[J] = f32x4{0.f, 0.f, 0.f, 0.f};
                            if (J <= I) {
                                const TC *krow = &sm.k[(16 * J + pp) * SM::LQ];
#pragma unroll
                                for (int s = 0; s < NSE; ++s) {
                                    Frag<TC> fk;
                                    lds_frag_straight(fk, krow + 32 * s, g);
                                    accA[J] = mma(fk, fqs[s], accA[J]);
                                }
#pragma unroll
                                for (int r = 0; r < 4; ++r) {
                                    float a = to_operand<TC>(accA[J][r]);
                                    if (J == I && 4 * g + r > pp) a = 0.f;  // causal mask j <= i
                                    accA[J][r] = a;
                                    part += a;
                                }
                            }
                        }
                    }
                    const float den = sum_over_groups(part);
                    const int row_local = 16 * I + pp;
                    const bool valid = row_local < nrows;
                    const long grow = (long)r0 + row_local;
                    if (p.den && wave == 0 && g == 0 && valid) p.den[bh * N + grow] = den;
                    const float inv = 1.0f / den;
#pragma unroll
                    for (int cs = 0; cs < CBW; ++cs) {
                        const int cb = wave + 4 * cs;
                        if (cb < CBT) {
                            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                            if (MODE == MODE_CAUSAL) {
                                const TC *vrow = &sm.vt[(16 * cb + pp) * SM::LT];
#pragma unroll
                                for (int J0 = 0; J0 < 4; J0 += 2) {
                                    if (J0 <= I) {
                                        Frag<TC> fa, fb;
                                        lds_frag_split(fa, vrow + 16 * J0, vrow + 16 * J0 + 16, g);
                                        acc_to_frag(fb, accA[J0], accA[J0 + 1]);
                                        acc = mma(fa, fb, acc);
                                    }
                                }
                            }
#pragma unroll
                            for (int s = 0; s < NSE; ++s) acc = mma(fragS[cs][s], fqp[s], acc);
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

        // ---- state carry: S(cb) += phi(K_c)^T V_c(cb) ----
        if (NEED_K) {
#pragma unroll
            for (int cs = 0; cs < CBW; ++cs) {
                const int cb = wave + 4 * cs;
                if (cb < CBT) {
                    const TC *vrow = &sm.vt[(16 * cb + pp) * SM::LT];
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        if (s < nts) {
                            Frag<TC> fv;
                            lds_frag_straight(fv, vrow + 32 * s, g);
#pragma unroll
                            for (int E = 0; E < NE; ++E) {
                                Frag<TC> fk;
                                lds_frag_straight(fk, &sm.kt[(16 * E + pp) * SM::LT + 32 * s], g);
                                accS[cs][E] = mma(fk, fv, accS[cs][E]);
                            }
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
        Sdst = p.seg_out + (bh * p.P + seg) * (long)(DK * DV + DK);
        zdst = Sdst + DK * DV;
    } else if (MODE == MODE_CAUSAL && seg == p.P - 1 && p.S_fin) {
        Sdst = p.S_fin + bh * (long)(DK * DV);
        zdst = p.z_fin + bh * (long)DK;
    }
    if (Sdst) {
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
        if (wave == 0) {
            if (lane < DK) zdst[lane] = zreg[0];
            if (lane + 64 < DK) zdst[lane + 64] = zreg[1];
        }
    }
}

}  // namespace la
