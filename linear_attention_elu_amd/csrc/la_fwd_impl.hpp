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
// global loads into registers ahead of use, applies phi to q and k while
// writing the rows to LDS (row-major, 16-byte writes), and every matrix
// operand is then read from those row-major tiles -- with plain reads where
// the contraction runs over features and with the gfx950 transpose read
// (ds_read_b64_tr_b16) where it runs over tokens.  When two sets of tiles fit
// in LDS they are double buffered: one step writes chunk c + 1 into one
// buffer while it computes chunk c from the other, with a single barrier per
// chunk, so the vector work of staging overlaps the matrix and LDS work.
// The chunks of a segment whose rows are all valid run in a loop of their
// own (unrolled by two, so buffer offsets are immediates), addressed from a
// uniform per-chunk base plus fixed per-lane offsets, without row masks; the
// last one or two chunks run a general loop with clamped loads and masks.
// The chunk size is a template parameter, so every tile loop is unrolled.
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

#include <type_traits>

#include "la_device.hpp"

namespace la {

enum { MODE_AGG = 0, MODE_CAUSAL = 1, MODE_APPLY = 2 };

constexpr int kThreads = 256;  // four waves

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
    int N;
    int L;                  // tokens per segment of this launch (a multiple of the chunk size)
    int state_P;            // segments per (bh) in the state array
    int state_mult;         // segment s of this launch starts at state slot s * state_mult
    int out_bf16;
};

// LDS layout for one chunk of CT tokens held as TC; only the tiles a mode
// reads are allocated.  Byte offsets inside one buffer: q, k, v, then the
// per-token z weights.
template <int DK, int DV, typename TC, int CT, int MODE> struct FwdTiles {
    static constexpr int DKP = DK < 32 ? 32 : DK;        // feature dim padded to a K step
    static constexpr int PAD = 16 / sizeof(TC);          // 16-byte row padding
    static constexpr int LQ = DKP + PAD;                  // row length of q, k tiles
    static constexpr int LV = DV + PAD;                   // row length of the v tile
    static constexpr int ROWS = CT < 32 ? 32 : CT;        // chunk rows padded to a token K step
    static constexpr int QB = MODE != MODE_AGG ? ROWS * LQ * (int)sizeof(TC) : 0;
    static constexpr int KB = MODE != MODE_APPLY ? ROWS * LQ * (int)sizeof(TC) : 0;
    static constexpr int VB = MODE != MODE_APPLY ? ROWS * LV * (int)sizeof(TC) : 0;
    static constexpr int WB = MODE == MODE_AGG ? ROWS * 4 : 0;
    static constexpr int OFF_Q = 0, OFF_K = QB, OFF_V = QB + KB, OFF_W = QB + KB + VB;
    static constexpr int BUF = QB + KB + VB + WB;          // bytes per buffer (multiple of 16)
    static constexpr int NBUF = 2 * BUF <= 64 * 1024 ? 2 : 1;  // double buffer when it stays small
    static constexpr int LDS_WG = (160 * 1024) / (NBUF * BUF);  // workgroups per CU that LDS allows
};

// Waves per SIMD the compiler must leave room for (registers are split among
// them) in the d <= 64 bf16 kernels: as many workgroups as LDS admits, capped
// where the causal chunk loop needs more registers than that would leave
// (two waves for 64-token chunks, three for smaller ones); one otherwise.
template <int DK, int DV, typename TI, int CT, int MODE> constexpr int fwd_waves_per_eu() {
    constexpr int lds = FwdTiles<DK, DV, TI, CT, MODE>::LDS_WG;
    constexpr int cap = MODE == MODE_CAUSAL ? (CT == 64 ? 2 : 3) : 4;
    return (sizeof(TI) == 2 && DK <= 64 && DV <= 64) ? (lds < 1 ? 1 : lds > cap ? cap : lds) : 1;
}

#define LA_INLINE __attribute__((always_inline))

template <int DK, int DV, typename TI, int MODE, int CT>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(fwd_waves_per_eu<DK, DV, TI, CT, MODE>())))
la_chunk_kernel(const FwdParams p) {
    using TC = TI;  // matrix operands keep the input precision
    using T = FwdTiles<DK, DV, TC, CT, MODE>;
    constexpr int NBUF = T::NBUF;
    constexpr int VEC = Store<TI>::VEC;
    constexpr int NE = DK / 16;            // feature tiles
    constexpr int NSE = (DK + 31) / 32;    // feature K steps
    constexpr int CBT = DV / 16;           // value-column blocks in total
    constexpr int CBW = (CBT + 3) / 4;     // per wave (at most)
    constexpr int NB = CT / 16;            // query/key row blocks per chunk
    constexpr int NP = (NB + 1) / 2;       // pairs of row blocks (token K steps)
    constexpr int VQ = DK / VEC;           // 16-byte vectors per q/k row
    constexpr int VV = DV / VEC;           // per v row
    constexpr int NLQ = (CT * VQ + kThreads - 1) / kThreads;
    constexpr int NLV = (CT * VV + kThreads - 1) / kThreads;
    constexpr int RSQ = kThreads / VQ;     // rows between a thread's q/k vectors
    constexpr int RSV = kThreads / VV;
    constexpr bool NEED_Q = MODE != MODE_AGG;
    constexpr bool NEED_K = MODE != MODE_APPLY;
    constexpr int NKS = MODE == MODE_AGG ? NLQ : 1;  // per-vector phi(k) factors

    __shared__ __attribute__((aligned(16))) char smem[NBUF * T::BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;
    const int pp = lane & 15;
    const long bh = blockIdx.x;
    const int seg = blockIdx.y;
    const int N = p.N;
    const int row_begin = seg * p.L;
    const int row_end = min(N, row_begin + p.L);
    const int nch = (row_end - row_begin + CT - 1) / CT;
    const int nfull = (row_end - row_begin) / CT;   // chunks with all CT rows valid
    const bool has_cols = wave < CBT;               // waves without value columns only stage data
    const bool weighted = MODE == MODE_AGG && p.zw != nullptr;
    const bool kscaled = MODE == MODE_AGG && p.kscale != nullptr;

    // Segment bases (uniform); chunk c starts CT rows further per chunk.
    const long seg_row0 = bh * N + row_begin;
    const char *qs = static_cast<const char *>(p.q) + seg_row0 * DK * (long)sizeof(TI);
    const char *ks = static_cast<const char *>(p.k) + seg_row0 * DK * (long)sizeof(TI);
    const char *vs = static_cast<const char *>(p.v) + seg_row0 * DV * (long)sizeof(TI);

    // Per-lane offsets of this thread's first staged vector (row, column).
    const int rq0 = tid / VQ, cq0 = (tid % VQ) * VEC;
    const int rv0 = tid / VV, cv0 = (tid % VV) * VEC;
    const unsigned gq0 = (unsigned)(rq0 * DK + cq0) * sizeof(TI);
    const unsigned gv0 = (unsigned)(rv0 * DV + cv0) * sizeof(TI);
    const int lq0 = (rq0 * T::LQ + cq0) * (int)sizeof(TC);
    const int lv0 = (rv0 * T::LV + cv0) * (int)sizeof(TC);

    // ---- zero the tile storage once: padding rows and columns stay zero ----
    for (int i = tid; i < NBUF * T::BUF / 16; i += kThreads)
        reinterpret_cast<uint4 *>(smem)[i] = make_uint4(0u, 0u, 0u, 0u);

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
    auto refresh_state_frags = [&]() LA_INLINE {
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
    // causal mask on a diagonal score tile: row 4g + r <= column pp
    bool diag_keep[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) diag_keep[r] = 4 * g + r <= pp;

    // ---- register prefetch of one chunk ----
    uint4 rq[NEED_Q ? NLQ : 1], rk[NEED_K ? NLQ : 1], rv[NEED_K ? NLV : 1];
    float rw = 0.f;
    float rks[NKS];
    // Full chunk c: every row is valid; uniform base plus fixed lane offsets.
    auto load_full = [&](int c) LA_INLINE {
        const long r0 = (long)c * CT;
        if (weighted) rw = tid < CT ? p.zw[seg_row0 + r0 + tid] : 0.f;
        if (kscaled) {
#pragma unroll
            for (int i = 0; i < NKS; ++i) rks[i] = p.kscale[seg_row0 + r0 + min(rq0 + i * RSQ, CT - 1)];
        }
        const char *qc = qs + r0 * DK * (long)sizeof(TI);
        const char *kc = ks + r0 * DK * (long)sizeof(TI);
        const char *vc = vs + r0 * DV * (long)sizeof(TI);
        // A thread's vectors past the chunk (only when CT * VQ is not a
        // multiple of the block) re-read the chunk's last row.
        if (NEED_Q) {
#pragma unroll
            for (int i = 0; i < NLQ; ++i) {
                const unsigned off = (CT * VQ) % kThreads != 0 && i == NLQ - 1
                                         ? (unsigned)((min(rq0 + i * RSQ, CT - 1) * DK + cq0) * sizeof(TI))
                                         : gq0 + (unsigned)(i * RSQ * DK * sizeof(TI));
                rq[i] = *reinterpret_cast<const uint4 *>(qc + off);
            }
        }
        if (NEED_K) {
#pragma unroll
            for (int i = 0; i < NLQ; ++i) {
                const unsigned off = (CT * VQ) % kThreads != 0 && i == NLQ - 1
                                         ? (unsigned)((min(rq0 + i * RSQ, CT - 1) * DK + cq0) * sizeof(TI))
                                         : gq0 + (unsigned)(i * RSQ * DK * sizeof(TI));
                rk[i] = *reinterpret_cast<const uint4 *>(kc + off);
            }
#pragma unroll
            for (int i = 0; i < NLV; ++i) {
                const unsigned off = (CT * VV) % kThreads != 0 && i == NLV - 1
                                         ? (unsigned)((min(rv0 + i * RSV, CT - 1) * DV + cv0) * sizeof(TI))
                                         : gv0 + (unsigned)(i * RSV * DV * sizeof(TI));
                rv[i] = *reinterpret_cast<const uint4 *>(vc + off);
            }
        }
    };
    // Any chunk c: rows clamped to the segment's last row (the duplicates
    // are replaced by zeros when staged).
    auto load_any = [&](int c) LA_INLINE {
        const int r0 = c * CT;
        const int last = row_end - row_begin - 1;  // segment-relative
        if (r0 + CT - 1 <= last) {
            load_full(c);
            return;
        }
        if (weighted) rw = (tid < CT && r0 + tid <= last) ? p.zw[seg_row0 + r0 + tid] : 0.f;
        if (kscaled) {
#pragma unroll
            for (int i = 0; i < NKS; ++i) rks[i] = p.kscale[seg_row0 + min(r0 + rq0 + i * RSQ, last)];
        }
        if (NEED_Q) {
#pragma unroll
            for (int i = 0; i < NLQ; ++i) {
                const long row = min(r0 + rq0 + i * RSQ, last);
                rq[i] = *reinterpret_cast<const uint4 *>(qs + (row * DK + cq0) * (long)sizeof(TI));
            }
        }
        if (NEED_K) {
#pragma unroll
            for (int i = 0; i < NLQ; ++i) {
                const long row = min(r0 + rq0 + i * RSQ, last);
                rk[i] = *reinterpret_cast<const uint4 *>(ks + (row * DK + cq0) * (long)sizeof(TI));
            }
#pragma unroll
            for (int i = 0; i < NLV; ++i) {
                const long row = min(r0 + rv0 + i * RSV, last);
                rv[i] = *reinterpret_cast<const uint4 *>(vs + (row * DV + cv0) * (long)sizeof(TI));
            }
        }
    };

    // phi (times a factor) of a 16-byte vector of inputs, as a 16-byte vector of TC.
    auto phi16 = [&](const uint4 &u, float scale) LA_INLINE {
        float x[VEC];
        unpack16(u, x, TI());
        Frag<TC> w;
#pragma unroll
        for (int t = 0; t < VEC; ++t) w.set(t, MODE == MODE_AGG ? phi(x[t]) * scale : phi(x[t]));
        if constexpr (sizeof(TC) == 2) {
            return __builtin_bit_cast(uint4, w.v);
        } else {
            return make_uint4(__float_as_uint(w.get(0)), __float_as_uint(w.get(1)), __float_as_uint(w.get(2)),
                              __float_as_uint(w.get(3)));
        }
    };
    // Stage the prefetched chunk into LDS buffer b.  FULL: all CT rows valid;
    // otherwise rows at or beyond nrows are written as zeros (they add nothing).
    auto stage = [&](auto full_tag, int b, int nrows) LA_INLINE {
        constexpr bool FULL = decltype(full_tag)::value;
        char *buf = smem + b * T::BUF;
        if (weighted && tid < T::ROWS) reinterpret_cast<float *>(buf + T::OFF_W)[tid] = rw;  // zero past the rows
        auto keep = [&](int row) { return FULL || row < nrows; };
        if (NEED_Q) {
#pragma unroll
            for (int i = 0; i < NLQ; ++i) {
                const int row = rq0 + i * RSQ;
                if ((CT * VQ) % kThreads == 0 || row < CT) {
                    uint4 out = phi16(rq[i], 1.0f);
                    if (!keep(row)) out = make_uint4(0u, 0u, 0u, 0u);
                    *reinterpret_cast<uint4 *>(buf + T::OFF_Q + lq0 + i * RSQ * T::LQ * (int)sizeof(TC)) = out;
                }
            }
        }
        if (NEED_K) {
#pragma unroll
            for (int i = 0; i < NLQ; ++i) {
                const int row = rq0 + i * RSQ;
                if ((CT * VQ) % kThreads == 0 || row < CT) {
                    uint4 out = phi16(rk[i], kscaled ? rks[MODE == MODE_AGG ? i : 0] : 1.0f);
                    if (!keep(row)) out = make_uint4(0u, 0u, 0u, 0u);
                    *reinterpret_cast<uint4 *>(buf + T::OFF_K + lq0 + i * RSQ * T::LQ * (int)sizeof(TC)) = out;
                }
            }
#pragma unroll
            for (int i = 0; i < NLV; ++i) {
                const int row = rv0 + i * RSV;
                if ((CT * VV) % kThreads == 0 || row < CT) {
                    uint4 out = rv[i];
                    if (!keep(row)) out = make_uint4(0u, 0u, 0u, 0u);
                    *reinterpret_cast<uint4 *>(buf + T::OFF_V + lv0 + i * RSV * T::LV * (int)sizeof(TC)) = out;
                }
            }
        }
    };

    // Compute chunk c from LDS buffer b (FULL: all CT rows valid).  All
    // matrix work is one straight-line block; the stores come last.
    auto compute = [&](auto full_tag, int b, int c, int nrows) LA_INLINE {
        constexpr bool FULL = decltype(full_tag)::value;
        const char *buf = smem + b * T::BUF;
        const TC *sq = reinterpret_cast<const TC *>(buf + T::OFF_Q);
        const TC *sk = reinterpret_cast<const TC *>(buf + T::OFF_K);
        const TC *sv = reinterpret_cast<const TC *>(buf + T::OFF_V);
        if (NEED_Q && has_cols) {
            f32x4 outv[CBW][NB];
            float den[NB];
            // V^T(cb) in the split assignment over tokens (A operand of the intra product)
            Frag<TC> fvt[CBW][NP];
            if (MODE == MODE_CAUSAL) {
#pragma unroll
                for (int cs = 0; cs < CBW; ++cs)
#pragma unroll
                    for (int jp = 0; jp < NP; ++jp)
                        if (wave + 4 * cs < CBT)
                            lds_frag_tr(fvt[cs][jp], sv, T::LV, 32 * jp + 4 * g, 32 * jp + 16 + 4 * g,
                                        16 * (wave + 4 * cs), pp);
            }
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                const TC *qrow = &sq[(16 * I + pp) * T::LQ];
                Frag<TC> fq[NSE];
#pragma unroll
                for (int s = 0; s < NSE; ++s) lds_frag_split(fq[s], qrow + 32 * s, qrow + 32 * s + 16, g);
                // den_i = phi(q_i) . z + sum_{j <= i} A_ij, both on the matrix
                // cores: every accumulator slot of lane (i, g) ends up holding den_i.
                f32x4 accD = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < NSE; ++s) accD = mma(fragZ[s], fq[s], accD);
                Frag<TC> fb[NP];  // A^T key-block pairs as B operands (split over tokens)
                if (MODE == MODE_CAUSAL) {
                    f32x4 accA[2 * NP];
#pragma unroll
                    for (int J = 0; J < 2 * NP; ++J) {
                        accA[J] = f32x4{0.f, 0.f, 0.f, 0.f};
                        if (J <= I) {
#pragma unroll
                            for (int s = 0; s < NSE; ++s) {
                                Frag<TC> fk;  // phi(K) rows of key block J, split over features
                                const TC *krow = &sk[(16 * J + pp) * T::LQ + 32 * s];
                                lds_frag_split(fk, krow, krow + 16, g);
                                accA[J] = mma(fk, fq[s], accA[J]);
                            }
                        }
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) accA[I][r] = diag_keep[r] ? accA[I][r] : 0.f;  // j <= i
#pragma unroll
                    for (int jp = 0; jp < NP; ++jp) {
                        if (2 * jp <= I) {
                            acc_to_frag(fb[jp], accA[2 * jp], accA[2 * jp + 1]);
                            accD = mma(ones, fb[jp], accD);
                        }
                    }
                }
                den[I] = accD[0];
                const float inv = __builtin_amdgcn_rcpf(accD[0]);
#pragma unroll
                for (int cs = 0; cs < CBW; ++cs) {
                    if (wave + 4 * cs < CBT) {
                        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                        if (MODE == MODE_CAUSAL) {
#pragma unroll
                            for (int jp = 0; jp < NP; ++jp)
                                if (2 * jp <= I) acc = mma(fvt[cs][jp], fb[jp], acc);
                        }
#pragma unroll
                        for (int s = 0; s < NSE; ++s) acc = mma(fragS[cs][s], fq[s], acc);
                        outv[cs][I] = acc * inv;
                    }
                }
            }
            // stores: row 16 I + pp of the chunk, columns 16 cb + 4g .. + 3
            const long crow0 = seg_row0 + (long)c * CT;
            if (p.out_bf16) {
                char *oc = static_cast<char *>(p.o) + crow0 * DV * 2;
#pragma unroll
                for (int cs = 0; cs < CBW; ++cs)
#pragma unroll
                    for (int I = 0; I < NB; ++I)
                        if (wave + 4 * cs < CBT && (FULL || 16 * I + pp < nrows))
                            *reinterpret_cast<uint2 *>(oc + (unsigned)(((16 * I + pp) * DV + 16 * (wave + 4 * cs) + 4 * g) * 2)) =
                                pack_bf16x4(outv[cs][I]);
            } else {
                char *oc = static_cast<char *>(p.o) + crow0 * DV * 4;
#pragma unroll
                for (int cs = 0; cs < CBW; ++cs)
#pragma unroll
                    for (int I = 0; I < NB; ++I)
                        if (wave + 4 * cs < CBT && (FULL || 16 * I + pp < nrows))
                            *reinterpret_cast<f32x4 *>(oc + (unsigned)(((16 * I + pp) * DV + 16 * (wave + 4 * cs) + 4 * g) * 4)) =
                                outv[cs][I];
            }
            if (p.den && wave == 0 && g == 0) {
#pragma unroll
                for (int I = 0; I < NB; ++I)
                    if (FULL || 16 * I + pp < nrows) p.den[crow0 + 16 * I + pp] = den[I];
            }
        }

        // ---- state carry: S(cb) += phi(K_c)^T V_c(cb), z += phi(K_c)^T 1 ----
        if (NEED_K && has_cols) {
            const float *sw = reinterpret_cast<const float *>(buf + T::OFF_W);
#pragma unroll
            for (int s = 0; s < NP; ++s) {
                Frag<TC> fkt[NE];
                // z weights over this step's tokens (straight assignment), as a
                // value and its rounding remainder when the operands are bf16
                Frag<TC> fw = ones, fw_lo;
                if (weighted) {
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const float x = sw[32 * s + 8 * g + t];
                        fw.set(t, x);
                        fw_lo.set(t, x - fw.get(t));
                    }
                }
#pragma unroll
                for (int E = 0; E < NE; ++E) {
                    lds_frag_tr(fkt[E], sk, T::LQ, 32 * s + 8 * g, 32 * s + 8 * g + 4, 16 * E, pp);
                    accZ[E] = mma(fkt[E], fw, accZ[E]);
                    if (weighted && sizeof(TC) == 2) accZ[E] = mma(fkt[E], fw_lo, accZ[E]);
                }
#pragma unroll
                for (int cs = 0; cs < CBW; ++cs) {
                    const int cb = wave + 4 * cs;
                    if (cb < CBT) {
                        Frag<TC> fv;
                        lds_frag_tr(fv, sv, T::LV, 32 * s + 8 * g, 32 * s + 8 * g + 4, 16 * cb, pp);
#pragma unroll
                        for (int E = 0; E < NE; ++E) accS[cs][E] = mma(fkt[E], fv, accS[cs][E]);
                    }
                }
            }
            if (MODE == MODE_CAUSAL) refresh_state_frags();
        }
    };

    using Full = std::integral_constant<bool, true>;
    using Part = std::integral_constant<bool, false>;
    auto rows_of = [&](int c) { return min(CT, row_end - row_begin - c * CT); };

    if (nch > 0) {
        load_any(0);
        __syncthreads();  // the zero fill is complete before any tile write
        stage(Part{}, 0, rows_of(0));
        if (nch > 1) load_any(1);
        __syncthreads();
    }
    int ch = 0;
    if constexpr (NBUF == 2) {
        // Steady state, two chunks per trip: chunks ch .. ch + 3 are full.
        // Stage the next chunk, prefetch the one after, compute this one.
        for (; ch + 3 < nfull; ch += 2) {
            stage(Full{}, 1, CT);
            load_full(ch + 2);
            compute(Full{}, 0, ch, CT);
            __syncthreads();
            stage(Full{}, 0, CT);
            load_full(ch + 3);
            compute(Full{}, 1, ch + 1, CT);
            __syncthreads();
        }
        for (; ch < nch; ++ch) {
            const int b = ch & 1;
            if (ch + 1 < nch) {
                stage(Part{}, b ^ 1, rows_of(ch + 1));
                if (ch + 2 < nch) load_any(ch + 2);
            }
            compute(Part{}, b, ch, rows_of(ch));
            __syncthreads();
        }
    } else {
        for (; ch + 2 < nfull; ++ch) {
            compute(Full{}, 0, ch, CT);
            __syncthreads();
            stage(Full{}, 0, CT);
            load_full(ch + 2);
            __syncthreads();
        }
        for (; ch < nch; ++ch) {
            compute(Part{}, 0, ch, rows_of(ch));
            __syncthreads();
            if (ch + 1 < nch) {
                stage(Part{}, 0, rows_of(ch + 1));
                if (ch + 2 < nch) load_any(ch + 2);
                __syncthreads();
            }
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

#undef LA_INLINE

}  // namespace la
