// la_fwd_impl.hpp -- chunked forward kernels (causal and non-causal) for gfx950.
//
// One kernel template serves three modes over a segment of one (batch, head):
//   MODE_AGG    -- sum phi(K)^T V and sum phi(K) over the segment (no output);
//   MODE_CAUSAL -- the chunk loop of the causal form, starting from the state
//                  carried into the segment;
//   MODE_APPLY  -- the non-causal read-out phi(Q) S / phi(Q) z with a fixed state;
//   MODE_AGGW   -- MODE_AGG with a per-token factor on each phi(k) row and
//                  per-token weights in the z sum (the non-causal backward's
//                  total of (phi(q) / den)^T [dO, -eps]).
// Chunked causal form (itwiki "선형 어텐션", table "Comparison of forms", chunked
// row, and section "Implementation"): inside a chunk of C tokens the causal
// scores are a masked matrix product, between chunks the state
// S = sum phi(k) v^T, z = sum phi(k) is carried.  The sequence of one
// (batch, head) is cut into P segments of whole chunks; the states entering
// the segments come from an exclusive prefix sum of per-segment aggregates
// (the prefix sum is a scan and can be taken in parallel: blog digest
// "Theoretical significance / prefix-sum parallelism").
//
// For bf16 with d_k, d_v <= 64 a workgroup is eight waves with two roles, one
// wave of each role on every SIMD, so that the vector work of one overlaps
// the matrix work of the other:
//   * staging waves (4..7) load q, k, v rows with 16-byte global loads two
//     chunks ahead into registers (two register sets, alternating), apply phi
//     to q and k and write the rows to LDS (row-major, 16-byte writes);
//   * compute waves (0..3) read every matrix operand from those row-major
//     tiles -- with plain reads where the contraction runs over features and
//     with the gfx950 transpose read (ds_read_b64_tr_b16) where it runs over
//     tokens -- run the MFMA work and store the outputs.
// The tiles are double buffered: while the compute waves work on chunk c the
// staging waves fill chunk c + 1, with a single barrier per chunk.  The
// aggregate passes (no outputs) use the same split layout at d = 128 too, one
// workgroup per CU.  Wider heads in the causal and read-out passes, and fp32,
// whose compute waves need more registers than two waves per SIMD leave, use
// four waves that do both jobs in turn (stage chunk c + 1, compute chunk c)
// with one register set, or two (loads two chunks ahead) in the bf16 causal
// loop without decay.  Chunks
// whose rows are all valid run an unrolled loop (buffer and register-set
// indices are constants) with fixed per-lane offsets from a uniform base and
// no row masks; the last chunks run a general loop with clamped loads.
//
// Compute split: compute wave w owns value-column blocks cb = w, w + 4, ...
// (16 columns each).  Its slice S[:, cb] of the state lives in accumulator
// registers for the whole segment and is fed back to the matrix cores as an
// operand through the split K assignment (see la_device.hpp), so the carry
// never leaves the registers; the normaliser z is carried the same way, as
// phi(K)^T times an all-ones operand.  Each compute wave computes the
// transposed score tiles A^T = phi(K) phi(Q)^T itself and the transposed
// output O^T(cb) = V^T(cb) A^T + S(cb)^T phi(Q)^T, which puts each query's
// normaliser in the lanes that store that query's outputs.
#pragma once

#include <type_traits>
#include <utility>

#include "la_device.hpp"

namespace la {

enum { MODE_AGG = 0, MODE_CAUSAL = 1, MODE_APPLY = 2, MODE_AGGW = 3 };

constexpr int kRoleThreads = 256;  // four waves per role

// Separate staging and compute waves (eight per workgroup) where the compute
// waves fit in the registers two waves per SIMD leave: bf16 with d_k, d_v <=
// 64, and the aggregate passes without decay (no outputs: their compute waves
// hold only the state) at every width; otherwise four waves take both roles.
// At d = 128, B=8, H=16, N=8192 the split aggregate took 77 us where four
// waves took 105; with decay its tables spill and four waves were faster.
template <int DK, int DV, typename TI, int MODE = MODE_CAUSAL, bool DECAY = false> constexpr bool fwd_split() {
    return sizeof(TI) == 2 && ((DK <= 64 && DV <= 64) || ((MODE == MODE_AGG || MODE == MODE_AGGW) && !DECAY));
}
template <int DK, int DV, typename TI, int MODE = MODE_CAUSAL, bool DECAY = false> constexpr int fwd_threads() {
    return fwd_split<DK, DV, TI, MODE, DECAY>() ? 2 * kRoleThreads : kRoleThreads;
}
// A wide aggregate pass (d_k or d_v of 128) in the split layout: one
// workgroup per CU (its compute waves hold a 128-wide state).
template <int DK, int DV, typename TI, int MODE, bool DECAY> constexpr bool fwd_wide_agg() {
    return fwd_split<DK, DV, TI, MODE, DECAY>() && (MODE == MODE_AGG || MODE == MODE_AGGW) && (DK > 64 || DV > 64);
}

struct FwdParams {
    const void *q;
    const void *k;
    const void *v;
    void *o;
    float *den;             // nullable, [BH][N]
    const float *seg_state; // per (bh, segment) entering state [DK*DV + DK], or null
    const float *S0;        // per-bh initial state, used only when seg_state is null
    const float *z0;
    float *seg_out;         // MODE_AGG(W): per (bh, segment) aggregates
    const float *zw;        // MODE_AGGW: per-token weights [BH][N] for z
    const float *kscale;    // MODE_AGGW: per-token factors [BH][N] applied to phi(k) rows
    float *S_fin;           // final state of the last segment (nullable)
    float *z_fin;
    int N;
    int L;                  // tokens per segment of this launch (a multiple of the chunk size)
    int state_P;            // segments per (bh) in the state array
    int state_mult;         // segment s of this launch starts at state slot s * state_mult
    int seg_base;           // segment of workgroup row blockIdx.y: seg_base + blockIdx.y
    const float *gamma;     // MODE_CAUSAL, MODE_AGG: per-head decay [H], or null for none
    int H;                  // heads (bh % H is the head of workgroup column bh)
    int sum_P;              // MODE_APPLY: the total state is the sum of slots 0 .. sum_P - 1 (>= 1)
    int phi_id;             // feature map: 0 = elu + 1, 1 = identity (q and k are already features)
    const void *W;          // PRF instantiations: random directions [H][DK][DK] in the input type
};

// LDS layout for one chunk of CT tokens held as TC; only the tiles a mode
// reads are allocated.  Byte offsets inside one buffer: q, k, v, then the
// per-token z weights.
template <int DK, int DV, typename TC, int CT, int MODE, bool DECAY = false> struct FwdTiles {
    static constexpr int DKP = DK < 32 ? 32 : DK;        // feature dim padded to a K step
    // Row padding, in elements, against LDS bank conflicts (64 banks of 4
    // bytes; a 64-lane 8-byte read is served 32 lanes per cycle): 16 bytes
    // suit the row-wise operand reads of the q and k tiles; the v tile is
    // read only transposed, four rows per lane group with the lane groups
    // four rows apart, which 32 bytes of bf16 padding make conflict-free.
    static constexpr int PAD = 16 / sizeof(TC);
    static constexpr int PADV = sizeof(TC) == 2 ? 16 : 4;
    static constexpr int LQ = DKP + PAD;                  // row length of q, k tiles
    static constexpr int LV = DV + PADV;                  // row length of the v tile
    static constexpr int ROWS = CT < 32 ? 32 : CT;        // chunk rows padded to a token K step
    static constexpr int QB = MODE == MODE_CAUSAL || MODE == MODE_APPLY ? ROWS * LQ * (int)sizeof(TC) : 0;
    static constexpr int KB = MODE != MODE_APPLY ? ROWS * LQ * (int)sizeof(TC) : 0;
    static constexpr int VB = MODE != MODE_APPLY ? ROWS * LV * (int)sizeof(TC) : 0;
    static constexpr int WB = MODE == MODE_AGGW ? ROWS * 4 : 0;
    static constexpr int OFF_Q = 0, OFF_K = QB, OFF_V = QB + KB, OFF_W = QB + KB + VB;
    static constexpr int BUF = QB + KB + VB + WB;          // bytes per buffer (multiple of 16)
    // Double buffering where it leaves room: a split workgroup has its CU's
    // LDS to itself; four-wave workgroups keep the buffers small.
    static constexpr int NBUF = 2 * BUF <= (fwd_split<DK, DV, TC, MODE, DECAY>() ? 150 : 64) * 1024 ? 2 : 1;
};

// Waves per SIMD the compiler must leave room for (registers are split among
// them).  A split workgroup puts two waves on every SIMD; its causal chunk
// loop needs the registers of one workgroup per CU, its aggregate and
// read-out passes fit two.  Four-wave workgroups get all registers.
// (The read-out with random features keeps the directions in its staging
// waves' registers as well, and gets the registers of two waves per SIMD.)
template <int DK, int DV, typename TI, int CT, int MODE, bool DECAY, bool PRF = false> constexpr int fwd_waves_per_eu() {
    return fwd_split<DK, DV, TI, MODE, DECAY>()
               ? ((MODE == MODE_CAUSAL || fwd_wide_agg<DK, DV, TI, MODE, DECAY>() || (PRF && MODE == MODE_APPLY)) ? 2 : 4)
               : 1;
}

#define LA_INLINE __attribute__((always_inline))

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N - 1>{}).
template <typename F, int... Is>
__device__ LA_INLINE void static_for_impl(F &&f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F> __device__ LA_INLINE void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// OBF: the output o is bf16 (else fp32).  DECAY (MODE_CAUSAL and MODE_AGG):
// the per-head decay of p.gamma, any value in [0, 1]; a separate
// instantiation, so that the plain kernels keep their registers.  PRF: the
// staging waves apply Performer's positive random features with as many
// directions as input features (p.W, m = DK) instead of elu + 1 (split bf16
// layout at CT = 64; see the staging code).  XCARRY (decayed MODE_AGG on bf16
// operands, for the backward): the carry weights and the weighted values enter the MFMAs as a
// value and its rounding remainder (see the decay factors below).
template <int DK, int DV, typename TI, int MODE, int CT, bool OBF, bool DECAY = false, bool PRF = false,
          bool XCARRY = false>
__global__ void __launch_bounds__((fwd_threads<DK, DV, TI, MODE, DECAY>()))
__attribute__((amdgpu_waves_per_eu(fwd_waves_per_eu<DK, DV, TI, CT, MODE, DECAY, PRF>())))
la_chunk_kernel(const FwdParams p) {
    using TC = TI;  // matrix operands keep the input precision
    using T = FwdTiles<DK, DV, TC, CT, MODE, DECAY>;
    constexpr bool SPLIT = fwd_split<DK, DV, TI, MODE, DECAY>();
    constexpr int kThreads = fwd_threads<DK, DV, TI, MODE, DECAY>();
    constexpr int NBUF = T::NBUF;
    // Register sets of the staging waves, i.e. chunks loaded ahead.  The
    // causal chunk loop runs one workgroup per CU and its staging waves have
    // registers to spare under the compute waves' allocation: four sets keep
    // about 96 KB of loads in flight per CU (two sets measured about 2%
    // slower).  The aggregate and read-out passes, two workgroups per CU,
    // keep two.  A power of two, and even where NBUF = 2.
    constexpr int NSET = (SPLIT && MODE == MODE_CAUSAL) ? 4 : 2;
    static_assert(NSET == 2 || NSET == 4 || NSET == 8, "register sets: 2, 4 or 8");
    // Four-wave causal loop on bf16 with two buffers: loads two chunks ahead
    // (both register sets) instead of one; decayed kernels would spill.
    constexpr bool PF2 = !SPLIT && MODE == MODE_CAUSAL && !DECAY && sizeof(TI) == 2 && T::NBUF == 2;
    constexpr int VEC = Store<TI>::VEC;
    constexpr int NE = DK / 16;            // feature tiles
    constexpr int NSE = (DK + 31) / 32;    // feature K steps
    constexpr int CBT = DV / 16;           // value-column blocks in total
    constexpr int CBW = (CBT + 3) / 4;     // per compute wave (at most)
    constexpr int NB = CT / 16;            // query/key row blocks per chunk
    constexpr int NP = (NB + 1) / 2;       // pairs of row blocks (token K steps)
    constexpr int VQ = DK / VEC;           // 16-byte vectors per q/k row
    constexpr int VV = DV / VEC;           // per v row
    constexpr int NLQ = (CT * VQ + kRoleThreads - 1) / kRoleThreads;  // vectors per staging thread
    constexpr int NLV = (CT * VV + kRoleThreads - 1) / kRoleThreads;
    constexpr int RSQ = kRoleThreads / VQ; // rows between a staging thread's q/k vectors
    constexpr int RSV = kRoleThreads / VV;
    constexpr bool NEED_Q = MODE == MODE_CAUSAL || MODE == MODE_APPLY;
    constexpr bool AGGM = MODE == MODE_AGG || MODE == MODE_AGGW;  // aggregate only
    constexpr bool WEIGHTED = MODE == MODE_AGGW;
    constexpr bool NEED_K = MODE != MODE_APPLY;
    constexpr int NKS = WEIGHTED ? NLQ : 1;  // per-vector phi(k) factors
    static_assert(!PRF || (SPLIT && CT == 64 && NLQ == DK / 32 && !DECAY && !WEIGHTED),
                  "random features in the staging waves: split bf16 layout, 64-token chunks");
    using Full = std::integral_constant<bool, true>;
    using Part = std::integral_constant<bool, false>;
    using S0t = std::integral_constant<int, 0>;
    using S1t = std::integral_constant<int, 1>;

    __shared__ __attribute__((aligned(16))) char smem[NBUF * T::BUF];

    const int tid = threadIdx.x;
    const bool stager = SPLIT && tid >= kRoleThreads;  // uniform per wave
    const int lane = tid & 63;
    const int wave = (tid >> 6) & 3;          // index inside the role
    const int g = lane >> 4;
    const int pp = lane & 15;
    const long bh = blockIdx.x;
    const int seg = p.seg_base + (int)blockIdx.y;
    // Per-head decay gamma (RetNet row of the itwiki variants table):
    // S_i = gamma S_{i-1} + phi(k_i) v_i^T, z likewise.  Inside a chunk every
    // score carries gamma^(tau_i - tau_j) (tau the row in the chunk), the carried
    // state is read as gamma^(tau_i + 1) S, and a chunk of R rows updates it to
    // gamma^R S + sum_j gamma^(R - 1 - tau_j) phi(k_j) v_j^T.  Every factor is a
    // power gamma^e with e >= 0, applied to MFMA results (scores, inter-chunk
    // terms) or to the phi(k) operand of the carry, so any gamma in [0, 1] stays
    // in range; the factors of full chunks are per-lane tables computed once.
    static_assert(!DECAY || MODE == MODE_CAUSAL || MODE == MODE_AGG, "decay: causal chunk loop and its aggregate");
    static_assert(!XCARRY || (DECAY && MODE == MODE_AGG && sizeof(TI) == 2),
                  "value-plus-remainder carry: decayed aggregate on bf16 operands");
    constexpr bool decay = DECAY;
    const float gam = decay ? p.gamma[bh % p.H] : 1.0f;
    const float lg_gam = decay ? __builtin_log2f(gam) : 0.0f;  // -inf for gamma = 0
    // gamma^e for an integer e >= 0 (gamma^0 = 1 also for gamma = 0)
    auto gpow = [&](int e) { return e == 0 ? 1.0f : __builtin_amdgcn_exp2f((float)e * lg_gam); };
    const int N = p.N;
    const int row_begin = seg * p.L;
    const int row_end = min(N, row_begin + p.L);
    const int nch = (row_end - row_begin + CT - 1) / CT;
    const int nfull = (row_end - row_begin) / CT;   // chunks with all CT rows valid
    const long seg_row0 = bh * N + row_begin;
    auto rows_of = [&](int c) { return min(CT, row_end - row_begin - c * CT); };
    if (nch <= 0) return;  // no launched segment is empty; uniform for the workgroup

    // ---- zero the tile storage once: padding rows and columns stay zero ----
    for (int i = tid; i < NBUF * T::BUF / 16; i += kThreads)
        reinterpret_cast<uint4 *>(smem)[i] = make_uint4(0u, 0u, 0u, 0u);

    // ================= staging (both layouts) =================
    const int sid = SPLIT ? tid - kRoleThreads : tid;  // staging thread index 0..255
        constexpr bool weighted = WEIGHTED, kscaled = WEIGHTED;
        const char *qs = static_cast<const char *>(p.q) + seg_row0 * DK * (long)sizeof(TI);
        const char *ks = static_cast<const char *>(p.k) + seg_row0 * DK * (long)sizeof(TI);
        const char *vs = static_cast<const char *>(p.v) + seg_row0 * DV * (long)sizeof(TI);
        // This thread's first vector (row, column); vector i is RSQ (RSV) rows further.
        const int rq0 = sid / VQ, cq0 = (sid % VQ) * VEC;
        const int rv0 = sid / VV, cv0 = (sid % VV) * VEC;
        const unsigned gq0 = (unsigned)(rq0 * DK + cq0) * sizeof(TI);
        const unsigned gv0 = (unsigned)(rv0 * DV + cv0) * sizeof(TI);
        const int lq0 = (rq0 * T::LQ + cq0) * (int)sizeof(TC);
        const int lv0 = (rv0 * T::LV + cv0) * (int)sizeof(TC);
        // PRF: staging wave w loads q, k rows 16 w + p of the chunk in the
        // operand layout of the projection: lane (g, p) holds elements
        // 32 i + 8 g .. + 7 of its row in vector i (NLQ = DK / 32 vectors).
        const int prow = 16 * wave + pp;
        const unsigned gp0 = (unsigned)(prow * DK + 8 * g) * sizeof(TI);
        // PRF: the directions of this head as A operands, held by the staging
        // waves for the whole segment: wf[F][i] is rows 16 F + p, columns
        // 32 i + 8 g .. + 7 of W (features x input elements).
        Frag<TC> wf[PRF ? DK / 16 : 1][PRF ? NLQ : 1];
        if constexpr (PRF) {
            if (stager) {
                const TC *Wh = static_cast<const TC *>(p.W) + (bh % p.H) * (long)(DK * DK);
#pragma unroll
                for (int F = 0; F < DK / 16; ++F)
#pragma unroll
                    for (int i = 0; i < NLQ; ++i)
                        lds_frag_straight(wf[F][i], Wh + (16 * F + pp) * DK + 32 * i, g);
            }
        }
        // Vectors past the chunk exist only when CT * VQ is not a multiple of
        // the role size; they re-read the chunk's last row and are not staged.
        auto q_on = [&](int i) { return (CT * VQ) % kRoleThreads == 0 || rq0 + i * RSQ < CT; };
        auto v_on = [&](int i) { return (CT * VV) % kRoleThreads == 0 || rv0 + i * RSV < CT; };

        // NSET register sets; chunk j lives in set j % NSET.
        uint4 rq[NSET][NEED_Q ? NLQ : 1], rk[NSET][NEED_K ? NLQ : 1], rv[NSET][NEED_K ? NLV : 1];
        float rw[NSET] = {};
        float rks[NSET][NKS];

        // Load chunk c into set S.  FULL: all rows valid (uniform base, fixed
        // lane offsets); otherwise row indices are clamped to the segment.
        auto load = [&](auto set_tag, auto full_tag, int c) LA_INLINE {
            constexpr int S = decltype(set_tag)::value;
            constexpr bool FULL = decltype(full_tag)::value;
            const int r0 = c * CT;
            const int last = FULL ? r0 + CT - 1 : row_end - row_begin - 1;  // segment-relative
            if (weighted) rw[S] = (sid < CT && r0 + sid <= last) ? p.zw[seg_row0 + r0 + sid] : 0.f;
            if (kscaled) {
#pragma unroll
                for (int i = 0; i < NKS; ++i) {
                    const int row = min(r0 + rq0 + i * RSQ, last);
                    rks[S][i] = p.kscale[seg_row0 + row];
                }
            }
            if constexpr (FULL) {
                const char *qc = qs + (long)r0 * DK * (long)sizeof(TI);
                const char *kc = ks + (long)r0 * DK * (long)sizeof(TI);
                const char *vc = vs + (long)r0 * DV * (long)sizeof(TI);
                auto offq = [&](int i) {
                    if constexpr (PRF) return gp0 + (unsigned)(32 * i * sizeof(TI));
                    return (CT * VQ) % kRoleThreads != 0 && i == NLQ - 1
                               ? (unsigned)((min(rq0 + i * RSQ, CT - 1) * DK + cq0) * sizeof(TI))
                               : gq0 + (unsigned)(i * RSQ * DK * sizeof(TI));
                };
                auto offv = [&](int i) {
                    return (CT * VV) % kRoleThreads != 0 && i == NLV - 1
                               ? (unsigned)((min(rv0 + i * RSV, CT - 1) * DV + cv0) * sizeof(TI))
                               : gv0 + (unsigned)(i * RSV * DV * sizeof(TI));
                };
                if (NEED_Q) {
#pragma unroll
                    for (int i = 0; i < NLQ; ++i) rq[S][i] = load_stream16(qc + offq(i));
                }
                if (NEED_K) {
#pragma unroll
                    for (int i = 0; i < NLQ; ++i) rk[S][i] = load_stream16(kc + offq(i));
#pragma unroll
                    for (int i = 0; i < NLV; ++i) rv[S][i] = load_stream16(vc + offv(i));
                }
            } else {
                // (PRF: row prow of the chunk, elements 32 i + 8 g .. + 7)
                auto qrow = [&](int i) -> long { return PRF ? min(r0 + prow, last) : min(r0 + rq0 + i * RSQ, last); };
                auto qcol = [&](int i) { return PRF ? 32 * i + 8 * g : cq0; };
                if (NEED_Q) {
#pragma unroll
                    for (int i = 0; i < NLQ; ++i)
                        rq[S][i] = load_stream16(qs + (qrow(i) * DK + qcol(i)) * (long)sizeof(TI));
                }
                if (NEED_K) {
#pragma unroll
                    for (int i = 0; i < NLQ; ++i)
                        rk[S][i] = load_stream16(ks + (qrow(i) * DK + qcol(i)) * (long)sizeof(TI));
#pragma unroll
                    for (int i = 0; i < NLV; ++i) {
                        const long row = min(r0 + rv0 + i * RSV, last);
                        rv[S][i] = load_stream16(vs + (row * DV + cv0) * (long)sizeof(TI));
                    }
                }
            }
        };
        // Any chunk: one code path (clamped rows), so every load sequence
        // has the same instructions and the waits computed for it stay exact.
        auto load_any = [&](auto set_tag, int c) LA_INLINE { load(set_tag, Part{}, c); };

        // phi (times a factor) of a 16-byte vector of inputs, as a 16-byte vector of TC.
        const bool ident = p.phi_id != 0;  // uniform: the feature map is the identity
        auto phi16 = [&](const uint4 &u, float scale) LA_INLINE {
            float x[VEC];
            unpack16(u, x, TI());
            Frag<TC> w;
#pragma unroll
            for (int t = 0; t < VEC; ++t) {
                const float f = ident ? x[t] : phi(x[t]);
                w.set(t, WEIGHTED ? f * scale : f);
            }
            if constexpr (sizeof(TC) == 2) {
                return __builtin_bit_cast(uint4, w.v);
            } else {
                return make_uint4(__float_as_uint(w.get(0)), __float_as_uint(w.get(1)), __float_as_uint(w.get(2)),
                                  __float_as_uint(w.get(3)));
            }
        };
        // Random features of this wave's 16 rows (PRF): phi(x)^T tiles
        // W[16F.., :] x^T on the matrix cores, so that lane (g, p) holds
        // features 16 F + 4 g + r of row prow, written to the tile as four
        // consecutive elements; |x|^2 from the same fragments (the four lane
        // groups hold a row's elements between them).  A row past the chunk
        // is written as zeros.
        auto project = [&](const auto &x, char *tile, bool live) LA_INLINE {
            if constexpr (PRF) {
            constexpr int NF = DK / 16;
            f32x4 acc[NF];
#pragma unroll
            for (int F = 0; F < NF; ++F) acc[F] = f32x4{0.f, 0.f, 0.f, 0.f};
            float nx = 0.f;
#pragma unroll
            for (int i = 0; i < NLQ; ++i) {
                Frag<TC> fx;
                if constexpr (sizeof(TC) == 2) fx.v = __builtin_bit_cast(bf16x8, x[i]);
#pragma unroll
                for (int t = 0; t < 8; ++t) nx += fx.get(t) * fx.get(t);
#pragma unroll
                for (int F = 0; F < NF; ++F) acc[F] = mma(wf[F][i], fx, acc[F]);
            }
            nx = sum_over_groups(nx);
            const float scale = __builtin_amdgcn_rsqf((float)DK);
#pragma unroll
            for (int F = 0; F < NF; ++F) {
                f32x4 f;
#pragma unroll
                for (int r = 0; r < 4; ++r) f[r] = live ? __expf(acc[F][r] - 0.5f * nx) * scale : 0.f;
                *reinterpret_cast<uint2 *>(tile + (prow * T::LQ + 16 * F + 4 * g) * (int)sizeof(TC)) = pack_bf16x4(f);
            }
            }
        };
        // Write set S into LDS buffer b.  FULL: all CT rows valid; otherwise
        // rows at or beyond nrows are written as zeros (they add nothing).
        auto stage = [&](auto set_tag, auto full_tag, int b, int nrows) LA_INLINE {
            constexpr int S = decltype(set_tag)::value;
            constexpr bool FULL = decltype(full_tag)::value;
            char *buf = smem + b * T::BUF;
            if (weighted && sid < T::ROWS) reinterpret_cast<float *>(buf + T::OFF_W)[sid] = rw[S];
            auto keep = [&](int row) { return FULL || row < nrows; };
            if constexpr (PRF && NEED_Q) project(rq[S], buf + T::OFF_Q, keep(prow));
            if constexpr (PRF && NEED_K) project(rk[S], buf + T::OFF_K, keep(prow));
            if (NEED_Q && !PRF) {
#pragma unroll
                for (int i = 0; i < NLQ; ++i) {
                    if (q_on(i)) {
                        uint4 out = phi16(rq[S][i], 1.0f);
                        if (!keep(rq0 + i * RSQ)) out = make_uint4(0u, 0u, 0u, 0u);
                        *reinterpret_cast<uint4 *>(buf + T::OFF_Q + lq0 + i * RSQ * T::LQ * (int)sizeof(TC)) = out;
                    }
                }
            }
            if (NEED_K) {
#pragma unroll
                for (int i = 0; i < NLQ; ++i) {
                    if (q_on(i) && !PRF) {
                        uint4 out = phi16(rk[S][i], kscaled ? rks[S][WEIGHTED ? i : 0] : 1.0f);
                        if (!keep(rq0 + i * RSQ)) out = make_uint4(0u, 0u, 0u, 0u);
                        *reinterpret_cast<uint4 *>(buf + T::OFF_K + lq0 + i * RSQ * T::LQ * (int)sizeof(TC)) = out;
                    }
                }
#pragma unroll
                for (int i = 0; i < NLV; ++i) {
                    if (v_on(i)) {
                        uint4 out = rv[S][i];
                        if (!keep(rv0 + i * RSV)) out = make_uint4(0u, 0u, 0u, 0u);
                        *reinterpret_cast<uint4 *>(buf + T::OFF_V + lv0 + i * RSV * T::LV * (int)sizeof(TC)) = out;
                    }
                }
            }
        };
        // One step of the split layout's general loop at chunk j: stage chunk
        // j from its register set, then refill that set with chunk j + NSET.
        auto step_split = [&](auto set_tag, int j) LA_INLINE {
            const int b = NBUF == 2 ? (j & 1) : 0;
            if (j < nfull) stage(set_tag, Full{}, b, CT);
            else stage(set_tag, Part{}, b, rows_of(j));
            if (j + NSET < nch) load_any(set_tag, j + NSET);
        };
        auto step_split_any = [&](int j) LA_INLINE {  // j >= 0
            static_for<NSET>([&](auto u) LA_INLINE {
                if ((j & (NSET - 1)) == decltype(u)::value) step_split(u, j);
            });
        };

    if constexpr (SPLIT) {
      if (stager) {
        // ================= staging waves: their whole loop =================
        // Step j stages chunk j (register set j % NSET) into buffer j & 1 and
        // refills that set with chunk j + NSET, then meets the compute waves
        // at a barrier.  The loop starts at j = -NSET with loads only, so
        // every load of the steady state is issued by the same instructions
        // and the wait before staging a set covers that set's loads, not the
        // later sets'.
        __syncthreads();  // the zero fill is complete before any tile write
        int j = -NSET;
        if constexpr (NBUF == 2) {
            // (the first trip, j = -NSET, always runs: it loads chunks 0 .. NSET - 1)
            for (; j + NSET - 1 < nfull; j += NSET) {  // chunks j .. j + NSET - 1 are full
                static_for<NSET>([&](auto u) LA_INLINE {
                    constexpr int U = decltype(u)::value;
                    if (j >= 0) stage(u, Full{}, U & 1, CT);
                    load_any(u, j + U + NSET);
                    if (j >= 0) __syncthreads();
                });
            }
            for (; j < nch; ++j) {
                step_split_any(j);
                __syncthreads();
            }
        } else {
            static_for<NSET>([&](auto u) LA_INLINE { load_any(u, decltype(u)::value); });
            for (j = 0; j < nch; ++j) {
                if (j > 0) __syncthreads();  // the compute waves are done with the buffer
                step_split_any(j);
                __syncthreads();
            }
        }
        return;
      }
    }

    // ================= compute (both layouts) =================
    // wave = tid / 64 < 4: with a multiple of four column blocks every wave
    // owns CBW of them, and the tests below fold away.
    auto col_ok = [&](int cs) { return CBT % 4 == 0 || wave + 4 * cs < CBT; };
    const bool has_cols = col_ok(0);                // waves without value columns only wait

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
    // 16E + 4g + r; for z every column holds the same value.  The non-causal
    // read-out sums the per-segment aggregates itself, slot by slot in a fixed
    // order (a few slots; no separate total pass).
    f32x4 accS[CBW][NE];
    f32x4 accZ[NE];
    const int nsum = MODE == MODE_APPLY ? p.sum_P : 1;
#pragma unroll
    for (int E = 0; E < NE; ++E) {
#pragma unroll
        for (int r = 0; r < 4; ++r) accZ[E][r] = 0.0f;
#pragma unroll
        for (int cs = 0; cs < CBW; ++cs)
#pragma unroll
            for (int r = 0; r < 4; ++r) accS[cs][E][r] = 0.0f;
    }
    for (int t = 0; t < nsum; ++t) {
        const float *St = Sin ? Sin + t * (long)(DK * DV + DK) : nullptr;
        const float *zt = zin ? zin + t * (long)(DK * DV + DK) : nullptr;
#pragma unroll
        for (int E = 0; E < NE; ++E) {
#pragma unroll
            for (int r = 0; r < 4; ++r) accZ[E][r] += zt ? zt[16 * E + 4 * g + r] : 0.0f;
#pragma unroll
            for (int cs = 0; cs < CBW; ++cs) {
                const int cb = wave + 4 * cs;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    accS[cs][E][r] += (St && col_ok(cs)) ? St[(16 * E + 4 * g + r) * DV + 16 * cb + pp] : 0.0f;
            }
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
    if (!AGGM) refresh_state_frags();
    Frag<TC> ones;
    frag_ones(ones);
    // causal mask on a diagonal score tile: row 4g + r <= column pp
    bool diag_keep[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) diag_keep[r] = 4 * g + r <= pp;

    // Decay factors, per lane (see the decay note above):
    //   dfq[I]    inter-chunk read of query row 16 I + pp: gamma^(16 I + pp + 1);
    //   dsc[D][r] score of key 16 J + 4g + r for query 16 I + pp, D = I - J:
    //             gamma^(16 D + pp - 4g - r), zero above the diagonal;
    //   dcwf[s]   carry weights of the tokens of token K step s of a full chunk,
    //             gamma^(CT - 1 - token), as an operand (slot t: the token of
    //             the split assignment).  With XCARRY the weights are recomputed
    //             in fp32 per step instead (fewer registers than a table), and
    //             both they and the weighted values enter the carry as a bf16
    //             value plus its bf16 remainder.
    // The backward takes its segment states from this aggregate.  There the
    // per-token e = -(g . out) den meets g . v in dk and the two cancel to a
    // small part of either under a fast decay, so errors of the carried state
    // reach dk magnified.  With the weights and the weighted values rounded to
    // bf16 once, each carried term has a relative error up to 2^-9; as value
    // plus remainder, about 2^-17.  The forward's output needs no more than the
    // single rounding.
    constexpr bool decay_out = decay && NEED_Q;
    constexpr bool DLO = XCARRY;
    float dfq[decay_out ? NB : 1];
    float dsc[decay_out ? NB : 1][4];
    Frag<TC> dcwf[decay && !DLO ? NP : 1];
    if constexpr (decay_out) {
#pragma unroll
        for (int I = 0; I < NB; ++I) {
            dfq[I] = gpow(16 * I + pp + 1);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int e = 16 * I + pp - 4 * g - r;
                dsc[I][r] = e >= 0 ? gpow(e) : 0.0f;
            }
        }
    }
    // token of slot t in token K step s (split assignment)
    auto slot_token = [&](int s, int t) { return 32 * s + (t < 4 ? 4 * g + t : 16 + 4 * g + t - 4); };
    if constexpr (decay && !DLO) {
#pragma unroll
        for (int s = 0; s < NP; ++s)
#pragma unroll
            for (int t = 0; t < 8; ++t) dcwf[s].set(t, slot_token(s, t) < CT ? gpow(CT - 1 - slot_token(s, t)) : 0.0f);
    }
    const float g_chunk = decay ? gpow(CT) : 1.0f;  // gamma^R for a full chunk

    // Store outputs of chunk c.  part = I >= 0: row block I (row 16 I + pp
    // of the chunk, columns 16 cb + 4g .. + 3) in bf16 (OBF) or fp32;
    // part = -1: den, when asked for.  FULL: all CT rows valid.  The output
    // type is a template parameter, so on full chunks the stores of the row
    // blocks need no branch; the den of row block I = wave is written by wave
    // `wave`, all four lane groups holding the same value.
    auto store_out = [&](auto full_tag, int c, int nrows, int part, const f32x4 (&outv)[CBW][NB],
                         const float (&den)[NB]) LA_INLINE {
        constexpr bool FULL = decltype(full_tag)::value;
        if constexpr (!NEED_Q) return;
        if (!has_cols) return;
        const long crow0 = seg_row0 + (long)c * CT;
        if (part >= 0) {
            const int I = part;
            char *oc = static_cast<char *>(p.o) + crow0 * DV * (OBF ? 2 : 4);
#pragma unroll
            for (int cs = 0; cs < CBW; ++cs) {
                if (col_ok(cs) && (FULL || 16 * I + pp < nrows)) {
                    const unsigned off = (unsigned)((16 * I + pp) * DV + 16 * (wave + 4 * cs) + 4 * g);
                    if constexpr (OBF) *reinterpret_cast<uint2 *>(oc + off * 2) = pack_bf16x4(outv[cs][I]);
                    else *reinterpret_cast<f32x4 *>(oc + off * 4) = outv[cs][I];
                }
            }
        } else if (p.den) {
            if constexpr (NB == 4 && CBT % 4 == 0) {
                // a vector (not the array) is indexed by the wave, so the
                // array stays in registers
                const f32x4 dv = {den[0], den[1], den[2], den[3]};
                const float d = dv[wave];
                if (FULL || 16 * wave + pp < nrows) p.den[crow0 + 16 * wave + pp] = d;
            } else if (wave == 0 && g == 0) {
#pragma unroll
                for (int I = 0; I < NB; ++I)
                    if (FULL || 16 * I + pp < nrows) p.den[crow0 + 16 * I + pp] = den[I];
            }
        }
    };

    // Per-lane bases of the split-fragment reads of the q and k tiles (row
    // pp, slot 4g), one per 32-feature step and half, so that no two of
    // these reads are merged (see lds_opaque).  Tile offsets are added as
    // element counts.
    lds_cptr<TC> fbase[NSE][2];
#pragma unroll
    for (int s = 0; s < NSE; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            fbase[s][h] = lds_opaque(reinterpret_cast<const TC *>(smem) + pp * T::LQ + 4 * g + 32 * s + 16 * h);

    // Outputs of one chunk, one row block I at a time (four-wave kernels:
    // their registers hold one block's operands at a time).
    auto outputs_by_block = [&](int qoff, int koff, const TC *sv, f32x4 (&outv)[CBW][NB], float (&den)[NB],
                                auto &&store) LA_INLINE {
        // V^T(cb) in the split assignment over tokens (A operand of the intra product)
        Frag<TC> fvt[CBW][NP];
        if (MODE == MODE_CAUSAL) {
#pragma unroll
            for (int cs = 0; cs < CBW; ++cs)
#pragma unroll
                for (int jp = 0; jp < NP; ++jp)
                    if (col_ok(cs))
                        lds_frag_tr(fvt[cs][jp], sv, T::LV, 32 * jp + 4 * g, 32 * jp + 16 + 4 * g,
                                    16 * (wave + 4 * cs), pp);
        }
#pragma unroll
        for (int I = 0; I < NB; ++I) {
            Frag<TC> fq[NSE];
#pragma unroll
            for (int s = 0; s < NSE; ++s) lds_frag_split_at(fq[s], fbase[s][0], fbase[s][1], qoff + 16 * I * T::LQ);
            // den_i = phi(q_i) . z + sum_{j <= i} A_ij, both on the matrix
            // cores: every accumulator slot of lane (i, g) ends up holding den_i.
            f32x4 accD = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NSE; ++s) accD = mma(fragZ[s], fq[s], accD);
            if constexpr (decay_out) accD = accD * dfq[I];
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
                            lds_frag_split_at(fk, fbase[s][0], fbase[s][1], koff + 16 * J * T::LQ);
                            accA[J] = mma(fk, fq[s], accA[J]);
                        }
                        if constexpr (decay_out) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) accA[J][r] *= dsc[I - J][r];
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
                if (col_ok(cs)) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (decay_out) {  // the decayed inter-chunk read first, then the chunk's own
#pragma unroll
                        for (int s = 0; s < NSE; ++s) acc = mma(fragS[cs][s], fq[s], acc);
                        acc = acc * dfq[I];
#pragma unroll
                        for (int jp = 0; jp < NP; ++jp)
                            if (2 * jp <= I) acc = mma(fvt[cs][jp], fb[jp], acc);
                    } else {
                        if (MODE == MODE_CAUSAL) {
#pragma unroll
                            for (int jp = 0; jp < NP; ++jp)
                                if (2 * jp <= I) acc = mma(fvt[cs][jp], fb[jp], acc);
                        }
#pragma unroll
                        for (int s = 0; s < NSE; ++s) acc = mma(fragS[cs][s], fq[s], acc);
                    }
                    outv[cs][I] = acc * inv;
                }
            }
            store(I, outv, den);
        }
    };

    // Outputs of one chunk in phases over all row blocks at once (split
    // kernels, whose compute waves have the registers): every operand read is
    // issued first, then the row blocks' score tiles and products, so the LDS
    // latency is paid once per chunk and the matrix-core latencies of one
    // block hide behind the work of the next.
    auto outputs_phased = [&](int qoff, int koff, const TC *sv, f32x4 (&outv)[CBW][NB], float (&den)[NB],
                              auto &&store) LA_INLINE {
        constexpr bool CAUSAL = MODE == MODE_CAUSAL;
        Frag<TC> fk[CAUSAL ? NB : 1][NSE];  // phi(K) rows of block J (A operand)
        Frag<TC> fvt[CBW][NP];           // V^T(cb) over token pairs (A operand)
        if constexpr (CAUSAL) {
#pragma unroll
            for (int J = 0; J < NB; ++J)
#pragma unroll
                for (int s = 0; s < NSE; ++s) lds_frag_split_at(fk[J][s], fbase[s][0], fbase[s][1], koff + 16 * J * T::LQ);
#pragma unroll
            for (int cs = 0; cs < CBW; ++cs)
#pragma unroll
                for (int jp = 0; jp < NP; ++jp)
                    if (col_ok(cs))
                        lds_frag_tr(fvt[cs][jp], sv, T::LV, 32 * jp + 4 * g, 32 * jp + 16 + 4 * g,
                                    16 * (wave + 4 * cs), pp);
        }
#pragma unroll
        for (int I = 0; I < NB; ++I) {
            Frag<TC> fq[NSE];  // phi(Q) rows of block I, split over features (B operand)
#pragma unroll
            for (int s = 0; s < NSE; ++s) lds_frag_split_at(fq[s], fbase[s][0], fbase[s][1], qoff + 16 * I * T::LQ);
            // den_i = phi(q_i) . z + sum_{j <= i} A_ij, on the matrix cores:
            // every accumulator slot of lane (i, g) ends up holding den_i.
            f32x4 accD = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NSE; ++s) accD = mma(fragZ[s], fq[s], accD);
            if constexpr (decay_out) accD = accD * dfq[I];
            Frag<TC> fb[NP];  // A^T key-block pairs as B operands (split over tokens)
            if constexpr (CAUSAL) {
                // score tiles A^T(J, I) for J <= I
                f32x4 accA[2 * NP];
#pragma unroll
                for (int J = 0; J < 2 * NP; ++J) {
                    accA[J] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (J <= I) {
#pragma unroll
                        for (int s = 0; s < NSE; ++s) accA[J] = mma(fk[J][s], fq[s], accA[J]);
                        if constexpr (decay_out) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) accA[J][r] *= dsc[I - J][r];
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
                if (col_ok(cs)) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (decay_out) {  // the decayed inter-chunk read first, then the chunk's own
#pragma unroll
                        for (int s = 0; s < NSE; ++s) acc = mma(fragS[cs][s], fq[s], acc);
                        acc = acc * dfq[I];
#pragma unroll
                        for (int jp = 0; jp < NP; ++jp)
                            if (2 * jp <= I) acc = mma(fvt[cs][jp], fb[jp], acc);
                    } else {
                        if constexpr (CAUSAL) {
#pragma unroll
                            for (int jp = 0; jp < NP; ++jp)
                                if (2 * jp <= I) acc = mma(fvt[cs][jp], fb[jp], acc);
                        }
#pragma unroll
                        for (int s = 0; s < NSE; ++s) acc = mma(fragS[cs][s], fq[s], acc);
                    }
                    outv[cs][I] = acc * inv;
                }
            }
            store(I, outv, den);
        }
    };

    // Compute the chunk in LDS buffer b: outputs into outv/den, `store(I)`
    // writes row block I as soon as it is done and `store(-1)` the den, then
    // the state carry.
    auto compute = [&](int b, int crows, auto &&store) LA_INLINE {
        const char *buf = smem + b * T::BUF;
        const int qoff = (b * T::BUF + T::OFF_Q) / (int)sizeof(TC);  // tile offsets in elements
        const int koff = (b * T::BUF + T::OFF_K) / (int)sizeof(TC);
        const TC *sk = reinterpret_cast<const TC *>(buf + T::OFF_K);
        const TC *sv = reinterpret_cast<const TC *>(buf + T::OFF_V);
        f32x4 outv[CBW][NB];  // outputs of the chunk, held until their stores
        float den[NB];
        if constexpr (SPLIT) {
            if (NEED_Q && has_cols) outputs_phased(qoff, koff, sv, outv, den, store);
        } else {
            if (NEED_Q && has_cols) outputs_by_block(qoff, koff, sv, outv, den, store);
        }
        store(-1, outv, den);

        // ---- state carry: S(cb) += phi(K_c)^T V_c(cb), z += phi(K_c)^T 1 ----
        // (decay: S = gamma^R S + sum_j gamma^(R - 1 - tau_j) phi(k_j) v_j^T, z
        // likewise: token j is the contraction index, so its weight scales the
        // 16-column V^T operand, and it replaces the all-ones operand of z)
        if constexpr (decay) {
            if (NEED_K && has_cols) {
                const float gR = crows == CT ? g_chunk : gpow(crows);
#pragma unroll
                for (int E = 0; E < NE; ++E) {
                    accZ[E] = accZ[E] * gR;
#pragma unroll
                    for (int cs = 0; cs < CBW; ++cs) accS[cs][E] = accS[cs][E] * gR;
                }
            }
        }
        if (NEED_K && has_cols) {
            const float *sw = reinterpret_cast<const float *>(buf + T::OFF_W);
            // (one token step at a time with the value-plus-remainder carry:
            // unrolled, its operands of both steps spill at d = 64)
            constexpr int kCarryUnroll = DLO ? 1 : NP;
#pragma unroll kCarryUnroll
            for (int s = 0; s < NP; ++s) {
                Frag<TC> fkt[NE];
                // z weights over this step's tokens (split assignment), as a
                // value and its rounding remainder when the operands are bf16
                Frag<TC> fw = ones, fw_lo;
                if (weighted) {
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const float x = sw[32 * s + (t < 4 ? 4 * g + t : 16 + 4 * g + t - 4)];
                        fw.set(t, x);
                        fw_lo.set(t, x - fw.get(t));
                    }
                }
                float cw[DLO ? 8 : 1];  // fp32 carry weights (DLO)
                if constexpr (DLO) {
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        cw[t] = slot_token(s, t) < crows ? gpow(crows - 1 - slot_token(s, t)) : 0.0f;
                        fw.set(t, cw[t]);
                        fw_lo.set(t, cw[t] - fw.get(t));
                    }
                } else if constexpr (decay) {  // carry weights of this step's tokens
                    if (crows == CT) {
                        fw = dcwf[s];
                    } else {
#pragma unroll
                        for (int t = 0; t < 8; ++t)
                            fw.set(t, slot_token(s, t) < crows ? gpow(crows - 1 - slot_token(s, t)) : 0.0f);
                    }
                }
#pragma unroll
                for (int E = 0; E < NE; ++E) {
                    lds_frag_tr(fkt[E], sk, T::LQ, 32 * s + 4 * g, 32 * s + 16 + 4 * g, 16 * E, pp);
                    accZ[E] = mma(fkt[E], fw, accZ[E]);
                    if ((weighted && sizeof(TC) == 2) || DLO) accZ[E] = mma(fkt[E], fw_lo, accZ[E]);
                }
#pragma unroll
                for (int cs = 0; cs < CBW; ++cs) {
                    const int cb = wave + 4 * cs;
                    if (col_ok(cs)) {
                        Frag<TC> fv, fv_lo;
                        lds_frag_tr(fv, sv, T::LV, 32 * s + 4 * g, 32 * s + 16 + 4 * g, 16 * cb, pp);
                        if constexpr (DLO) {
#pragma unroll
                            for (int t = 0; t < 8; ++t) {
                                const float x = fv.get(t) * cw[t];
                                fv.set(t, x);
                                fv_lo.set(t, x - fv.get(t));
                            }
                        } else if constexpr (decay) {
#pragma unroll
                            for (int t = 0; t < 8; ++t) fv.set(t, fv.get(t) * fw.get(t));
                        }
#pragma unroll
                        for (int E = 0; E < NE; ++E) {
                            accS[cs][E] = mma(fkt[E], fv, accS[cs][E]);
                            if constexpr (DLO) accS[cs][E] = mma(fkt[E], fv_lo, accS[cs][E]);
                        }
                    }
                }
            }
            if (MODE == MODE_CAUSAL) refresh_state_frags();
        }
    };

    if constexpr (SPLIT) {
        // Compute step j: wait for chunk j, compute it (the barrier before
        // step j + 2 frees its buffer).
        __syncthreads();  // zero fill
        int j = 0;
        if constexpr (NBUF == 2) {
            for (; j + 3 < nfull; j += 2) {  // same trip count as the staging waves
                __syncthreads();
                compute(0, CT, [&](int part, auto &o, auto &d) LA_INLINE { store_out(Full{}, j, CT, part, o, d); });
                __syncthreads();
                compute(1, CT, [&](int part, auto &o, auto &d) LA_INLINE { store_out(Full{}, j + 1, CT, part, o, d); });
            }
        }
        for (; j < nch; ++j) {
            const int b = NBUF == 2 ? (j & 1) : 0;
            __syncthreads();
            if (j < nfull) compute(b, CT, [&](int part, auto &o, auto &d) LA_INLINE { store_out(Full{}, j, CT, part, o, d); });
            else compute(b, rows_of(j), [&](int part, auto &o, auto &d) LA_INLINE { store_out(Part{}, j, rows_of(j), part, o, d); });
            if (NBUF == 1 && j + 1 < nch) __syncthreads();  // the staging waves refill the single buffer
        }
    } else if constexpr (PF2) {
        // ---- four waves in both roles, loads two chunks ahead: chunk j is
        // loaded into register set j & 1; step ch stages chunk ch + 1 into
        // buffer (ch + 1) & 1, refills its set with chunk ch + 3 and computes
        // chunk ch.  Absent chunks load clamped rows and are never staged. ----
        load_any(S0t{}, 0);
        load_any(S1t{}, 1);
        __syncthreads();  // the zero fill is complete before any tile write
        stage(S0t{}, Part{}, 0, rows_of(0));
        load_any(S0t{}, 2);
        __syncthreads();
        int ch = 0;
        // Pairs of full steps: chunks ch .. ch + 4 are full.
        for (; ch + 4 < nfull; ch += 2) {
            stage(S1t{}, Full{}, 1, CT);
            load(S1t{}, Full{}, ch + 3);
            compute(0, CT, [&](int part, auto &o, auto &d) LA_INLINE { store_out(Full{}, ch, CT, part, o, d); });
            __syncthreads();
            stage(S0t{}, Full{}, 0, CT);
            load(S0t{}, Full{}, ch + 4);
            compute(1, CT, [&](int part, auto &o, auto &d) LA_INLINE { store_out(Full{}, ch + 1, CT, part, o, d); });
            __syncthreads();
        }
        for (; ch < nch; ++ch) {
            const int b = ch & 1;
            if (ch + 1 < nch) {
                static_for<2>([&](auto u) LA_INLINE {
                    if (((ch + 1) & 1) == decltype(u)::value) {
                        if (ch + 1 < nfull) stage(u, Full{}, b ^ 1, CT);
                        else stage(u, Part{}, b ^ 1, rows_of(ch + 1));
                        if (ch + 3 < nch) load_any(u, ch + 3);
                    }
                });
            }
            if (ch < nfull) compute(b, CT, [&](int part, auto &o, auto &d) LA_INLINE { store_out(Full{}, ch, CT, part, o, d); });
            else compute(b, rows_of(ch), [&](int part, auto &o, auto &d) LA_INLINE { store_out(Part{}, ch, rows_of(ch), part, o, d); });
            __syncthreads();
        }
    } else {
        // ---- four waves in both roles: stage chunk c + 1, compute chunk c ----
        load_any(S0t{}, 0);
        __syncthreads();  // the zero fill is complete before any tile write
        stage(S0t{}, Part{}, 0, rows_of(0));
        load_any(S0t{}, 1);  // clamped rows when there is no chunk 1
        __syncthreads();
        int ch = 0;
        // Full chunks.
        if constexpr (NBUF == 2) {
            for (; ch + 2 < nfull; ++ch) {  // chunks ch .. ch + 2 are full
                const int b = ch & 1;
                stage(S0t{}, Full{}, b ^ 1, CT);
                load(S0t{}, Full{}, ch + 2);
                compute(b, CT, [&](int part, auto &o, auto &d) LA_INLINE { store_out(Full{}, ch, CT, part, o, d); });
                __syncthreads();
            }
        } else {
            for (; ch + 2 < nfull; ++ch) {
                compute(0, CT, [&](int part, auto &o, auto &d) LA_INLINE { store_out(Full{}, ch, CT, part, o, d); });
                __syncthreads();
                stage(S0t{}, Full{}, 0, CT);
                load(S0t{}, Full{}, ch + 2);
                __syncthreads();
            }
        }
        for (; ch < nch; ++ch) {
            const int b = NBUF == 2 ? (ch & 1) : 0;
            if (NBUF == 2 && ch + 1 < nch) {
                if (ch + 1 < nfull) stage(S0t{}, Full{}, b ^ 1, CT);
                else stage(S0t{}, Part{}, b ^ 1, rows_of(ch + 1));
                if (ch + 2 < nch) load_any(S0t{}, ch + 2);
            }
            if (ch < nfull) compute(b, CT, [&](int part, auto &o, auto &d) LA_INLINE { store_out(Full{}, ch, CT, part, o, d); });
            else compute(b, rows_of(ch), [&](int part, auto &o, auto &d) LA_INLINE { store_out(Part{}, ch, rows_of(ch), part, o, d); });
            __syncthreads();
            if (NBUF == 1 && ch + 1 < nch) {
                if (ch + 1 < nfull) stage(S0t{}, Full{}, 0, CT);
                else stage(S0t{}, Part{}, 0, rows_of(ch + 1));
                if (ch + 2 < nch) load_any(S0t{}, ch + 2);
                __syncthreads();
            }
        }
    }

    // ---- write the segment's resulting state ----
    float *Sdst = nullptr;
    float *zdst = nullptr;
    if (AGGM) {
        Sdst = p.seg_out + (bh * p.state_P + seg) * (long)(DK * DV + DK);
        zdst = Sdst + DK * DV;
    } else if (MODE == MODE_CAUSAL && blockIdx.y == gridDim.y - 1 && p.S_fin) {
        Sdst = p.S_fin + bh * (long)(DK * DV);
        zdst = p.z_fin + bh * (long)DK;
    }
    if (Sdst && has_cols) {
#pragma unroll
        for (int cs = 0; cs < CBW; ++cs) {
            const int cb = wave + 4 * cs;
            if (col_ok(cs)) {
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
