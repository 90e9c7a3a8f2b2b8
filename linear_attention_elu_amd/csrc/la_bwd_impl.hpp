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
// Workgroups have eight waves; the next chunk's rows are loaded into
// registers while the current chunk is computed.  Per chunk, the token-pair
// products (M, and A in the dk/dv sweep) are formed once, one 16 x 16 block
// per wave, and handed to every wave through LDS.  The feature-dimension work
// is split by blocks of 16: in the dq sweep wave w owns feature block w of dq
// and the rows S[16w.., :] of the state, held as accumulators of S^T so that
// they feed the matrix cores as an operand over the value index; in the dk/dv
// sweep wave w owns feature block w of dk with R[16w.., :] in accumulators,
// and value block w of dv, which needs R contracted over features: a copy of
// R in LDS, read with the transpose read.
//
// Non-causal form (NC = true; blog digest "Method / key components 2)"):
// the same gradient with full sums instead of prefix and suffix sums, so every
// token reads the totals S, z (dq sweep) and R, r (dk/dv sweep): no masked
// in-chunk products, no carry, and each sweep loads only the rows it needs
// (q, dO for dq; k, v for dk, dv).  The totals come as a few per-segment
// sums that each workgroup adds up in its prologue, in a fixed order.
//
// LDS row strides: tiles read row-wise (two 8-byte pieces per lane, rows p =
// 0..15) are padded to a stride of 4 (mod 8) times an odd number of banks,
// tiles read with the transpose read (rows 4g..4g+3 per lane group) to 8
// times an odd number; each pattern is then free of bank conflicts.
#pragma once

#include <type_traits>

#include "la_device.hpp"

namespace la {

constexpr int kBwdThreads = 512;
constexpr int kBwdWaves = 8;

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
    int sum_P;               // non-causal: the totals are the sums of slots 0 .. sum_P - 1
    int phi_id;              // feature map: 0 = elu + 1, 1 = identity (phi' = 1)
    const float *gamma;      // DECAY: per-head decay [H]
    int H;                   // heads (bh % H is the head of workgroup column bh)
    float *suf_out;          // causal dq sweep: per (bh, segment) suffix sums of its segment, or null
    int suf_P;               // segments per bh in suf_out
};

// Per-head decay (itwiki "선형 어텐션", table of later variants, RetNet row):
// S_i = gamma S_{i-1} + phi(k_i) v_i^T, z likewise.  Its gradient is the one
// above with every pair (i, j <= i) weighed by gamma^(i - j): the in-chunk
// products M and A carry gamma^(tau_i - tau_j) (tau the row in the chunk), the
// dq sweep reads the carried S, z as gamma^(tau_i + 1) S, and the dk/dv sweep
// reads the suffix state entering from the right, normalised at the next
// chunk's first token, as gamma^(R - tau_j) R (R the rows of the chunk).  The
// carries are S = gamma^R S + sum_j gamma^(R - 1 - tau_j) phi(k_j) v_j^T and
// R = gamma^R R + sum_i gamma^(tau_i) (phi(q_i) a_i) g_i^T.  All exponents are
// >= 0, so any gamma in [0, 1] is in range.
struct Decay {
    float lg;  // log2(gamma): -inf for gamma = 0
    __device__ __forceinline__ float pow(int e) const {  // gamma^e, e >= 0
        return e <= 0 ? 1.0f : __builtin_amdgcn_exp2f((float)e * lg);
    }
};

template <typename TI, int DK, int DV> constexpr int bwd_cmax() {
    // fp32 and bf16-pair tiles take twice the bf16 bytes
    return ((sizeof(TI) == 4 || std::is_same<TI, bf16p>::value) && (DK > 64 || DV > 64)) ? 32 : 64;
}

// Leading dimensions (elements) of a tile of D columns (padded to >= 32).
template <typename TC, int D> struct BwdLd {
    static constexpr int DP = D < 32 ? 32 : D;
    static constexpr int ROW = DP + (sizeof(TC) == 2 ? 8 : 4);  // row-wise reads
    static constexpr int TR = DP + (sizeof(TC) == 2 ? 16 : 4);  // transpose reads
};

// Block b of the lower triangle of a 4 x 4 block grid, row by row:
// (0,0), (1,0), (1,1), (2,0), ...
__device__ __forceinline__ void lower_block(int b, int &I, int &J) {
    I = (b >= 1) + (b >= 3) + (b >= 6);
    J = b - I * (I + 1) / 2;
}

// One chunk of rows of a [N][D] tensor held in registers between its global
// load and its LDS store, so that the loads of chunk c + 1 are in flight while
// chunk c is computed.  Every lane issues the same number of loads (rows past
// the chunk's end are clamped to its last row and zeroed at the store), which
// keeps the wait before the store exact.
template <typename T> struct plane_of {
    static constexpr int value = 0;
};
template <int PL> struct plane_of<bf16pl<PL>> {
    static constexpr int value = PL;
};

template <typename TI, int D, int NT, int CM> struct RowRegs {
    static constexpr bool HALVES = std::is_same<TI, bf16h>::value;  // two bf16 planes, `plane` elements apart
    static constexpr int VEC = Store<TI>::VEC;
    static constexpr int VPR = D / VEC;  // 16-byte vectors per row (of one plane)
    static constexpr int NV = CM * VPR;
    static constexpr int NIT = (NV + NT - 1) / NT;
    uint4 u[NIT];
    uint4 ul[HALVES ? NIT : 1];  // the remainder plane's vectors

    __device__ __forceinline__ void load(const void *src, long row_base, int r0, int nrows, int tid, long plane = 0) {
        constexpr long ES = HALVES ? 2 : (long)sizeof(TI);  // bytes per element of a plane
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int idx = tid + it * NT;
            const int row = min(idx / VPR, nrows - 1);
            const int col = (idx % VPR) * VEC;
            const char *at = static_cast<const char *>(src) + ((row_base + r0 + row) * D + col) * ES;
            u[it] = load_stream16(at);
            if constexpr (HALVES) ul[it] = load_stream16(at + plane * ES);
        }
    }

    // phi of the loaded values, in place (16-byte vectors of TI); nothing for
    // the identity map.
    __device__ __forceinline__ void apply_phi(bool ident) {
        if constexpr (HALVES) {
            return;  // features given (identity map only)
        } else {
            if (ident) return;
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                float x[VEC];
                unpack16(u[it], x, TI());
                if constexpr (sizeof(TI) == 2) {
                    const f32x4 a = {phi(x[0]), phi(x[1]), phi(x[2]), phi(x[3])};
                    const f32x4 b = {phi(x[4]), phi(x[5]), phi(x[6]), phi(x[7])};
                    const uint2 pa = pack_bf16x4(a), pb = pack_bf16x4(b);
                    u[it] = make_uint4(pa.x, pa.y, pb.x, pb.y);
                } else {
                    u[it] = make_uint4(__float_as_uint(phi(x[0])), __float_as_uint(phi(x[1])),
                                       __float_as_uint(phi(x[2])), __float_as_uint(phi(x[3])));
                }
            }
        }
    }

    // Rows [0, CM) of the tile (leading dimension LD) from the registers; zero
    // past nrows (FULL: the caller knows nrows == CM).  Loaded value and
    // remainder planes go to the two planes of a pair tile.
    template <int LD, bool FULL, typename TT>
    __device__ __forceinline__ void store(TT *tile, int nrows, int tid) const {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int idx = tid + it * NT;
            if (NV % NT != 0 && idx >= NV) continue;
            const int row = idx / VPR;
            const int col = (idx % VPR) * VEC;
            uint4 w = (FULL || row < nrows) ? u[it] : make_uint4(0, 0, 0, 0);
            if constexpr (HALVES) {  // value plane and remainder plane into the tile's two planes
                const uint4 l = (FULL || row < nrows) ? ul[it] : make_uint4(0, 0, 0, 0);
                *reinterpret_cast<uint4 *>(tile + row * LD + col) = w;
                *reinterpret_cast<uint4 *>(tile + row * LD + col + plane_of<TT>::value) = l;
            } else {
                static_assert(std::is_same<TT, TI>::value, "staging: tile of the loaded type, or planes into pairs");
                *reinterpret_cast<uint4 *>(tile + row * LD + col) = w;
            }
        }
    }
};

// (TI = bf16p, the pair sweeps: fp32 outputs, as for TI = float.)
template <typename TI>
__device__ __forceinline__ void store4(void *dst, long idx, const f32x4 &a) {
    if constexpr (std::is_same<TI, __bf16>::value) {
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(dst) + idx) = pack_bf16x4(a);
    } else {
        *reinterpret_cast<f32x4 *>(static_cast<float *>(dst) + idx) = a;
    }
}

// ---------------------------------------------------------------------------
// dq sweep (forward over chunks, state S, z).  It also forms, once a chunk's
// a = 1 / den and e = eps * den are known, its segment's share of the dk/dv
// sweep's suffix state: R_seg = sum_i (phi(q_i) a_i) g_i^T and
// r_seg = sum_i (phi(q_i) a_i) e_i over the segment (token p of the segment
// weighs gamma^p with a decay), so no separate pass re-reads q and dO.
// ---------------------------------------------------------------------------
// Tile types.  Input type TI, except with bf16-pair sweeps (TI = bf16p):
//   bwd_tv  v and dO: bf16 tiles (their values are bf16 exactly), whose
//           fragments meet pairs in two-MFMA products;
//   bwd_ts  element of a plane, for strides: bf16;
//   bwd_pt  the other tiles: two bf16 planes, the remainder plane PL elements
//           after the value plane (NPL planes in all).
template <typename TI> constexpr bool bwd_pair() { return std::is_same<TI, bf16p>::value; }
template <typename TI> using bwd_tv = typename std::conditional<bwd_pair<TI>(), __bf16, TI>::type;
template <typename TI> using bwd_ts = typename std::conditional<bwd_pair<TI>(), __bf16, TI>::type;
template <typename TI, int PL> using bwd_pt = typename std::conditional<bwd_pair<TI>(), bf16pl<PL>, TI>::type;
template <typename TI> constexpr int bwd_npl() { return bwd_pair<TI>() ? 2 : 1; }

template <int DK, int DV, typename TI, bool DEC = false> struct DqSmem {
    static constexpr int CM = bwd_cmax<TI, DK, DV>();
    using TS = bwd_ts<TI>;
    static constexpr int NPL = bwd_npl<TI>();
    static constexpr int LK = BwdLd<TS, DK>::TR;   // phi(K): transpose reads
    static constexpr int LQ = BwdLd<TS, DK>::ROW;  // phi(Q): row reads
    using TV = bwd_tv<TI>;
    static constexpr int LV = BwdLd<TV, DV>::TR;   // V: transpose reads (state), row reads (M)
    static constexpr int LG = BwdLd<TV, DV>::ROW;  // dO: row reads
    static constexpr int LM = BwdLd<TS, CM>::ROW;  // M[i][j]
    static constexpr bool LO = std::is_same<TI, __bf16>::value;  // M kept as value + remainder
    alignas(16) bwd_pt<TI, CM * LK> k[NPL * CM * LK];
    alignas(16) bwd_pt<TI, CM * LQ> q[NPL * CM * LQ];
    alignas(16) TV v[CM * LV];
    alignas(16) TV g[CM * LG];
    alignas(16) bwd_pt<TI, CM * LM> mh[NPL * CM * LM];
    alignas(16) bwd_pt<TI, CM * LM> ml[LO ? CM * LM : 4];
    alignas(16) float red[kBwdWaves][CM][2];  // per-wave partial phi(q).X and phi(q).z
    // decay weights gamma^(i - j) of query i and token j <= i, as value + remainder
    alignas(16) TI dh[DEC ? CM * LM : 8];
    alignas(16) TI dl[DEC && LO ? CM * LM : 8];
};

template <int DK, int DV, typename TI, bool NC = false, bool DECAY = false>
__global__ void __launch_bounds__(kBwdThreads)
la_bwd_dq_kernel(const BwdParams p) {
    using TC = TI;
    using TV = bwd_tv<TI>;  // v and dO tiles and fragments
    constexpr bool dec = DECAY && !NC;
    using SM = DqSmem<DK, DV, TI, dec>;
    constexpr int NW = kBwdWaves;
    constexpr int EB = DK / 16;          // feature blocks, one per wave
    constexpr int CV = DV / 16;          // value tiles of the state
    constexpr int NSV = (DV + 31) / 32;  // value K steps
    constexpr int NIB = SM::CM / 16;     // 16-row blocks of a full chunk
    constexpr int NTS = SM::CM / 32;     // 32-token K steps of a full chunk
    static_assert(EB <= NW, "one feature block per wave");
    __shared__ SM sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, pp = lane & 15;
    const long bh = blockIdx.x;
    const int seg = blockIdx.y;
    const int C = p.C, N = p.N;
    const int row_begin = seg * p.L;
    const int row_end = min(N, row_begin + p.L);
    const int nch = (row_end - row_begin + C - 1) / C;
    const int nib = C / 16;
    const bool ident = p.phi_id != 0;  // uniform: identity feature map
    const bool active = EB >= NW || wave < EB;
    const int eb = wave;

    {
        uint32_t *w = reinterpret_cast<uint32_t *>(&sm);
        for (int i = tid; i < (int)(sizeof(SM) / 4); i += kBwdThreads) w[i] = 0u;
    }
    const Decay dcy{dec ? __builtin_log2f(p.gamma[bh % p.H]) : 0.0f};
    if constexpr (dec) {
        __syncthreads();  // the zero fill is done; the first chunk's barrier orders these writes
        for (int idx = tid; idx < SM::CM * SM::CM; idx += kBwdThreads) {
            const int i = idx / SM::CM, j = idx % SM::CM;
            const float w = j <= i ? dcy.pow(i - j) : 0.0f;
            sm.dh[i * SM::LM + j] = static_cast<TC>(w);
            if constexpr (SM::LO) sm.dl[i * SM::LM + j] = static_cast<TC>(w - static_cast<float>(static_cast<TC>(w)));
        }
    }

    // S^T(c', eb) tiles: lane (pp, g) holds S[16 eb + pp][16 c' + 4g + r]; z(eb): z[16 eb + 4g + r].
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 accS[CV];
    f32x4 accZ = zero4;
#pragma unroll
    for (int cv = 0; cv < CV; ++cv) accS[cv] = zero4;
    if (p.state && active) {
        const float *Sin = p.state + (bh * p.state_P + (long)seg * p.state_mult) * (long)(DK * DV + DK);
        // non-causal: the per-segment sums, added slot by slot in a fixed order
        for (int t = 0; t < (NC ? p.sum_P : 1); ++t, Sin += DK * DV + DK) {
#pragma unroll
            for (int r = 0; r < 4; ++r) accZ[r] += Sin[DK * DV + 16 * eb + 4 * g + r];
#pragma unroll
            for (int cv = 0; cv < CV; ++cv)
#pragma unroll
                for (int r = 0; r < 4; ++r) accS[cv][r] += Sin[(16 * eb + pp) * DV + 16 * cv + 4 * g + r];
        }
    }
    // this segment's suffix sums (segment 0's are never read): R^T(c', eb) tiles,
    // lane (pp, g) holding R[16 eb + pp][16 c' + 4g + r], and r(eb) as r[16 eb + 4g + r]
    const bool suf = !NC && p.suf_out != nullptr && seg > 0;  // uniform
    f32x4 accRs[NC ? 1 : CV];
    f32x4 accrs = zero4;
#pragma unroll
    for (int cv = 0; cv < (NC ? 1 : CV); ++cv) accRs[cv] = zero4;
    Frag<TC> fragS[NSV];  // S rows e, split over the value index
    // Non-causal, or decayed, with bf16 operands: S also as its rounding
    // remainder, so that X = S g and z meet at fp32-level accuracy in
    // X - z (phi(q) . X) / den, whose two terms cancel exactly for a single
    // token (non-causal) and to O(gamma) of their size for a fast decay.
    constexpr bool SLO = (NC || dec) && std::is_same<TC, __bf16>::value;
    Frag<TC> fragS_lo[SLO ? NSV : 1];
    auto refresh = [&]() {
#pragma unroll
        for (int s = 0; s < NSV; ++s) {
            acc_to_frag(fragS[s], accS[2 * s], (2 * s + 1 < CV) ? accS[2 * s + 1] : zero4);
            if constexpr (SLO) acc_to_frag_lo(fragS_lo[s], accS[2 * s], (2 * s + 1 < CV) ? accS[2 * s + 1] : zero4);
        }
    };
    refresh();
    Frag<TV> ones;
    frag_ones(ones);

    // q, k: two bf16 planes (value, remainder) for bf16-pair sweeps
    using TQ = typename std::conditional<std::is_same<TI, bf16p>::value, bf16h, TI>::type;
    const long fplane = (long)gridDim.x * N * DK;  // elements per plane
    RowRegs<TQ, DK, kBwdThreads, SM::CM> xk, xq;
    RowRegs<TV, DV, kBwdThreads, SM::CM> xv, xg;
    auto fetch = [&](int ch) {
        const int r0 = row_begin + ch * C;
        const int nrows = min(C, row_end - r0);
        if constexpr (!NC) xk.load(p.k, bh * N, r0, nrows, tid, fplane);
        xq.load(p.q, bh * N, r0, nrows, tid, fplane);
        if constexpr (!NC) xv.load(p.v, bh * N, r0, nrows, tid);
        xg.load(p.g, bh * N, r0, nrows, tid);
    };
    if (nch > 0) {
        fetch(0);
        if constexpr (!NC) xk.apply_phi(ident);
        xq.apply_phi(ident);
    }

    // per-lane bases of the row-wise reads: row pp, column 4g
    const lds_vptr<TV> gb = lds_v(sm.g + pp * SM::LG + 4 * g);
    const lds_vptr<TV> vb = lds_v(sm.v + pp * SM::LV + 4 * g);
    const auto qb = lds_v(sm.q + pp * SM::LQ + 16 * eb + 4 * g);
    const auto mhb = lds_v(sm.mh + pp * SM::LM + 4 * g);
    const auto mlb = lds_v(sm.ml + (SM::LO ? pp * SM::LM + 4 * g : 0));
    const auto dhb = lds_v(sm.dh + (dec ? pp * SM::LM + 4 * g : 0));
    const auto dlb = lds_v(sm.dl + (dec && SM::LO ? pp * SM::LM + 4 * g : 0));

    for (int ch = 0; ch < nch; ++ch) {
        const int r0 = row_begin + ch * C;
        const int nrows = min(C, row_end - r0);
        __syncthreads();  // previous chunk's tile reads done
        // (phi(k), phi(q) were applied in registers during the previous chunk)
        if (nrows == SM::CM) {
            if constexpr (!NC) xk.template store<SM::LK, true>(sm.k, nrows, tid);
            xq.template store<SM::LQ, true>(sm.q, nrows, tid);
            if constexpr (!NC) xv.template store<SM::LV, true>(sm.v, nrows, tid);
            xg.template store<SM::LG, true>(sm.g, nrows, tid);
        } else {
            if constexpr (!NC) xk.template store<SM::LK, false>(sm.k, nrows, tid);
            xq.template store<SM::LQ, false>(sm.q, nrows, tid);
            if constexpr (!NC) xv.template store<SM::LV, false>(sm.v, nrows, tid);
            xg.template store<SM::LG, false>(sm.g, nrows, tid);
        }
        __syncthreads();
        if (ch + 1 < nch) fetch(ch + 1);

        // Masked M_ij = g_i . v_j (j <= i) over the blocks I >= J, one block
        // per wave and pass; blocks above the diagonal stay zero in LDS.
        for (int b = wave; !NC && b < nib * (nib + 1) / 2; b += NW) {
            int I, J;
            lower_block(b, I, J);
            f32x4 acc = zero4;
#pragma unroll
            for (int s = 0; s < NSV; ++s) {
                Frag<TV> fv, fg;
                lds_frag_split_v(fv, vb, 16 * J * SM::LV + 32 * s);
                lds_frag_split_v(fg, gb, 16 * I * SM::LG + 32 * s);
                acc = mma(fv, fg, acc);
            }
            // lane: tokens j = 16 J + 4g + r of query i = 16 I + pp
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int e = 16 * (I - J) + pp - 4 * g - r;  // i - j
                if (I == J && e < 0) acc[r] = 0.f;
                else if constexpr (dec) acc[r] *= dcy.pow(e);
            }
            const int off = (16 * I + pp) * SM::LM + 16 * J + 4 * g;
            lds_put4_pair(sm.mh + off, sm.ml + (SM::LO ? off : 0), acc);
        }
        __syncthreads();

        // X(eb, I) = sum_{j<=i} M_ij phi(k_j) + S g_i and Z(eb, I) = z_i, both
        // with rows e = 16 eb + 4g + r of query column i = 16 I + pp.
        f32x4 X[NIB], Z[NIB];
        Frag<TC> fkt[NTS];  // phi(K) over tokens (split), features 16 eb + pp
        if (active) {
#pragma unroll
            for (int jp = 0; jp < NTS; ++jp)
                if constexpr (!NC) lds_frag_tr(fkt[jp], sm.k, SM::LK, 32 * jp + 4 * g, 32 * jp + 16 + 4 * g, 16 * eb, pp);
#pragma unroll
            for (int I = 0; I < NIB; ++I) {
                X[I] = zero4;
                Z[I] = zero4;
                if (I < nib) {
                    Frag<TV> fg[NSV];
#pragma unroll
                    for (int s = 0; s < NSV; ++s) lds_frag_split_v(fg[s], gb, 16 * I * SM::LG + 32 * s);
                    f32x4 ax = zero4, az = accZ;
                    if constexpr (dec) {  // the carried state's terms first, decayed by gamma^(tau_i + 1)
#pragma unroll
                        for (int s = 0; s < NSV; ++s) {
                            ax = mma(fragS[s], fg[s], ax);
                            if constexpr (SLO) ax = mma(fragS_lo[s], fg[s], ax);
                        }
                        const float gi = dcy.pow(16 * I + pp + 1);
                        ax = ax * gi;
                        az = accZ * gi;
                    }
#pragma unroll
                    for (int jp = 0; jp < NTS; ++jp) {
                        if (!NC && 2 * jp <= I) {
                            Frag<TC> fm;
                            Frag<TV> ftr;
                            lds_frag_split_v(fm, mhb, 16 * I * SM::LM + 32 * jp);
                            ax = mma(fkt[jp], fm, ax);
                            if constexpr (SM::LO) {
                                lds_frag_split_v(fm, mlb, 16 * I * SM::LM + 32 * jp);
                                ax = mma(fkt[jp], fm, ax);
                            }
                            if constexpr (dec) {  // decay weights over the same tokens (value + remainder)
                                lds_frag_split_v(ftr, dhb, 16 * I * SM::LM + 32 * jp);
                                az = mma(fkt[jp], ftr, az);
                                if constexpr (SM::LO) {
                                    lds_frag_split_v(ftr, dlb, 16 * I * SM::LM + 32 * jp);
                                    az = mma(fkt[jp], ftr, az);
                                }
                            } else {
                                const int i = 16 * I + pp;
#pragma unroll
                                for (int t = 0; t < 4; ++t) {  // causal all-ones mask over the same tokens
                                    ftr.set(t, 32 * jp + 4 * g + t <= i ? 1.f : 0.f);
                                    ftr.set(t + 4, 32 * jp + 16 + 4 * g + t <= i ? 1.f : 0.f);
                                }
                                az = mma(fkt[jp], ftr, az);
                            }
                        }
                    }
                    if constexpr (!dec) {
#pragma unroll
                        for (int s = 0; s < NSV; ++s) {
                            ax = mma(fragS[s], fg[s], ax);
                            if constexpr (SLO) ax = mma(fragS_lo[s], fg[s], ax);
                        }
                    }
                    const f32x4 fq = lds_get4(qb, 16 * I * SM::LQ);
                    float px = 0.f, pz = 0.f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        px += fq[r] * ax[r];
                        pz += fq[r] * az[r];
                    }
                    px = sum_over_groups_swap(px);
                    pz = sum_over_groups_swap(pz);
                    if (g == 0) {
                        sm.red[wave][16 * I + pp][0] = px;
                        sm.red[wave][16 * I + pp][1] = pz;
                    }
                    X[I] = ax;
                    Z[I] = az;
                }
            }
        }
        __syncthreads();  // partial dot products of every wave are in LDS
        float a_row[NIB], e_row[NIB];  // a and e of query 16 I + pp
#pragma unroll
        for (int I = 0; I < NIB; ++I) a_row[I] = e_row[I] = 0.f;
        if (active) {
#pragma unroll
            for (int I = 0; I < NIB; ++I) {
                if (I < nib) {
                    const int row_local = 16 * I + pp;
                    float t = 0.f, den = 0.f;
#pragma unroll
                    for (int w = 0; w < EB; ++w) {
                        t += sm.red[w][row_local][0];
                        den += sm.red[w][row_local][1];
                    }
                    const float inv = __builtin_amdgcn_rcpf(den);
                    const float coef = t * inv;
                    const bool valid = row_local < nrows;
                    const long orow = bh * N + r0 + row_local;
                    if (wave == 0 && g == 0 && valid) {
                        p.inv_den[orow] = inv;
                        p.eps[orow] = -coef;
                    }
                    a_row[I] = valid ? inv : 0.f;  // every lane group holds its rows' values
                    e_row[I] = valid ? -coef : 0.f;
                    const f32x4 fq = lds_get4(qb, 16 * I * SM::LQ);
                    f32x4 out;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        out[r] = (X[I][r] - Z[I][r] * coef) * inv * (ident ? 1.0f : fminf(fq[r], 1.0f));
                    // pair sweeps (random features): u = dphi(q) * phi(q), what the
                    // chain rule through the map takes
                    if constexpr (bwd_pair<TI>()) out = out * fq;
                    if (valid) store4<TI>(p.dq, orow * DK + 16 * eb + 4 * g, out);
                }
            }
        }
        if constexpr (!NC) {
            if (suf && active) {
                {
                    // R_seg^T(c', eb) += dO^T(c') (w a phi(Q))(eb), r_seg(eb) += (w a phi(Q))(eb)^T e,
                    // w = gamma^(position in the segment) (1 without decay).  The
                    // operands run over tokens: slot t of lane group g is token
                    // 32 s + 4g + t (+16), whose a and e lane 4g + t holds.
#pragma unroll
                    for (int s = 0; s < NTS; ++s) {
                        f32x4 a0, a1, e0, e1;
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            a0[t] = __shfl(a_row[2 * s], 4 * g + t, 64);
                            a1[t] = __shfl(a_row[2 * s + 1], 4 * g + t, 64);
                            e0[t] = __shfl(e_row[2 * s], 4 * g + t, 64);
                            e1[t] = __shfl(e_row[2 * s + 1], 4 * g + t, 64);
                        }
                        Frag<TC> fqt, fq, fe, fe_lo;
                        lds_frag_tr(fqt, sm.q, SM::LQ, 32 * s + 4 * g, 32 * s + 16 + 4 * g, 16 * eb, pp);
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const float w0 = dec ? dcy.pow(ch * C + 32 * s + 4 * g + t) : 1.0f;
                            const float w1 = dec ? dcy.pow(ch * C + 32 * s + 16 + 4 * g + t) : 1.0f;
                            fq.set(t, fqt.get(t) * (a0[t] * w0));
                            fq.set(t + 4, fqt.get(t + 4) * (a1[t] * w1));
                            fe.set(t, e0[t]);
                            fe.set(t + 4, e1[t]);
                            fe_lo.set(t, e0[t] - fe.get(t));
                            fe_lo.set(t + 4, e1[t] - fe.get(t + 4));
                        }
                        accrs = mma(fq, fe, accrs);
                        if constexpr (SM::LO) accrs = mma(fq, fe_lo, accrs);
#pragma unroll
                        for (int cv = 0; cv < CV; ++cv) {
                            Frag<TV> fgc;
                            lds_frag_tr(fgc, sm.g, SM::LG, 32 * s + 4 * g, 32 * s + 16 + 4 * g, 16 * cv, pp);
                            accRs[cv] = mma(fgc, fq, accRs[cv]);
                        }
                    }
                }
            }
        }
        // phi of the next chunk's rows (after the last chunk the registers are not used again)
        if constexpr (!NC) xk.apply_phi(ident);
        xq.apply_phi(ident);
        if (active && !NC) {
            // state carry: S^T(c', eb) += V^T(c') phi(K)(eb), z(eb) += phi(K)(eb)^T 1
            // (token rows past the chunk are zero in the tiles; with decay the
            // state first decays by gamma^R and token j weighs gamma^(R - 1 - tau_j))
            if constexpr (dec) {
                const float gR = dcy.pow(nrows);
                accZ = accZ * gR;
#pragma unroll
                for (int cv = 0; cv < CV; ++cv) accS[cv] = accS[cv] * gR;
            }
#pragma unroll
            for (int s = 0; s < NTS; ++s) {
                // weighted phi(k) as a value and its remainder (bf16), as in the
                // aggregate that feeds the segment states
                Frag<TC> fkl;
                if constexpr (dec) {
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const int tok = 32 * s + (t < 4 ? 4 * g + t : 16 + 4 * g + t - 4);
                        const float x = tok < nrows ? fkt[s].get(t) * dcy.pow(nrows - 1 - tok) : 0.0f;
                        fkt[s].set(t, x);
                        if constexpr (SLO) fkl.set(t, x - fkt[s].get(t));
                    }
                }
                accZ = mma(fkt[s], ones, accZ);
                if constexpr (dec && SLO) accZ = mma(fkl, ones, accZ);
#pragma unroll
                for (int cv = 0; cv < CV; ++cv) {
                    Frag<TV> fvt;
                    lds_frag_tr(fvt, sm.v, SM::LV, 32 * s + 4 * g, 32 * s + 16 + 4 * g, 16 * cv, pp);
                    accS[cv] = mma(fvt, fkt[s], accS[cv]);
                    if constexpr (dec && SLO) accS[cv] = mma(fvt, fkl, accS[cv]);
                }
            }
            refresh();
        }
    }
    if constexpr (!NC) {
        if (suf && active) {
            float *Rs = p.suf_out + (bh * p.suf_P + seg) * (long)(DK * DV + DK);
#pragma unroll
            for (int cv = 0; cv < CV; ++cv)
#pragma unroll
                for (int r = 0; r < 4; ++r) Rs[(16 * eb + pp) * DV + 16 * cv + 4 * g + r] = accRs[cv][r];
            if (pp == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r) Rs[DK * DV + 16 * eb + 4 * g + r] = accrs[r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// dk / dv sweep (backward over chunks, state R, r).
// ---------------------------------------------------------------------------
template <int DK, int DV, typename TI> struct DkvSmem {
    static constexpr int CM = bwd_cmax<TI, DK, DV>();
    using TS = bwd_ts<TI>;
    static constexpr int NPL = bwd_npl<TI>();
    static constexpr int LQ = BwdLd<TS, DK>::TR;   // phi(Q): transpose reads (dk, state), row reads (A)
    static constexpr int LK = BwdLd<TS, DK>::ROW;  // phi(K): row reads
    using TV = bwd_tv<TI>;
    static constexpr int LV = BwdLd<TV, DV>::ROW;  // V: row reads
    static constexpr int LG = BwdLd<TV, DV>::TR;   // dO: transpose reads (dv, state), row reads (M)
    static constexpr int LR = BwdLd<TS, DV>::TR;   // R[e][c']: transpose reads
    static constexpr int LM = BwdLd<TS, CM>::ROW;  // M[j][i], A[j][i]
    static constexpr int RROWS = DK < 32 ? 32 : DK;
    static constexpr bool LO = std::is_same<TI, __bf16>::value;
    alignas(16) bwd_pt<TI, CM * LQ> q[NPL * CM * LQ];
    alignas(16) bwd_pt<TI, CM * LK> k[NPL * CM * LK];
    alignas(16) TV v[CM * LV];
    alignas(16) TV g[CM * LG];
    alignas(16) bwd_pt<TI, RROWS * LR> R[NPL * RROWS * LR];  // copy of the suffix state R[e][c'] for the dv product
    alignas(16) bwd_pt<TI, CM * LM> mh[NPL * CM * LM];
    alignas(16) bwd_pt<TI, CM * LM> ml[LO ? CM * LM : 4];
    alignas(16) bwd_pt<TI, CM * LM> at[NPL * CM * LM];
    alignas(16) float e[CM];  // e = eps * den
    alignas(16) float a[CM];  // a = 1 / den
};

template <int DK, int DV, typename TI, bool NC = false, bool DECAY = false>
__global__ void __launch_bounds__(kBwdThreads)
la_bwd_dkdv_kernel(const BwdParams p) {
    using TC = TI;
    using TV = bwd_tv<TI>;  // v and dO tiles and fragments
    constexpr bool dec = DECAY && !NC;
    using SM = DkvSmem<DK, DV, TI>;
    constexpr int NW = kBwdWaves;
    constexpr int EB = DK / 16, CB = DV / 16, CV = DV / 16;
    constexpr int NSV = (DV + 31) / 32;
    constexpr int NSE = (DK + 31) / 32;
    constexpr int NIB = SM::CM / 16;
    constexpr int NTS = SM::CM / 32;
    static_assert(EB <= NW && CB <= NW, "one feature block and one value block per wave");
    __shared__ SM sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, pp = lane & 15;
    const long bh = blockIdx.x;
    const int seg = blockIdx.y;
    const int C = p.C, N = p.N;
    const int row_begin = seg * p.L;
    const int row_end = min(N, row_begin + p.L);
    const int nch = (row_end - row_begin + C - 1) / C;
    const int nib = C / 16;
    const bool ident = p.phi_id != 0;  // uniform: identity feature map
    const bool has_e = EB >= NW || wave < EB, has_c = CB >= NW || wave < CB;
    const int eb = wave, cb = wave;

    {
        uint32_t *w = reinterpret_cast<uint32_t *>(&sm);
        for (int i = tid; i < (int)(sizeof(SM) / 4); i += kBwdThreads) w[i] = 0u;
    }
    __syncthreads();
    const Decay dcy{dec ? __builtin_log2f(p.gamma[bh % p.H]) : 0.0f};

    // R^T(c', eb) tiles: lane (pp, g) holds R[16 eb + pp][16 c' + 4g + r]; r(eb): r[16 eb + 4g + r].
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 accR[CV];
    f32x4 accr = zero4;
#pragma unroll
    for (int cv = 0; cv < CV; ++cv) accR[cv] = zero4;
    if (p.state && has_e) {
        // suffix state after this segment: the exclusive suffix of its last fine
        // segment (non-causal: the total, in slot 0)
        const long last = NC ? 0 : min((long)(seg + 1) * p.state_mult, (long)p.state_P) - 1;
        const float *Rin = p.state + (bh * p.state_P + last) * (long)(DK * DV + DK);
        for (int t = 0; t < (NC ? p.sum_P : 1); ++t, Rin += DK * DV + DK) {
#pragma unroll
            for (int r = 0; r < 4; ++r) accr[r] += Rin[DK * DV + 16 * eb + 4 * g + r];
#pragma unroll
            for (int cv = 0; cv < CV; ++cv)
#pragma unroll
                for (int r = 0; r < 4; ++r) accR[cv][r] += Rin[(16 * eb + pp) * DV + 16 * cv + 4 * g + r];
        }
    }
    Frag<TC> fragR[NSV];  // R rows e, split over the value index
    // Non-causal, or decayed, with bf16 operands: R also as its rounding
    // remainder, so that R v_j and r meet at fp32-level accuracy (they cancel
    // for a single token, and to O(gamma) of their size for a fast decay).
    constexpr bool RLO = (NC || dec) && std::is_same<TC, __bf16>::value;
    Frag<TC> fragR_lo[RLO ? NSV : 1];
    auto refresh = [&]() {
#pragma unroll
        for (int s = 0; s < NSV; ++s) {
            acc_to_frag(fragR[s], accR[2 * s], (2 * s + 1 < CV) ? accR[2 * s + 1] : zero4);
            if constexpr (RLO) acc_to_frag_lo(fragR_lo[s], accR[2 * s], (2 * s + 1 < CV) ? accR[2 * s + 1] : zero4);
        }
#pragma unroll
        for (int cv = 0; cv < CV; ++cv) lds_put4(&sm.R[(16 * eb + pp) * SM::LR + 16 * cv + 4 * g], accR[cv]);
    };
    if (has_e) refresh();

    using TQ = typename std::conditional<std::is_same<TI, bf16p>::value, bf16h, TI>::type;
    const long fplane = (long)gridDim.x * N * DK;  // elements per plane
    RowRegs<TQ, DK, kBwdThreads, SM::CM> xq, xk;
    RowRegs<TV, DV, kBwdThreads, SM::CM> xv, xg;
    float xe = 0.f, xa = 0.f;  // e and a of token tid (tid < CM)
    auto fetch = [&](int ch) {
        const int r0 = row_begin + ch * C;
        const int nrows = min(C, row_end - r0);
        if constexpr (!NC) xq.load(p.q, bh * N, r0, nrows, tid, fplane);
        xk.load(p.k, bh * N, r0, nrows, tid, fplane);
        xv.load(p.v, bh * N, r0, nrows, tid);
        if constexpr (!NC) xg.load(p.g, bh * N, r0, nrows, tid);
        if (!NC && tid < SM::CM) {
            const long t = bh * N + r0 + min(tid, nrows - 1);
            xe = p.eps[t];
            xa = p.inv_den[t];
        }
    };
    if (nch > 0) {
        fetch(nch - 1);
        if constexpr (!NC) xq.apply_phi(ident);
        xk.apply_phi(ident);
    }

    // per-lane bases of the row-wise reads: row pp, column 4g
    const auto qb = lds_v(sm.q + pp * SM::LQ + 4 * g);
    const auto kb = lds_v(sm.k + pp * SM::LK + 4 * g);
    const lds_vptr<TV> vb = lds_v(sm.v + pp * SM::LV + 4 * g);
    const lds_vptr<TV> gb = lds_v(sm.g + pp * SM::LG + 4 * g);
    const auto mhb = lds_v(sm.mh + pp * SM::LM + 4 * g);
    const auto mlb = lds_v(sm.ml + (SM::LO ? pp * SM::LM + 4 * g : 0));
    const auto atb = lds_v(sm.at + pp * SM::LM + 4 * g);

    for (int ch = nch - 1; ch >= 0; --ch) {
        const int r0 = row_begin + ch * C;
        const int nrows = min(C, row_end - r0);
        __syncthreads();  // previous chunk's tile reads done
        // (phi(q), phi(k) were applied in registers during the previous chunk)
        if (nrows == SM::CM) {
            if constexpr (!NC) xq.template store<SM::LQ, true>(sm.q, nrows, tid);
            xk.template store<SM::LK, true>(sm.k, nrows, tid);
            xv.template store<SM::LV, true>(sm.v, nrows, tid);
            if constexpr (!NC) xg.template store<SM::LG, true>(sm.g, nrows, tid);
        } else {
            if constexpr (!NC) xq.template store<SM::LQ, false>(sm.q, nrows, tid);
            xk.template store<SM::LK, false>(sm.k, nrows, tid);
            xv.template store<SM::LV, false>(sm.v, nrows, tid);
            if constexpr (!NC) xg.template store<SM::LG, false>(sm.g, nrows, tid);
        }
        if (!NC && tid < SM::CM) {
            sm.e[tid] = tid < nrows ? xe : 0.f;
            sm.a[tid] = tid < nrows ? xa : 0.f;
        }
        __syncthreads();
        if (ch > 0) fetch(ch - 1);

        // Over the blocks I >= J, one block per wave and pass (M blocks, then A blocks):
        //   M_ij = (g_i . v_j + e_i) a_i,  A_ij = (phi(q_i) . phi(k_j)) a_i  (i >= j),
        // stored transposed, [j][i]; blocks above the diagonal stay zero in LDS.
        const int nblk = nib * (nib + 1) / 2;
        for (int b = wave; !NC && b < 2 * nblk; b += NW) {
            const bool is_a = b >= nblk;
            int I, J;
            lower_block(is_a ? b - nblk : b, I, J);
            f32x4 acc = zero4;
            if (!is_a) {
#pragma unroll
                for (int s = 0; s < NSV; ++s) {
                    Frag<TV> fg, fv;
                    lds_frag_split_v(fg, gb, 16 * I * SM::LG + 32 * s);
                    lds_frag_split_v(fv, vb, 16 * J * SM::LV + 32 * s);
                    acc = mma(fg, fv, acc);
                }
            } else {
#pragma unroll
                for (int s = 0; s < NSE; ++s) {
                    Frag<TC> fq, fk;
                    lds_frag_split_v(fq, qb, 16 * I * SM::LQ + 32 * s);
                    lds_frag_split_v(fk, kb, 16 * J * SM::LK + 32 * s);
                    acc = mma(fq, fk, acc);
                }
            }
            // lane: queries i = 16 I + 4g + r of token j = 16 J + pp
            const f32x4 ev = *reinterpret_cast<const f32x4 *>(&sm.e[16 * I + 4 * g]);
            const f32x4 av = *reinterpret_cast<const f32x4 *>(&sm.a[16 * I + 4 * g]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int e = 16 * (I - J) + 4 * g + r - pp;  // i - j
                const bool keep = !(I == J && e < 0);
                const float w = dec && keep ? dcy.pow(e) : 1.0f;
                // bf16 pairs: g_i . v_j as the dq sweep's M tile held it, the
                // value e_i was formed from (a lone token's g . v + e is then 0)
                const float gv = std::is_same<TC, bf16p>::value && !is_a ? to_operand<TC>(acc[r]) : acc[r];
                acc[r] = keep ? (is_a ? acc[r] : gv + ev[r]) * av[r] * w : 0.f;
            }
            const int off = (16 * J + pp) * SM::LM + 16 * I + 4 * g;
            if (!is_a)
                lds_put4_pair(sm.mh + off, sm.ml + (SM::LO ? off : 0), acc);
            else
                lds_put4(sm.at + off, acc);
        }
        // R^T rows c' = 16 cb + pp over features (split): A operand of the dv product
        Frag<TC> frt[NSE];
        if (has_c) {
#pragma unroll
            for (int s = 0; s < NSE; ++s)
                lds_frag_tr(frt[s], sm.R, SM::LR, 32 * s + 4 * g, 32 * s + 16 + 4 * g, 16 * cb, pp);
        }
        __syncthreads();  // M and A blocks are in LDS; R copy reads done

        Frag<TC> fqt[NTS];  // phi(Q) (features 16 eb + pp) over queries
        Frag<TV> fgt[NTS];  // dO (values 16 cb + pp) over queries
        if (has_e && !NC) {
#pragma unroll
            for (int ip = 0; ip < NTS; ++ip)
                lds_frag_tr(fqt[ip], sm.q, SM::LQ, 32 * ip + 4 * g, 32 * ip + 16 + 4 * g, 16 * eb, pp);
        }
        if (has_c && !NC) {
#pragma unroll
            for (int ip = 0; ip < NTS; ++ip)
                lds_frag_tr(fgt[ip], sm.g, SM::LG, 32 * ip + 4 * g, 32 * ip + 16 + 4 * g, 16 * cb, pp);
        }
#pragma unroll
        for (int J = 0; J < NIB; ++J) {
            if (J < nib) {
                const int row_local = 16 * J + pp;
                const bool valid = row_local < nrows;
                const long orow = bh * N + r0 + row_local;
                if (has_e) {
                    // dk(eb, J) = sum_i phi(q_i)(eb) M_ij + R(eb, :) v_j + r(eb), times phi'(k_j)
                    // (decay: the suffix terms first, times gamma^(R - tau_j))
                    f32x4 acc = zero4;
                    if constexpr (dec) {
#pragma unroll
                        for (int s = 0; s < NSV; ++s) {
                            Frag<TV> fv;
                            lds_frag_split_v(fv, vb, 16 * J * SM::LV + 32 * s);
                            acc = mma(fragR[s], fv, acc);
                            if constexpr (RLO) acc = mma(fragR_lo[s], fv, acc);
                        }
                        acc = (acc + accr) * dcy.pow(nrows - row_local);
                    }
#pragma unroll
                    for (int ip = 0; ip < NTS; ++ip) {
                        if (!NC && 2 * ip + 1 >= J) {
                            Frag<TC> fm;
                            lds_frag_split_v(fm, mhb, 16 * J * SM::LM + 32 * ip);
                            acc = mma(fqt[ip], fm, acc);
                            if constexpr (SM::LO) {
                                lds_frag_split_v(fm, mlb, 16 * J * SM::LM + 32 * ip);
                                acc = mma(fqt[ip], fm, acc);
                            }
                        }
                    }
                    if constexpr (!dec) {
#pragma unroll
                        for (int s = 0; s < NSV; ++s) {
                            Frag<TV> fv;
                            lds_frag_split_v(fv, vb, 16 * J * SM::LV + 32 * s);
                            acc = mma(fragR[s], fv, acc);
                            if constexpr (RLO) acc = mma(fragR_lo[s], fv, acc);
                        }
                        acc = acc + accr;
                    }
                    const f32x4 kd = lds_get4(kb, 16 * J * SM::LK + 16 * eb);
                    f32x4 out;
#pragma unroll
                    for (int r = 0; r < 4; ++r) out[r] = acc[r] * (ident ? 1.0f : fminf(kd[r], 1.0f));
                    if constexpr (bwd_pair<TI>()) out = out * kd;  // u = dphi(k) * phi(k)
                    if (valid) store4<TI>(p.dk, orow * DK + 16 * eb + 4 * g, out);
                }
                if (has_c) {
                    // dv(cb, J) = sum_i dO_i(cb) A_ij + R^T(cb, :) phi(k_j)
                    // (decay: the suffix term first, times gamma^(R - tau_j))
                    f32x4 acc = zero4;
                    if constexpr (dec) {
#pragma unroll
                        for (int s = 0; s < NSE; ++s) {
                            Frag<TC> fk;
                            lds_frag_split_v(fk, kb, 16 * J * SM::LK + 32 * s);
                            acc = mma(frt[s], fk, acc);
                        }
                        acc = acc * dcy.pow(nrows - row_local);
                    }
#pragma unroll
                    for (int ip = 0; ip < NTS; ++ip) {
                        if (!NC && 2 * ip + 1 >= J) {
                            Frag<TC> fa;
                            lds_frag_split_v(fa, atb, 16 * J * SM::LM + 32 * ip);
                            acc = mma(fgt[ip], fa, acc);
                        }
                    }
                    if constexpr (!dec) {
#pragma unroll
                        for (int s = 0; s < NSE; ++s) {
                            Frag<TC> fk;
                            lds_frag_split_v(fk, kb, 16 * J * SM::LK + 32 * s);
                            acc = mma(frt[s], fk, acc);
                        }
                    }
                    if (valid) store4<TV>(p.dv, orow * DV + 16 * cb + 4 * g, acc);
                }
            }
        }
        // phi of the previous chunk's rows (after the first chunk the registers are not used again)
        if constexpr (!NC) xq.apply_phi(ident);
        xk.apply_phi(ident);
        if (has_e && !NC) {
            // state carry: R^T(c', eb) += dO^T(c') (a phi(Q))(eb), r(eb) += (a phi(Q))(eb)^T e
            // (a = 0 for token rows past the chunk; with decay the state first
            // decays by gamma^R and query i weighs gamma^(tau_i))
            if constexpr (dec) {
                const float gR = dcy.pow(nrows);
                accr = accr * gR;
#pragma unroll
                for (int cv = 0; cv < CV; ++cv) accR[cv] = accR[cv] * gR;
            }
#pragma unroll
            for (int s = 0; s < NTS; ++s) {
                {
                    const f32x4 a0 = *reinterpret_cast<const f32x4 *>(&sm.a[32 * s + 4 * g]);
                    const f32x4 a1 = *reinterpret_cast<const f32x4 *>(&sm.a[32 * s + 16 + 4 * g]);
                    const f32x4 e0 = *reinterpret_cast<const f32x4 *>(&sm.e[32 * s + 4 * g]);
                    const f32x4 e1 = *reinterpret_cast<const f32x4 *>(&sm.e[32 * s + 16 + 4 * g]);
                    // e as a pair of operands (value and rounding remainder) so that
                    // r keeps fp32-level accuracy with bf16 operands
                    Frag<TC> fq, fe, fe_lo;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float w0 = dec ? dcy.pow(32 * s + 4 * g + t) : 1.0f;
                        const float w1 = dec ? dcy.pow(32 * s + 16 + 4 * g + t) : 1.0f;
                        fq.set(t, fqt[s].get(t) * (a0[t] * w0));
                        fq.set(t + 4, fqt[s].get(t + 4) * (a1[t] * w1));
                        fe.set(t, e0[t]);
                        fe.set(t + 4, e1[t]);
                        fe_lo.set(t, e0[t] - fe.get(t));
                        fe_lo.set(t + 4, e1[t] - fe.get(t + 4));
                    }
                    accr = mma(fq, fe, accr);
                    if constexpr (SM::LO) accr = mma(fq, fe_lo, accr);
#pragma unroll
                    for (int cv = 0; cv < CV; ++cv) {
                        Frag<TV> fgc;
                        lds_frag_tr(fgc, sm.g, SM::LG, 32 * s + 4 * g, 32 * s + 16 + 4 * g, 16 * cv, pp);
                        accR[cv] = mma(fgc, fq, accR[cv]);
                    }
                }
            }
            refresh();  // the R copy's readers of this chunk passed the barrier above
        }
    }
}

}  // namespace la
