// la_fwd_launch.hpp -- host launch sequence of the chunked forward.
//
// Causal:     [P > 1]  aggregate per segment -> exclusive prefix over segments
//             then the chunk loop of every segment from its entering state.
// Non-causal: aggregate per segment -> total over segments -> read-out.
#pragma once

#include "la_fwd_impl.hpp"
#include "la_internal.h"

namespace la {

// Resident workgroups of one instantiation of the chunk kernel (cached).
template <int DK, int DV, typename TI, int MODE, int CT, bool OBF = false, bool DECAY = false, bool PRF = false,
          bool XCARRY = false>
long chunk_resident() {
    static OccCache cache;
    return resident_workgroups(reinterpret_cast<const void *>(&la_chunk_kernel<DK, DV, TI, MODE, CT, OBF, DECAY, PRF, XCARRY>),
                               cache, fwd_threads<DK, DV, TI, MODE, DECAY>());
}

// Workgroup target for the fine segments of an aggregate pass that feeds
// `want` causal segments per (b, h).  The pass sums only the fine segments
// before the last causal segment, (want - 1) * mult per (b, h), so mult fine
// segments per causal segment are chosen to fill one round of the `resident`
// aggregate workgroups.  At B=8, H=16, N=8192, d=128 (two causal segments
// per (b, h)) a single fine segment each left half of the CUs idle.
inline long fine_target(long BH, long want, long resident) {
    long t = resident;
    if (want > 1) {
        const long mult = resident / ((want - 1) * BH);
        if (mult > 1) t = mult * want * BH;
    }
    return t < kMaxTargetWg ? t : kMaxTargetWg;
}

// Aggregate segments per (b, h) of the non-causal form (at most).  At B=4,
// H=8, N=4096, d=64 the forward took 29.1 us with 2, 24.6 with 4, 23.6 with
// 6, 23.8 with 8 and 29.2 with 16 (each read-out workgroup sums them: d_k
// (d_v + 1) floats apiece), against 26.9 us with a separate total pass; the
// backward 66.1 us with 4, 65.2 with 6, 66.5 with 8.  A 128-wide state
// (66 KB) keeps four, so that the read-out prologues stay short.
template <int DK, int DV> constexpr int nc_agg_segments() { return (DK <= 64 && DV <= 64) ? 6 : 4; }

// Causal chunks per (b, h) up to which the split-layout forward runs one
// segment per (b, h) (no aggregate pass and no scan).
constexpr long kOneSegmentChunks = 16;

// DECAY: the causal form with a per-head decay (d.gamma non-null).  PRF: the
// random-feature map in the staging waves (d.phi_id 2, d.W).  CT: the chunk
// of the causal and read-out kernels; CTA: that of the aggregate pass.
template <int DK, int DV, typename TI, int CT, int CTA, bool OBF, bool DECAY, bool PRF = false>
hipError_t run_fwd_ct(const FwdDesc &d, bool causal) {
    const long BH = (long)d.B * d.H;
    auto agg_kernel = &la_chunk_kernel<DK, DV, TI, MODE_AGG, CTA, false, DECAY, PRF>;
    auto main_kernel = causal ? &la_chunk_kernel<DK, DV, TI, MODE_CAUSAL, CT, OBF, DECAY, PRF>
                              : &la_chunk_kernel<DK, DV, TI, MODE_APPLY, CT, OBF, false, PRF>;
    // Each launch aims at one round of resident workgroups.  The aggregate
    // pass uses fine segments; a causal segment is a run of `mult` of them.
    const long target_main = causal ? chunk_resident<DK, DV, TI, MODE_CAUSAL, CT, OBF, DECAY, PRF>()
                                    : chunk_resident<DK, DV, TI, MODE_APPLY, CT, OBF, false, PRF>();
    long want_main = (target_main + BH - 1) / BH;
    // A short sequence runs as one segment per (b, h) in the split layout:
    // at B=8, H=8, d=64, C=64 the three launches of a four-way split took
    // 20.3 us at N=512 and 26.5 at N=1024, one segment 13.8 and 23.8; from
    // N=2048 (32 chunks) on the split is faster (35.4 against 42.7 us).
    if (causal && fwd_split<DK, DV, TI, MODE_CAUSAL, DECAY>() && (d.N + CT - 1) / CT <= kOneSegmentChunks)
        want_main = 1;
    long target_agg = chunk_resident<DK, DV, TI, MODE_AGG, CTA, false, DECAY, PRF>();
    if (causal) target_agg = fine_target(BH, want_main, target_agg);
    // A workspace holding at most d.ws_states segment states (a fixed scratch):
    // fewer segments per (b, h), down to one, which stores no state at all.
    if (causal && d.ws_states > 0) {
        const long per_bh = d.ws_states / BH;
        const long cap = per_bh >= 1 ? per_bh * BH : BH;
        if (cap < target_agg) target_agg = cap;
    }
    int Lf = 0;
    const int Pf = plan_segments(BH, d.N, d.C, target_agg, &Lf);
    const int mult = (int)((Pf + want_main - 1) / want_main);
    const int Pm = (Pf + mult - 1) / mult;

    FwdParams p{};
    p.q = d.q;
    p.k = d.k;
    p.v = d.v;
    p.o = d.o;
    p.den = d.den;
    p.N = d.N;
    p.state_P = Pf;
    p.phi_id = d.phi_id;
    p.W = d.W;
    p.H = d.H;
    hipError_t err;

    if (causal) {
        p.S_fin = d.S_out;
        p.z_fin = d.z_out;
        p.gamma = d.gamma;
        p.H = d.H;
        if (Pm > 1) {
            // Only the segments before the last one need their sums: the
            // last causal segment starts at fine slot (Pm - 1) * mult.
            const int nagg = (Pm - 1) * mult;
            p.seg_out = d.ws;
            p.L = Lf;
            p.state_mult = 1;
            agg_kernel<<<dim3((unsigned)BH, (unsigned)nagg), fwd_threads<DK, DV, TI, MODE_AGG, DECAY>(), 0, d.stream>>>(p);
            if ((err = hipGetLastError()) != hipSuccess) return err;
            if ((err = launch_seg_scan(d.ws, d.S0, d.z0, BH, Pf, DK, DV, 0, nagg, d.stream, d.gamma, d.H, Lf)) !=
                hipSuccess)
                return err;
            p.seg_state = d.ws;
            p.state_mult = mult;
            p.L = Lf * mult;
            main_kernel<<<dim3((unsigned)BH, (unsigned)Pm), fwd_threads<DK, DV, TI, MODE_CAUSAL, DECAY>(), 0, d.stream>>>(p);
        } else {
            p.S0 = d.S0;
            p.z0 = d.z0;
            p.L = d.N;
            main_kernel<<<dim3((unsigned)BH, 1u), fwd_threads<DK, DV, TI, MODE_CAUSAL, DECAY>(), 0, d.stream>>>(p);
        }
        return hipGetLastError();
    }

    // Non-causal: a few aggregate segments per (b, h), summed by every
    // read-out workgroup in its prologue (no total pass, no extra launch).
    int Ln = 0;
    // (a target within kMaxTargetWg keeps Pn within the workspace the query sized)
    const long target_nc = BH * (long)nc_agg_segments<DK, DV>() < kMaxTargetWg ? BH * (long)nc_agg_segments<DK, DV>()
                                                                                : kMaxTargetWg;
    const int Pn = plan_segments(BH, d.N, d.C, target_nc, &Ln);
    p.seg_out = d.ws;
    p.L = Ln;
    p.state_P = Pn;
    p.state_mult = 1;
    agg_kernel<<<dim3((unsigned)BH, (unsigned)Pn), fwd_threads<DK, DV, TI, MODE_AGG>(), 0, d.stream>>>(p);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // The read-out is independent per row: split it on its own.
    int La = 0;
    const int Pa = plan_segments(BH, d.N, d.C, target_main, &La);
    p.seg_state = d.ws;
    p.sum_P = Pn;
    p.L = La;
    main_kernel<<<dim3((unsigned)BH, (unsigned)Pa), fwd_threads<DK, DV, TI, MODE_APPLY>(), 0, d.stream>>>(p);
    return hipGetLastError();
}

// Chunk sizes the kernels run at for a requested C.  The result does not
// depend on them, and segment lengths stay multiples of the requested C.
//   fwd_chunk: the aggregate passes (forward and backward); fp32 operands
//     with a 128-wide head dimension tile 64-token chunks as two of 32.
//   fwd_main_chunk: the causal chunk loop and the read-out; every 128-wide
//     head dimension tiles at 32 (the four-wave bf16 causal kernel spills at
//     64 and runs 5% faster at 32; its aggregate pass runs faster at 64).
template <int DK, int DV, typename TI> constexpr int fwd_chunk(int C) {
    return (sizeof(TI) == 4 && (DK == 128 || DV == 128) && C > 32) ? 32 : C;
}
template <int DK, int DV, typename TI> constexpr int fwd_main_chunk(int C) {
    return ((DK == 128 || DV == 128) && C > 32) ? 32 : C;
}

template <int DK, int DV, typename TI>
hipError_t run_fwd_t(const FwdDesc &d, bool causal) {
    const bool obf = d.out_bf16 != 0;
    const bool dec = causal && d.gamma != nullptr;
    if (d.phi_id == kPhiPrfFused) {
        // random features in the staging waves: the split bf16 layout at
        // 64-token chunks, as many directions as input features
        if constexpr (prf_fused_ok<DK, DV, TI>()) {
            if (!dec && d.C == 64)
                return obf ? run_fwd_ct<DK, DV, TI, 64, 64, true, false, true>(d, causal)
                           : run_fwd_ct<DK, DV, TI, 64, 64, false, false, true>(d, causal);
        }
        return hipErrorInvalidValue;
    }
    auto pick = [&](auto ct, auto cta) {
        constexpr int CT = decltype(ct)::value, CTA = decltype(cta)::value;
        if (dec) return obf ? run_fwd_ct<DK, DV, TI, CT, CTA, true, true>(d, causal)
                            : run_fwd_ct<DK, DV, TI, CT, CTA, false, true>(d, causal);
        return obf ? run_fwd_ct<DK, DV, TI, CT, CTA, true, false>(d, causal)
                   : run_fwd_ct<DK, DV, TI, CT, CTA, false, false>(d, causal);
    };
    using I16 = std::integral_constant<int, 16>;
    using I32 = std::integral_constant<int, 32>;
    using I64 = std::integral_constant<int, 64>;
    if constexpr (sizeof(TI) == 2 && (DK == 128 || DV == 128)) {
        if (fwd_main_chunk<DK, DV, TI>(d.C) == 32 && fwd_chunk<DK, DV, TI>(d.C) == 64) return pick(I32{}, I64{});
    }
    switch (fwd_main_chunk<DK, DV, TI>(d.C)) {
        case 16: return pick(I16{}, I16{});
        case 32: return pick(I32{}, I32{});
        case 64: return pick(I64{}, I64{});
        default: return hipErrorInvalidValue;
    }
}

template <int DK>
hipError_t run_fwd_dk(const FwdDesc &d, bool causal) {
    switch (d.DV) {
        case 16: return d.in_bf16 ? run_fwd_t<DK, 16, __bf16>(d, causal) : run_fwd_t<DK, 16, float>(d, causal);
        case 32: return d.in_bf16 ? run_fwd_t<DK, 32, __bf16>(d, causal) : run_fwd_t<DK, 32, float>(d, causal);
        case 64: return d.in_bf16 ? run_fwd_t<DK, 64, __bf16>(d, causal) : run_fwd_t<DK, 64, float>(d, causal);
        case 128: return d.in_bf16 ? run_fwd_t<DK, 128, __bf16>(d, causal) : run_fwd_t<DK, 128, float>(d, causal);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace la
