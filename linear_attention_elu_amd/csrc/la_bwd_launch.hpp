// la_bwd_launch.hpp -- host launch sequence of the cumulative-sum backward.
//
//   [P > 1]     aggregates of phi(K)^T V, phi(K)^T 1 per segment -> exclusive prefix
//   dq sweep    forward over the chunks of every segment; leaves 1/den and eps
//               per token and each segment's (phi(Q)/den)^T dO, (phi(Q)/den)^T e
//   [P > 1]     exclusive suffix over the segments
//   dk/dv sweep backward over the chunks of every segment
#pragma once

#include "la_bwd_impl.hpp"
#include "la_fwd_launch.hpp"
#include "la_internal.h"

namespace la {

inline size_t bwd_align(size_t x) { return (x + 255) & ~size_t(255); }

struct BwdLayout {
    size_t inv_den, eps, pre, suf, total;
};

inline BwdLayout bwd_layout(long BH, int N, int DK, int DV, int Pmax) {
    BwdLayout l{};
    l.inv_den = 0;
    l.eps = bwd_align(l.inv_den + (size_t)BH * N * sizeof(float));
    l.pre = bwd_align(l.eps + (size_t)BH * N * sizeof(float));
    const size_t st = (size_t)BH * Pmax * state_floats(DK, DV) * sizeof(float);
    l.suf = bwd_align(l.pre + st);
    l.total = bwd_align(l.suf + st);
    return l;
}

// Gradient of the non-causal form: the totals S, z and R, r replace the
// prefix and suffix states, so the sequence splits freely.
//   aggregates of phi(K)^T V, phi(K)^T 1 over a few segments
//   dq sweep (non-causal; sums them)      leaves 1/den and eps per token
//   aggregates of (phi(Q)/den)^T dO, (phi(Q)/den)^T e over a few segments
//   dk/dv sweep (non-causal; sums them)
template <int DK, int DV, typename TI, int CT>
hipError_t run_bwd_nc_ct(const BwdDesc &d) {
    const long BH = (long)d.B * d.H;
    int Lmax = 0;
    const int Pmax = plan_segments(BH, d.N, d.C, kMaxTargetWg, &Lmax);
    const BwdLayout lay = bwd_layout(BH, d.N, DK, DV, Pmax);
    char *ws = reinterpret_cast<char *>(d.ws);
    float *inv_den = reinterpret_cast<float *>(ws + lay.inv_den);
    float *eps = reinterpret_cast<float *>(ws + lay.eps);
    float *tot = reinterpret_cast<float *>(ws + lay.pre);
    float *rtot = reinterpret_cast<float *>(ws + lay.suf);
    hipError_t err;

    auto agg_kernel = &la_chunk_kernel<DK, DV, TI, MODE_AGG, CT, false>;
    auto aggw_kernel = &la_chunk_kernel<DK, DV, TI, MODE_AGGW, CT, false>;
    auto dq_kernel = &la_bwd_dq_kernel<DK, DV, TI, true>;
    auto dkdv_kernel = &la_bwd_dkdv_kernel<DK, DV, TI, true>;
    static OccCache occ_dq, occ_kv;
    const long target_dq = resident_workgroups(reinterpret_cast<const void *>(dq_kernel), occ_dq, kBwdThreads);
    const long target_kv = resident_workgroups(reinterpret_cast<const void *>(dkdv_kernel), occ_kv, kBwdThreads);
    // a few aggregate segments per (b, h), as in the non-causal forward (a
    // target within kMaxTargetWg keeps Pf within the workspace the query sized)
    const long target_agg = BH * (long)nc_agg_segments<DK, DV>() < kMaxTargetWg ? BH * (long)nc_agg_segments<DK, DV>()
                                                                                 : kMaxTargetWg;
    int Lf = 0;
    const int Pf = plan_segments(BH, d.N, d.C, target_agg, &Lf);

    FwdParams a{};
    a.N = d.N;
    a.phi_id = d.phi_id;
    a.L = Lf;
    a.state_P = Pf;
    a.state_mult = 1;
    a.k = d.k;
    a.v = d.v;
    a.seg_out = tot;
    agg_kernel<<<dim3((unsigned)BH, (unsigned)Pf), fwd_threads<DK, DV, TI, MODE_AGG>(), 0, d.stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;

    BwdParams b{};
    b.q = d.q;
    b.k = d.k;
    b.v = d.v;
    b.g = d.dO;
    b.inv_den = inv_den;
    b.eps = eps;
    b.dq = d.dq;
    b.dk = d.dk;
    b.dv = d.dv;
    b.N = d.N;
    b.phi_id = d.phi_id;
    b.C = d.C < bwd_cmax<TI, DK, DV>() ? d.C : bwd_cmax<TI, DK, DV>();
    b.state_P = Pf;
    b.state_mult = 0;  // every segment reads slots 0 .. Pf - 1
    b.sum_P = Pf;
    int Lq = 0, Lkv = 0;
    const int Pq = plan_segments(BH, d.N, d.C, target_dq, &Lq);
    const int Pkv = plan_segments(BH, d.N, d.C, target_kv, &Lkv);

    b.state = tot;
    b.L = Lq;
    dq_kernel<<<dim3((unsigned)BH, (unsigned)Pq), kBwdThreads, 0, d.stream>>>(b);
    if ((err = hipGetLastError()) != hipSuccess) return err;

    a.k = d.q;  // (a phi(Q))^T dO and (a phi(Q))^T e, a = 1 / den
    a.v = d.dO;
    a.kscale = inv_den;
    a.zw = eps;
    a.seg_out = rtot;
    aggw_kernel<<<dim3((unsigned)BH, (unsigned)Pf), fwd_threads<DK, DV, TI, MODE_AGGW>(), 0, d.stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;

    b.state = rtot;
    b.L = Lkv;
    dkdv_kernel<<<dim3((unsigned)BH, (unsigned)Pkv), kBwdThreads, 0, d.stream>>>(b);
    return hipGetLastError();
}

template <int DK, int DV, typename TI>
hipError_t run_bwd_nc_t(const BwdDesc &d) {
    switch (fwd_chunk<DK, DV, TI>(d.C)) {
        case 16: return run_bwd_nc_ct<DK, DV, TI, 16>(d);
        case 32: return run_bwd_nc_ct<DK, DV, TI, 32>(d);
        case 64: return run_bwd_nc_ct<DK, DV, TI, 64>(d);
        default: return hipErrorInvalidValue;
    }
}

// DECAY: the causal form with a per-head decay (d.gamma non-null).  TI =
// bf16p: sweeps that multiply bf16 value-plus-remainder operands, on q and k
// given as two bf16 planes (value, remainder) and bf16 v, dO; the prefix
// aggregate is then the sum of two bf16 passes (type TA), one per plane of k,
// each product of bf16 values exact in fp32.
template <int DK, int DV, typename TI, bool DECAY>
hipError_t run_bwd_causal_t(const BwdDesc &d) {
    constexpr bool PAIR = std::is_same<TI, bf16p>::value;
    using TA = typename std::conditional<PAIR, __bf16, TI>::type;
    static_assert(!DECAY || !PAIR, "bf16-pair sweeps: no decay");
    const long BH = (long)d.B * d.H;
    int Lmax = 0;
    const int Pmax = plan_segments(BH, d.N, d.C, kMaxTargetWg, &Lmax);
    const BwdLayout lay = bwd_layout(BH, d.N, DK, DV, Pmax);
    char *ws = reinterpret_cast<char *>(d.ws);
    float *inv_den = reinterpret_cast<float *>(ws + lay.inv_den);
    float *eps = reinterpret_cast<float *>(ws + lay.eps);
    float *pre = reinterpret_cast<float *>(ws + lay.pre);
    float *suf = reinterpret_cast<float *>(ws + lay.suf);
    hipError_t err;

    // The prefix aggregate reuses the forward's chunk kernel at the caller's
    // chunk size (the suffix sums come from the dq sweep); decayed on bf16
    // operands, in its value-plus-remainder carry variant.
    constexpr bool XC = DECAY && sizeof(TA) == 2;
    void (*agg_kernel)(const FwdParams) = nullptr;
    long target_agg = 0;
    switch (fwd_chunk<DK, DV, TA>(d.C)) {
        case 16:
            agg_kernel = &la_chunk_kernel<DK, DV, TA, MODE_AGG, 16, false, DECAY, false, XC>;
            target_agg = chunk_resident<DK, DV, TA, MODE_AGG, 16, false, DECAY, false, XC>();
            break;
        case 32:
            agg_kernel = &la_chunk_kernel<DK, DV, TA, MODE_AGG, 32, false, DECAY, false, XC>;
            target_agg = chunk_resident<DK, DV, TA, MODE_AGG, 32, false, DECAY, false, XC>();
            break;
        case 64:
            agg_kernel = &la_chunk_kernel<DK, DV, TA, MODE_AGG, 64, false, DECAY, false, XC>;
            target_agg = chunk_resident<DK, DV, TA, MODE_AGG, 64, false, DECAY, false, XC>();
            break;
        default: return hipErrorInvalidValue;
    }
    auto dq_kernel = &la_bwd_dq_kernel<DK, DV, TI, false, DECAY>;
    auto dkdv_kernel = &la_bwd_dkdv_kernel<DK, DV, TI, false, DECAY>;
    static OccCache occ_dq, occ_kv;
    const long target_dq = resident_workgroups(reinterpret_cast<const void *>(dq_kernel), occ_dq, kBwdThreads);
    const long target_kv = resident_workgroups(reinterpret_cast<const void *>(dkdv_kernel), occ_kv, kBwdThreads);
    const long target_sweep = target_dq < target_kv ? target_dq : target_kv;
    int Lf = 0;
    const int Pf = plan_segments(BH, d.N, d.C, fine_target(BH, (target_sweep + BH - 1) / BH, target_agg), &Lf);
    auto split = [&](long target, int *mult) {
        const long want = (target + BH - 1) / BH;
        *mult = (int)((Pf + want - 1) / want);
        return (Pf + *mult - 1) / *mult;
    };
    // One split for both sweeps: the dq sweep leaves each segment's suffix sums
    // for the dk/dv sweep's segments.
    int mult = 1;
    const int Pc = split(target_sweep, &mult);
    const int Lc = Lf * mult;

    FwdParams a{};
    a.N = d.N;
    a.phi_id = d.phi_id;
    a.L = Lf;
    a.state_P = Pf;
    a.state_mult = 1;
    a.gamma = d.gamma;
    a.H = d.H;
    if (Pc > 1) {
        // prefix sums: the last segment's own fine segments are not needed
        const int nagg = (Pc - 1) * mult;
        a.k = d.k;
        a.v = d.v;
        a.seg_out = pre;
        a.seg_base = 0;
        agg_kernel<<<dim3((unsigned)BH, (unsigned)nagg), fwd_threads<DK, DV, TA, MODE_AGG, DECAY>(), 0, d.stream>>>(a);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        if constexpr (PAIR) {  // the remainder half of k
            a.k = static_cast<const __bf16 *>(d.k) + BH * d.N * (long)DK;
            a.seg_out = d.agg_lo;
            agg_kernel<<<dim3((unsigned)BH, (unsigned)nagg), fwd_threads<DK, DV, TA, MODE_AGG, DECAY>(), 0,
                         d.stream>>>(a);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
        if ((err = launch_seg_scan(pre, nullptr, nullptr, BH, Pf, DK, DV, 0, nagg, d.stream, d.gamma, d.H, Lf,
                                   PAIR ? d.agg_lo : nullptr)) != hipSuccess)
            return err;
    }

    BwdParams b{};
    b.q = d.q;
    b.k = d.k;
    b.v = d.v;
    b.g = d.dO;
    b.inv_den = inv_den;
    b.eps = eps;
    b.dq = d.dq;
    b.dk = d.dk;
    b.dv = d.dv;
    b.N = d.N;
    b.phi_id = d.phi_id;
    b.C = d.C < bwd_cmax<TI, DK, DV>() ? d.C : bwd_cmax<TI, DK, DV>();
    b.state_P = Pf;
    b.gamma = d.gamma;
    b.H = d.H;

    // dq sweep: reads the prefix states at fine slots, writes each segment's
    // suffix sums to slot [bh][segment] of `suf` (segments 1 .. Pc - 1)
    b.state = Pc > 1 ? pre : nullptr;
    b.state_mult = mult;
    b.L = Pc > 1 ? Lc : d.N;
    b.suf_out = Pc > 1 ? suf : nullptr;
    b.suf_P = Pc;
    dq_kernel<<<dim3((unsigned)BH, (unsigned)Pc), kBwdThreads, 0, d.stream>>>(b);
    if ((err = hipGetLastError()) != hipSuccess) return err;

    if (Pc > 1) {
        // exclusive suffix over the segments: slot s receives the sums after segment s
        if ((err = launch_seg_scan(suf, nullptr, nullptr, BH, Pc, DK, DV, 2, 1, d.stream, d.gamma, d.H, Lc)) !=
            hipSuccess)
            return err;
    }
    b.suf_out = nullptr;
    b.state = Pc > 1 ? suf : nullptr;
    b.state_P = Pc;
    b.state_mult = 1;
    b.L = Pc > 1 ? Lc : d.N;
    dkdv_kernel<<<dim3((unsigned)BH, (unsigned)Pc), kBwdThreads, 0, d.stream>>>(b);
    return hipGetLastError();
}

template <int DK, int DV, typename TI>
hipError_t run_bwd_t(const BwdDesc &d) {
    if constexpr (std::is_same<TI, bf16p>::value) {
        if (d.noncausal || d.gamma || !d.agg_lo) return hipErrorInvalidValue;
        return run_bwd_causal_t<DK, DV, TI, false>(d);
    } else {
        if (d.noncausal) return run_bwd_nc_t<DK, DV, TI>(d);
        return d.gamma ? run_bwd_causal_t<DK, DV, TI, true>(d) : run_bwd_causal_t<DK, DV, TI, false>(d);
    }
}

// bf16-pair sweeps are built for the widths the random features give the state
// (m in {32, 64, 128}).
template <int DK, int DV>
hipError_t run_bwd_pair(const BwdDesc &d) {
    if constexpr (DK >= 32) return run_bwd_t<DK, DV, bf16p>(d);
    else return hipErrorInvalidValue;
}

template <int DK>
hipError_t run_bwd_dk(const BwdDesc &d) {
    switch (d.DV) {
        case 16: return d.pair_ops ? run_bwd_pair<DK, 16>(d)
                          : d.in_bf16 ? run_bwd_t<DK, 16, __bf16>(d) : run_bwd_t<DK, 16, float>(d);
        case 32: return d.pair_ops ? run_bwd_pair<DK, 32>(d)
                          : d.in_bf16 ? run_bwd_t<DK, 32, __bf16>(d) : run_bwd_t<DK, 32, float>(d);
        case 64: return d.pair_ops ? run_bwd_pair<DK, 64>(d)
                          : d.in_bf16 ? run_bwd_t<DK, 64, __bf16>(d) : run_bwd_t<DK, 64, float>(d);
        case 128: return d.pair_ops ? run_bwd_pair<DK, 128>(d)
                          : d.in_bf16 ? run_bwd_t<DK, 128, __bf16>(d) : run_bwd_t<DK, 128, float>(d);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace la
