// la_fwd_launch.hpp -- host launch sequence of the chunked forward.
//
// Causal:     [P > 1]  aggregate per segment -> exclusive prefix over segments
//             then the chunk loop of every segment from its entering state.
// Non-causal: aggregate per segment -> total over segments -> read-out.
#pragma once

#include "la_fwd_impl.hpp"
#include "la_internal.h"

namespace la {

template <int DK, int DV, typename TI>
hipError_t run_fwd_t(const FwdDesc &d, bool causal) {
    const long BH = (long)d.B * d.H;
    int L = 0;
    const int P = plan_segments(BH, d.N, d.C, &L);

    FwdParams p{};
    p.q = d.q;
    p.k = d.k;
    p.v = d.v;
    p.o = d.o;
    p.den = d.den;
    p.N = d.N;
    p.C = d.C;
    p.L = L;
    p.P = P;
    p.out_bf16 = d.out_bf16;

    const dim3 grid((unsigned)BH, (unsigned)P);
    hipError_t err;

    if (causal) {
        p.S_fin = d.S_out;
        p.z_fin = d.z_out;
        if (P > 1) {
            p.seg_out = d.ws;
            la_chunk_kernel<DK, DV, TI, MODE_AGG><<<grid, kThreads, 0, d.stream>>>(p);
            if ((err = hipGetLastError()) != hipSuccess) return err;
            if ((err = launch_seg_scan(d.ws, d.S0, d.z0, BH, P, DK, DV, 0, d.stream)) != hipSuccess) return err;
            p.seg_state = d.ws;
        } else {
            p.S0 = d.S0;
            p.z0 = d.z0;
        }
        la_chunk_kernel<DK, DV, TI, MODE_CAUSAL><<<grid, kThreads, 0, d.stream>>>(p);
        return hipGetLastError();
    }

    p.seg_out = d.ws;
    la_chunk_kernel<DK, DV, TI, MODE_AGG><<<grid, kThreads, 0, d.stream>>>(p);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (P > 1) {
        if ((err = launch_seg_scan(d.ws, nullptr, nullptr, BH, P, DK, DV, 1, d.stream)) != hipSuccess) return err;
    }
    p.seg_state = d.ws;
    la_chunk_kernel<DK, DV, TI, MODE_APPLY><<<grid, kThreads, 0, d.stream>>>(p);
    return hipGetLastError();
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
