// la_decode.hip -- one recurrent decode step for every (batch, head) on gfx950.
//
// Recurrent form (blog digest "Method / key components 4)"; velog review 3.6
// "Transformers and RNNs"; itwiki "선형 어텐션", section "Causal masking and
// the recurrent form"): S += phi(k) v^T, z += phi(k), then
// o = phi(q)^T S / phi(q)^T z, the update coming before the read.
//
// The step is bound by streaming the fp32 state through HBM (read and write
// d_k x d_v floats per (batch, head) against O(d) other bytes), so the kernel
// is plain VALU work laid out for coalescing: one wave per (batch, head);
// the wave's lanes cover a row of S with 16-byte accesses (d_v / 4 lanes per
// row) and 64 / (d_v / 4) rows at a time, so each wave-wide access is one
// contiguous block of S.  Column sums of phi(q) * S are reduced across the
// rows a wave holds with lane shuffles; phi(q) . z across the wave.
//
// With a per-head decay (itwiki "선형 어텐션", table of later variants, RetNet
// row) the update is S = gamma_h S + phi(k) v^T, z = gamma_h z + phi(k); a
// null gamma is gamma = 1, the plain step.  The feature map is a template
// parameter (elu + 1, identity, or positive random features computed per
// step from the directions W).
#include "la_device.hpp"
#include "la_internal.h"

namespace la {

// Feature maps of the decode step: FM_ELU1 phi = elu + 1 (DK = d_k), FM_ID
// phi(x) = x (q and k are features), FM_PRF positive random features
// phi(x)_r = exp(w_r . x - |x|^2 / 2) / sqrt(DK), r < DK, from the din-wide
// q and k rows and the directions W [H][DK][din] (itwiki "선형 어텐션",
// section "특징 사상 선택").
enum { FM_ELU1 = 0, FM_ID = 1, FM_PRF = 2 };

template <int DK, int DV, typename TI, int FM>
__global__ void __launch_bounds__(256)
la_decode_kernel(float *__restrict__ S, float *__restrict__ z, const void *__restrict__ q,
                 const void *__restrict__ k, const void *__restrict__ v, void *__restrict__ o, long BH,
                 const float *__restrict__ gamma, int H, const void *__restrict__ W, int din) {
    constexpr int CV = DV / 4;   // lanes per row of S (one float4 each)
    constexpr int RG = 64 / CV;  // rows of S a wave covers per access
    constexpr int RPL = DK / RG; // accesses per lane
    constexpr int NFH = (DK + 63) / 64;  // features per lane (random features)
    const int lane = threadIdx.x & 63;
    const long bh = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (bh >= BH) return;  // whole waves leave; no block-wide barrier follows
    const float gm = gamma ? gamma[bh % H] : 1.0f;

    const int cg = lane % CV;
    const int r0 = lane / CV;
    float *Sb = S + bh * (long)DK * DV;
    const long qk0 = bh * (long)(FM == FM_PRF ? din : DK);

    // Random features: lane l computes features l, l + 64 of q and k.
    float fqh[NFH], fkh[NFH];
    if constexpr (FM == FM_PRF) {
        float nq = 0.f, nk = 0.f;
        for (int i = 0; i < din; ++i) {
            const float xq = Store<TI>::load(q, qk0 + i), xk = Store<TI>::load(k, qk0 + i);
            nq += xq * xq;
            nk += xk * xk;
        }
        const float scale = __builtin_amdgcn_rsqf((float)DK);
#pragma unroll
        for (int h = 0; h < NFH; ++h) {
            const int e = lane + 64 * h;
            float aq = 0.f, ak = 0.f;
            if (e < DK) {
                const long w0 = ((bh % H) * (long)DK + e) * din;
                for (int i = 0; i < din; ++i) {
                    const float w = Store<TI>::load(W, w0 + i);
                    aq += w * Store<TI>::load(q, qk0 + i);
                    ak += w * Store<TI>::load(k, qk0 + i);
                }
            }
            fqh[h] = __expf(aq - 0.5f * nq) * scale;
            fkh[h] = __expf(ak - 0.5f * nk) * scale;
        }
    }
    // phi(q_e), phi(k_e) for a feature index e (wave-uniform control flow)
    auto feat = [&](const void *x, const float (&fh)[NFH], int e) {
        if constexpr (FM == FM_PRF) {
            float r = __shfl(fh[0], e & 63, 64);
#pragma unroll
            for (int h = 1; h < NFH; ++h) {
                const float t = __shfl(fh[h], e & 63, 64);
                r = (e >> 6) == h ? t : r;
            }
            return r;
        } else if constexpr (FM == FM_ID) {
            return Store<TI>::load(x, qk0 + e);
        } else {
            return phi(Store<TI>::load(x, qk0 + e));
        }
    };

    // The normaliser's operands (z, and q, k at this lane's features) are
    // loaded here, with the other loads of the step: issued after the state's
    // stores they cost a second memory round trip per step.
    float zr[NFH], qr[NFH], kr[NFH];
#pragma unroll
    for (int h = 0; h < NFH; ++h) {
        const int e = min(lane + 64 * h, DK - 1);  // lanes past d_k re-read the last feature, unused
        zr[h] = z[bh * (long)DK + e];
        if constexpr (FM != FM_PRF) {
            qr[h] = Store<TI>::load(q, qk0 + e);
            kr[h] = Store<TI>::load(k, qk0 + e);
        }
    }
    float vv[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) vv[t] = Store<TI>::load(v, bh * (long)DV + 4 * cg + t);

    // Accesses are issued in groups of up to eight so that loads overlap
    // without holding the whole slice of S in registers.
    constexpr int GRP = RPL < 8 ? RPL : 8;
    float num[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t0 = 0; t0 < RPL; t0 += GRP) {
        f32x4 sreg[GRP];
#pragma unroll
        for (int t = 0; t < GRP; ++t)
            sreg[t] = *reinterpret_cast<const f32x4 *>(Sb + (long)(r0 + RG * (t0 + t)) * DV + 4 * cg);
#pragma unroll
        for (int t = 0; t < GRP; ++t) {
            const int e = r0 + RG * (t0 + t);
            const float fk = feat(k, fkh, e);
            const float fq = feat(q, fqh, e);
            f32x4 s = sreg[t];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                s[c] = gm * s[c] + fk * vv[c];
                num[c] += fq * s[c];
            }
            *reinterpret_cast<f32x4 *>(Sb + (long)e * DV + 4 * cg) = s;
        }
    }
    // column sums over the RG row groups of the wave
#pragma unroll
    for (int off = CV; off < 64; off *= 2)
#pragma unroll
        for (int c = 0; c < 4; ++c) num[c] += __shfl_xor(num[c], off, 64);

    // (computed on every lane, so that the loads above have a use outside the
    // store's branch and stay where they are issued)
    float dpart = 0.f;
#pragma unroll
    for (int h = 0; h < NFH; ++h) {
        const int e = lane + 64 * h;
        float fk, fq;
        if constexpr (FM == FM_PRF) {
            fk = fkh[h];
            fq = fqh[h];
        } else if constexpr (FM == FM_ID) {
            fk = kr[h];
            fq = qr[h];
        } else {
            fk = phi(kr[h]);
            fq = phi(qr[h]);
        }
        const float zn = gm * zr[h] + fk;
        dpart += e < DK ? fq * zn : 0.f;
        if (e < DK) z[bh * (long)DK + e] = zn;
    }
#pragma unroll
    for (int off = 1; off < 64; off *= 2) dpart += __shfl_xor(dpart, off, 64);

    if (lane < CV) {
        const long ob = bh * (long)DV + 4 * cg;
        if (sizeof(TI) == 4) {
            f32x4 w = {num[0] / dpart, num[1] / dpart, num[2] / dpart, num[3] / dpart};
            *reinterpret_cast<f32x4 *>(static_cast<float *>(o) + ob) = w;
        } else {
            uint2 w;
            w.x = (uint32_t)f32_to_bf16_bits(num[0] / dpart) | ((uint32_t)f32_to_bf16_bits(num[1] / dpart) << 16);
            w.y = (uint32_t)f32_to_bf16_bits(num[2] / dpart) | ((uint32_t)f32_to_bf16_bits(num[3] / dpart) << 16);
            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(o) + ob) = w;
        }
    }
}

template <int DK, int DV, typename TI>
static void launch_decode(const DecodeDesc &d, dim3 grid, long BH) {
    switch (d.fm) {
        case FM_ID:
            la_decode_kernel<DK, DV, TI, FM_ID><<<grid, 256, 0, d.stream>>>(d.S, d.z, d.q, d.k, d.v, d.o, BH, d.gamma,
                                                                            d.H, nullptr, d.DK);
            break;
        case FM_PRF:
            la_decode_kernel<DK, DV, TI, FM_PRF><<<grid, 256, 0, d.stream>>>(d.S, d.z, d.q, d.k, d.v, d.o, BH,
                                                                             d.gamma, d.H, d.W, d.din);
            break;
        default:
            la_decode_kernel<DK, DV, TI, FM_ELU1><<<grid, 256, 0, d.stream>>>(d.S, d.z, d.q, d.k, d.v, d.o, BH,
                                                                              d.gamma, d.H, nullptr, d.DK);
    }
}

template <int DK, int DV>
static hipError_t run_decode_t(const DecodeDesc &d) {
    const long BH = (long)d.B * d.H;
    const dim3 grid((unsigned)((BH + 3) / 4));
    if (d.in_bf16) launch_decode<DK, DV, __bf16>(d, grid, BH);
    else launch_decode<DK, DV, float>(d, grid, BH);
    return hipGetLastError();
}

template <int DK>
static hipError_t run_decode_dk(const DecodeDesc &d) {
    switch (d.DV) {
        case 16: return run_decode_t<DK, 16>(d);
        case 32: return run_decode_t<DK, 32>(d);
        case 64: return run_decode_t<DK, 64>(d);
        case 128: return run_decode_t<DK, 128>(d);
        default: return hipErrorInvalidValue;
    }
}

hipError_t run_decode(const DecodeDesc &d) {
    switch (d.DK) {
        case 16: return run_decode_dk<16>(d);
        case 32: return run_decode_dk<32>(d);
        case 64: return run_decode_dk<64>(d);
        case 128: return run_decode_dk<128>(d);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace la
