// la_device.hpp -- device-side building blocks for the gfx950 kernels.
//
// MFMA fragment conventions (wave64, 16x16 tiles).  Lane l belongs to lane
// group g = l / 16 and has position p = l % 16 inside the group.
//   * A operand (16 x 32, M x K): lane l supplies row m = p and eight K values.
//   * B operand (32 x 16, K x N): lane l supplies column n = p and eight K values.
//   * Accumulator (16 x 16): lane l holds rows m = 4g + r (r = 0..3) of column n = p.
// The hardware pairs A's and B's K values lane group by lane group and slot by
// slot, so any assignment of the 32 K indices to (g, slot) works as long as
// both operands use the same one.  Two assignments are used:
//   * "straight": slot t of group g is K index 8g + t;
//   * "split":    slot t < 4 of group g is 4g + t, slot t >= 4 is 16 + 4g + (t - 4).
// The split assignment is exactly the row set an accumulator lane holds over
// two stacked 16 x 16 tiles, so an accumulator can be fed back as an operand
// without leaving registers.
//
// bf16 path: one v_mfma_f32_16x16x32_bf16 per 32-wide K step.
// fp32 path: eight v_mfma_f32_16x16x4_f32, slot t of every group forming the
// four K values of the t-th instruction -- the same pairing, in fp32.
// bf16-pair path (bf16p, fp32 data): four v_mfma_f32_16x16x32_bf16 per K
// step on each operand's bf16 value and bf16 remainder -- the bf16 pairing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Scalar helpers
// ---------------------------------------------------------------------------

// phi(x) = elu(x) + 1 (slope 1): x + 1 above zero, exp(x) at or below zero.
// Evaluated as max(x + 1, exp(-|x|)) without a compare: at or below zero
// exp(x) >= 1 + x (exp is convex), above zero exp(-x) < 1 < x + 1.  Where the
// two candidates are within an ulp of each other (|x| tiny) both are exp(x)
// to fp32 rounding.  NaN propagates; exp(-inf) = 0 gives phi(-inf) = 0.
__device__ __forceinline__ float phi(float x) {
    return fmaxf(x + 1.0f, __builtin_amdgcn_exp2f(-fabsf(x) * 1.44269504088896341f));
}

// phi'(x): 1 above zero, exp(x) at or below zero.
__device__ __forceinline__ float dphi(float x) { return x > 0.0f ? 1.0f : __expf(x); }

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ __bf16 f32_to_bf16(float x) { return static_cast<__bf16>(x); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    __bf16 b = static_cast<__bf16>(x);
    return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float round_bf16(float x) {
    return static_cast<float>(static_cast<__bf16>(x));
}

// Streaming global loads: nontemporal loads of data a kernel reads once (on
// gfx950 they raise a plain streaming read from about 6.4 to 7.0 TB/s).
// Stores stay ordinary: the output rows are written in 32-byte pieces by
// four waves, which the L2 merges before they reach HBM.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const void *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Four floats to four bf16 (round to nearest even), packed in 8 bytes.
__device__ __forceinline__ uint2 pack_bf16x4(const f32x4 &x) {
    const bf16x4 b = __builtin_convertvector(x, bf16x4);
    return __builtin_bit_cast(uint2, b);
}

// ---------------------------------------------------------------------------
// Compute-type traits: the type matrix operands are staged in (LDS and
// registers) and the 32-wide K step built on it.
// ---------------------------------------------------------------------------
template <typename TC> struct Frag;

template <> struct Frag<__bf16> {
    bf16x8 v;
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = static_cast<__bf16>(0.0f);
    }
    __device__ __forceinline__ void set(int t, float x) { v[t] = static_cast<__bf16>(x); }
    __device__ __forceinline__ float get(int t) const { return static_cast<float>(v[t]); }
};

template <> struct Frag<float> {
    float v[8];
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = 0.0f;
    }
    __device__ __forceinline__ void set(int t, float x) { v[t] = x; }
    __device__ __forceinline__ float get(int t) const { return v[t]; }
};

__device__ __forceinline__ f32x4 mma(const Frag<__bf16> &a, const Frag<__bf16> &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma(const Frag<float> &a, const Frag<float> &b, f32x4 c) {
#pragma unroll
    for (int t = 0; t < 8; ++t) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[t], b.v[t], c, 0, 0, 0);
    return c;
}

// fp32 values as bf16 pairs: a bf16 value and the bf16 rounding of what it
// leaves out, about 16 significant bits together.  In LDS a pair tile is two
// bf16 planes of one layout (bf16pl<PL>: the remainder plane PL elements after
// the value plane), read with the bf16 loaders.  A product of two pairs is
// hi*hi + hi*lo + lo*hi + lo*lo on the bf16 matrix cores, each product of
// halves exact in fp32.  lo*lo lies below the pair's own rounding, but without
// it the product of two pair values is no longer exact, and terms that must
// cancel (X and z (phi(q) . X) / den of a lone token) miss each other by a
// part in 2^18.  Four bf16 MFMAs against eight fp32 MFMAs of twice the time
// each; operands keep about 16 bits instead of 24.
struct bf16p {};
template <int PL> struct bf16pl {
    __bf16 x;
};

__device__ __forceinline__ float bf16p_value(float x) {
    const float h = round_bf16(x);
    return h + round_bf16(x - h);
}

template <> struct Frag<bf16p> {
    bf16x8 hi, lo;
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int t = 0; t < 8; ++t) hi[t] = lo[t] = static_cast<__bf16>(0.0f);
    }
    __device__ __forceinline__ void set(int t, float x) {
        hi[t] = static_cast<__bf16>(x);
        lo[t] = static_cast<__bf16>(x - static_cast<float>(hi[t]));
    }
    __device__ __forceinline__ float get(int t) const { return static_cast<float>(hi[t]) + static_cast<float>(lo[t]); }
};

__device__ __forceinline__ f32x4 mma(const Frag<bf16p> &a, const Frag<bf16p> &b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.lo, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, c, 0, 0, 0);
}

// A pair with a bf16 operand (a value a bf16 holds exactly): two MFMAs, each
// product of halves exact in fp32 as above.
__device__ __forceinline__ f32x4 mma(const Frag<bf16p> &a, const Frag<__bf16> &b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.v, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<__bf16> &a, const Frag<bf16p> &b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.lo, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.hi, c, 0, 0, 0);
}

// Round a value to what the operand type can hold (identity for fp32).
template <typename TC> __device__ __forceinline__ float to_operand(float x);
template <> __device__ __forceinline__ float to_operand<__bf16>(float x) { return round_bf16(x); }
template <> __device__ __forceinline__ float to_operand<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_operand<bf16p>(float x) { return bf16p_value(x); }

// ---------------------------------------------------------------------------
// LDS fragment reads.  `row` points at the first element of the operand row
// (or column, for transposed tiles) inside an LDS tile of TC.
// ---------------------------------------------------------------------------

// Straight assignment: eight consecutive elements starting at row[8g].
__device__ __forceinline__ void lds_frag_straight(Frag<__bf16> &f, const __bf16 *row, int g) {
    f.v = *reinterpret_cast<const bf16x8 *>(row + 8 * g);
}
__device__ __forceinline__ void lds_frag_straight(Frag<float> &f, const float *row, int g) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(row + 8 * g);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(row + 8 * g + 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f.v[t] = a[t];
        f.v[t + 4] = b[t];
    }
}

// Split assignment over two 16-element halves: row0[4g..4g+3] then row1[4g..4g+3].
__device__ __forceinline__ void lds_frag_split(Frag<__bf16> &f, const __bf16 *row0, const __bf16 *row1, int g) {
    const bf16x4 a = *reinterpret_cast<const bf16x4 *>(row0 + 4 * g);
    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(row1 + 4 * g);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f.v[t] = a[t];
        f.v[t + 4] = b[t];
    }
}
__device__ __forceinline__ void lds_frag_split(Frag<float> &f, const float *row0, const float *row1, int g) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(row0 + 4 * g);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(row1 + 4 * g);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f.v[t] = a[t];
        f.v[t + 4] = b[t];
    }
}

// A copy of an LDS address the compiler cannot relate to other addresses
// (a register move it does not see through).  Reads from bases made this way
// are never merged with each other: the compiler would otherwise pair the
// two 8-byte halves of split fragments (32 or 64 bytes apart) into one
// ds_read2_b64, which on gfx950 serves a wave with several times the bank
// conflicts of two ds_read_b64 (LDS conflict counters: 16 against 4 cycles
// per fragment at a 144-byte row stride).
template <typename T> using lds_cptr = const T __attribute__((address_space(3))) *;

template <typename TC> __device__ __forceinline__ lds_cptr<TC> lds_opaque(const TC *p) {
    uint32_t a = (uint32_t)(uintptr_t)(lds_cptr<TC>)p;  // generic -> LDS address
    asm("v_mov_b32 %0, %1" : "=v"(a) : "v"(a));
    return (lds_cptr<TC>)(uintptr_t)a;
}

// Split-assignment fragment from two per-lane LDS bases (the lane's slots
// 0..3 at lo[off..], slots 4..7 at hi[off..]).
template <typename TC>
__device__ __forceinline__ void lds_frag_split_at(Frag<TC> &f, lds_cptr<TC> lo, lds_cptr<TC> hi, int off) {
    if constexpr (sizeof(TC) == 2) {
        const bf16x4 a = *reinterpret_cast<lds_cptr<bf16x4>>(lo + off);
        const bf16x4 b = *reinterpret_cast<lds_cptr<bf16x4>>(hi + off);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f.v[t] = a[t];
            f.v[t + 4] = b[t];
        }
    } else {
        const f32x4 a = *reinterpret_cast<lds_cptr<f32x4>>(lo + off);
        const f32x4 b = *reinterpret_cast<lds_cptr<f32x4>>(hi + off);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f.v[t] = a[t];
            f.v[t + 4] = b[t];
        }
    }
}

// Volatile LDS accesses: each stays a separate ds_read_b64 / ds_write_b64 with
// an immediate offset from one base register (the compiler does not pair
// volatile accesses into ds_read2 / ds_write2).
template <typename T> using lds_vptr = const volatile T __attribute__((address_space(3))) *;
template <typename T> using lds_wptr = volatile T __attribute__((address_space(3))) *;

template <typename T> __device__ __forceinline__ lds_vptr<T> lds_v(const T *p) {
    return (lds_vptr<T>)(lds_cptr<T>)p;
}
template <typename T> __device__ __forceinline__ lds_wptr<T> lds_w(T *p) {
    return (lds_wptr<T>)(T __attribute__((address_space(3))) *)p;
}

// Four consecutive elements at base[off] as floats.
__device__ __forceinline__ f32x4 lds_get4(lds_vptr<__bf16> base, int off) {
    const bf16x4 b = *reinterpret_cast<lds_vptr<bf16x4>>(base + off);
    return __builtin_convertvector(b, f32x4);
}
__device__ __forceinline__ f32x4 lds_get4(lds_vptr<float> base, int off) {
    return *reinterpret_cast<lds_vptr<f32x4>>(base + off);
}
template <int PL> __device__ __forceinline__ f32x4 lds_get4(lds_vptr<bf16pl<PL>> base, int off) {
    const lds_vptr<__bf16> b = reinterpret_cast<lds_vptr<__bf16>>(base);
    return lds_get4(b, off) + lds_get4(b, off + PL);
}

// Split-assignment fragment: slots 0..3 from base[off..], slots 4..7 from
// base[off + 16..] (base = the lane's address of row p, column 4g).
__device__ __forceinline__ void lds_frag_split_v(Frag<__bf16> &f, lds_vptr<__bf16> base, int off) {
    const bf16x4 a = *reinterpret_cast<lds_vptr<bf16x4>>(base + off);
    const bf16x4 b = *reinterpret_cast<lds_vptr<bf16x4>>(base + off + 16);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f.v[t] = a[t];
        f.v[t + 4] = b[t];
    }
}
template <int PL> __device__ __forceinline__ void lds_frag_split_v(Frag<bf16p> &f, lds_vptr<bf16pl<PL>> base, int off) {
    const lds_vptr<__bf16> b = reinterpret_cast<lds_vptr<__bf16>>(base);
    Frag<__bf16> h, l;
    lds_frag_split_v(h, b, off);
    lds_frag_split_v(l, b, off + PL);
    f.hi = h.v;
    f.lo = l.v;
}
__device__ __forceinline__ void lds_frag_split_v(Frag<float> &f, lds_vptr<float> base, int off) {
    const f32x4 a = *reinterpret_cast<lds_vptr<f32x4>>(base + off);
    const f32x4 b = *reinterpret_cast<lds_vptr<f32x4>>(base + off + 16);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f.v[t] = a[t];
        f.v[t + 4] = b[t];
    }
}

// Four floats stored as four elements of the tile type at p[0..3].
__device__ __forceinline__ void lds_put4(__bf16 *p, const f32x4 &x) {
    *reinterpret_cast<lds_wptr<bf16x4>>(lds_w(p)) = __builtin_convertvector(x, bf16x4);
}
__device__ __forceinline__ void lds_put4(float *p, const f32x4 &x) {
    *reinterpret_cast<lds_wptr<f32x4>>(lds_w(p)) = x;
}

// Four floats as an operand value (hi) and, for bf16, the bf16 rounding of
// what that value leaves out (lo): hi + lo carries about 16 significant bits.
__device__ __forceinline__ void lds_put4_pair(__bf16 *hi, __bf16 *lo, const f32x4 &x) {
    const bf16x4 h = __builtin_convertvector(x, bf16x4);
    const f32x4 r = x - __builtin_convertvector(h, f32x4);
    *reinterpret_cast<lds_wptr<bf16x4>>(lds_w(hi)) = h;
    *reinterpret_cast<lds_wptr<bf16x4>>(lds_w(lo)) = __builtin_convertvector(r, bf16x4);
}
__device__ __forceinline__ void lds_put4_pair(float *hi, float *, const f32x4 &x) { lds_put4(hi, x); }
template <int PL> __device__ __forceinline__ void lds_put4(bf16pl<PL> *p, const f32x4 &x) {
    __bf16 *b = reinterpret_cast<__bf16 *>(p);
    lds_put4_pair(b, b + PL, x);
}
template <int PL> __device__ __forceinline__ void lds_put4_pair(bf16pl<PL> *hi, bf16pl<PL> *, const f32x4 &x) {
    lds_put4(hi, x);
}

// Transposed reads of a row-major tile (LDS), for operands whose K index is
// the tile's row index.  The result slots t = 0..3 of the lane at position p
// are tile[row0 + t][col0 + p] and slots 4..7 are tile[row1 + t][col0 + p];
// row0 and row1 must be the same for the 16 lanes of a lane group.
//
// bf16: one ds_read_b64_tr_b16 per half.  Inside each group of 16 lanes that
// instruction hands lane i the element i % 4 of the 8-byte rows fetched by
// lanes i / 4, i / 4 + 4, i / 4 + 8 and i / 4 + 12; so lane a fetches row
// row0 + a / 4 at columns col0 + 4 (a % 4) .. + 3.
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x4 lds_tr4(const __bf16 *tile, int ld, int row0, int col0, int p) {
    const __bf16 *a = tile + (row0 + (p >> 2)) * ld + col0 + 4 * (p & 3);
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(a));
    return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ void lds_frag_tr(Frag<__bf16> &f, const __bf16 *tile, int ld, int row0, int row1,
                                            int col0, int p) {
    const bf16x4 a = lds_tr4(tile, ld, row0, col0, p);
    const bf16x4 b = lds_tr4(tile, ld, row1, col0, p);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f.v[t] = a[t];
        f.v[t + 4] = b[t];
    }
}

// fp32 tiles: plain strided reads (the fp32 path is not bandwidth-critical).
__device__ __forceinline__ void lds_frag_tr(Frag<float> &f, const float *tile, int ld, int row0, int row1,
                                            int col0, int p) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f.v[t] = tile[(row0 + t) * ld + col0 + p];
        f.v[t + 4] = tile[(row1 + t) * ld + col0 + p];
    }
}

template <int PL>
__device__ __forceinline__ void lds_frag_tr(Frag<bf16p> &f, const bf16pl<PL> *tile, int ld, int row0, int row1,
                                            int col0, int p) {
    const __bf16 *b = reinterpret_cast<const __bf16 *>(tile);
    Frag<__bf16> h, l;
    lds_frag_tr(h, b, ld, row0, row1, col0, p);
    lds_frag_tr(l, b + PL, ld, row0, row1, col0, p);
    f.hi = h.v;
    f.lo = l.v;
}

template <typename TC> __device__ __forceinline__ void frag_ones(Frag<TC> &f) {
#pragma unroll
    for (int t = 0; t < 8; ++t) f.set(t, 1.0f);
}

// Build a split-assignment fragment from two accumulator tiles (lane holds
// rows 4g..4g+3 of each), rounding to the operand type.
template <typename TC>
__device__ __forceinline__ void acc_to_frag(Frag<TC> &f, const f32x4 &lo, const f32x4 &hi) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f.set(t, lo[t]);
        f.set(t + 4, hi[t]);
    }
}

// The rounding remainder of acc_to_frag: slot values x - TC(x), rounded to TC
// (zero for fp32 operands).  A product with f plus one with this remainder
// reproduces the fp32 accumulator values to about 16 significant bits.
template <typename TC>
__device__ __forceinline__ void acc_to_frag_lo(Frag<TC> &f, const f32x4 &lo, const f32x4 &hi) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f.set(t, lo[t] - to_operand<TC>(lo[t]));
        f.set(t + 4, hi[t] - to_operand<TC>(hi[t]));
    }
}

// ---------------------------------------------------------------------------
// Global memory element access for the two storage types.
// ---------------------------------------------------------------------------
template <typename TS> struct Store;

template <> struct Store<float> {
    static constexpr int VEC = 4;  // elements per 16-byte vector
    __device__ __forceinline__ static float load(const void *p, long i) {
        return static_cast<const float *>(p)[i];
    }
};

// fp32 values held in global memory as two bf16 planes (value, remainder) of
// one layout; staged into bf16-pair tiles.
struct bf16h {};
template <> struct Store<bf16h> {
    static constexpr int VEC = 8;  // elements per 16-byte vector of one plane
};

template <> struct Store<__bf16> {
    static constexpr int VEC = 8;
    __device__ __forceinline__ static float load(const void *p, long i) {
        return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
    }
};

// Unpack a 16-byte vector of storage elements to floats (VEC of them).
__device__ __forceinline__ void unpack16(const uint4 &u, float *out, float) {
    out[0] = __uint_as_float(u.x);
    out[1] = __uint_as_float(u.y);
    out[2] = __uint_as_float(u.z);
    out[3] = __uint_as_float(u.w);
}
__device__ __forceinline__ void unpack16(const uint4 &u, float *out, __bf16) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(w[i] << 16);
        out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// Sum over the four lane groups (lanes p, p+16, p+32, p+48).
__device__ __forceinline__ float sum_over_groups(float x) {
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

// The same sum with the gfx950 lane swaps (VALU, no LDS round trip): the
// 16-lane swap pairs rows 0-1 and 2-3 of the wave, the 32-lane swap its halves.
__device__ __forceinline__ float sum_over_groups_swap(float x) {
    const unsigned u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const unsigned v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace la
