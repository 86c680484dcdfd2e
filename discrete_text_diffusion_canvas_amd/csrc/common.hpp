// Shared device helpers for the gfx950 kernels: storage types, conversions,
// wavefront reductions and MFMA fragment types. CDNA4 only (wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

constexpr int WAVE = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---- bf16 <-> f32 (bf16 held as raw uint16_t in memory) ----
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// f32 -> bf16, round to nearest even, NaN stays NaN (quiet bit set): gfx950's
// v_cvt_pk_bf16_f32. Its results equal, for every one of the 2^32 inputs, the
// integer recipe u += 0x7fff + ((u >> 16) & 1) (NaN: (u >> 16) | 0x40),
// checked exhaustively on the device. f2bf2 packs two (a low, b high).
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ uint16_t f2bf(float f) { return (uint16_t)(f2bf2(f, 0.f) & 0xffffu); }

// round an f32 to the nearest bf16 value, kept as f32
__device__ __forceinline__ float round_bf(float f) { return bf2f(f2bf(f)); }

// ---- OCP e4m3fn byte -> f32 (exact; NaN code 0x7f/0xff -> NaN) ----
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    uint32_t s = (b & 0x80u) << 24;
    uint32_t e = (b >> 3) & 0xfu;
    uint32_t m = b & 0x7u;
    if (e == 0) {  // subnormal: m/8 * 2^-6 = m * 2^-9
        float v = (float)m * 0.001953125f;
        return __uint_as_float(__float_as_uint(v) | s);
    }
    if (e == 0xf && m == 0x7) return __uint_as_float(0x7fc00000u | s);
    // bias 7 -> bias 127: exponent + 120
    return __uint_as_float(s | ((e + 120u) << 23) | (m << 20));
}

// ---- wavefront reductions ----
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, WAVE));
    return v;
}

// Combine a value with the one in lane l ^ 16 (or l ^ 32) through gfx950's
// v_permlane16_swap / v_permlane32_swap with both operands the same register:
// each lane gets the pair {its value, the partner's} (checked on the device),
// so a commutative op leaves both lanes with the same bits. VALU only, no
// LDS round trip.
__device__ __forceinline__ float xor16_max(float v) {
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Max over the wavefront, the result in every lane: DPP moves inside each row
// of 16 lanes (swap neighbours, swap pairs, mirror halves of 8, mirror the
// row), then the two permlane swaps across rows. VALU only.
#define DG_MAX_DPP_STEP(v, ctrl) \
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, 0xF, 0xF, false)))
__device__ __forceinline__ float wave_max(float v) {
    DG_MAX_DPP_STEP(v, 0xB1);
    DG_MAX_DPP_STEP(v, 0x4E);
    DG_MAX_DPP_STEP(v, 0x141);
    DG_MAX_DPP_STEP(v, 0x140);
    return xor32_max(xor16_max(v));
}
#undef DG_MAX_DPP_STEP

// (value, index) argmax with lowest index on equal values
struct ArgMax {
    float v;
    int i;
};
__device__ __forceinline__ ArgMax argmax_merge(ArgMax a, ArgMax b) {
    if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
    return a;
}
// The merge is commutative and associative, so any pairing tree leaves the
// same result in every lane. Inside each row of 16 lanes the pairs come from
// DPP moves (swap neighbours, swap pairs, mirror halves of 8, mirror the
// row); the two cross-row steps are permlane swaps.
#define DG_ARGMAX_DPP_STEP(a, ctrl)                                                                       \
    a = argmax_merge(a, ArgMax{__builtin_bit_cast(float, __builtin_amdgcn_update_dpp(                    \
                                   0, __builtin_bit_cast(int, a.v), ctrl, 0xF, 0xF, false)),             \
                               __builtin_amdgcn_update_dpp(0, a.i, ctrl, 0xF, 0xF, false)})
__device__ __forceinline__ ArgMax wave_argmax(ArgMax a) {
    DG_ARGMAX_DPP_STEP(a, 0xB1);
    DG_ARGMAX_DPP_STEP(a, 0x4E);
    DG_ARGMAX_DPP_STEP(a, 0x141);
    DG_ARGMAX_DPP_STEP(a, 0x140);
    {   // cross-row steps: the swaps move v and i with the same lane pattern
        const auto v = __builtin_amdgcn_permlane16_swap(__float_as_uint(a.v), __float_as_uint(a.v), false, false);
        const auto i = __builtin_amdgcn_permlane16_swap((unsigned)a.i, (unsigned)a.i, false, false);
        a = argmax_merge(ArgMax{__uint_as_float(v[0]), (int)i[0]}, ArgMax{__uint_as_float(v[1]), (int)i[1]});
    }
    {
        const auto v = __builtin_amdgcn_permlane32_swap(__float_as_uint(a.v), __float_as_uint(a.v), false, false);
        const auto i = __builtin_amdgcn_permlane32_swap((unsigned)a.i, (unsigned)a.i, false, false);
        a = argmax_merge(ArgMax{__uint_as_float(v[0]), (int)i[0]}, ArgMax{__uint_as_float(v[1]), (int)i[1]});
    }
    return a;
}
#undef DG_ARGMAX_DPP_STEP

// Base-2 entropy partials of a set of tempered logits z2 = z * log2(e):
// m = max z2, s = sum 2^(z2-m), t = sum 2^(z2-m) (z2-m).
struct EntPart {
    float m, s, t;
};
// merge two partials onto the larger max
__device__ __forceinline__ EntPart ent_merge(EntPart a, EntPart b) {
    if (b.m > a.m) { EntPart c = a; a = b; b = c; }
    if (b.s == 0.f) return a;
    float d = b.m - a.m;  // <= 0
    float f = exp2f(d);
    a.s += b.s * f;
    a.t += f * (b.t + d * b.s);
    return a;
}
// Merge over the wavefront, the result in every lane: the DPP and permlane
// pairing of wave_max. The merge is commutative (bit for bit), so both lanes
// of every pair hold the same partial after each step.
#define DG_ENT_DPP_STEP(a, ctrl)                                                                              \
    a = ent_merge(a, EntPart{__builtin_bit_cast(float, __builtin_amdgcn_update_dpp(                           \
                                 0, __builtin_bit_cast(int, a.m), ctrl, 0xF, 0xF, false)),                    \
                             __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(                           \
                                 0, __builtin_bit_cast(int, a.s), ctrl, 0xF, 0xF, false)),                    \
                             __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(                           \
                                 0, __builtin_bit_cast(int, a.t), ctrl, 0xF, 0xF, false))})
#define DG_ENT_PERM_STEP(a, swap)                                                                             \
    {                                                                                                         \
        const auto m = swap(__float_as_uint(a.m), __float_as_uint(a.m), false, false);                        \
        const auto s = swap(__float_as_uint(a.s), __float_as_uint(a.s), false, false);                        \
        const auto t = swap(__float_as_uint(a.t), __float_as_uint(a.t), false, false);                        \
        a = ent_merge(EntPart{__uint_as_float(m[0]), __uint_as_float(s[0]), __uint_as_float(t[0])},           \
                      EntPart{__uint_as_float(m[1]), __uint_as_float(s[1]), __uint_as_float(t[1])});          \
    }
__device__ __forceinline__ EntPart wave_ent(EntPart a) {
    DG_ENT_DPP_STEP(a, 0xB1);
    DG_ENT_DPP_STEP(a, 0x4E);
    DG_ENT_DPP_STEP(a, 0x141);
    DG_ENT_DPP_STEP(a, 0x140);
    DG_ENT_PERM_STEP(a, __builtin_amdgcn_permlane16_swap);
    DG_ENT_PERM_STEP(a, __builtin_amdgcn_permlane32_swap);
    return a;
}
#undef DG_ENT_DPP_STEP
#undef DG_ENT_PERM_STEP

// Per-row partial written by the logit-statistics producers (LM-head epilogue
// and the standalone statistics kernel) and merged by the merge kernel.
struct RowPart {
    float m2;    // max of z2 over the tile (-inf if empty)
    float s;     // sum 2^(z2 - m2)
    float t;     // sum 2^(z2 - m2) (z2 - m2)
    float lmax;  // max raw (biased) logit over the tile
    int amax;    // its lowest column index (-1 if empty)
    int pad[3];  // Gumbel-max draws: [0] best z - log(-log u) (float bits), [1] its column (-1: none)
};

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC'11), written from the paper's description: ten rounds, each
// multiplying words 0 and 2 by fixed odd constants, swapping the high halves
// into the other words xor the round key; the key advances by two Weyl
// constants.
__device__ __forceinline__ u32x4 philox10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        uint32_t lo0 = 0xD2511F53u * c[0], hi0 = __umulhi(0xD2511F53u, c[0]);
        uint32_t lo1 = 0xCD9E8D57u * c[2], hi1 = __umulhi(0xCD9E8D57u, c[2]);
        u32x4 o;
        o[0] = hi1 ^ c[1] ^ k0;
        o[1] = lo1;
        o[2] = hi0 ^ c[3] ^ k1;
        o[3] = lo0;
        c = o;
    }
    return c;
}

// Gumbel noise -log(-log u) of one Philox word: u = (top 23 bits + 1/2) *
// 2^-23, exact in float32 and inside (0, 1).
__device__ __forceinline__ float gumbel_of(uint32_t w) {
    const float u = ((float)(w >> 9) + 0.5f) * 1.1920928955078125e-7f;
    return -logf(-logf(u));
}

}  // namespace dg
