// ggrms_epilogue.hpp -- the fused gated group-RMSNorm's per-unit arithmetic
// as gfx950 device functions, for any kernel that holds a (row, group) unit
// in registers: the library's own kernels (which load the unit from global
// memory) and a producer kernel that computes y itself and normalises it in
// its epilogue, before y ever reaches HBM.
//
// Per (row n, group g) unit of G contiguous columns, col = g*G + j (the page
// "gated_group_rmsnorm", math block):
//   a_j  = f32(y) * silu(f32(gate))                      (widen, gate)
//   m2   = sum_j a_j^2                                    (group reduction, f32)
//   nf   = rsqrt(m2 / G + eps)                            (eps after the mean)
//   out  = cast(w[col] * f32(cast(a_j * nf, dtype)), dtype) with the inner cast
//          only when round_intermediate is set,
// and the norm-first operator of the page "com.microsoft.GatedRMSNorm"
// (Description section): a_j = f32(y), out = cast(((a_j * nf) * w) *
// silu(gate)), every intermediate f32.
//
// How a caller uses it.  The unit's G elements are spread over the lanes that
// own it; a lane holds K slots, each one VB-byte vector of y and of gate in
// their storage format (Packet<T, VB>: N = VB / sizeof(T) elements).
//   1. gate_and_square: gates every slot and returns the lane's share of m2
//      (slots that hold no element of the unit, and pieces of a slot that
//      belong to a neighbouring unit, add nothing).
//   2. The caller sums the shares over the unit's lanes, in a fixed order so
//      every lane gets the same bits (segment_sum below covers lanes of one
//      wave; across waves the caller adds per-wave sums through LDS).
//   3. norm_factor turns the sum into the normaliser; finish applies it, the
//      optional intermediate cast, the weight and the narrowing cast, giving
//      each slot's output vector in storage format, ready for the caller's
//      own stores.
// A lane whose vector straddles the boundary of two units uses
// gate_and_square2 and finish_by_piece, which keep the two units' pieces
// apart.
// Steps 1 and 3 are per lane; a caller is free to lay slots over lanes as its
// own tile dictates, as long as step 2 combines exactly the unit's lanes.
// Results are deterministic and, for a given grouping of lanes, identical to
// the library's kernels bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ggrms {

using u16 = unsigned short;
using u32 = unsigned int;
typedef u16 u16x2 __attribute__((ext_vector_type(2)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Element types.  kSize = bytes per element.
struct TF32 { static constexpr int kSize = 4; };
struct TF16 { static constexpr int kSize = 2; };
struct TBF16 { static constexpr int kSize = 2; };

// Storage word for a VB-byte vector.
template <int VB> struct VecWord;
template <> struct VecWord<16> { using type = u32x4; };
template <> struct VecWord<8> { using type = u32x2; };
template <> struct VecWord<4> { using type = u32; };
template <> struct VecWord<2> { using type = u16; };

// ------------------------------------------------------------ conversions
// 16-bit -> f32 widening is exact.  f32 -> 16-bit narrowing uses the gfx950
// conversion instructions (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32), which round
// to nearest even under the default mode and keep subnormals.

template <class T> struct Cvt;

template <> struct Cvt<TF32> {
    static constexpr int kPerWord = 1;
    __device__ static inline void unpack_word(u32 w, float* f) { f[0] = __uint_as_float(w); }
    __device__ static inline u32 pack_word(const float* f) { return __float_as_uint(f[0]); }
    __device__ static inline void round_trip(float*) {}
};

template <> struct Cvt<TBF16> {
    static constexpr int kPerWord = 2;
    __device__ static inline void unpack_word(u32 w, float* f) {
        f[0] = __uint_as_float(w << 16);
        f[1] = __uint_as_float(w & 0xFFFF0000u);
    }
    __device__ static inline u32 pack_word(const float* f) {
        f32x2 v = {f[0], f[1]};
        return __builtin_bit_cast(u32, __builtin_convertvector(v, bf16x2));
    }
    __device__ static inline float unpack_half(u16 h) { return __uint_as_float((u32)h << 16); }
    __device__ static inline u16 pack_half(float f) {
        return __builtin_bit_cast(u16, (__bf16)f);
    }
    __device__ static inline void round_trip(float* f) { unpack_word(pack_word(f), f); }
};

template <> struct Cvt<TF16> {
    static constexpr int kPerWord = 2;
    __device__ static inline void unpack_word(u32 w, float* f) {
        f32x2 v = __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
        f[0] = v.x;
        f[1] = v.y;
    }
    __device__ static inline u32 pack_word(const float* f) {
        f32x2 v = {f[0], f[1]};
        return __builtin_bit_cast(u32, __builtin_convertvector(v, f16x2));
    }
    __device__ static inline float unpack_half(u16 h) {
        return (float)__builtin_bit_cast(_Float16, h);
    }
    __device__ static inline u16 pack_half(float f) {
        return __builtin_bit_cast(u16, (_Float16)f);
    }
    __device__ static inline void round_trip(float* f) { unpack_word(pack_word(f), f); }
};

// A VB-byte vector of T: N elements.
template <class T, int VB> struct Packet {
    static constexpr int N = VB / T::kSize;
    using W = typename VecWord<VB>::type;

    __device__ static inline void unpack(const W& v, float (&f)[N]) {
        if constexpr (VB == 2) {
            f[0] = Cvt<T>::unpack_half(v);
        } else if constexpr (VB == 4) {
            Cvt<T>::unpack_word(v, f);
        } else {
#pragma unroll
            for (int i = 0; i < VB / 4; ++i) Cvt<T>::unpack_word(v[i], f + i * Cvt<T>::kPerWord);
        }
    }

    __device__ static inline W pack(const float (&f)[N]) {
        if constexpr (VB == 2) {
            return Cvt<T>::pack_half(f[0]);
        } else if constexpr (VB == 4) {
            return Cvt<T>::pack_word(f);
        } else {
            W v;
#pragma unroll
            for (int i = 0; i < VB / 4; ++i) v[i] = Cvt<T>::pack_word(f + i * Cvt<T>::kPerWord);
            return v;
        }
    }

    // cast to T and back, element-wise
    __device__ static inline void round_trip(float (&f)[N]) {
        if constexpr (VB == 2) {
            f[0] = Cvt<T>::unpack_half(Cvt<T>::pack_half(f[0]));
        } else {
#pragma unroll
            for (int i = 0; i < N; i += Cvt<T>::kPerWord) Cvt<T>::round_trip(f + i);
        }
    }
};

// 32-bit word i of a VB-byte vector (VB >= 4).
template <int VB, class W> __device__ inline uint32_t word_of(const W& v, int i) {
    if constexpr (VB == 4)
        return (uint32_t)v;
    else
        return v[i];
}

// ------------------------------------------------------------ arithmetic

// silu(x) = x / (1 + e^-x): e^-x by v_exp_f32 (2^t with t = -x*log2 e), the
// reciprocal by v_rcp_f32, five VALU operations.  The reciprocal is only
// trusted while its result is a normal number, i.e. while 1 + e^-x < 2^126
// (x > -87.33); below that it may flush to zero where the quotient is a tiny
// non-zero number.  silu_exact scales both operands by 2^-64 once the
// denominator passes 2^64, which keeps the reciprocal normal and changes no
// bits elsewhere (power-of-two scalings are exact); kernels take it only when
// some gate of the wave is below kSiluFastMin.
constexpr float kSiluFastMin = -87.0f;

// Whether some gate is below kSiluFastMin, from the raw bits: for negative
// numbers the sign-magnitude pattern, read as an unsigned integer of the
// element's width, grows with the magnitude, so the lane keeps the largest
// pattern of its gate words (one packed 16-bit maximum per two bf16/fp16
// gates, no widening) and compares it with the pattern of -87 at the end.
// A NaN with its sign bit set also selects the exact form, which gives it
// the same result.
template <class T> __device__ inline u32 gate_max_word(u32 acc, u32 w) {
    if constexpr (T::kSize == 4)
        return acc > w ? acc : w;
    else
        return __builtin_bit_cast(u32, __builtin_elementwise_max(__builtin_bit_cast(u16x2, acc),
                                                                  __builtin_bit_cast(u16x2, w)));
}
template <class T> struct FastMinBits;  // bit pattern of kSiluFastMin (-87)
template <> struct FastMinBits<TF32> { static constexpr u32 v = 0xC2AE0000u; };
template <> struct FastMinBits<TBF16> { static constexpr u32 v = 0xC2AEu; };
template <> struct FastMinBits<TF16> { static constexpr u32 v = 0xD570u; };
template <class T> __device__ inline bool gate_below_fast_min(u32 acc) {
    if constexpr (T::kSize == 4) {
        return acc > FastMinBits<T>::v;
    } else {
        const u32 lo = acc & 0xFFFFu, hi = acc >> 16;
        return (lo > hi ? lo : hi) > FastMinBits<T>::v;
    }
}

__device__ inline float silu_fast(float x) {
    const float e = __builtin_amdgcn_exp2f(x * -1.4426950408889634f);
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}

__device__ inline float silu_exact(float x) {
    const float e = __builtin_amdgcn_exp2f(x * -1.4426950408889634f);
    const float d = 1.0f + e;
    const float sc = d > 0x1p64f ? 0x1p-64f : 1.0f;
    return (x * sc) * __builtin_amdgcn_rcpf(d * sc);
}

// -0.0f that the compiler cannot see through (a v_mov of the bit pattern),
// so that fma(x, b, nz) is kept as an FMA instead of being folded into a
// multiply.
__device__ inline float opaque_neg_zero() {
    float z;
    asm("v_mov_b32 %0, 0x80000000" : "=v"(z));
    return z;
}

// f32(half h of the fp16 pair `word`) * b, rounded once, as fma(x, b, -0):
// gfx950 issues it as one v_fma_mix_f32, which widens the 16-bit operand
// exactly inside the FMA and so saves the separate v_cvt_f32_f16 of each fp16
// operand; the addend -0 leaves every product -- a zero's sign included -- as
// the f32 multiply of the widened value gives it.  The compiler emits the
// instruction itself, so its hazard checks cover it (a transcendental's result
// read by the next VALU instruction needs a wait state).  gfx950 has no bf16
// form.
__device__ inline float mul_f16(uint32_t word, int h, float b, float nz) {
    const _Float16 x = __builtin_bit_cast(_Float16, (u16)(h ? word >> 16 : word & 0xFFFFu));
    return __builtin_fmaf((float)x, b, nz);
}

// silu_fast of half h of an fp16 pair, and y * silu(gate) for element h of
// the pairs yw, gw, with the widening folded into the multiplies: the same
// operations in the same order as y * silu_fast(gate) on widened values.
__device__ inline float gated_f16(uint32_t yw, uint32_t gw, int h, float nz) {
    const float e = __builtin_amdgcn_exp2f(mul_f16(gw, h, -1.4426950408889634f, nz));
    const float s = mul_f16(gw, h, __builtin_amdgcn_rcpf(1.0f + e), nz);
    return mul_f16(yw, h, s, nz);
}

// DPP move with all rows and banks enabled.
template <int CTRL> __device__ inline float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ inline float readlane(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over aligned segments of SEG lanes (SEG a power of two, <= 64).  Every
// lane of a segment gets the same bits.  Steps: swap neighbours, swap pairs
// (quad_perm), mirror within 8 (row_half_mirror), mirror within 16
// (row_mirror); then whole 16-lane rows are combined with v_readlane.
template <int SEG> __device__ inline float segment_sum(float v) {
    if constexpr (SEG >= 2) v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    if constexpr (SEG >= 4) v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    if constexpr (SEG >= 8) v += dpp<0x141>(v);  // row_half_mirror
    if constexpr (SEG >= 16) v += dpp<0x140>(v); // row_mirror
    if constexpr (SEG == 32) {
        const float r0 = readlane(v, 0), r1 = readlane(v, 16);
        const float r2 = readlane(v, 32), r3 = readlane(v, 48);
        v = (threadIdx.x & 32) ? (r2 + r3) : (r0 + r1);
    }
    if constexpr (SEG == 64) {
        const float r0 = readlane(v, 0), r1 = readlane(v, 16);
        const float r2 = readlane(v, 32), r3 = readlane(v, 48);
        v = (r0 + r1) + (r2 + r3);
    }
    return v;
}

// nf = 1/sqrt(m2/G + eps): the mean and eps in one fused multiply-add with
// 1/G rounded once on the host, then v_rsq_f32 (about 1 ulp).  The result is
// within a few f32 ulp of the correctly rounded steps (divide, add, square
// root, divide), for a few VALU operations instead of ~35 IEEE-exact ones
// per lane.  An argument below FLT_MIN is scaled by 2^64 first and the
// result by 2^32, so tiny means are not flushed; 0 gives +inf, inf gives 0,
// NaN stays NaN.
__device__ inline float norm_factor(float m2, float ginv, float eps) {
    const float v = __builtin_fmaf(m2, ginv, eps);
    const bool tiny = v < 0x1p-126f;
    const float r = __builtin_amdgcn_rsqf(tiny ? v * 0x1p64f : v);
    return tiny ? r * 0x1p32f : r;
}

// ------------------------------------------------------------ per-unit steps

namespace epi {

// What a lane holds of one unit between the two steps: K slots of N
// elements.  a: gate first, y * silu(gate); norm first, y.  s: norm first,
// silu(gate) (unused gate first).
template <class T, int VB, int K, bool NBG> struct LaneUnit {
    using P = Packet<T, VB>;
    using W = typename P::W;
    static constexpr int N = P::N;
    float a[K][N];
    float s[NBG ? K : 1][N];
};

// fp16 gate first multiplies fp16 operands without a separate widening
// (mul_f16); other types and the norm-first operator widen first.
template <class T, int VB, bool NBG>
constexpr bool kMixMul = std::is_same<T, TF16>::value && VB >= 4 && !NBG;

// Step 1 (A1 widen, A2 gate, A3 this lane's share of the sum of squares).
//
//   yr, gr   the lane's K slots of y and gate, as loaded (storage format).
//   live(k)  whether slot k holds any element of the unit; a slot that does
//            not (a lane past the unit's end, holding a copy of some other
//            vector) is computed like the others and its sum dropped, so no
//            load needs predication.
//   owned(k, q)  whether piece q (PB bytes, VB / PB pieces per slot) of slot
//            k belongs to the unit; only consulted when PB < VB, for units
//            whose boundaries fall inside a vector ("packed" groups, whose
//            byte length is not a multiple of the vector).  Unit boundaries
//            never split a piece.
//
// Each slot's elements are squared and added in element order with fused
// multiply-adds, a piece that is not owned leaving the running sum as it is
// (one select per piece, not per element); the slots' sums are added in slot
// order.  When some gate of the wave is deep in silu's underflow range (below
// -87; it must be called by every lane of the wave), the wave redoes silu
// with the exact form, which gives identical bits for every other gate.
template <class T, int VB, int PB, int K, bool NBG, class Live, class Owned>
__device__ __forceinline__ float gate_and_square(
    const typename VecWord<VB>::type (&yr)[K], const typename VecWord<VB>::type (&gr)[K],
    LaneUnit<T, VB, K, NBG>& L, Live live, Owned owned) {
    using P = Packet<T, VB>;
    constexpr int N = P::N;
    constexpr int PE = PB / T::kSize;  // elements per piece
    constexpr int NPIECE = VB / PB;
    constexpr bool kMix = kMixMul<T, VB, NBG>;
    const float nz = kMix ? opaque_neg_zero() : 0.0f;

    // one slot's share, given a way to produce its gated values
    auto slot_sum = [&](int k, auto value) {
        float part = 0.0f;
#pragma unroll
        for (int q = 0; q < NPIECE; ++q) {
            float p = part;
#pragma unroll
            for (int i = 0; i < PE; ++i) {
                const int e = q * PE + i;
                const float x = value(e);
                L.a[k][e] = x;
                p = __builtin_fmaf(x, x, p);
            }
            if constexpr (NPIECE > 1)
                part = owned(k, q) ? p : part;
            else
                part = p;
        }
        return part;
    };

    float acc = 0.0f;
    u32 gmax = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        float yf[N], gf[N];
        if constexpr (!kMix) {
            P::unpack(yr[k], yf);
            P::unpack(gr[k], gf);
        }
        if constexpr (VB <= 4) {
            gmax = gate_max_word<T>(gmax, (u32)gr[k]);
        } else {
#pragma unroll
            for (int i = 0; i < VB / 4; ++i) gmax = gate_max_word<T>(gmax, gr[k][i]);
        }
        if constexpr (NBG) {
#pragma unroll
            for (int e = 0; e < N; ++e) L.s[k][e] = silu_fast(gf[e]);
        }
        const float part = slot_sum(k, [&](int e) {
            if constexpr (kMix)
                return gated_f16(word_of<VB>(yr[k], e / 2), word_of<VB>(gr[k], e / 2), e & 1, nz);
            else if constexpr (NBG)
                return yf[e];
            else
                return yf[e] * silu_fast(gf[e]);
        });
        acc += live(k) ? part : 0.0f;
    }
    // Rare: a gate deep in silu's underflow range.  Redo the wave's silu with
    // the exact form (identical bits for every other gate).
    const bool exact_silu = __builtin_expect(__any(gate_below_fast_min<T>(gmax)), 0);
    if (NBG && exact_silu) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float gf[N];
            P::unpack(gr[k], gf);
#pragma unroll
            for (int e = 0; e < N; ++e) L.s[k][e] = silu_exact(gf[e]);
        }
    }
    if (!NBG && exact_silu) {
        acc = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float yf[N], gf[N];
            P::unpack(yr[k], yf);
            P::unpack(gr[k], gf);
            const float part = slot_sum(k, [&](int e) { return yf[e] * silu_exact(gf[e]); });
            acc += live(k) ? part : 0.0f;
        }
    }
    return acc;
}

// Step 1 for a lane whose slots hold elements of two consecutive units: each
// PB-byte piece goes to the first unit's share, s_first, or -- where
// second(k, q) holds -- to the second unit's, s_second (each a chain over its
// pieces in element order, slots added in slot order, as gate_and_square
// does for one unit).  Slots that are not live add to neither.
template <class T, int VB, int PB, int K, bool NBG, class Live, class Second>
__device__ __forceinline__ void gate_and_square2(
    const typename VecWord<VB>::type (&yr)[K], const typename VecWord<VB>::type (&gr)[K],
    LaneUnit<T, VB, K, NBG>& L, Live live, Second second, float& s_first, float& s_second) {
    static_assert(VB >= 4, "whole 32-bit words per slot");
    using P = Packet<T, VB>;
    constexpr int N = P::N;
    constexpr int PE = PB / T::kSize;
    constexpr int NPIECE = VB / PB;
    constexpr bool kMix = kMixMul<T, VB, NBG>;
    const float nz = kMix ? opaque_neg_zero() : 0.0f;

    auto slot_sums = [&](int k, auto value, float& p0, float& p1) {
        p0 = 0.0f;
        p1 = 0.0f;
#pragma unroll
        for (int q = 0; q < NPIECE; ++q) {
            const bool to1 = second(k, q);
            float p = to1 ? p1 : p0;
#pragma unroll
            for (int i = 0; i < PE; ++i) {
                const int e = q * PE + i;
                const float x = value(e);
                L.a[k][e] = x;
                p = __builtin_fmaf(x, x, p);
            }
            p0 = to1 ? p0 : p;
            p1 = to1 ? p : p1;
        }
    };

    float acc0 = 0.0f, acc1 = 0.0f;
    u32 gmax = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        float yf[N], gf[N];
        if constexpr (!kMix) {
            P::unpack(yr[k], yf);
            P::unpack(gr[k], gf);
        }
#pragma unroll
        for (int i = 0; i < VB / 4; ++i) gmax = gate_max_word<T>(gmax, word_of<VB>(gr[k], i));
        if constexpr (NBG) {
#pragma unroll
            for (int e = 0; e < N; ++e) L.s[k][e] = silu_fast(gf[e]);
        }
        float p0, p1;
        slot_sums(k, [&](int e) {
            if constexpr (kMix)
                return gated_f16(word_of<VB>(yr[k], e / 2), word_of<VB>(gr[k], e / 2), e & 1, nz);
            else if constexpr (NBG)
                return yf[e];
            else
                return yf[e] * silu_fast(gf[e]);
        }, p0, p1);
        acc0 += live(k) ? p0 : 0.0f;
        acc1 += live(k) ? p1 : 0.0f;
    }
    const bool exact_silu = __builtin_expect(__any(gate_below_fast_min<T>(gmax)), 0);
    if (NBG && exact_silu) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float gf[N];
            P::unpack(gr[k], gf);
#pragma unroll
            for (int e = 0; e < N; ++e) L.s[k][e] = silu_exact(gf[e]);
        }
    }
    if (!NBG && exact_silu) {
        acc0 = 0.0f;
        acc1 = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float yf[N], gf[N];
            P::unpack(yr[k], yf);
            P::unpack(gr[k], gf);
            float p0, p1;
            slot_sums(k, [&](int e) { return yf[e] * silu_exact(gf[e]); }, p0, p1);
            acc0 += live(k) ? p0 : 0.0f;
            acc1 += live(k) ? p1 : 0.0f;
        }
    }
    s_first = acc0;
    s_second = acc1;
}

// Step 3 (A5 scale and optional intermediate cast, A6 weight and narrowing
// cast): the output vector of every slot, in storage format, from the unit's
// normaliser nf = norm_factor(m2, 1/G, eps) (A4; the same bits on every lane
// of the unit, as m2 is) and the slots' f32 weights.  RI: cast a*nf to T and
// back before the weight multiply (gate first only).  finish_by_piece takes
// the normaliser per PE-element piece, nf(k, q), for slots that hold the
// elements of two units.
template <bool RI, int PE, class T, int VB, int K, bool NBG, class NF>
__device__ __forceinline__ void finish_by_piece(const LaneUnit<T, VB, K, NBG>& L, NF nf,
                                                const float (&w)[K][Packet<T, VB>::N],
                                                typename VecWord<VB>::type (&res)[K]) {
    using P = Packet<T, VB>;
    using W = typename P::W;
    constexpr int N = P::N;
    constexpr bool kMix = kMixMul<T, VB, NBG>;
    const float nz = kMix ? opaque_neg_zero() : 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        float t[N];
#pragma unroll
        for (int e = 0; e < N; ++e) t[e] = L.a[k][e] * nf(k, e / PE);
        if constexpr (NBG) {
            // ((y * nf) * w) * silu(gate), every intermediate f32
#pragma unroll
            for (int e = 0; e < N; ++e) t[e] = (t[e] * w[k][e]) * L.s[k][e];
        } else if constexpr (RI && kMix) {
            // cast to fp16, then weight * f32(cast) with the widening folded in
            const W h = P::pack(t);
#pragma unroll
            for (int e = 0; e < N; ++e) t[e] = mul_f16(word_of<VB>(h, e / 2), e & 1, w[k][e], nz);
        } else {
            if constexpr (RI) P::round_trip(t);
#pragma unroll
            for (int e = 0; e < N; ++e) t[e] = w[k][e] * t[e];
        }
        res[k] = P::pack(t);
    }
}

template <bool RI, class T, int VB, int K, bool NBG>
__device__ __forceinline__ void finish(const LaneUnit<T, VB, K, NBG>& L, float nf,
                                       const float (&w)[K][Packet<T, VB>::N],
                                       typename VecWord<VB>::type (&res)[K]) {
    finish_by_piece<RI, Packet<T, VB>::N>(L, [nf](int, int) { return nf; }, w, res);
}

}  // namespace epi
}  // namespace ggrms
