// ggrms_kernels.hpp -- gfx950 (CDNA4) kernels of the fused gated
// group-RMSNorm: how each launch shape maps (row, group) units onto lanes,
// loads them, combines their sums and stores them.  The per-unit arithmetic
// (widen, gate, sum of squares, normaliser, casts, weight) is the epilogue in
// ggrms_epilogue.hpp, which these kernels call on units they load from global
// memory.
//
// The op is HBM-bound (two 16-bit input streams and one output stream; a few
// VALU ops per element), so the design is about moving bytes:
//   * every y/gate/out access is a VB-byte vector (16 B when alignment allows),
//     one vector per lane per step, so a wave instruction covers a contiguous
//     64*VB-byte run; groups whose byte length is not a multiple of 16 in
//     rows that are keep 16-byte vectors counted from the row start
//     ("packed", boundary vectors stored in PB-byte pieces);
//   * large jobs stream y/gate/out with the non-temporal hint, small ones
//     (decode) keep their lines cached (the NT template argument);
//   * a unit is read once into registers; its reduction happens in registers
//     and the outputs are written from the same registers (single pass);
//   * lanes past the end of a group re-load the group's last vector (an L1/L2
//     hit, no extra HBM traffic) and contribute 0, so no load is predicated
//     and all loads of a lane are issued before the first use;
//   * the group sum uses DPP row operations inside 16-lane rows and
//     v_readlane across rows: no LDS and no barrier unless a group spans
//     several waves (BLOCK), where one LDS slot per wave and one barrier
//     combine the partial sums;
//   * every lane of a group ends with a bit-identical m2 (the same additions
//     in the same order), so nf is uniform over the group and the result is
//     deterministic run to run;
//   * VALU work is kept low (it runs about half busy at the HBM rate): one
//     exp and one reciprocal per silu, the normaliser as a fused multiply-add
//     and v_rsq_f32, the silu-underflow test on raw gate bits, fp16 operands
//     multiplied without a separate widening (v_fma_mix_f32), and packed
//     groups leaving a neighbour's elements out with one select per piece;
//   * which workgroup takes which rows and groups (row-major or XCD-banded
//     order, WAVE workgroups of one or four waves) is a launch argument and
//     changes no result bit.
// Nothing here uses MFMA: there is no contraction to feed it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ggrms_epilogue.hpp"
#include "ggrms_internal.h"

namespace ggrms {

// Accesses of y, gate and out.  Each is touched once per launch; with NT they
// carry the non-temporal hint (the nt bit), which on gfx950 takes a large
// two-read-one-write stream from ~72% to ~81% of HBM peak against plain
// accesses.  Small jobs (decode) use plain accesses: their inputs are usually
// still in L2 from the kernel that wrote them and their output is read next,
// so keeping lines cached is worth more than streaming them.  The weight,
// re-read by every row, always stays cached.
template <bool NT, class W> __device__ inline W load_stream(const W* p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}
template <bool NT, class W> __device__ inline void store_stream(W* p, W v) {
    if constexpr (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// N consecutive f32 weights; p is aligned to min(16, 4N) bytes.
template <int N> __device__ inline void load_weights(const float* p, float (&w)[N]) {
    if constexpr (N >= 4) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            f32x4 v = *reinterpret_cast<const f32x4*>(p + i);
            w[i] = v.x; w[i + 1] = v.y; w[i + 2] = v.z; w[i + 3] = v.w;
        }
    } else if constexpr (N == 2) {
        f32x2 v = *reinterpret_cast<const f32x2*>(p);
        w[0] = v.x; w[1] = v.y;
    } else {
        w[0] = p[0];
    }
}

// The N weights of a packed vector when one [G] weight is shared by every
// group, piece by piece: piece q (PE elements) of the vector is columns
// base + q*PE .. + PE - 1 of its group, inside [0, G) for the pieces the unit
// owns; a neighbour's piece of a boundary vector (never stored by this unit)
// reads a clamped place.  G and the vector's start are multiples of PE, so
// every piece's weights are PE consecutive floats aligned to 4*PE bytes: two
// 16-byte loads per 16-byte vector of 16-bit values for 8-byte pieces (as
// with a weight per column), 8-byte loads for 4-byte pieces, one 4-byte load
// per element for 2-byte pieces.
template <int N, int PE> __device__ inline void load_weights_shared(const float* w, int32_t base,
                                                                    int32_t G, float (&r)[N]) {
#pragma unroll
    for (int q = 0; q < N / PE; ++q) {
        int32_t i = base + q * PE;
        i = i < 0 ? 0 : (i > G - PE ? G - PE : i);
        float piece[PE];
        load_weights<PE>(w + i, piece);
#pragma unroll
        for (int e = 0; e < PE; ++e) r[q * PE + e] = piece[e];
    }
}

// s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(15): gfx9 encoding (vmcnt in bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8) -- waits for vector memory only.
constexpr int kWaitVmcnt0 = 0x0F70;

__device__ inline uint32_t fast_div(uint32_t n, uint32_t m, uint32_t s) {
    return (__umulhi(n, m) + n) >> s;
}

// Materialises the argument words that only one tile order reads in scalar
// registers at the kernel's entry, so that every argument is fetched in one
// round of scalar loads.  Otherwise the compiler sinks those loads into the
// order's branch, and the row-major path waits for a second round trip to
// the argument block before it can address its first vector -- which is on
// the critical path of a small launch such as decode.
__device__ __forceinline__ void fetch_args_together(const KArgs& a) {
    asm volatile("" ::"s"(a.groups), "s"(a.div_m), "s"(a.xc), "s"(a.xc_m), "s"(a.bits));
}

// Fields of KArgs::bits, and what the kernels derive from the arguments.
__device__ inline uint32_t div_shift(const KArgs& a) { return (a.bits >> kBitDivShift) & 31u; }
__device__ inline uint32_t xc_shift(const KArgs& a) { return (a.bits >> kBitXcShift) & 31u; }
__device__ inline bool round_intermediate(const KArgs& a) { return (a.bits & kBitRound) != 0; }
__device__ inline bool banded(const KArgs& a) { return (a.bits & kBitBand) != 0; }
__device__ inline uint32_t super_shift(const KArgs& a) { return (a.bits >> kBitSuperShift) & 7u; }
// the weight's offset between groups: G (one weight per column) or 0 (shared)
__device__ inline int64_t weight_group_stride(const KArgs& a) {
    return (a.bits & kBitShared) ? 0 : (int64_t)a.G;
}
__device__ inline uint32_t row_div(const KArgs& a, uint32_t x) {  // x / groups
    return fast_div(x, a.div_m, div_shift(a));
}

// Magic numbers for x / d, d = 1..7 (the short block of the banded order),
// by the same round-up method as the host's: l = ceil(log2 d),
// m = floor(2^32 (2^l - d) / d) + 1.
struct SmallMagic { uint32_t m[8], s[8]; };
constexpr SmallMagic small_magic() {
    SmallMagic r{};
    for (uint32_t d = 1; d < 8; ++d) {
        uint32_t l = 0;
        while ((1u << l) < d) ++l;
        r.m[d] = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
        r.s[d] = l;
    }
    return r;
}
constexpr SmallMagic kSmallMagic = small_magic();

// ------------------------------------------------------------ one unit

// Where the output multiply takes its weights from: each lane loads its own
// from global memory, or the workgroup staged the group's weights in LDS.
enum class WSource { Global, Lds };

// A PB-byte piece of a VB-byte vector (PB < VB), written alone.
template <int PB, class W> __device__ inline void store_piece(char* p, const W& v, int piece) {
    if constexpr (PB == 8) {
        const u32x2 h = piece ? u32x2{v[2], v[3]} : u32x2{v[0], v[1]};
        *reinterpret_cast<u32x2*>(p) = h;
    } else if constexpr (PB == 4) {
        *reinterpret_cast<u32*>(p) = v[piece];
    } else {
        *reinterpret_cast<u16*>(p) = (u16)(v[piece >> 1] >> (16 * (piece & 1)));
    }
}
template <bool NT, int PB, class W>
__device__ inline void store_piece_stream(char* p, const W& v, int piece) {
    if constexpr (!NT) {
        store_piece<PB>(p, v, piece);
    } else if constexpr (PB == 8) {
        const u32x2 h = piece ? u32x2{v[2], v[3]} : u32x2{v[0], v[1]};
        __builtin_nontemporal_store(h, reinterpret_cast<u32x2*>(p));
    } else if constexpr (PB == 4) {
        __builtin_nontemporal_store(v[piece], reinterpret_cast<u32*>(p));
    } else {
        __builtin_nontemporal_store((u16)(v[piece >> 1] >> (16 * (piece & 1))),
                                    reinterpret_cast<u16*>(p));
    }
}

// The 16-byte vector whose PB-byte pieces are those of `own` where
// mine(q) holds and those of `other` elsewhere.
template <int PB, class Mine>
__device__ inline u32x4 merge_pieces(const u32x4& own, const u32x4& other, Mine mine) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (PB >= 4) {
            r[i] = mine(i * 4 / PB) ? own[i] : other[i];
        } else {
            const u32 lo = mine(2 * i) ? own[i] : other[i];
            const u32 hi = mine(2 * i + 1) ? own[i] : other[i];
            r[i] = (lo & 0xFFFFu) | (hi & 0xFFFF0000u);
        }
    }
    return r;
}

// Lane `sl` of the SEG lanes that own the unit (row n, group g) loads VPT
// vectors (indices sl, sl+SEG, ...), runs the epilogue's per-unit steps on
// them, sums its share with `reduce`, and stores if `store_ok`.  With
// WSource::Lds, `wl` points at the group's weights in LDS, valid once
// `reduce` has passed its barrier.
//
// PB == VB: every group starts on a vector boundary and spans a.nvec whole
// vectors.  PB < VB (packed): the group's byte length is not a multiple of
// the 16-byte vector but the rows are, so vectors are counted from the row's
// start and the unit takes the vectors that hold any of its elements; a
// vector on a group boundary also holds a neighbour's elements, which are
// left out of the sum and not written by this unit: such a vector is stored
// whole by the left unit's lane when both units sit on segments of one wave,
// and in PB-byte pieces otherwise (PB = gcd(group bytes, 16), so a group
// boundary never splits a piece).  Reads stay inside the row; every element
// is written by exactly one unit.
template <class T, int VB, int PB, int SEG, int VPT, bool NBG, bool NT, WSource WS, class Reduce>
__device__ __forceinline__ void unit_pass(const KArgs& a, uint32_t n, uint32_t g, uint32_t sl,
                                          bool store_ok, const float* wl, Reduce reduce) {
    using P = Packet<T, VB>;
    using W = typename P::W;
    constexpr int N = P::N;
    using S = typename VecWord<T::kSize>::type;  // element storage
    constexpr bool kPacked = PB < VB;
    constexpr int PE = PB / T::kSize;  // elements per piece
    static_assert(!kPacked || (VB == 16 && WS == WSource::Global), "packed: 16-byte vectors");
    // With three or more vectors per lane the per-lane weights are loaded
    // after the reduction, so they are not live at the same time as the
    // inputs: 4 vectors drop from ~140 to ~110 VGPRs (3 -> 4 waves per SIMD;
    // 512 x 4 runs 14-18% faster) and the 1024-lane shape, capped at 128
    // VGPRs, no longer spills.  Narrower shapes keep the early loads, which
    // overlap the input stream.
    constexpr bool kLateWeights = WS == WSource::Global && VPT >= 3;

    const int64_t col0 = (int64_t)g * a.G;
    const int64_t cbase = kPacked ? 0 : col0;  // column of vector 0
    const W* yv = reinterpret_cast<const W*>(static_cast<const S*>(a.y) + (int64_t)n * a.sy + cbase);
    const W* gv =
        reinterpret_cast<const W*>(static_cast<const S*>(a.gate) + (int64_t)n * a.sg + cbase);
    W* ov = reinterpret_cast<W*>(static_cast<S*>(a.out) + (int64_t)n * a.so + cbase);
    const float* wp = kPacked ? a.w : a.w + (int64_t)g * weight_group_stride(a);
    // vectors of this unit: v0 .. v0 + nv - 1 (packed: those holding any of
    // columns col0 .. col0 + G - 1)
    uint32_t v0 = 0, nv = a.nvec;
    if constexpr (kPacked) {
        v0 = (uint32_t)(col0 / N);
        nv = (uint32_t)((col0 + a.G + N - 1) / N) - v0;
    }

    W yr[VPT], gr[VPT];
    float wr[VPT][N];
    uint32_t ci[VPT];
    int32_t rel[VPT];  // packed: column of the vector's first element minus col0
    // packed groups with one shared [G] weight: weights by element (see
    // load_weights_shared); otherwise the vector's N consecutive weights
    const bool wshared = kPacked && (a.bits & kBitShared) != 0;
    auto weights_of = [&](int k, float (&r)[N]) {
        if (kPacked && wshared)
            load_weights_shared<N, (PE < N ? PE : N)>(a.w, rel[k], (int32_t)a.G, r);
        else
            load_weights<N>(wp + (int64_t)ci[k] * N, r);
    };
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const uint32_t idx = sl + k * SEG;
        ci[k] = v0 + (idx < nv ? idx : nv - 1);
        rel[k] = kPacked ? (int32_t)((int64_t)ci[k] * N - col0) : 0;
        yr[k] = load_stream<NT>(yv + ci[k]);
        gr[k] = load_stream<NT>(gv + ci[k]);
        if constexpr (WS == WSource::Global && !kLateWeights) weights_of(k, wr[k]);
    }
    // whether piece q of vector k belongs to the unit (packed groups only)
    auto owned = [&](int k, int q) { return (uint32_t)(rel[k] + q * PE) < a.G; };
    // lanes past the group's end hold a copy of its last vector
    auto live = [&](int k) { return sl + k * SEG < nv; };

    epi::LaneUnit<T, VB, VPT, NBG> L;
    const float acc = epi::gate_and_square<T, VB, PB, VPT, NBG>(yr, gr, L, live, owned);
    const float m2 = reduce(acc);
    const float nf = norm_factor(m2, a.Ginv, a.eps);
    if constexpr (WS == WSource::Lds) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) load_weights<N>(wl + ci[k] * N, wr[k]);  // v0 == 0 here
    } else if constexpr (kLateWeights) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) weights_of(k, wr[k]);
    }

    // Wait for every load (the weights included) before the first store:
    // vmcnt retires in issue order on gfx9, so a weight load still counted
    // when a store is issued would later force a wait on that store's
    // completion between the wave's stores.  The builtin form lets the
    // compiler's wait insertion see the wait.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    // Packed groups on lane segments of one wave (one vector per lane): a
    // vector on the boundary between two groups of the wave is the last
    // vector of the left group's segment and the first of the next segment.
    // The left lane takes the right unit's pieces of it from lane 0 of the
    // next segment (ds_bpermute) and stores the whole vector; the right lane
    // stores nothing there.  Boundary vectors shared with a group outside
    // the wave (or with the next row's first group) keep the piece stores.
    // Same bytes, one 16-byte store in place of two partial ones (377 MB of
    // 100-wide fp16 groups: 63.1 against 67.1 us).  In either tile order a
    // wave's segments hold consecutive units, so segment s + 1 holds group
    // g + 1 of the same row whenever g + 1 < groups.
    constexpr bool kMerge = kPacked && VPT == 1 && SEG < 64 && WS == WSource::Global;
    const uint32_t seg = (threadIdx.x & 63u) / SEG;
    const bool has_right = seg + 1 < 64u / SEG && g + 1 < a.groups;  // next segment: group g+1
    const bool has_left = seg > 0 && g > 0;                            // previous one: group g-1
    auto store = [&](auto ri_tag) {
        W res[VPT];
        epi::finish<decltype(ri_tag)::value>(L, nf, wr, res);
        W nb{};
        if constexpr (kMerge) {
            const int src = (int)((((seg + 1) * SEG) & 63u) << 2);
#pragma unroll
            for (int i = 0; i < VB / 4; ++i)
                nb[i] = (u32)__builtin_amdgcn_ds_bpermute(src, (int)res[0][i]);
        }
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const uint32_t idx = sl + k * SEG;
            if (!store_ok || idx >= nv) continue;
            if constexpr (kMerge) {
                if (rel[k] < 0 && has_left) continue;  // stored whole by the left lane
                if (rel[k] + N > (int32_t)a.G && has_right) {
                    store_stream<NT>(ov + v0 + idx,
                                     merge_pieces<PB>(res[k], nb, [&](int q) { return owned(k, q); }));
                    continue;
                }
            }
            if constexpr (kPacked) {
                if (rel[k] < 0 || rel[k] + N > (int32_t)a.G) {
                    // a vector on a group boundary: only this unit's pieces
                    char* base = reinterpret_cast<char*>(ov + v0 + idx);
#pragma unroll
                    for (int q = 0; q < VB / PB; ++q)
                        if (owned(k, q)) store_piece_stream<NT, PB>(base + q * PB, res[k], q);
                    continue;
                }
            }
            store_stream<NT>(ov + v0 + idx, res[k]);
        }
    };
    if (!NBG && round_intermediate(a))
        store(std::true_type{});
    else
        store(std::false_type{});
}

// ------------------------------------------------------------ kernels

// Tile (row or row tile rt, tile column c) of workgroup blockIdx.x in the
// XCD-banded order over R x C tiles (C = KArgs::xc): XCD x = b % 8 takes, in
// each block of 8 rows numbered column-major by super-tiles of S tiles of one
// row (S = 1: by tiles), the tiles x*C .. x*C + C-1, block after block; then
// its share of the short block of the last R % 8 rows (numbered by tiles).
// With C % S == 0 a bijection of the launch's R * C workgroups onto its
// tiles.
__device__ inline void xcd_band_tile(const KArgs& a, uint32_t R, uint32_t& rt, uint32_t& c) {
    const uint32_t b = blockIdx.x;
    const uint32_t x = b % kXcds, k = b / kXcds;
    const uint32_t C = a.xc;
    const uint32_t fullk = (R / kXcds) * C;  // each XCD's workgroups in the full blocks
    if (k < fullk) {
        const uint32_t blk = fast_div(k, a.xc_m, xc_shift(a));
        const uint32_t idx = x * C + (k - blk * C);  // = (s * 8 + r) * S + t
        const uint32_t ss = super_shift(a);
        const uint32_t q = idx >> ss;
        c = ((q / kXcds) << ss) | (idx & ((1u << ss) - 1u));
        rt = blk * kXcds + q % kXcds;
    } else {
        const uint32_t rr = R % kXcds;  // >= 1 here
        const uint32_t t2 = rr * C;     // tiles of the short block
        const uint32_t q2 = t2 / kXcds, r2 = t2 % kXcds;
        const uint32_t idx = x * q2 + (x < r2 ? x : r2) + (k - fullk);
        c = fast_div(idx, kSmallMagic.m[rr], kSmallMagic.s[rr]);
        rt = (R - rr) + (idx - c * rr);
    }
}

// WAVE: SEG (<= 64) lanes per unit, workgroups of 64 or 256 threads (the
// launch's choice), no LDS, no barrier.  Row-major order: each workgroup
// takes the next threads / SEG units of the (row, group) sequence.
// XCD-banded order: the workgroup takes threads / SEG consecutive groups of
// one row.
template <class T, int VB, int PB, int SEG, int VPT, bool NBG, bool NT>
__global__ __launch_bounds__(kWaveBlock) void ggrms_wave_kernel(KArgs a) {
    fetch_args_together(a);
    uint32_t n, g;
    if (banded(a)) {
        uint32_t c;
        xcd_band_tile(a, a.rows, n, c);
        g = c * (blockDim.x / SEG) + threadIdx.x / SEG;
        if (g >= a.groups) return;  // the row's last tile may be partial
    } else {
        const uint32_t unit = (blockIdx.x * (uint32_t)blockDim.x + threadIdx.x) / SEG;
        if (unit >= a.rows * a.groups) return;  // whole segments leave together
        n = row_div(a, unit);
        g = unit - n * a.groups;
    }
    unit_pass<T, VB, PB, SEG, VPT, NBG, NT, WSource::Global>(a, n, g, threadIdx.x & (SEG - 1),
                                                             true, nullptr,
                                                             [](float v) { return segment_sum<SEG>(v); });
}

// BLOCK: a unit spans SEG/64 waves; the per-wave sums meet in LDS after one
// barrier and every wave adds them in the same order.  A workgroup holds UPB
// units: UPB consecutive rows of one group (row-major order: workgroup b
// takes row tile b / groups, group b % groups; or the XCD-banded order).
// With UPB > 1 the group's f32 weights are fetched once
// per workgroup -- contiguous 16-byte loads spread over all its threads --
// and parked in LDS before the reduction barrier, instead of every unit
// fetching its own copy: weight traffic from L2 falls by UPB and the L1
// miss slots it held go back to the HBM streams.
template <class T, int VB, int PB, int SEG, int VPT, int UPB, bool NBG, bool NT>
__global__ __launch_bounds__(SEG * UPB) void ggrms_block_kernel(KArgs a) {
    fetch_args_together(a);
    constexpr int BT = SEG * UPB;
    constexpr int WPG = SEG / 64;
    constexpr int N = Packet<T, VB>::N;
    __shared__ float part[BT / 64];
    extern __shared__ __attribute__((aligned(16))) float wl[];  // a.G floats when UPB > 1
    // row tile and group: row-major (the groups of a row tile in turn) or
    // XCD-banded (kBitBand)
    uint32_t tile, g;
    if (banded(a)) {
        xcd_band_tile(a, (a.rows + UPB - 1) / UPB, tile, g);
    } else {
        tile = row_div(a, blockIdx.x);
        g = blockIdx.x - tile * a.groups;
    }
    const uint32_t u = threadIdx.x / SEG;
    uint32_t n = tile * UPB + u;
    const bool live = n < a.rows;
    if (!live) n = a.rows - 1;  // stay in bounds and reach the barrier
    const uint32_t wave = threadIdx.x >> 6;

    // Staged weights: G/4 float4 of the group, thread j takes j, j+BT, ...
    constexpr int SV = UPB > 1 ? (VPT * N + 4 * UPB - 1) / (4 * UPB) : 1;
    f32x4 wst[SV];
    if constexpr (UPB > 1) {
        const f32x4* src = reinterpret_cast<const f32x4*>(a.w + (int64_t)g * weight_group_stride(a));
        const uint32_t nw4 = a.G / 4;
#pragma unroll
        for (int i = 0; i < SV; ++i) {
            const uint32_t j = threadIdx.x + i * BT;
            if (j < nw4) wst[i] = src[j];
        }
    }
    constexpr WSource WS = UPB > 1 ? WSource::Lds : WSource::Global;
    unit_pass<T, VB, PB, SEG, VPT, NBG, NT, WS>(a, n, g, threadIdx.x & (SEG - 1), live, wl, [&](float v) {
        const float s = segment_sum<64>(v);
        if ((threadIdx.x & 63) == 0) part[wave] = s;
        if constexpr (UPB > 1) {
            const uint32_t nw4 = a.G / 4;
#pragma unroll
            for (int i = 0; i < SV; ++i) {
                const uint32_t j = threadIdx.x + i * BT;
                if (j < nw4) reinterpret_cast<f32x4*>(wl)[j] = wst[i];
            }
        }
        __syncthreads();
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < WPG; ++i) m += part[u * WPG + i];
        return m;
    });
}

// RUN: one wave takes a run of gpw = a.nvec consecutive packed groups of one
// row (tile (row, run) of the job's rows x runs_per_row = a.xc tiles), VPT
// 16-byte vectors per lane (vector i of the run on lane i % 64, slot i / 64,
// so every load instruction covers 64 consecutive vectors), the vectors
// counted from the row start.  100-wide fp16 groups (12.5 vectors) fill 125
// of 128 slots ten groups at a time, where 16-lane segments per group fill 13
// of 16 and load every boundary vector twice; when gpw groups span a whole
// number of vectors (the planner's choice where it can), every run starts on
// a vector boundary and the wave stores whole vectors only.  A vector on a
// group boundary holds pieces of two groups, whose sums are kept apart
// (gate_and_square2).  The groups' sums meet in LDS: each lane parks its
// slots' two shares, then lane j adds group j's shares in vector order (the
// piece of its first vector that follows the boundary, then the first share
// of each vector that starts inside the group), forms its normaliser and
// parks it; every lane reads back the normalisers of its pieces' groups.
// The vectors and their order depend on the group alone, so any run length
// gives the same bits.
// The workgroup is one wave, so its two barriers only order the LDS
// accesses.  A vector whose pieces belong to groups of two runs is stored in
// pieces by both waves.
template <class T, int PB, int VPT, bool NBG, bool NT>
__global__ __launch_bounds__(64) void ggrms_run_kernel(KArgs a) {
    constexpr int VB = 16;
    using P = Packet<T, VB>;
    using W = typename P::W;
    constexpr int N = P::N;
    constexpr int PE = PB / T::kSize;  // elements per piece
    constexpr int NP = VB / PB;        // pieces per vector
    static_assert(PB < VB, "runs are built for packed groups");
    using S = typename VecWord<T::kSize>::type;
    __shared__ float share0[64 * VPT], share1[64 * VPT];
    __shared__ float nfs[kRunMaxGroups];
    // one [G] weight shared by every group (G <= 64 * kRunStage): staged in
    // a.G floats of dynamic LDS, fetched after the inputs and parked before
    // the first barrier
    extern __shared__ float wsh[];
    fetch_args_together(a);
    const bool wshared = (a.bits & kBitShared) != 0;

    uint32_t n, c;  // row, run
    if (banded(a)) {
        xcd_band_tile(a, a.rows, n, c);
    } else {
        n = row_div(a, blockIdx.x);  // runs per row (div_m holds its magic number)
        c = blockIdx.x - n * a.xc;
    }
    const uint32_t gpw = a.nvec;
    const uint32_t g0 = c * gpw;
    const int32_t cnt = (int32_t)(a.groups - g0 < gpw ? a.groups - g0 : gpw);
    const int64_t e0 = (int64_t)g0 * a.G;                // the run's first element in the row
    const int64_t e1 = e0 + (int64_t)cnt * a.G;          // one past its last
    const uint32_t v0 = (uint32_t)(e0 / N);
    const uint32_t nv = (uint32_t)((e1 + N - 1) / N) - v0;  // <= 64 * VPT (the planner's gpw)
    const int32_t lead = (int32_t)(e0 - (int64_t)v0 * N);   // vector v0's elements before the run
    const uint32_t l = threadIdx.x;
    const int32_t G = (int32_t)a.G;

    const W* yv = reinterpret_cast<const W*>(static_cast<const S*>(a.y) + (int64_t)n * a.sy);
    const W* gv = reinterpret_cast<const W*>(static_cast<const S*>(a.gate) + (int64_t)n * a.sg);
    W yr[VPT][1], gr[VPT][1];
    float wr[VPT][1][N];
    uint32_t vi[VPT];
    bool lv[VPT];
    // kv: the group (relative to g0) of the vector's first element, -1 for a
    // vector that starts in the previous run; bnd: elements of group kv in
    // the vector (>= N: all of them)
    int32_t kv[VPT], bnd[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const uint32_t idx = l + 64u * k;
        lv[k] = idx < nv;
        vi[k] = v0 + (lv[k] ? idx : nv - 1);
        const int32_t off = (int32_t)((int64_t)vi[k] * N - e0);  // >= -(N - 1)
        int32_t kk = -1;
        if (off >= 0) {  // off / G, by the f32 reciprocal and exact corrections
            kk = (int32_t)((float)off * a.Ginv);
            kk -= kk * G > off ? 1 : 0;
            kk += (kk + 1) * G <= off ? 1 : 0;
        }
        kv[k] = kk;
        bnd[k] = (kk + 1) * G - off;
        yr[k][0] = load_stream<NT>(yv + vi[k]);
        gr[k][0] = load_stream<NT>(gv + vi[k]);
        if (!wshared) load_weights<N>(a.w + (int64_t)vi[k] * N, wr[k][0]);
    }
    float wst[kRunStage];
    if (wshared) {
#pragma unroll
        for (int j = 0; j < kRunStage; ++j) {
            const uint32_t i = l + 64u * j;
            wst[j] = i < a.G ? a.w[i] : 0.0f;
        }
    }

    epi::LaneUnit<T, VB, 1, NBG> L[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        float s_k, s_k1;  // 0 for a slot past the run's end
        epi::gate_and_square2<T, VB, PB, 1, NBG>(
            yr[k], gr[k], L[k], [&](int) { return lv[k]; },
            [&](int, int q) { return q * PE >= bnd[k]; }, s_k, s_k1);
        share0[l + 64u * k] = s_k;
        share1[l + 64u * k] = s_k1;
    }
    if (wshared) {
#pragma unroll
        for (int j = 0; j < kRunStage; ++j)
            if (l + 64u * j < a.G) wsh[l + 64u * j] = wst[j];
    }
    __syncthreads();
    if ((int32_t)l < cnt) {
        // group l: its first element is element s of the run's vectors
        const int32_t s = lead + (int32_t)l * G;
        const int32_t f = s / N, hi = (s + G - 1) / N;
        const bool straddle = s % N != 0;  // vector f starts in group l - 1
        float m2 = straddle ? share1[f] : 0.0f;
        for (int32_t i = straddle ? f + 1 : f; i <= hi; ++i) m2 += share0[i];
        nfs[l] = norm_factor(m2, a.Ginv, a.eps);
    }
    __syncthreads();
    float nf_k[VPT], nf_k1[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        nf_k[k] = kv[k] >= 0 ? nfs[kv[k]] : 0.0f;
        nf_k1[k] = kv[k] + 1 < cnt ? nfs[kv[k] + 1] : 0.0f;
        if (wshared) {
            // element e is column off + e of group kv, or column off + e - G
            // of group kv + 1 (e >= bnd); a slot past the run reads a clamped
            // place (its results are not stored)
            const int32_t off = (int32_t)((int64_t)vi[k] * N - e0) - kv[k] * G;
#pragma unroll
            for (int e = 0; e < N; ++e) {
                int32_t col = off + e - (e >= bnd[k] ? G : 0);
                col = col < 0 ? 0 : (col >= G ? G - 1 : col);
                wr[k][0][e] = wsh[col];
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    W* ov = reinterpret_cast<W*>(static_cast<S*>(a.out) + (int64_t)n * a.so);
    auto store = [&](auto ri_tag) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            W res[1];
            auto nf = [&](int, int q) { return q * PE >= bnd[k] ? nf_k1[k] : nf_k[k]; };
            epi::finish_by_piece<decltype(ri_tag)::value, PE>(L[k], nf, wr[k], res);
            if (!lv[k]) continue;
            const bool own_k = kv[k] >= 0, own_k1 = kv[k] + 1 < cnt;
            if (bnd[k] >= N ? own_k : (own_k && own_k1)) {
                store_stream<NT>(ov + vi[k], res[0]);
            } else {
#pragma unroll
                for (int q = 0; q < NP; ++q)
                    if (q * PE >= bnd[k] ? own_k1 : own_k)
                        store_piece_stream<NT, PB>(reinterpret_cast<char*>(ov + vi[k]) + q * PB,
                                                   res[0], q);
            }
        }
    };
    if (!NBG && round_intermediate(a))
        store(std::true_type{});
    else
        store(std::false_type{});
}

// ROWS: wide groups (513-2048 16-byte vectors) in large jobs.  The grid is
// one workgroup per compute unit (a.xc = S rows per group): workgroup b takes
// group b % groups and rows b / groups, + S, + 2S, ...  Its SEG lanes hold VPT
// vectors of a row each (the slots and the order of the sums are those of
// the BLOCK kernel with the same lanes and vectors, so both give the same
// bits), its weights stay in registers for every row, and it keeps the rows
// two ahead in flight: the inputs of row i + 2S are requested as soon as row
// i's inputs have been turned into gated values, before row i's barrier and
// stores.  All y/gate/out accesses are buffer accesses over the unit's
// vectors: a lane past the group's end, or a prefetch past the last row,
// gets an offset outside the unit, which the hardware drops (stores) or
// answers with zeros without touching memory (loads).  No path through the
// loop then skips a memory operation, so the compiler's counts of
// outstanding operations stay exact and a row's loads never wait for the
// previous row's stores (memory counters retire in order).
template <class T, int SEG, int VPT, bool NBG, bool NT>
__global__ __launch_bounds__(SEG) void ggrms_rows_kernel(KArgs a) {
    constexpr int VB = 16;
    using P = Packet<T, VB>;
    using W = typename P::W;
    constexpr int N = P::N;
    constexpr int WPG = SEG / 64;
    constexpr int D = 2;             // rows in flight per workgroup
    constexpr int kFmt = 0x00020000;  // word 3 of a raw buffer resource: 32-bit data
    constexpr int kPol = NT ? 2 : 0;  // cache policy operand: nt
    using S = typename VecWord<T::kSize>::type;
    __shared__ float part[D][WPG];

    const uint32_t n0 = row_div(a, blockIdx.x);
    const uint32_t g = blockIdx.x - n0 * a.groups;
    const uint32_t stride = a.xc, rows = a.rows, nvec = a.nvec;
    const uint32_t sl = threadIdx.x;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int beyond = (int)(nvec * VB);  // an offset outside the unit
    uint32_t ci[VPT];
    bool lv[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const uint32_t idx = sl + k * SEG;
        lv[k] = idx < nvec;
        ci[k] = lv[k] ? idx : nvec - 1;
    }
    float wr[VPT][N];
    const float* wp = a.w + (int64_t)g * weight_group_stride(a);
#pragma unroll
    for (int k = 0; k < VPT; ++k) load_weights<N>(wp + (int64_t)ci[k] * N, wr[k]);

    // the unit (row n, group g) of a [rows, width] view with row stride ld
    auto unit_rsrc = [&](const void* base, int64_t ld, uint32_t n) {
        return __builtin_amdgcn_make_buffer_rsrc(
            const_cast<S*>(static_cast<const S*>(base)) + (int64_t)n * ld + (int64_t)g * a.G, 0,
            beyond, kFmt);
    };
    auto load_unit = [&](uint32_t n, bool want, W (&yr)[VPT], W (&gr)[VPT]) {
        const auto ry = unit_rsrc(a.y, a.sy, n), rg = unit_rsrc(a.gate, a.sg, n);
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int off = want && lv[k] ? (int)(ci[k] * VB) : beyond;
            yr[k] = __builtin_amdgcn_raw_buffer_load_b128(ry, off, 0, kPol);
            gr[k] = __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, kPol);
        }
    };

    W yb[D][VPT], gb[D][VPT];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const uint32_t nd = n0 + d * stride;
        load_unit(nd < rows ? nd : n0, nd < rows, yb[d], gb[d]);
    }
    // The weights and the first rows have landed before the loop: inside it
    // the compiler's waits then follow only the loop's own loads and stores.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    auto live = [&](int k) { return lv[k]; };
    auto owned = [](int, int) { return true; };
    // the loop, one copy per rounding mode (no branch inside it)
    auto run = [&](auto ri_tag) __attribute__((always_inline)) {
        constexpr bool RI = decltype(ri_tag)::value;
        auto pass = [&](uint32_t n, W (&yr)[VPT], W (&gr)[VPT], float* pt)
            __attribute__((always_inline)) {
            epi::LaneUnit<T, VB, VPT, NBG> L;
            const float acc = epi::gate_and_square<T, VB, VB, VPT, NBG>(yr, gr, L, live, owned);
            // the raw inputs are now in L: their registers take the row D ahead
            const uint32_t nn = n + D * stride;
            load_unit(nn < rows ? nn : n, nn < rows, yr, gr);
            const float s = segment_sum<64>(acc);
            if ((threadIdx.x & 63) == 0) pt[wave] = s;
            __syncthreads();
            float m2 = 0.0f;
#pragma unroll
            for (int i = 0; i < WPG; ++i) m2 += pt[i];
            const float nf = norm_factor(m2, a.Ginv, a.eps);
            W res[VPT];
            epi::finish<RI>(L, nf, wr, res);
            const auto ro = unit_rsrc(a.out, a.so, n);
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int off = lv[k] ? (int)(ci[k] * VB) : beyond;
                __builtin_amdgcn_raw_buffer_store_b128(res[k], ro, off, 0, kPol);
            }
        };
        // D rows per trip, so that each row's registers and partial-sum slot are
        // fixed (consecutive rows use different slots: a wave still reading one
        // row's partial sums never meets the next row's writes)
        uint32_t n = n0;
        for (; n + (D - 1) * stride < rows; n += D * stride) {
#pragma unroll
            for (int d = 0; d < D; ++d) pass(n + d * stride, yb[d], gb[d], part[d]);
        }
#pragma unroll
        for (int d = 0; d < D - 1; ++d)
            if (n + d * stride < rows) pass(n + d * stride, yb[d], gb[d], part[d]);
    };
    if (!NBG && round_intermediate(a))
        run(std::true_type{});
    else
        run(std::false_type{});
}

// WIDE: one 1024-thread workgroup per unit, for groups with more vectors than
// the BLOCK shapes hold in registers.  Pass 1 reads the group and reduces;
// pass 2 reads it again and writes (the only path that reads inputs twice).
template <class T, int VB, bool NBG, bool NT>
__global__ __launch_bounds__(kWideBlock) void ggrms_wide_kernel(KArgs a) {
    using P = Packet<T, VB>;
    using W = typename P::W;
    constexpr int N = P::N;
    using S = typename VecWord<T::kSize>::type;
    __shared__ float part[kWideBlock / 64];

    const uint32_t unit = blockIdx.x;
    const uint32_t n = row_div(a, unit);
    const uint32_t g = unit - n * a.groups;
    const int64_t col0 = (int64_t)g * a.G;
    const W* yv = reinterpret_cast<const W*>(static_cast<const S*>(a.y) + (int64_t)n * a.sy + col0);
    const W* gv =
        reinterpret_cast<const W*>(static_cast<const S*>(a.gate) + (int64_t)n * a.sg + col0);
    W* ov = reinterpret_cast<W*>(static_cast<S*>(a.out) + (int64_t)n * a.so + col0);
    const float* wp = a.w + (int64_t)g * weight_group_stride(a);

    float acc = 0.0f;
    for (uint32_t i = threadIdx.x; i < a.nvec; i += kWideBlock) {
        float yf[N], gf[N];
        P::unpack(yv[i], yf);
        if constexpr (!NBG) P::unpack(gv[i], gf);
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const float x = NBG ? yf[e] : yf[e] * silu_exact(gf[e]);
            acc = __builtin_fmaf(x, x, acc);
        }
    }
    const float s = segment_sum<64>(acc);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    float m2 = 0.0f;
#pragma unroll
    for (int i = 0; i < kWideBlock / 64; ++i) m2 += part[i];
    const float nf = norm_factor(m2, a.Ginv, a.eps);

    for (uint32_t i = threadIdx.x; i < a.nvec; i += kWideBlock) {
        float yf[N], gf[N], wv[N], t[N];
        P::unpack(load_stream<NT>(yv + i), yf);
        P::unpack(load_stream<NT>(gv + i), gf);
        load_weights<N>(wp + (int64_t)i * N, wv);
        if constexpr (NBG) {
#pragma unroll
            for (int e = 0; e < N; ++e) t[e] = ((yf[e] * nf) * wv[e]) * silu_exact(gf[e]);
        } else {
#pragma unroll
            for (int e = 0; e < N; ++e) t[e] = yf[e] * silu_exact(gf[e]) * nf;
            if (round_intermediate(a)) P::round_trip(t);
#pragma unroll
            for (int e = 0; e < N; ++e) t[e] = wv[e] * t[e];
        }
        store_stream<NT>(ov + i, P::pack(t));
    }
}

// ------------------------------------------------------------ table

// PB == VB: group-aligned vectors; PB < VB (VB == 16): packed groups, built
// for every WAVE shape and for the BLOCK shapes with one row per workgroup.
template <class T, int VB, int PB, bool NBG, bool NT>
inline const void* pick_vb(int kernel, int lanes, int vpt, int upb) {
    constexpr bool kPacked = PB < VB;
#define GG_W(L, V)                      \
    if (lanes == L && vpt == V)         \
    return reinterpret_cast<const void*>(&ggrms_wave_kernel<T, VB, PB, L, V, NBG, NT>)
#define GG_B(L, V, U)                     \
    if (lanes == L && vpt == V && upb == U) \
    return reinterpret_cast<const void*>(&ggrms_block_kernel<T, VB, PB, L, V, U, NBG, NT>)
#define GG_B4(L, U) GG_B(L, 1, U); GG_B(L, 2, U); GG_B(L, 3, U); GG_B(L, 4, U)
    if (kernel == GGRMS_KERNEL_WAVE) {
        if (upb != 1) return nullptr;
        GG_W(1, 1); GG_W(2, 1); GG_W(4, 1); GG_W(8, 1); GG_W(16, 1); GG_W(32, 1);
        GG_W(64, 1); GG_W(64, 2); GG_W(64, 3); GG_W(64, 4);
        // packed groups: two vectors per lane on half the lanes (the same
        // slots; each wave's fixed work over twice the elements, every
        // boundary vector stored in pieces), for forced shapes
        if constexpr (kPacked) {
            GG_W(8, 2); GG_W(16, 2); GG_W(32, 2);
        }
    } else if (kernel == GGRMS_KERNEL_BLOCK) {
        GG_B4(128, 1); GG_B4(256, 1); GG_B4(512, 1); GG_B4(1024, 1);
        GG_B(256, 6, 1);
        if constexpr (!kPacked) {
            GG_B4(128, 2); GG_B4(128, 4);
            GG_B4(256, 2);
        }
    } else if (kernel == GGRMS_KERNEL_WIDE) {
        if constexpr (kPacked) return nullptr;
        if (upb != 1) return nullptr;
        return reinterpret_cast<const void*>(&ggrms_wide_kernel<T, VB, NBG, NT>);
    } else if (kernel == GGRMS_KERNEL_ROWS) {
        if constexpr (VB == 16 && !kPacked) {
            if (upb != 1) return nullptr;
#define GG_R(L, V)              \
    if (lanes == L && vpt == V) \
    return reinterpret_cast<const void*>(&ggrms_rows_kernel<T, L, V, NBG, NT>)
            GG_R(256, 3); GG_R(320, 2); GG_R(384, 2); GG_R(448, 2); GG_R(512, 2);
            GG_R(768, 2); GG_R(1024, 2);
#undef GG_R
        }
        return nullptr;
    } else if (kernel == GGRMS_KERNEL_RUN) {
        if constexpr (kPacked) {
            if (lanes == 64 && vpt == 1 && upb == 1)
                return reinterpret_cast<const void*>(&ggrms_run_kernel<T, PB, 1, NBG, NT>);
            if (lanes == 64 && vpt == 2 && upb == 1)
                return reinterpret_cast<const void*>(&ggrms_run_kernel<T, PB, 2, NBG, NT>);
        }
        return nullptr;
    }
#undef GG_W
#undef GG_B
#undef GG_B4
    return nullptr;
}

// vb: vector bytes; pb: piece bytes (== vb for group-aligned vectors, 2, 4 or
// 8 with vb == 16 for packed groups).
template <class T, bool NBG, bool NT>
inline const void* pick_type(int kernel, int vb, int pb, int lanes, int vpt, int upb) {
    if (pb == vb) {
        switch (vb) {
        case 16: return pick_vb<T, 16, 16, NBG, NT>(kernel, lanes, vpt, upb);
        case 8: return pick_vb<T, 8, 8, NBG, NT>(kernel, lanes, vpt, upb);
        case 4: return pick_vb<T, 4, 4, NBG, NT>(kernel, lanes, vpt, upb);
        case 2:
            if constexpr (T::kSize == 2) return pick_vb<T, 2, 2, NBG, NT>(kernel, lanes, vpt, upb);
            return nullptr;
        default: return nullptr;
        }
    }
    if (vb != 16) return nullptr;
    switch (pb) {
    case 8: return pick_vb<T, 16, 8, NBG, NT>(kernel, lanes, vpt, upb);
    case 4: return pick_vb<T, 16, 4, NBG, NT>(kernel, lanes, vpt, upb);
    case 2:
        if constexpr (T::kSize == 2) return pick_vb<T, 16, 2, NBG, NT>(kernel, lanes, vpt, upb);
        return nullptr;
    default: return nullptr;
    }
}

}  // namespace ggrms
