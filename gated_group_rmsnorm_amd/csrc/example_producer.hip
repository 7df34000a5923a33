// example_producer.hip -- the per-unit epilogue (ggrms_epilogue.hpp) called
// from a kernel that computes y itself, so that y never reaches HBM: the
// hand-off that fusing the norm into the kernel producing y needs.
//
// The page "gated_group_rmsnorm" places this math inside the Mamba-2 scan
// (the norm_before_gate=False branch of its combined scan), and the standalone
// op is a port of it.  The pages do not define the scan, so the producer here
// is a stand-in with a plain definition: y = bf16(x @ wt^T), a bf16 matrix
// product on the matrix cores (v_mfma_f32_16x16x32_bf16), whose output tile
// arrives in the accumulator layout of the MFMA instruction, like any
// contraction's.  What carries over to a real producer is the hand-off:
//   * a workgroup owns whole (row, group) units -- here row tiles of 16 rows
//     x one group of G columns, its 16 waves sharing the group's columns;
//   * the accumulators are rounded to the storage type (the values the
//     standalone op would have read back) and re-laid through LDS from the
//     MFMA layout (lane = column, 4 consecutive rows per lane) to the
//     epilogue's (lane = 16 bytes of one row);
//   * each wave then takes one row of the tile and runs the epilogue's steps
//     on it: gate_and_square on y from LDS and the gate from global memory,
//     segment_sum over the unit's 64 lanes, norm_factor, finish, one
//     16-byte store per slot.  gate, the weight and out are the only HBM
//     traffic of the norm; a separate norm kernel would also write and then
//     read y.
// The slots lie as in the library's WAVE kernel with 64 lanes x 2 vectors,
// so for the same y the outputs equal that launch's bit for bit.
//
// This file is an example of the epilogue's use, built as its own library
// (libggrms_example.so); it is not part of libggrms's interface.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ggrms_epilogue.hpp"

namespace {

using namespace ggrms;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kRowsPerTile = 16;   // one MFMA tile of rows
constexpr int kWaves = 16;         // one wave per row of a tile in the epilogue
constexpr int kMaxTilesPerWg = 16;  // row tiles one workgroup takes in turn, at most
constexpr int kCus = 256;           // compute units of the part
constexpr int kMaxGroup = 1024;    // 128 vectors of bf16: two per lane
constexpr int kMaxK = 64;          // two MFMA k steps of 32; their B fragments stay in registers
constexpr int kLdsPad = 8;         // bf16 elements of padding per re-lay row
constexpr int kXPad = 8;           // and per staged row of x: 144-byte rows, so that
                                   // 16 lanes reading 16 rows hit 64 distinct banks
constexpr int NT = kMaxGroup / 16 / kWaves;  // column tiles per wave, at most
constexpr int kWaitVmcnt0 = 0x0F70;  // s_waitcnt vmcnt(0), expcnt and lgkmcnt at their maxima
constexpr int kBufferFormat = 0x00020000;  // word 3 of a raw gfx9 buffer resource (32-bit data)
constexpr int kNonTemporal = 2;            // cache policy operand of a buffer access: nt

struct ExArgs {
    const u16* x;      // [rows, K] bf16
    const u16* wt;     // [width, K] bf16
    const u32x4* gate; // [rows, width] bf16, as 16-byte vectors
    const float* w;    // [width] f32
    void* out;         // [rows, width] bf16
    uint32_t rows, width, K, G;
    uint32_t tiles_per_wg;  // 1 .. kMaxTilesPerWg
    float Ginv, eps;
};

constexpr int kDppSwapPairs = 0xB1;  // DPP quad_perm [1, 0, 3, 2]: swap lanes 2i and 2i+1

// One workgroup of 16 waves: group g, row tiles blockIdx.x * tiles_per_wg
// onwards (16 rows each; the last workgroup's may be fewer).  The multiply:
// the group's G / 16 column tiles of 16 go round the waves (wave w: tiles w,
// w + 16, ...), each an MFMA tile whose B fragments (wt for those columns)
// are loaded once and reused for every row tile.  The epilogue: wave w takes
// row w of each tile, so every wave has one unit per tile.  What keeps the
// memory latency off the loop:
//   * the workgroup's rows of x and the group's weights are staged in LDS
//     up front;
//   * the gate of a wave's row two tiles ahead is requested before its
//     stores of this tile: a global load issued after a store waits for
//     that store's completion as well (memory counters retire in order), so
//     a load issued after the stores would expose the store and the load
//     latency once per tile, and two tiles of gate in flight per wave keep
//     the bytes in flight up while every tile passes a barrier;
//   * the re-lay buffer alternates between two halves, so each tile needs
//     one barrier.
// PRODUCE: store y itself (the producer of an unfused pipeline).
template <bool RI, bool PRODUCE>
__global__ __launch_bounds__(kWaves * 64) void example_gemm_norm_kernel(ExArgs a) {
    // rows of 2064 bytes keep every 16-byte vector of a row 16-byte aligned
    __shared__ __attribute__((aligned(16))) u16 ys[2][kRowsPerTile][kMaxGroup + kLdsPad];
    __shared__ __attribute__((aligned(16))) u16 xs[kMaxTilesPerWg * kRowsPerTile][kMaxK + kXPad];
    __shared__ __attribute__((aligned(16))) float ws[kMaxGroup];
    const uint32_t lane = threadIdx.x & 63;
    // the wave's index, in a scalar register (the same on every lane)
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t g = blockIdx.y;
    const uint32_t G = a.G;
    const uint32_t nct = G / 16;  // column tiles of the group
    const uint32_t ntiles = a.rows / kRowsPerTile;
    const uint32_t t0 = blockIdx.x * a.tiles_per_wg;
    const uint32_t t1 = t0 + a.tiles_per_wg < ntiles ? t0 + a.tiles_per_wg : ntiles;

    // the epilogue's slots: a row's group is nvec = G/8 vectors, lane l holds
    // vectors l and l + 64 (the same columns for every row)
    const uint32_t nvec = G / 8;
    constexpr int K = 2;
    uint32_t ci[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const uint32_t idx = lane + k * 64;
        ci[k] = idx < nvec ? idx : nvec - 1;  // past the end: a copy of the last vector
    }
    auto live = [&](int k) { return lane + k * 64 < nvec; };
    auto owned = [](int, int) { return true; };
    // The gate of the unit (row n, group g) into g_out, by buffer loads: with
    // want false, or for a lane past the group's end, the offset lies outside
    // the unit and the load returns zeros without touching memory -- every
    // path issues the same loads (the compiler's counts stay exact) and no
    // byte is fetched twice.
    auto load_gate = [&](uint32_t n, bool want, u32x4 (&g_out)[K]) {
        const __amdgpu_buffer_rsrc_t gb = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<u32x4*>(a.gate) + ((size_t)n * a.width + (size_t)g * G) / 8, 0,
            (int)(nvec * 16), kBufferFormat);
#pragma unroll
        for (int k = 0; k < K; ++k)
            g_out[k] = __builtin_amdgcn_raw_buffer_load_b128(
                gb, want && live(k) ? (int)(ci[k] * 16) : (int)(nvec * 16), 0, kNonTemporal);
    };
    // the gate of this wave's row of the first two tiles
    u32x4 gA[K] = {}, gB[K] = {};
    if constexpr (!PRODUCE) {
        load_gate(t0 * kRowsPerTile + wave, true, gA);
        load_gate((t0 + 1 < t1 ? t0 + 1 : t0) * kRowsPerTile + wave, t0 + 1 < t1, gB);
    }

    // x rows of the workgroup's tiles into LDS, 16 bytes at a time, zero
    // past column K: every tile then takes both k steps of 32, the
    // missing ones adding products of zeros (exactly +0, which leaves every
    // sum as it is)
    {
        const uint32_t r0 = t0 * kRowsPerTile, nr = (t1 - t0) * kRowsPerTile;
        const uint32_t per_row = a.K / 8;  // 16-byte pieces of x per row
        for (uint32_t i = threadIdx.x; i < nr * (kMaxK / 8); i += blockDim.x) {
            const uint32_t r = i / (kMaxK / 8), c = i % (kMaxK / 8);
            u32x4 v = {0u, 0u, 0u, 0u};
            if (c < per_row) v = *reinterpret_cast<const u32x4*>(a.x + (size_t)(r0 + r) * a.K + c * 8);
            *reinterpret_cast<u32x4*>(&xs[r][c * 8]) = v;
        }
    }
    // the group's weights into LDS
    if constexpr (!PRODUCE) {
        for (uint32_t i = threadIdx.x; i < G / 4; i += blockDim.x)
            *reinterpret_cast<f32x4*>(&ws[4 * i]) =
                *reinterpret_cast<const f32x4*>(a.w + (size_t)g * G + 4 * i);
    }

    // v_mfma_f32_16x16x32_bf16: lane l supplies 8 consecutive k of row
    // l % 16 of A and of column l % 16 of B, the k chunk chosen by l / 16, and
    // holds D[4*(l/16) + i][l % 16] (i = 0..3).  The k index is free to
    // permute (the same way for A and B): at k step h (0, 1), lane l's chunk
    // is x[.][16*(l/16) + 8h .. + 7], so over the two steps a lane reads 32
    // contiguous bytes of one row of x, and of one row of wt for B, as two
    // 16-byte accesses.
    const uint32_t m = lane & 15, q = lane >> 4;
    // B for the wave's column tiles (zero past K and past the group's end)
    u32x4 bw[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const bool ok = wave + t * kWaves < nct && 16 * q < a.K;
        const uint32_t col = g * G + (wave + t * kWaves) * 16 + m;
        const u32x4* p = reinterpret_cast<const u32x4*>(a.wt + (size_t)col * a.K + 16 * q);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            bw[t][h] = u32x4{0u, 0u, 0u, 0u};
            if (ok) bw[t][h] = p[h];
        }
    }
    // Every load so far has landed before the loop starts (s_waitcnt vmcnt(0);
    // the other counters untouched), so that inside the loop the compiler's
    // waits track only the loop's own gate loads and stores and never hold a
    // tile's gate behind that tile's stores.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();  // xs and ws are complete

    // One row tile, re-laid through buffer yb, with the gate of this wave's
    // row in gcur; gcur then receives the gate of the tile two ahead.
    auto tile_pass = [&](uint32_t tile, u16 (*yb)[kMaxGroup + kLdsPad], u32x4 (&gcur)[K])
        __attribute__((always_inline)) {
        // --- producer: the tile of y in MFMA accumulators, rounded to bf16
        // and re-laid: D[4*(l/16) + i][l % 16] -> yb[row][column in group].
        // The buffer was last read two tiles ago, before every wave passed
        // the previous tile's barrier.  Each k step's A fragment feeds the
        // NT independent accumulator chains.
        f32x4v acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
        u32x4 xa[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            xa[h] = *reinterpret_cast<const u32x4*>(&xs[(tile - t0) * kRowsPerTile + m][16 * q + 8 * h]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bf16x8 av = __builtin_bit_cast(bf16x8, xa[h]);
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    av, __builtin_bit_cast(bf16x8, bw[t][h]), acc[t], 0, 0, 0);
        }
        // Lanes m and m + 1 (m even) hold columns c and c + 1 of rows 4q..4q+3;
        // after one swap of a bf16 pair between them, the even lane writes
        // rows 4q and 4q+1 and the odd lane rows 4q+2 and 4q+3, each as
        // 32-bit words of both columns (64 distinct banks per write).
        const bool odd = m & 1;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (wave + t * kWaves >= nct) break;
            const uint32_t c = (wave + t * kWaves) * 16 + (m & ~1u);
            const float r01[2] = {acc[t][0], acc[t][1]}, r23[2] = {acc[t][2], acc[t][3]};
            const u32 p0 = Cvt<TBF16>::pack_word(r01);  // rows 4q, 4q+1 (low half: 4q)
            const u32 p1 = Cvt<TBF16>::pack_word(r23);  // rows 4q+2, 4q+3
            const u32 recv = (u32)__builtin_amdgcn_update_dpp(0, (int)(odd ? p0 : p1), kDppSwapPairs,
                                                              0xF, 0xF, false);
            const u32 mine = odd ? p1 : p0;
            // even lane: (own, partner's) element of each row; odd: (partner's, own)
            const u32 lo = odd ? recv : mine, hi = odd ? mine : recv;
            const uint32_t row = 4 * q + (odd ? 2 : 0);
            *reinterpret_cast<u32*>(&yb[row][c]) = (lo & 0xFFFFu) | (hi << 16);
            *reinterpret_cast<u32*>(&yb[row + 1][c]) = (lo >> 16) | (hi & 0xFFFF0000u);
        }
        __syncthreads();

        // --- epilogue: wave w takes row w of the tile
        const uint32_t n = tile * kRowsPerTile + wave;
        u32x4 yr[K];
#pragma unroll
        for (int k = 0; k < K; ++k) yr[k] = *reinterpret_cast<const u32x4*>(&yb[wave][ci[k] * 8]);
        // out's unit (row n, group g) as a buffer of nvec vectors: a lane
        // past the group's end gets an offset outside it, and the buffer
        // store drops it -- no predicated store, so no path through the loop
        // skips one and the compiler's count of the memory operations after
        // the gate loads stays exact
        const __amdgpu_buffer_rsrc_t ob = __builtin_amdgcn_make_buffer_rsrc(
            static_cast<u16*>(a.out) + (size_t)n * a.width + (size_t)g * G, 0, (int)(nvec * 16),
            kBufferFormat);
        int off[K];
#pragma unroll
        for (int k = 0; k < K; ++k) off[k] = live(k) ? (int)(ci[k] * 16) : (int)(nvec * 16);
        if constexpr (PRODUCE) {  // the unfused producer: y goes to memory
#pragma unroll
            for (int k = 0; k < K; ++k)
                __builtin_amdgcn_raw_buffer_store_b128(yr[k], ob, off[k], 0, kNonTemporal);
            return;
        }
        epi::LaneUnit<TBF16, 16, K, false> L;
        const float part = epi::gate_and_square<TBF16, 16, 16, K, false>(yr, gcur, L, live, owned);
        const float m2 = segment_sum<64>(part);
        const float nf = norm_factor(m2, a.Ginv, a.eps);
        float wr[K][8];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const f32x4 w0 = *reinterpret_cast<const f32x4*>(&ws[ci[k] * 8]);
            const f32x4 w1 = *reinterpret_cast<const f32x4*>(&ws[ci[k] * 8 + 4]);
            wr[k][0] = w0.x; wr[k][1] = w0.y; wr[k][2] = w0.z; wr[k][3] = w0.w;
            wr[k][4] = w1.x; wr[k][5] = w1.y; wr[k][6] = w1.z; wr[k][7] = w1.w;
        }
        u32x4 res[K];
        epi::finish<RI>(L, nf, wr, res);
        // the gate two tiles ahead, before this tile's stores (past the last
        // tile: loads that fetch nothing, so that no path skips them)
        const bool more = tile + 2 < t1;
        load_gate(more ? n + 2 * kRowsPerTile : n, more, gcur);
#pragma unroll
        for (int k = 0; k < K; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(res[k], ob, off[k], 0, kNonTemporal);
    };

    // tiles in pairs, so that the two gate buffers and the two re-lay
    // buffers keep fixed registers and addresses
    uint32_t tile = t0;
    for (; tile + 1 < t1; tile += 2) {
        tile_pass(tile, ys[0], gA);
        tile_pass(tile + 1, ys[1], gB);
    }
    if (tile < t1) tile_pass(tile, ys[0], gA);
}

}  // namespace

// y = bf16(x @ wt^T) for x [rows, K] and wt [width, K], then the gated group
// RMSNorm of y with gate [rows, width], f32 norm_weight [width], group_size
// G, into out [rows, width]; all bf16 except the weight, contiguous rows,
// 16-byte aligned pointers.  produce_only = 1 stores y itself into out (the
// producer of an unfused pipeline).  rows % 16 == 0, K % 16 == 0, width % G
// == 0, K <= 64, G a multiple of 64 up to 1024.  Returns 0 on success, 1 for
// arguments outside these limits, 2 if the launch fails.  Enqueued on
// `stream` (a hipStream_t; NULL is the default stream).
extern "C" __attribute__((visibility("default"))) int ggrms_example_gemm_norm(
    const void* x, const void* wt, const void* gate, const float* norm_weight, void* out,
    int64_t rows, int64_t width, int64_t K, int64_t group_size, float eps,
    int round_intermediate, int produce_only, void* stream) {
    if (!x || !wt || !gate || !norm_weight || !out) return 1;
    if (rows <= 0 || width <= 0 || K <= 0 || group_size <= 0) return 1;
    if (rows % kRowsPerTile || K % 16 || K > kMaxK || width % group_size || group_size > kMaxGroup)
        return 1;
    if (rows > ((int64_t)1 << 30) || width / group_size > 65535) return 1;
    if (((uintptr_t)x | (uintptr_t)wt | (uintptr_t)gate | (uintptr_t)norm_weight |
         (uintptr_t)out) % 16)
        return 1;
    if (group_size % 64) return 1;
    const void* fn =
        produce_only ? (round_intermediate
                            ? reinterpret_cast<const void*>(&example_gemm_norm_kernel<true, true>)
                            : reinterpret_cast<const void*>(&example_gemm_norm_kernel<false, true>))
                     : (round_intermediate
                            ? reinterpret_cast<const void*>(&example_gemm_norm_kernel<true, false>)
                            : reinterpret_cast<const void*>(&example_gemm_norm_kernel<false, false>));
    ExArgs a;
    a.x = static_cast<const u16*>(x);
    a.wt = static_cast<const u16*>(wt);
    a.gate = static_cast<const u32x4*>(gate);
    a.w = norm_weight;
    a.out = out;
    a.rows = (uint32_t)rows;
    a.width = (uint32_t)width;
    a.K = (uint32_t)K;
    a.G = (uint32_t)group_size;
    a.Ginv = (float)(1.0 / (double)group_size);
    a.eps = eps;
    void* args[] = {&a};
    // Row tiles per workgroup: enough that the grid is about one workgroup
    // per compute unit (each workgroup is a whole CU's worth of waves and
    // loads its B fragments and x once), at most kMaxTilesPerWg.
    const int64_t tiles = rows / kRowsPerTile, groups = width / group_size;
    int64_t tpw = (tiles * groups + kCus - 1) / kCus;
    if (tpw < 1) tpw = 1;
    if (tpw > kMaxTilesPerWg) tpw = kMaxTilesPerWg;
    a.tiles_per_wg = (uint32_t)tpw;
    const dim3 grid((uint32_t)((tiles + tpw - 1) / tpw), (uint32_t)groups);
    if (hipLaunchKernel(fn, grid, dim3(kWaves * 64), args, 0,
                        static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return 2;
    return 0;
}
