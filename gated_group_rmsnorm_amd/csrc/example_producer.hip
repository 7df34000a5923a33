// example_producer.hip -- the per-unit epilogue (ggrms_epilogue.hpp) called
// from a kernel that computes y itself, so that y never reaches HBM: the
// hand-off that fusing the norm into the kernel producing y needs.
//
// The page "gated_group_rmsnorm" places this math inside the Mamba-2 scan
// (the norm_before_gate=False branch of its combined scan), and the standalone
// op is a port of it.  The pages do not define the scan, so the producer here
// is a stand-in with a plain definition: y = bf16(x @ wt^T), a bf16 matrix
// product on the matrix cores (v_mfma_f32_16x16x16_bf16), whose output tile
// arrives in the accumulator layout of the MFMA instruction, like any
// contraction's.  What carries over to a real producer is the hand-off:
//   * a workgroup owns whole (row, group) units -- here row tiles of 16 rows
//     x one group of G columns, G/64 waves each computing 64 of the columns;
//   * the accumulators are rounded to the storage type (the values the
//     standalone op would have read back) and re-laid through LDS from the
//     MFMA layout (lane = column, 4 consecutive rows per lane) to the
//     epilogue's (lane = 16 bytes of one row);
//   * each wave then takes rows of the tile and runs the epilogue's steps on
//     them: gate_and_square on y from LDS and the gate from global memory,
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

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kRowsPerTile = 16;   // one MFMA tile of rows
constexpr int kTilesPerGroup = 8;  // row tiles one workgroup takes in turn
constexpr int kMaxGroup = 1024;    // 128 vectors of bf16: two per lane
constexpr int kMaxK = 64;          // the B fragments of every k step stay in registers
constexpr int kLdsPad = 8;         // bf16 elements of padding per LDS row

struct ExArgs {
    const u16* x;      // [rows, K] bf16
    const u16* wt;     // [width, K] bf16
    const u32x4* gate; // [rows, width] bf16, as 16-byte vectors
    const float* w;    // [width] f32
    void* out;         // [rows, width] bf16
    uint32_t rows, width, K, G;
    float Ginv, eps;
    uint32_t produce_only;  // 1: store y itself (the unfused producer)
};

// One workgroup: group g, row tiles blockIdx.x * 8 .. + 7 (16 rows each, the
// last workgroup's may be fewer), G / 64 waves.  Wave w computes columns
// g*G + 64w .. 64w + 63 as four MFMA tiles of 16 columns; its B fragments (wt
// for those columns, every k step) are loaded once and reused for every row
// tile, and so are the lanes' weights of the epilogue.  The workgroup's rows
// of x are staged in LDS up front: a global load issued after a store is
// counted behind it (memory counters retire in order), so loading x tile by
// tile would make every tile wait for the previous tile's stores.
template <bool RI>
__global__ __launch_bounds__(kMaxGroup) void example_gemm_norm_kernel(ExArgs a) {
    constexpr int NT = 4;  // column tiles per wave
    // two re-lay buffers, used by alternate tiles: one barrier per tile; rows
    // of 2064 bytes keep every 16-byte vector of a row 16-byte aligned
    __shared__ __attribute__((aligned(16))) u16 ys[2][kRowsPerTile][kMaxGroup + kLdsPad];
    __shared__ __attribute__((aligned(16))) u16 xs[kTilesPerGroup * kRowsPerTile][kMaxK];
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t waves = blockDim.x >> 6;  // G / 64
    const uint32_t g = blockIdx.y;
    const uint32_t G = a.G;
    const uint32_t ccol0 = wave * 64;  // first column of this wave in the group
    const uint32_t ntiles = a.rows / kRowsPerTile;
    const uint32_t t0 = blockIdx.x * kTilesPerGroup;
    const uint32_t t1 = t0 + kTilesPerGroup < ntiles ? t0 + kTilesPerGroup : ntiles;
    const uint32_t nks = a.K / 16;  // k steps, <= kMaxK / 16

    // x rows of the workgroup's tiles into LDS, 16 bytes at a time
    {
        const uint32_t r0 = t0 * kRowsPerTile, nr = (t1 - t0) * kRowsPerTile;
        const uint32_t per_row = a.K / 8;  // 16-byte pieces per row
        for (uint32_t i = threadIdx.x; i < nr * per_row; i += blockDim.x) {
            const uint32_t r = i / per_row, c = i - r * per_row;
            *reinterpret_cast<u32x4*>(&xs[r][c * 8]) =
                *reinterpret_cast<const u32x4*>(a.x + (size_t)(r0 + r) * a.K + c * 8);
        }
    }

    // v_mfma_f32_16x16x16_bf16: lane l supplies A[l % 16][4*(l/16) + i] and
    // B[4*(l/16) + i][l % 16] (i = 0..3) and holds D[4*(l/16) + i][l % 16].
    const uint32_t m = lane & 15, kq = (lane >> 4) * 4;
    s16x4 bv[NT][kMaxK / 16];
#pragma unroll
    for (int ks = 0; ks < kMaxK / 16; ++ks) {
        if ((uint32_t)ks >= nks) break;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t col = g * G + ccol0 + t * 16 + m;
            bv[t][ks] = *reinterpret_cast<const s16x4*>(a.wt + (size_t)col * a.K + ks * 16 + kq);
        }
    }
    // the epilogue's slots: a row's group is nvec = G/8 vectors, lane l holds
    // vectors l and l + 64 (the same columns for every row)
    const uint32_t nvec = G / 8;
    constexpr int K = 2;
    uint32_t ci[K];
    float wr[K][8];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const uint32_t idx = lane + k * 64;
        ci[k] = idx < nvec ? idx : nvec - 1;  // past the end: a copy of the last vector
        const f32x4* wp = reinterpret_cast<const f32x4*>(a.w + (size_t)g * G + ci[k] * 8);
        const f32x4 w0 = wp[0], w1 = wp[1];
        wr[k][0] = w0.x; wr[k][1] = w0.y; wr[k][2] = w0.z; wr[k][3] = w0.w;
        wr[k][4] = w1.x; wr[k][5] = w1.y; wr[k][6] = w1.z; wr[k][7] = w1.w;
    }
    auto live = [&](int k) { return lane + k * 64 < nvec; };
    auto owned = [](int, int) { return true; };
    auto gate_at = [&](uint32_t n, int k) {
        return a.gate + ((size_t)n * a.width + (size_t)g * G) / 8 + ci[k];
    };
    __syncthreads();  // xs is complete

    for (uint32_t tile = t0; tile < t1; ++tile) {
        const uint32_t r0 = tile * kRowsPerTile;
        // the gate of this wave's first row of the tile, requested before the
        // multiply and the re-lay so that its latency overlaps them
        u32x4 gp[K] = {};
        if (!a.produce_only) {
#pragma unroll
            for (int k = 0; k < K; ++k) gp[k] = __builtin_nontemporal_load(gate_at(r0 + wave, k));
        }
        // --- producer: the tile of y in MFMA accumulators
        f32x4v acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < kMaxK / 16; ++ks) {
            if ((uint32_t)ks >= nks) break;
            const s16x4 av = *reinterpret_cast<const s16x4*>(&xs[(tile - t0) * kRowsPerTile + m][ks * 16 + kq]);
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv[t][ks], acc[t], 0, 0, 0);
        }
        // round to bf16 and re-lay: D[4*(l/16) + i][l % 16] -> yb[row][column in
        // group].  The buffer was last read two tiles ago, before every wave
        // passed the previous tile's barrier.
        u16 (*yb)[kMaxGroup + kLdsPad] = ys[(tile - t0) & 1];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                yb[kq + i][ccol0 + t * 16 + m] = Cvt<TBF16>::pack_half(acc[t][i]);
        }
        __syncthreads();

        // --- epilogue: wave w takes rows w, w + waves, ... of the tile
        for (uint32_t rr = wave; rr < kRowsPerTile; rr += waves) {
            const bool first = rr == wave;
            const uint32_t n = r0 + rr;
            u32x4 yr[K];
#pragma unroll
            for (int k = 0; k < K; ++k) yr[k] = *reinterpret_cast<const u32x4*>(&yb[rr][ci[k] * 8]);
            u32x4* ov = reinterpret_cast<u32x4*>(a.out) + ((size_t)n * a.width + (size_t)g * G) / 8;
            if (a.produce_only) {  // the unfused producer: y goes to memory
#pragma unroll
                for (int k = 0; k < K; ++k)
                    if (live(k)) __builtin_nontemporal_store(yr[k], ov + ci[k]);
                continue;
            }
            u32x4 gr[K];
#pragma unroll
            for (int k = 0; k < K; ++k)
                gr[k] = first ? gp[k] : __builtin_nontemporal_load(gate_at(n, k));
            epi::LaneUnit<TBF16, 16, K, false> L;
            const float part = epi::gate_and_square<TBF16, 16, 16, K, false>(yr, gr, L, live, owned);
            const float m2 = segment_sum<64>(part);
            const float nf = norm_factor(m2, a.Ginv, a.eps);
            u32x4 res[K];
            epi::finish<RI>(L, nf, wr, res);
#pragma unroll
            for (int k = 0; k < K; ++k)
                if (live(k)) __builtin_nontemporal_store(res[k], ov + ci[k]);
        }
    }
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
    const void* fn = round_intermediate ? reinterpret_cast<const void*>(&example_gemm_norm_kernel<true>)
                                        : reinterpret_cast<const void*>(&example_gemm_norm_kernel<false>);
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
    a.produce_only = produce_only != 0;
    void* args[] = {&a};
    const int64_t tiles = rows / kRowsPerTile;
    const dim3 grid((uint32_t)((tiles + kTilesPerGroup - 1) / kTilesPerGroup),
                    (uint32_t)(width / group_size));
    if (hipLaunchKernel(fn, grid, dim3((uint32_t)group_size), args, 0,
                        static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return 2;
    return 0;
}
