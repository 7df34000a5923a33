// bench_aux.hip -- measurement helpers for the benchmark (libggrms_bench.so).
// Not part of the product ABI.
//   * an empty kernel taking an argument block of the same size as the
//     normalisation kernels, launched with a caller-chosen grid: the floor
//     that a decode launch is compared against;
//   * a plain 16-byte vector copy of known size: the calibration that turns
//     the FETCH_SIZE / WRITE_SIZE counters into HBM bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ggrms_internal.h"

namespace {

__global__ void ggrms_bench_empty_kernel(ggrms::KArgs) {}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void ggrms_bench_copy_kernel(const u32x4* __restrict__ src,
                                                               u32x4* __restrict__ dst,
                                                               uint64_t n) {
    const uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

}  // namespace

extern "C" int ggrms_bench_empty(int64_t blocks, int threads, void* stream) {
    ggrms::KArgs a = {};
    void* args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void*>(&ggrms_bench_empty_kernel),
                           dim3((uint32_t)blocks), dim3((uint32_t)threads), args, 0,
                           static_cast<hipStream_t>(stream)) == hipSuccess
               ? 0
               : 1;
}

// Copies nbytes (a multiple of 16; both pointers 16-byte aligned).
extern "C" int ggrms_bench_copy(const void* src, void* dst, int64_t nbytes, void* stream) {
    if (nbytes <= 0 || nbytes % 16 || (uintptr_t)src % 16 || (uintptr_t)dst % 16) return 1;
    const uint64_t n = (uint64_t)nbytes / 16;
    const uint64_t blocks = (n + 255) / 256;
    if (blocks > 0xFFFFFFFFull / 256) return 1;
    void* args[] = {&src, &dst, (void*)&n};
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    args[0] = &s;
    args[1] = &d;
    return hipLaunchKernel(reinterpret_cast<const void*>(&ggrms_bench_copy_kernel),
                           dim3((uint32_t)blocks), dim3(256), args, 0,
                           static_cast<hipStream_t>(stream)) == hipSuccess
               ? 0
               : 1;
}
