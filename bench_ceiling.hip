// Streaming-read ceiling: the HBM read rate a plain kernel reaches on this
// part, the reference beside which bench.py --ceiling reports the GEMV.
// Measurement tool only (bench_ceiling.so, built beside bench.py); the
// product library does not contain or use it.
//
// Every workgroup reads 16-byte chunks in a grid-stride loop, four loads in
// flight per lane, and folds them with XOR; the result is stored only if it
// equals a value the caller passes in (practically never), which keeps the
// loads alive without writing anything.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWgs = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kWgs) void read_sweep_kernel(const u32x4_t *__restrict__ p, int64_t n16,
                                                          uint32_t *__restrict__ sink, uint32_t never) {
    uint32_t acc = 0;
    const int64_t step = (int64_t)gridDim.x * kWgs * kUnroll;
    for (int64_t i = (int64_t)blockIdx.x * kWgs * kUnroll + threadIdx.x; i < n16; i += step) {
        u32x4_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t k = i + u * kWgs;
            v[u] = k < n16 ? p[k] : u32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == never) sink[threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, `buf` 16-byte aligned) on `hip_stream`
// with `blocks` workgroups of 256 threads.  `sink` must hold 256 uint32.
// Returns 0, or -1 for bad arguments, -4 when the launch fails.
int qw3_read_sweep(const void *buf, int64_t bytes, int32_t blocks, uint32_t *sink, void *hip_stream) {
    if (!buf || !sink || bytes < 0 || bytes % 16 != 0 || blocks < 1 || ((uintptr_t)buf & 15) != 0) return -1;
    if (bytes == 0) return 0;
    hipLaunchKernelGGL(read_sweep_kernel, dim3((unsigned)blocks), dim3(kWgs), 0, (hipStream_t)hip_stream,
                       reinterpret_cast<const u32x4_t *>(buf), bytes / 16, sink, 0x9E3779B9u);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
