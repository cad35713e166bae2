// Device peak probes for the roofline figures: what the matrix cores and HBM of
// the device in hand actually sustain, measured next to the datasheet values.
//   * a bf16 matrix-core loop: every wave keeps eight independent accumulator
//     chains of v_mfma_f32_16x16x32_bf16 busy and touches no memory until its
//     final store, so the launch time is matrix-core issue time only;
//   * a plain device copy with 16-byte loads and stores, grid-stride, whose
//     bytes moved (read + write) over its time is the sustained HBM rate.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "../../../include/peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CHAINS = 8;
constexpr int THREADS = 256;

__global__ __launch_bounds__(THREADS) void k_mfma_loop(int iters, float* __restrict__ sink) {
  // operands depend on the lane so nothing folds; values stay small and finite
  bf16x8 a, b;
  for (int t = 0; t < 8; ++t) {
    a[t] = (__bf16)((float)((threadIdx.x + t) & 7) * 0.0078125f);
    b[t] = (__bf16)((float)((threadIdx.x * 3 + t) & 7) * 0.0078125f);
  }
  // eight named accumulators (an indexed array invites register shuffles between
  // iterations)
  const float z = (float)threadIdx.x * 0x1p-40f;   // distinct starting values keep them apart
  f32x4 c0 = {z, 0.f, 0.f, 0.f}, c1 = {0.f, z, 0.f, 0.f}, c2 = {0.f, 0.f, z, 0.f}, c3 = {0.f, 0.f, 0.f, z};
  f32x4 c4 = {2 * z, 0.f, 0.f, 0.f}, c5 = {0.f, 2 * z, 0.f, 0.f}, c6 = {0.f, 0.f, 2 * z, 0.f}, c7 = {0.f, 0.f, 0.f, 2 * z};
  // as one assembly block: the compiler otherwise moves the accumulators between
  // register files on every iteration.  Wait states around the block (the
  // compiler's hazard checks do not see into it): after the plain writes of the
  // starting values, and before the results are read.
  asm volatile("s_nop 7" ::);
  for (int it = 0; it < iters; ++it) {
    asm volatile(
        "v_mfma_f32_16x16x32_bf16 %0, %8, %9, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %8, %9, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %8, %9, %2\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %8, %9, %3\n\t"
        "v_mfma_f32_16x16x32_bf16 %4, %8, %9, %4\n\t"
        "v_mfma_f32_16x16x32_bf16 %5, %8, %9, %5\n\t"
        "v_mfma_f32_16x16x32_bf16 %6, %8, %9, %6\n\t"
        "v_mfma_f32_16x16x32_bf16 %7, %8, %9, %7"
        : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7)
        : "v"(a), "v"(b));
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::);
  const f32x4 t = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
  const float s = t[0] + t[1] + t[2] + t[3];
  sink[(size_t)blockIdx.x * THREADS + threadIdx.x] = s;
}

// Four 16-byte loads in flight per thread, then their four stores.
__global__ __launch_bounds__(THREADS) void k_copy16(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * THREADS;
  size_t i = (size_t)blockIdx.x * THREADS + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" {

double rece_peak_mfma_flops(int blocks, int iters) {
  // 16 x 16 x 32 multiply-adds per instruction, 2 flops each; 4 waves per block
  return 2.0 * 16 * 16 * 32 * CHAINS * (double)iters * (THREADS / 64) * (double)blocks;
}

int rece_peak_mfma_bf16(void* stream, int blocks, int iters, float* sink) {
  if (blocks <= 0 || iters <= 0 || !sink) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_mfma_loop, dim3(blocks), dim3(THREADS), 0, (hipStream_t)stream, iters, sink);
  return (int)hipGetLastError();
}

int rece_peak_copy(void* stream, const void* src, void* dst, size_t bytes) {
  if (!src || !dst || bytes % 16 != 0 || ((uintptr_t)src | (uintptr_t)dst) % 16 != 0)
    return (int)hipErrorInvalidValue;
  const size_t n = bytes / 16;
  if (n == 0) return 0;
  const size_t want = (n + THREADS - 1) / THREADS;
  const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(k_copy16, dim3(grid), dim3(THREADS), 0, (hipStream_t)stream,
                     (const uint4*)src, (uint4*)dst, n);
  return (int)hipGetLastError();
}

}  // extern "C"
