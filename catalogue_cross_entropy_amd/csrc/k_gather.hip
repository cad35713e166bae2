// Sorted copies between the sort and the chunk kernels: Xs[p] = X[perm_x[p]],
// Ys[q] = Y[perm_y[q]] (RECE page, Algorithm 1, the two sorting lines that reorder
// X and Y by bucket), so every chunk and every window is one contiguous block of
// rows.  The bucket variant gathers the rows each bucket took the same way.
#include "rece_device.h"
#include "rece_internal.h"

namespace rece {

// Copy rows src[perm[p]] -> dst[p]; one thread per 16-byte chunk.
__global__ __launch_bounds__(256) void k_gather_rows(const char* __restrict__ src, const int32_t* __restrict__ perm,
                                                     int64_t n, int row_bytes, char* __restrict__ dst) {
  const int cpr = row_bytes / 16;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n * cpr) return;
  const int64_t p = idx / cpr;
  const int c = (int)(idx % cpr);
  const int64_t e = perm[p];
  *reinterpret_cast<u32x4*>(dst + p * row_bytes + c * 16) =
      *reinterpret_cast<const u32x4*>(src + e * row_bytes + c * 16);
}

hipError_t launch_gather_rows(const void* src, const int32_t* perm, int64_t n, int row_bytes, void* dst,
                              hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t total = n * (row_bytes / 16);
  hipLaunchKernelGGL(k_gather_rows, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                     static_cast<const char*>(src), perm, n, row_bytes, static_cast<char*>(dst));
  return hipGetLastError();
}

}  // namespace rece
