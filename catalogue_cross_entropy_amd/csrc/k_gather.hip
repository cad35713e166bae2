// Layout kernels between the sort and the chunk kernels.
//   * sorted copies: Xs[p] = X[perm_x[p]], Ys[q] = Y[perm_y[q]] (RECE page,
//     Algorithm 1 sorting lines "X = X[argsort I]", "Y = Y[argsort J]"), so every
//     chunk and every window is one contiguous block of rows;
//   * for rounds rho > 0: the chunk that item perm_y_rho[q] had in an earlier
//     round r2, aligned with the round-rho order (duplicate tests stream it);
//   * backward records: per sorted position, what the backward kernels need of
//     it (log-sum-exp, upstream gradient, this round's threshold, positive id)
//     and its thresholds of earlier rounds.
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

__global__ __launch_bounds__(256) void k_prev_chunks(const int32_t* __restrict__ perm_y, const int32_t* __restrict__ inv_y2,
                                                     int64_t C, int n_c, int32_t* __restrict__ out) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q < C) out[q] = chunk_of(inv_y2[perm_y[q]], C, n_c);
}

hipError_t launch_prev_chunks(const int32_t* perm_y, const int32_t* inv_y2, int64_t C, int n_c, int32_t* out,
                              hipStream_t st) {
  hipLaunchKernelGGL(k_prev_chunks, dim3((unsigned)((C + 255) / 256)), dim3(256), 0, st, perm_y, inv_y2, C, n_c,
                     out);
  return hipGetLastError();
}

// rec[p], prev[r2][p] for the positions of round rho in sorted order.
__global__ __launch_bounds__(256) void k_bwd_records(BwdArgs a, const int32_t* __restrict__ perm_x, int rho,
                                                     PosRec* __restrict__ rec, PrevRow* __restrict__ prev) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= a.s) return;
  const int64_t i = perm_x[p];
  const int64_t o = (int64_t)rho * a.s + i;
  PosRec r;
  r.lse = a.lse[i];
  r.gb = a.dloss_pp ? a.dloss_pp[i] : a.dloss[0] / (float)a.npos;
  r.lo = a.thr_lo[o];
  r.hi = a.thr_hi[o];
  r.te = a.thr_e[o];
  r.tid = a.thr_id[o];
  r.pos = a.pos[i];
  r.i = (int32_t)i;
  r.lpos = a.lpos[i];
  r.pad0 = 0;
  r.pad1 = 0;
  if (a.sce) {   // the position's group of slots and this slot's place in it
    r.pad0 = a.sce_pstart[i];
    r.pad1 = a.sce_inv[p] - r.pad0;
  }
  rec[p] = r;
  for (int r2 = 0; r2 < rho; ++r2) {
    const int64_t o2 = (int64_t)r2 * a.s + i;
    PrevRow q;
    q.te = a.thr_e[o2];
    q.lo = a.thr_lo[o2];
    q.hi = a.thr_hi[o2];
    q.tid = a.thr_id[o2];
    q.cx = chunk_of(a.inv_x[o2], a.s, a.n_c);
    prev[(int64_t)r2 * a.s + p] = q;
  }
}

hipError_t launch_bwd_records(const BwdArgs& a, const int32_t* perm_x, int rho, PosRec* rec, PrevRow* prev,
                              hipStream_t st) {
  hipLaunchKernelGGL(k_bwd_records, dim3((unsigned)((a.s + 255) / 256)), dim3(256), 0, st, a, perm_x, rho, rec,
                     prev);
  return hipGetLastError();
}

}  // namespace rece
