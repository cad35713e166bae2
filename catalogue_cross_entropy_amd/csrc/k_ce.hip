// Per-position loss and its mean (RECE page, Section 3, Algorithm 1: the
// positive-logit line with the positive's original item id, the loss line
// -log(e^{l+} / (e^{l+} + sum e^{l-})) and the final mean over |X| positions).
//
// The kept negatives of all rounds arrive as one (shift, sum of exp) pair per
// round, duplicates already removed; this kernel adds the positive and takes
// the log.  The mean is a fixed-order two-stage reduction (bit-reproducible).
#include "rece_device.h"
#include "rece_internal.h"

namespace rece {

constexpr int CE_POS_PER_BLOCK = 16;   // 4 waves x 4 positions, 16 lanes each

template <class E, int D>
__global__ __launch_bounds__(256) void k_ce(CeArgs a) {
  __shared__ double part[CE_POS_PER_BLOCK];
  const E* X = reinterpret_cast<const E*>(a.X);
  const E* Y = reinterpret_cast<const E*>(a.Y);
  const int l = lane_id(), w = threadIdx.x >> 6;
  const int sub = l >> 4, li = l & 15;
  const int slot = w * 4 + sub;
  const int64_t i = (int64_t)blockIdx.x * CE_POS_PER_BLOCK + slot;
  float loss = 0.0f;
  if (i < a.s) {
    int j = a.pos[i];
    if (j < 0 || j >= a.C) {
      if (a.validate && li == 0) atomicOr(a.counters + CNT_ERROR, (uint32_t)ERRBIT_BAD_ID);
      j = j < 0 ? 0 : (int)(a.C - 1);
    }
    const E* x = X + i * D;
    const E* y = Y + (int64_t)j * D;
    float acc = 0.0f;
    for (int t = li; t < D; t += 16) acc = fmaf(to_f32(x[t]), to_f32(y[t]), acc);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) acc += __shfl_xor(acc, o);
    const float lpos = acc;
    float m = lpos;
    for (int r = 0; r < a.rounds; ++r) {
      const int64_t o = (int64_t)r * a.s + i;
      if (a.nmem[o] > 0) m = fmaxf(m, a.mshift[o]);
    }
    float Z = expf(lpos - m);
    for (int r = 0; r < a.rounds; ++r) {
      const int64_t o = (int64_t)r * a.s + i;
      if (a.nmem[o] > 0) Z += a.ssum[o] * expf(a.mshift[o] - m);
    }
    const float lse = m + logf(Z);
    loss = lse - lpos;
    if (li == 0) {
      a.lse[i] = lse;
      a.lpos[i] = lpos;
      if (a.loss_pp) a.loss_pp[i] = loss;
    }
  }
  if (li == 0) part[slot] = (double)loss;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int q = 0; q < CE_POS_PER_BLOCK; ++q) t += part[q];
    reinterpret_cast<double*>(a.partial)[blockIdx.x] = t;
  }
}

__global__ __launch_bounds__(256) void k_mean(const double* __restrict__ partial, int nb, int64_t s,
                                              float* __restrict__ loss) {
  __shared__ double sh[256];
  double t = 0.0;
  for (int q = threadIdx.x; q < nb; q += 256) t += partial[q];
  sh[threadIdx.x] = t;
  __syncthreads();
  for (int off = 128; off >= 1; off >>= 1) {
    if ((int)threadIdx.x < off) sh[threadIdx.x] += sh[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = (float)(sh[0] / (double)s);
}

int ce_blocks(int64_t s) { return (int)((s + CE_POS_PER_BLOCK - 1) / CE_POS_PER_BLOCK); }

template <class E, int D>
static hipError_t launch_ce_t(const CeArgs& a, float* loss, hipStream_t st) {
  const int nb = ce_blocks(a.s);
  hipLaunchKernelGGL((k_ce<E, D>), dim3(nb), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_mean, dim3(1), dim3(256), 0, st, reinterpret_cast<const double*>(a.partial), nb, a.s, loss);
  return hipGetLastError();
}

hipError_t launch_ce(bool bf16v, int d, const CeArgs& a, float* loss, hipStream_t st) {
#define RECE_CE(E, DD) \
  if (d == DD) return launch_ce_t<E, DD>(a, loss, st);
  if (bf16v) {
    RECE_CE(bf16, 32) RECE_CE(bf16, 64) RECE_CE(bf16, 128) RECE_CE(bf16, 256)
  } else {
    RECE_CE(float, 32) RECE_CE(float, 64) RECE_CE(float, 128) RECE_CE(float, 256)
  }
#undef RECE_CE
  return hipErrorInvalidValue;
}

}  // namespace rece
