// Per-position loss and its mean (RECE page, Section 3, Algorithm 1: the
// positive-logit line with the positive's original item id, the loss line
// -log(e^{l+} / (e^{l+} + sum e^{l-})) and the final mean over |X| positions).
//
// The kept negatives of all rounds arrive as one (shift, sum of exp) pair per
// round, duplicates already removed; this kernel adds the positive and takes
// the log.  The mean is a fixed-order two-stage reduction (bit-reproducible).
#include <algorithm>

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

// Rounds (RECE page, Section 3: the procedure repeated over rounds, with a
// minus-ln(count) term per logit).  The term makes the copies of a pair kept in
// several rounds count once, so a round's sum covers only the pairs no earlier
// round kept.  One wave per position: the earlier rounds' kept ids go into an LDS
// hash table (open addressing, at most half full), then each entry of round rho's
// list is looked up; a pair found is marked with bit 31 (the backward skips it),
// the others are summed as exp(logit - shift) in list order and a fixed tree.
constexpr int DEDUP_WAVES = 4;

__device__ __forceinline__ uint32_t dedup_hash(int id, int bits) {
  return ((uint32_t)id * 2654435761u) >> (32 - bits);
}

__global__ __launch_bounds__(64 * DEDUP_WAVES) void k_round_dedup(DedupArgs a) {
  extern __shared__ int32_t tab_all[];
  const int w = threadIdx.x >> 6, l = lane_id();
  const int64_t i = (int64_t)blockIdx.x * DEDUP_WAVES + w;
  const int k = a.k, rho = a.rho, bits = a.hash_bits;
  const int hs = bits ? 1 << bits : 0;
  int32_t* tab = tab_all + (size_t)w * hs;
  const bool live = i < a.s;
  for (int t = l; t < hs; t += WAVE) tab[t] = -1;
  __syncthreads();
  if (live && bits) {
    for (int r2 = 0; r2 < rho; ++r2) {
      const int32_t* lst = a.negs + ((int64_t)r2 * a.s + i) * k;
      for (int e = l; e < k; e += WAVE) {
        const int raw = lst[e];
        if (raw == -1) continue;
        const int id = raw & 0x7FFFFFFF;
        uint32_t h = dedup_hash(id, bits);
        for (int probe = 0; probe < hs; ++probe) {   // a free slot always exists
          const int old = atomicCAS(&tab[h], -1, id);
          if (old == -1 || old == id) break;
          h = (h + 1) & (uint32_t)(hs - 1);
        }
      }
    }
  }
  __syncthreads();
  if (!live) return;
  const int64_t o = (int64_t)rho * a.s + i;
  int32_t* mine = a.negs + o * k;
  const float* lg = a.negl + i * (int64_t)k;
  const float mx = a.mshift[o];
  float sum = 0.0f;
  int cnt = 0;
  for (int e = l; e < k; e += WAVE) {
    const int id = mine[e];
    if (id < 0) continue;
    bool dup = false;
    if (bits) {
      uint32_t h = dedup_hash(id, bits);
      for (int probe = 0; probe < hs; ++probe) {
        const int v = tab[h];
        if (v == id) {
          dup = true;
          break;
        }
        if (v == -1) break;
        h = (h + 1) & (uint32_t)(hs - 1);
      }
    } else {
      for (int r2 = 0; r2 < rho && !dup; ++r2) {
        const int32_t* lst = a.negs + ((int64_t)r2 * a.s + i) * k;
        for (int u = 0; u < k; ++u) {
          const int raw = lst[u];
          if (raw != -1 && (raw & 0x7FFFFFFF) == id) {
            dup = true;
            break;
          }
        }
      }
    }
    if (dup) {
      mine[e] = id | (int)0x80000000u;
    } else {
      sum += __expf(lg[e] - mx);
      ++cnt;
    }
  }
  sum = wave_sumf(sum);
#pragma unroll
  for (int off = 1; off < WAVE; off <<= 1) cnt += __shfl_xor(cnt, off);
  if (l == 0) {
    a.ssum[o] = sum;
    a.nmem[o] = cnt;
  }
}

int dedup_hash_bits(int rounds, int k) {
  const int64_t n = (int64_t)std::max(rounds - 1, 1) * std::max(k, 1);
  int bits = 6;
  while (((int64_t)1 << bits) < 2 * n) ++bits;
  // four waves of 2^bits int32 slots must fit the 160 KB of LDS a workgroup may take
  return ((size_t)DEDUP_WAVES << bits) * 4 <= 128 * 1024 ? bits : 0;
}

hipError_t launch_round_dedup(const DedupArgs& a, hipStream_t st) {
  const size_t lds = a.hash_bits ? ((size_t)DEDUP_WAVES << a.hash_bits) * 4 : 0;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_round_dedup),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const unsigned blocks = (unsigned)((a.s + DEDUP_WAVES - 1) / DEDUP_WAVES);
  hipLaunchKernelGGL(k_round_dedup, dim3(blocks), dim3(64 * DEDUP_WAVES), lds, st, a);
  return hipGetLastError();
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
