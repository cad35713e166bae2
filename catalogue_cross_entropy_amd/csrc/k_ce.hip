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
  __shared__ float cnt[CE_POS_PER_BLOCK];
  const E* X = reinterpret_cast<const E*>(a.X);
  const E* Y = reinterpret_cast<const E*>(a.Y);
  const int l = lane_id(), w = threadIdx.x >> 6;
  const int sub = l >> 4, li = l & 15;
  const int slot = w * 4 + sub;
  const int64_t i = (int64_t)blockIdx.x * CE_POS_PER_BLOCK + slot;
  float loss = 0.0f;
  float counted = 0.0f;
  if (i < a.s) {
    int j = a.pos[i];
    const bool pad = a.ignore && j < 0;
    if (j < 0 || j >= a.C) {
      if (a.validate && !pad && li == 0) atomicOr(a.counters + CNT_ERROR, (uint32_t)ERRBIT_BAD_ID);
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
    // (a padding position keeps a proper log-sum-exp, with item 0 standing in for its
    // positive, so that exp(logit - lse) stays bounded; its loss is 0)
    const float lse = m + logf(Z);
    loss = pad ? 0.0f : lse - lpos;
    counted = pad ? 0.0f : 1.0f;
    if (li == 0) {
      a.lse[i] = lse;
      a.lpos[i] = lpos;
      if (a.loss_pp) a.loss_pp[i] = loss;
    }
  }
  if (li == 0) {
    part[slot] = (double)loss;
    cnt[slot] = counted;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0, n = 0.0;
    for (int q = 0; q < CE_POS_PER_BLOCK; ++q) {
      t += part[q];
      n += cnt[q];
    }
    reinterpret_cast<double*>(a.partial)[2 * blockIdx.x] = t;
    reinterpret_cast<double*>(a.partial)[2 * blockIdx.x + 1] = n;
  }
}

// Mean over the positions counted (all of them without the padding mask; none
// counted gives 0), fixed order; also the weight 1 / count of a position in it.
__global__ __launch_bounds__(256) void k_mean(const double* __restrict__ partial, int nb, int64_t s, int ignore,
                                              float* __restrict__ loss, float* __restrict__ wmean) {
  __shared__ double sh[256], shn[256];
  double t = 0.0, c = 0.0;
  for (int q = threadIdx.x; q < nb; q += 256) {
    t += partial[2 * q];
    c += partial[2 * q + 1];
  }
  sh[threadIdx.x] = t;
  shn[threadIdx.x] = c;
  __syncthreads();
  for (int off = 128; off >= 1; off >>= 1) {
    if ((int)threadIdx.x < off) {
      sh[threadIdx.x] += sh[threadIdx.x + off];
      shn[threadIdx.x] += shn[threadIdx.x + off];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double n = ignore ? shn[0] : (double)s;
    loss[0] = n > 0.0 ? (float)(sh[0] / n) : 0.0f;
    if (wmean) wmean[0] = n > 0.0 ? (float)(1.0 / n) : 0.0f;
  }
}

// Rounds (RECE page, Section 3: the procedure repeated over rounds, with a
// minus-ln(count) term per logit).  The term makes the copies of a pair kept in
// several rounds count once, so a round's sum covers only the pairs no earlier
// round kept.  16 lanes per position (four positions per wave); lane `sub` takes
// eight consecutive list entries at a time (two 16-byte loads when k is a
// multiple of 4, so every cache line a load misses on is used whole).  The
// earlier rounds' kept ids go into the position's LDS hash table (open
// addressing, at most half full), then each entry of round rho's list is looked
// up; a pair found is marked with bit 31 (the backward skips it), the others are
// summed as exp(logit - shift) in a fixed order (per lane in list order, then a
// fixed tree over the 16 lanes).
constexpr int DEDUP_WAVES = 4;
constexpr int DEDUP_LPP = 16;                            // lanes per position
constexpr int DEDUP_PPB = DEDUP_WAVES * WAVE / DEDUP_LPP;  // positions per workgroup
constexpr int DEDUP_EPL = 8;                             // consecutive entries per lane and step
constexpr int DEDUP_CHUNK = DEDUP_LPP * DEDUP_EPL;       // list entries per step

__device__ __forceinline__ uint32_t dedup_hash(int id, int bits) {
  return ((uint32_t)id * 2654435761u) >> (32 - bits);
}

// Entries e0 + 8*sub .. +7 of a list of k (missing entries read as `pad`).
template <bool VEC, class T>
__device__ __forceinline__ void load8(const T* __restrict__ row, int e0, int sub, int k, T pad, T (&v)[DEDUP_EPL]) {
  const int e = e0 + DEDUP_EPL * sub;
  if constexpr (VEC) {   // k % 4 == 0: each quad is wholly inside or outside the list
#pragma unroll
    for (int h = 0; h < DEDUP_EPL / 4; ++h) {
      if (e + 4 * h < k) {
        typedef T T4 __attribute__((ext_vector_type(4)));
        const T4 q = *reinterpret_cast<const T4*>(row + e + 4 * h);
#pragma unroll
        for (int u = 0; u < 4; ++u) v[4 * h + u] = q[u];
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) v[4 * h + u] = pad;
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < DEDUP_EPL; ++u) v[u] = e + u < k ? row[e + u] : pad;
  }
}

// The eight entries of a lane walk their probe sequences (linear probing) in
// step, so each step has eight independent LDS accesses in flight.  The table
// always has a free slot, so every walk ends within the table size.
// find: bit u of the result is set when id[u] (>= 0) is in the table.
__device__ __forceinline__ uint32_t hash_find8(const int32_t* tab, int bits, const int (&id)[DEDUP_EPL]) {
  const uint32_t mask = (1u << bits) - 1u;
  uint32_t h[DEDUP_EPL];
  uint32_t open = 0, found = 0;
#pragma unroll
  for (int u = 0; u < DEDUP_EPL; ++u) {
    h[u] = dedup_hash(id[u], bits);
    open |= id[u] >= 0 ? 1u << u : 0u;
  }
  for (uint32_t step = 0; open && step <= mask; ++step) {
#pragma unroll
    for (int u = 0; u < DEDUP_EPL; ++u) {
      if (!((open >> u) & 1u)) continue;
      const int v = tab[h[u]];
      if (v == id[u]) found |= 1u << u;
      if (v == id[u] || v == -1) open &= ~(1u << u);
      h[u] = (h[u] + 1) & mask;
    }
  }
  return found;
}

// insert every id[u] >= 0 (an id already present stays once).
__device__ __forceinline__ void hash_insert8(int32_t* tab, int bits, const int (&id)[DEDUP_EPL]) {
  const uint32_t mask = (1u << bits) - 1u;
  uint32_t h[DEDUP_EPL];
  uint32_t open = 0;
#pragma unroll
  for (int u = 0; u < DEDUP_EPL; ++u) {
    h[u] = dedup_hash(id[u], bits);
    open |= id[u] >= 0 ? 1u << u : 0u;
  }
  for (uint32_t step = 0; open && step <= mask; ++step) {
#pragma unroll
    for (int u = 0; u < DEDUP_EPL; ++u) {
      if (!((open >> u) & 1u)) continue;
      const int old = atomicCAS(&tab[h[u]], -1, id[u]);
      if (old == -1 || old == id[u]) open &= ~(1u << u);
      h[u] = (h[u] + 1) & mask;
    }
  }
}

// Whether `id` is in one of the lists of rounds 0 .. rho - 1 (the scan used when
// the earlier ids do not fit the LDS tables).
__device__ __forceinline__ bool scan_find(const DedupArgs& a, int64_t i, int id) {
  for (int r2 = 0; r2 < a.rho; ++r2) {
    const int32_t* lst = a.negs + ((int64_t)r2 * a.s + i) * a.k;
    for (int t = 0; t < a.k; ++t) {
      const int raw = lst[t];
      if (raw != -1 && (raw & 0x7FFFFFFF) == id) return true;
    }
  }
  return false;
}

template <bool VEC, bool HASH>
__global__ __launch_bounds__(64 * DEDUP_WAVES) void k_round_dedup(DedupArgs a) {
  extern __shared__ int32_t tab_all[];
  const int q = threadIdx.x / DEDUP_LPP, sub = threadIdx.x % DEDUP_LPP;
  const int64_t i = (int64_t)blockIdx.x * DEDUP_PPB + q;
  const int k = a.k, rho = a.rho, bits = a.hash_bits;
  const bool live = i < a.s;
  int32_t* tab = tab_all + (HASH ? (size_t)q << bits : 0);
  if (HASH) {
    for (int t = sub; t < (1 << bits); t += DEDUP_LPP) tab[t] = -1;
    __syncthreads();
    if (live) {
      for (int r2 = 0; r2 < rho; ++r2) {
        const int32_t* lst = a.negs + ((int64_t)r2 * a.s + i) * k;
        for (int e0 = 0; e0 < k; e0 += DEDUP_CHUNK) {
          int raw[DEDUP_EPL];
          load8<VEC>(lst, e0, sub, k, -1, raw);
#pragma unroll
          for (int u = 0; u < DEDUP_EPL; ++u) raw[u] = raw[u] == -1 ? -1 : raw[u] & 0x7FFFFFFF;
          hash_insert8(tab, bits, raw);
        }
      }
    }
    __syncthreads();
  }
  if (!live) return;   // the rest needs no barrier
  const int64_t o = (int64_t)rho * a.s + i;
  int32_t* mine = a.negs + o * k;
  const float* lg = a.negl + i * (int64_t)k;
  const float mx = a.mshift[o];
  float sum = 0.0f;
  int cnt = 0;
  for (int e0 = 0; e0 < k; e0 += DEDUP_CHUNK) {
    int id[DEDUP_EPL];
    float lv[DEDUP_EPL];
    load8<VEC>(mine, e0, sub, k, -1, id);
    load8<VEC>(lg, e0, sub, k, 0.0f, lv);
    uint32_t dupm = 0;   // bit u: entry u was kept in an earlier round
    if (HASH) {
      dupm = hash_find8(tab, bits, id);
    } else {
#pragma unroll
      for (int u = 0; u < DEDUP_EPL; ++u)
        if (id[u] >= 0 && scan_find(a, i, id[u])) dupm |= 1u << u;
    }
#pragma unroll
    for (int u = 0; u < DEDUP_EPL; ++u) {
      const bool fresh = id[u] >= 0 && ((dupm >> u) & 1u) == 0;
      sum += fresh ? __expf(lv[u] - mx) : 0.0f;
      cnt += fresh ? 1 : 0;
    }
    if (dupm) {   // write the lane's entries back with the marks
      int outv[DEDUP_EPL];
#pragma unroll
      for (int u = 0; u < DEDUP_EPL; ++u) outv[u] = ((dupm >> u) & 1u) ? (id[u] | (int)0x80000000u) : id[u];
      const int e = e0 + DEDUP_EPL * sub;
      if constexpr (VEC) {
#pragma unroll
        for (int h = 0; h < DEDUP_EPL / 4; ++h)
          if (e + 4 * h < k)
            *reinterpret_cast<u32x4*>(mine + e + 4 * h) =
                u32x4{(uint32_t)outv[4 * h], (uint32_t)outv[4 * h + 1], (uint32_t)outv[4 * h + 2],
                      (uint32_t)outv[4 * h + 3]};
      } else {
#pragma unroll
        for (int u = 0; u < DEDUP_EPL; ++u)
          if ((dupm >> u) & 1u) mine[e + u] = outv[u];
      }
    }
  }
#pragma unroll
  for (int off = 1; off < DEDUP_LPP; off <<= 1) {
    sum += __shfl_xor(sum, off);
    cnt += __shfl_xor(cnt, off);
  }
  if (sub == 0) {
    a.ssum[o] = sum;
    a.nmem[o] = cnt;
  }
}

int dedup_hash_bits(int rounds, int k) {
  const int64_t n = (int64_t)std::max(rounds - 1, 1) * std::max(k, 1);
  // one table of 2^bits int32 slots per position of the workgroup, within 128 KB of
  // LDS: at most a quarter full (short probe walks), else at most half full
  for (int64_t fill : {4, 2}) {
    int bits = 4;
    while (((int64_t)1 << bits) < fill * n) ++bits;
    if (((size_t)DEDUP_PPB << bits) * 4 <= 128 * 1024) return bits;
  }
  return 0;
}

hipError_t launch_round_dedup(const DedupArgs& a, hipStream_t st) {
  const size_t lds = a.hash_bits ? ((size_t)DEDUP_PPB << a.hash_bits) * 4 : 0;
  auto kern = a.hash_bits ? (a.k % 4 == 0 ? k_round_dedup<true, true> : k_round_dedup<false, true>)
                          : (a.k % 4 == 0 ? k_round_dedup<true, false> : k_round_dedup<false, false>);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const unsigned blocks = (unsigned)((a.s + DEDUP_PPB - 1) / DEDUP_PPB);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * DEDUP_WAVES), lds, st, a);
  return hipGetLastError();
}

int ce_blocks(int64_t s) { return (int)((s + CE_POS_PER_BLOCK - 1) / CE_POS_PER_BLOCK); }

template <class E, int D>
static hipError_t launch_ce_t(const CeArgs& a, float* loss, hipStream_t st) {
  const int nb = ce_blocks(a.s);
  hipLaunchKernelGGL((k_ce<E, D>), dim3(nb), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_mean, dim3(1), dim3(256), 0, st, reinterpret_cast<const double*>(a.partial), nb, a.s, a.ignore,
                     loss, a.wmean);
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
