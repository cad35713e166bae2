// Exact k-th largest float of a short list held in LDS, computed by one wave.
#pragma once
#include "rece_device.h"

namespace rece {

constexpr int KTH_BINS = 256;

__device__ __forceinline__ int kth_bin_of(float v, float lo, float scale) {
  const float x = fminf(fmaxf((v - lo) * scale, 0.0f), (float)(KTH_BINS - 1));
  return (int)x;
}

// Exact k-th largest (1-based) of vals[0..n), 1 <= k <= n.  Histogram refinement
// until at most 64 values remain in range, then one value per lane, ranked by
// broadcasting each lane's value in turn.
__device__ inline float wave_kth_largest(const float* vals, int n, int k, uint32_t* hist, float* cand) {
  const int l = lane_id();
  float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
  for (int t = l; t < n; t += WAVE) {
    const float v = vals[t];
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  int kk = k;
  int m = n;
  for (int iter = 0; iter < 12; ++iter) {
    if (!(hi > lo)) return hi;
    if (m <= WAVE) {
      int cnt = 0;
      for (int base = 0; base < n; base += WAVE) {
        const int t = base + l;
        const float v = t < n ? vals[t] : 0.0f;
        const bool live = t < n && v >= lo && v <= hi;
        const uint64_t mk = ballot(live);
        if (live) cand[cnt + popc(mk & lanemask_lt())] = v;
        cnt += popc(mk);
      }
      wave_sync();
      const float c = l < m ? cand[l] : NEG_INF;
      int gt = 0, ge = 0;
      for (int u = 0; u < m; ++u) {
        const float cu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), u));
        gt += cu > c;
        ge += cu >= c;
      }
      const uint64_t ok = ballot(l < m && gt < kk && kk <= ge);
      const float r =
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), __builtin_ctzll(ok | (1ull << 63))));
      wave_sync();
      return r;
    }
    const float scale = (float)KTH_BINS / (hi - lo);
    for (int b = l; b < KTH_BINS; b += WAVE) hist[b] = 0u;
    wave_sync();
    for (int t = l; t < n; t += WAVE) {
      const float v = vals[t];
      if (v >= lo && v <= hi) atomicAdd(&hist[kth_bin_of(v, lo, scale)], 1u);
    }
    wave_sync();
    uint32_t h[4];
    uint32_t own = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      h[q] = hist[4 * l + q];
      own += h[q];
    }
    uint32_t suf = own;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_down(suf, o);
      if (l + o < 64) suf += y;
    }
    int myb = -1;
    uint32_t my_above = 0, my_cnt = 0;
    {
      uint32_t acc = suf - own;
#pragma unroll
      for (int q = 3; q >= 0; --q) {
        if (myb < 0 && acc + h[q] >= (uint32_t)kk) {
          myb = 4 * l + q;
          my_above = acc;
          my_cnt = h[q];
        }
        acc += h[q];
      }
    }
    const uint64_t hit = ballot(myb >= 0);
    const int src = 63 - __builtin_clzll(hit | 1ull);
    const int bstar = __shfl(myb, src);
    kk -= (int)__shfl(my_above, src);
    m = (int)__shfl(my_cnt, src);
    float nlo = __builtin_huge_valf(), nhi = -__builtin_huge_valf();
    for (int t = l; t < n; t += WAVE) {
      const float v = vals[t];
      if (v >= lo && v <= hi && kth_bin_of(v, lo, scale) == bstar) {
        nlo = fminf(nlo, v);
        nhi = fmaxf(nhi, v);
      }
    }
    lo = wave_min(nlo);
    hi = wave_max(nhi);
  }
  // more than 64 distinct values in a range that no longer splits: rank directly
  float result = lo;
  for (int base = 0; base < n; base += WAVE) {
    const int t = base + l;
    const float v = t < n ? vals[t] : 0.0f;
    bool ok = false;
    if (t < n && v >= lo && v <= hi) {
      int gt = 0, ge = 0;
      for (int u = 0; u < n; ++u) {
        const float x = vals[u];
        if (x >= lo && x <= hi) {
          gt += x > v;
          ge += x >= v;
        }
      }
      ok = gt < kk && kk <= ge;
    }
    const uint64_t okm = ballot(ok);
    if (okm) {
      result = __shfl(v, __builtin_ctzll(okm));
      break;
    }
  }
  return result;
}

}  // namespace rece
