// Exact k-th largest float of a short list held in LDS, computed by one wave, and
// the exact top-k of such a list (float64 near-tie ranking).
#pragma once
#include "rece_device.h"
#include "rece_internal.h"

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

constexpr int MG_NEAR = 256;   // near-tie entries ranked in float64 per step

struct MergeLds {
  int32_t* ids;    // [cap]
  float* vals;     // [cap]
  uint32_t* khist; // [256]
  float* cv;       // [64]
  int32_t* ci;     // [MG_NEAR] list index
  double* ce;      // [MG_NEAR] float64 logit
};
// LDS of one wave for a list of up to cap entries.
__host__ __device__ constexpr size_t topk_wave_bytes(int cap) {
  return (size_t)cap * 8 + 256 * 4 + 64 * 4 + MG_NEAR * 4 + MG_NEAR * 8;
}

__device__ inline MergeLds carve_topk(char* base, int cap) {
  MergeLds L;
  L.ids = reinterpret_cast<int32_t*>(base);
  L.vals = reinterpret_cast<float*>(base + (size_t)cap * 4);
  L.khist = reinterpret_cast<uint32_t*>(base + (size_t)cap * 8);
  L.cv = reinterpret_cast<float*>(base + (size_t)cap * 8 + 1024);
  L.ci = reinterpret_cast<int32_t*>(base + (size_t)cap * 8 + 1280);
  L.ce = reinterpret_cast<double*>(base + (size_t)cap * 8 + 1280 + MG_NEAR * 4);
  return L;
}

// Rank the near-tie band {t : lo <= vals[t] <= hi} of list[0..n) when it holds
// more entries than MG_NEAR: no float64 buffer, every comparison recomputes the
// other entry's float64 logit (64 at a time, one per lane).  Quadratic in the band
// and slow, but exact; reached only with hundreds of equal or nearly equal logits
// at the k-th place (repeated item vectors).  Entries ranked at or beyond `need`
// get value -inf; returns the element ranked need - 1 (te, tid).
template <class E, int D>
__device__ __forceinline__ void rank_band_wide(const MergeLds& L, int n, int need, float lo, float hi,
                                                         const E* xrow, const E* Y, double& te, int& tid,
                                                         uint32_t& nexact) {
  const int l = lane_id();
  constexpr uint32_t OUT = 0x80000000u;   // ranked out (ids are non-negative)
  uint32_t ndot = 0;
  for (int eb = 0; eb < n; eb += WAVE) {
    const int t = eb + l;
    const bool mine = t < n && L.vals[t] >= lo && L.vals[t] <= hi;
    const int mj = mine ? (int)((uint32_t)L.ids[t] & ~OUT) : 0;
    const double me = mine ? exact_dot<E, D>(xrow, Y + (int64_t)mj * D) : 0.0;
    int rank = 0;
    for (int ub = 0; ub < n; ub += WAVE) {
      const int u = ub + l;
      const bool inb = u < n && L.vals[u] >= lo && L.vals[u] <= hi;
      const int uj = inb ? (int)((uint32_t)L.ids[u] & ~OUT) : 0;
      const double ue = inb ? exact_dot<E, D>(xrow, Y + (int64_t)uj * D) : 0.0;
      uint64_t m = ballot(inb);
      ndot += (uint32_t)popc(m);
      while (m) {   // uniform loop over the batch's band entries
        const int q = __builtin_ctzll(m);
        m &= m - 1;
        const double eu = lane_val(ue, q);
        const int ju = lane_val(uj, q);
        rank += (eu > me) || (eu == me && ju < mj);
      }
    }
    const uint64_t tm = ballot(mine && rank == need - 1);
    if (tm) {
      const int tl = __builtin_ctzll(tm);
      te = __shfl(me, tl);
      tid = __shfl(mj, tl);
    }
    // marks go on the ids, so the band stays the same for the later batches
    if (mine && rank >= need) L.ids[t] = (int32_t)((uint32_t)mj | OUT);
    wave_sync();
  }
  for (int t = l; t < n; t += WAVE) {
    const uint32_t j = (uint32_t)L.ids[t];
    if (j & OUT) {
      L.ids[t] = (int32_t)(j & ~OUT);
      L.vals[t] = NEG_INF;
    }
  }
  wave_sync();
  if (l == 0) nexact += ndot;   // lane 0 keeps the wave's count
}

// Keep the k best of list[0..n) (n >= k) in (float64 logit desc, id asc) order,
// compacted to the front; returns the k-th kept element's float64 logit and id.
// The float32 k-th value a_k decides every entry more than 2*beta away from it;
// the entries within 2*beta of a_k are ranked on float64 values (coordinate-order
// scalar products), so the kept set is the one float64 values define.
template <class E, int D>
__device__ void reduce_to_k(const MergeLds& L, int n, int k, float beta, const E* xrow, const E* Y, double& te,
                            int& tid, uint32_t& nexact, uint32_t* counters) {
  (void)counters;
  const int l = lane_id();
  const float ak = wave_kth_largest(L.vals, n, k, L.khist, L.cv);
  const float lo = f_down((double)ak - 2.0 * (double)beta);
  const float hi = f_up((double)ak + 2.0 * (double)beta);
  int nabove = 0, na = 0;
  for (int base = 0; base < n; base += WAVE) {
    const int t = base + l;
    const float v = t < n ? L.vals[t] : NEG_INF;
    nabove += popc(ballot(t < n && v > hi));
    const bool nr = t < n && v >= lo && v <= hi;
    const uint64_t mk = ballot(nr);
    if (nr) {
      const int dst = na + popc(mk & lanemask_lt());
      if (dst < MG_NEAR) L.ci[dst] = t;
    }
    na += popc(mk);
  }
  const int need = k - nabove;   // near-ties kept (>= 1)
  te = 0.0;
  tid = 0;
  wave_sync();
  if (na > MG_NEAR) {
    rank_band_wide<E, D>(L, n, need, lo, hi, xrow, Y, te, tid, nexact);
  } else {
    for (int e = l; e < na; e += WAVE) L.ce[e] = exact_dot<E, D>(xrow, Y + (int64_t)L.ids[L.ci[e]] * D);
    if (l == 0) nexact += (uint32_t)na;
    wave_sync();
    for (int a0 = 0; a0 < na; a0 += WAVE) {
      const int e = a0 + l;
      int rank = 0;
      double me = 0.0;
      int mj = 0;
      if (e < na) {
        me = L.ce[e];
        mj = L.ids[L.ci[e]];
        for (int u = 0; u < na; ++u) {
          const double eu = L.ce[u];
          const int ju = L.ids[L.ci[u]];
          rank += (eu > me) || (eu == me && ju < mj);
        }
      }
      const uint64_t tm = ballot(e < na && rank == need - 1);
      if (tm) {
        const int tl = __builtin_ctzll(tm);
        te = __shfl(me, tl);
        tid = __shfl(mj, tl);
      }
      wave_sync();
      if (e < na && rank >= need) L.vals[L.ci[e]] = NEG_INF;   // ranked out
    }
  }
  wave_sync();
  // compact the kept entries (value >= lo after the ranked-out near-ties were dropped)
  int kept = 0;
  for (int base = 0; base < n; base += WAVE) {
    const int t = base + l;
    const float v = t < n ? L.vals[t] : NEG_INF;
    const int j = t < n ? L.ids[t] : -1;
    const bool keep = t < n && v >= lo && v != NEG_INF;
    const uint64_t mk = ballot(keep);
    wave_sync();
    if (keep) {
      const int dst = kept + popc(mk & lanemask_lt());   // dst <= t: in-place is safe chunk by chunk
      L.vals[dst] = v;
      L.ids[dst] = j;
    }
    kept += popc(mk);
    wave_sync();
  }
}

}  // namespace rece
