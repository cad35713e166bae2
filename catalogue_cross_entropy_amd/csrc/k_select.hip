// In-chunk logits and per-position top-k negatives (RECE page, Section 3,
// Algorithm 1: the chunk, window and "logits for wrong classes" lines, repeated
// over rounds; the top-k keeps the largest logits, which Section 3 argues carry
// the largest gradients).
//
// Grid: one workgroup per (X-chunk c, tile of 16*NW sorted positions).  Each
// wave owns 16 positions and keeps their fragments in registers.  The window
// (item chunks c, c-1, c+1 of the round's sorted order, cyclic) streams through
// LDS 64 items at a time; a 16x64 logit block per wave comes from the matrix
// cores and never leaves the chip.
//
// Selection per position: a logit enters the position's LDS candidate list when
// it exceeds the list's filter.  When a list nears its capacity, the wave finds
// its exact k-th largest value tau and keeps only entries >= tau - 2*beta, where
// beta bounds |float32 logit - float64 logit|; the k-th largest only grows, so
// every candidate that can still be among the float64 top-k stays.
// At the end the float32 k-th value a_k splits the list: entries above a_k + 2*beta
// are kept, entries below a_k - 2*beta dropped, and the few in between are
// recomputed in float64 and ranked (logit desc, id asc).  The k-th kept element
// (float64 logit, id) is the position's threshold: membership of any later pair
// is decided against it the same way, so no list of kept pairs is stored.
//
// Rounds: a pair already kept in an earlier round is skipped (the page's
// minus-ln(count) rule makes the multiset of copies a set).  The outputs per
// position are the threshold and the sum of exp(logit - shift) over the new pairs.
#include "rece_device.h"
#include "rece_internal.h"

namespace rece {

constexpr int NBINS = 256;

// Histogram bin of v in [lo, hi] with 256/(hi-lo) = scale; clamped (scale may be inf).
__device__ __forceinline__ int bin_of(float v, float lo, float scale) {
  const float x = fminf(fmaxf((v - lo) * scale, 0.0f), (float)(NBINS - 1));
  return (int)x;
}

struct WaveLds {
  float* vals;      // [16][cap]
  int32_t* ids;     // [16][cap]
  uint32_t* hist;   // [NBINS]
  float* cv;        // [ALIST]
  int32_t* ci;      // [ALIST] (buffer index)
  int32_t* cj;      // [ALIST] (item id)
  double* ce;       // [ALIST]
  int32_t* rint;    // [16 * 4]: i, pos, cnt, (spare)
  float* rflt;      // [16 * 2]: beta, thr
};

__host__ __device__ inline size_t wave_lds_bytes(int cap) {
  return (size_t)16 * cap * 8 + NBINS * 4 + ALIST * (4 + 4 + 4 + 8) + 16 * 4 * 4 + 16 * 2 * 4;
}

__device__ inline WaveLds carve(char* base, int cap) {
  WaveLds L;
  char* p = base;
  L.ce = reinterpret_cast<double*>(p);
  p += ALIST * 8;
  L.vals = reinterpret_cast<float*>(p);
  p += (size_t)16 * cap * 4;
  L.ids = reinterpret_cast<int32_t*>(p);
  p += (size_t)16 * cap * 4;
  L.hist = reinterpret_cast<uint32_t*>(p);
  p += NBINS * 4;
  L.cv = reinterpret_cast<float*>(p);
  p += ALIST * 4;
  L.ci = reinterpret_cast<int32_t*>(p);
  p += ALIST * 4;
  L.cj = reinterpret_cast<int32_t*>(p);
  p += ALIST * 4;
  L.rint = reinterpret_cast<int32_t*>(p);
  p += 16 * 4 * 4;
  L.rflt = reinterpret_cast<float*>(p);
  return L;
}

// Exact k-th largest (1-based) of vals[0..n), 1 <= k <= n.  Histogram refinement:
// 256 linear bins over the live value range, keep the bin holding the k-th value,
// repeat; a final list of at most ALIST values is ranked directly.
__device__ float wave_kth_largest(const float* vals, int n, int k, uint32_t* hist, float* cand) {
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
  for (int iter = 0; iter < 8; ++iter) {
    if (!(hi > lo)) return hi;
    const float scale = (float)NBINS / (hi - lo);
    for (int b = l; b < NBINS; b += WAVE) hist[b] = 0u;
    wave_sync();
    for (int t = l; t < n; t += WAVE) {
      const float v = vals[t];
      if (v >= lo && v <= hi) {
        atomicAdd(&hist[bin_of(v, lo, scale)], 1u);
      }
    }
    wave_sync();
    // lane l owns bins 4l..4l+3; suffix counts from the top
    uint32_t h[4];
    uint32_t own = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      h[q] = hist[4 * l + q];
      own += h[q];
    }
    uint32_t suf = own;   // inclusive suffix over lanes >= l
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_down(suf, o);
      if (l + o < 64) suf += y;
    }
    const uint32_t above_lane = suf - own;   // bins of lanes > l
    // the k-th largest lies in the highest bin b with count(bins >= b) >= kk
    int myb = -1;
    uint32_t my_above = 0;
    {
      uint32_t acc = above_lane;
#pragma unroll
      for (int q = 3; q >= 0; --q) {
        if (myb < 0 && acc + h[q] >= (uint32_t)kk) {
          myb = 4 * l + q;
          my_above = acc;
        }
        acc += h[q];
      }
    }
    // highest lane with a hit has the highest bin
    const uint64_t hit = ballot(myb >= 0);
    const int src = 63 - __builtin_clzll(hit);
    const int bstar = __shfl(myb, src);
    const int above = (int)__shfl(my_above, src);
    kk -= above;
    // range of the values in bin bstar
    float nlo = __builtin_huge_valf(), nhi = -__builtin_huge_valf();
    int m = 0;
    for (int t = l; t < n; t += WAVE) {
      const float v = vals[t];
      if (v >= lo && v <= hi && bin_of(v, lo, scale) == bstar) {
        nlo = fminf(nlo, v);
        nhi = fmaxf(nhi, v);
        ++m;
      }
    }
    nlo = wave_min(nlo);
    nhi = wave_max(nhi);
    m = wave_sum(m);
    lo = nlo;
    hi = nhi;
    if (m <= ALIST || !(hi > lo)) break;
  }
  if (!(hi > lo)) return hi;
  // rank the values in [lo, hi]: the answer v has #(>v) < kk <= #(>=v)
  float result = lo;
  int found = 0;
  for (int base = 0; base < n && !found; base += WAVE) {
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
      found = 1;
    }
  }
  (void)cand;
  return result;
}

// Keep entries >= thr of one candidate list, in order.  Returns the new count.
__device__ int compact_list(float* vals, int32_t* ids, int n, float thr) {
  const int l = lane_id();
  int out = 0;
  for (int base = 0; base < n; base += WAVE) {
    const int t = base + l;
    float v = 0.0f;
    int32_t id = 0;
    bool keep = false;
    if (t < n) {
      v = vals[t];
      id = ids[t];
      keep = v >= thr;
    }
    wave_sync();
    const uint64_t m = ballot(keep);
    if (keep) {
      const int dst = out + popc(m & lanemask_lt());
      vals[dst] = v;
      ids[dst] = id;
    }
    out += popc(m);
    wave_sync();
  }
  return out;
}

// Membership of pair (i, j) with float32 logit a in a round's kept set, given that
// round's threshold (float64 logit te, id tid) and its float32 outward bounds.
template <class E, int D>
__device__ __forceinline__ bool beats(float a, float lo, float hi, double te, int tid, const E* xrow,
                                      const E* Y, int j, uint32_t* counters) {
  if (a > hi) return true;
  if (a < lo) return false;
  const double e = exact_dot(xrow, Y + (int64_t)j * D, D);
  atomicAdd(counters + CNT_LOGIT_EXACT, 1u);
  return e > te || (e == te && j <= tid);
}

template <class E, int D, int NW>
__global__ __launch_bounds__(64 * NW) void k_select(SelectArgs p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int P = Pitch<E, D>::value;
  constexpr int TR = 16 * NW;
  const E* __restrict__ X = reinterpret_cast<const E*>(p.X);
  const E* __restrict__ Y = reinterpret_cast<const E*>(p.Y);
  E* ytile = reinterpret_cast<E*>(smem);
  int32_t* yid = reinterpret_cast<int32_t*>(smem + 64 * P * sizeof(E));
  const int w = threadIdx.x >> 6, l = lane_id(), g = l >> 4;
  WaveLds L = carve(smem + 64 * P * sizeof(E) + 64 * 4 + (size_t)w * wave_lds_bytes(p.cap), p.cap);
  const int cap = p.cap, k = p.k, n_c = p.n_c;

  const int c = blockIdx.x / p.tiles_per_chunk;
  const int tile = blockIdx.x % p.tiles_per_chunk;
  const int64_t x0 = chunk_start(c, p.s, n_c), x1 = chunk_start(c + 1, p.s, n_c);
  const int64_t tile0 = x0 + (int64_t)tile * TR;
  if (tile0 >= x1) return;   // whole workgroup leaves together
  const int64_t wrow0 = tile0 + 16 * w;

  // window chunks: own chunk first, then its neighbours (distinct, cyclic)
  int wc[3];
  int nwc = 0;
  wc[nwc++] = c;
  if (n_c >= 2) wc[nwc++] = (c + n_c - 1) % n_c;
  if (n_c >= 3) wc[nwc++] = (c + 1) % n_c;
  int64_t W = 0;
  for (int q = 0; q < nwc; ++q) W += chunk_start(wc[q] + 1, p.C, n_c) - chunk_start(wc[q], p.C, n_c);

  // fragments of this wave's 16 positions
  const int64_t pA = wrow0 + (l & 15);
  const int iA = pA < x1 ? p.perm_x[pA] : -1;
  Frag<E, D> afr;
  afr.load_global(iA >= 0 ? X + (int64_t)iA * D : nullptr);

  const float ymax = p.ynorm_max[0];
  // per-lane state of the output rows r = 4g + v
  int pos_v[4], cnt_v[4];
  float thr_v[4], beta_v[4];
  bool rv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t pr = wrow0 + 4 * g + v;
    rv[v] = pr < x1;
    const int i = rv[v] ? p.perm_x[pr] : 0;
    pos_v[v] = rv[v] ? p.pos[i] : -1;
    beta_v[v] = rv[v] ? p.beta_coef * p.xnorm[i] * ymax : 0.0f;
    cnt_v[v] = 0;
    thr_v[v] = NEG_INF;
    if ((l & 15) == 0) {
      L.rint[(4 * g + v) * 4 + 0] = rv[v] ? i : -1;
      L.rint[(4 * g + v) * 4 + 1] = pos_v[v];
      L.rflt[(4 * g + v) * 2 + 0] = beta_v[v];
    }
  }

  // select-all mode: every candidate of every window is kept (k >= window size)
  float om_v[4], os_v[4];
  int oc_v[4], oi_v[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    om_v[v] = NEG_INF;
    os_v[v] = 0.0f;
    oc_v[v] = 0;
    oi_v[v] = rv[v] ? p.perm_x[wrow0 + 4 * g + v] : 0;
  }

  if (k > 0) {
    for (int q = 0; q < nwc; ++q) {
      const int64_t y0 = chunk_start(wc[q], p.C, n_c), y1 = chunk_start(wc[q] + 1, p.C, n_c);
      for (int64_t q0 = y0; q0 < y1; q0 += 64) {
        __syncthreads();
        if (threadIdx.x < 64) yid[threadIdx.x] = q0 + threadIdx.x < y1 ? p.perm_y[q0 + threadIdx.x] : -1;
        __syncthreads();
        {
          constexpr int EPP = 16 / (int)sizeof(E);
          constexpr int PIECES = D / EPP;
          for (int pc = threadIdx.x; pc < 64 * PIECES; pc += 64 * NW) {
            const int nb = pc / PIECES, part = pc % PIECES;
            const int j = yid[nb];
            u32x4 val = {0u, 0u, 0u, 0u};
            if (j >= 0) val = *reinterpret_cast<const u32x4*>(Y + (int64_t)j * D + part * EPP);
            *reinterpret_cast<u32x4*>(ytile + nb * P + part * EPP) = val;
          }
        }
        __syncthreads();
        f32x4 acc[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          Frag<E, D> bf;
          bf.load_lds(ytile + (cb * 16 + (l & 15)) * P);
          acc[cb] = mma_block(afr, bf, f32x4{0.f, 0.f, 0.f, 0.f});
        }
        if (p.selall) {
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const int j = yid[cb * 16 + (l & 15)];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float a = acc[cb][v];
              const bool cand = rv[v] && j >= 0 && j != pos_v[v];
              if (p.negs) {
                const uint64_t m = ballot(cand);
                const uint32_t gm = (uint32_t)(m >> (16 * g)) & 0xFFFFu;
                if (cand) {
                  const int slot = cnt_v[v] + __popc(gm & ((1u << (l & 15)) - 1u));
                  if (slot < k) p.negs[((int64_t)p.rho * p.s + oi_v[v]) * k + slot] = j;
                }
                cnt_v[v] += __popc(gm);
              }
              bool dup = false;
              if (cand) {
                const E* xrow = X + (int64_t)oi_v[v] * D;
                for (int r2 = 0; r2 < p.rho && !dup; ++r2) {
                  const int64_t o2 = (int64_t)r2 * p.s + oi_v[v];
                  const int cx2 = chunk_of(p.inv_x[o2], p.s, n_c);
                  const int cy2 = chunk_of(p.inv_y[(int64_t)r2 * p.C + j], p.C, n_c);
                  if (!in_window(cx2, cy2, n_c)) continue;
                  dup = beats<E, D>(a, p.thr_lo[o2], p.thr_hi[o2], p.thr_e[o2], p.thr_id[o2], xrow, Y, j,
                                    p.counters);
                }
              }
              if (cand && !dup) {
                const float mn = fmaxf(om_v[v], a);
                os_v[v] = os_v[v] * expf(om_v[v] - mn) + expf(a - mn);
                om_v[v] = mn;
                oc_v[v] += 1;
              }
            }
          }
          continue;
        }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int j = yid[cb * 16 + (l & 15)];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float a = acc[cb][v];
            const bool pass = rv[v] && j >= 0 && j != pos_v[v] && a > thr_v[v];
            const uint64_t m = ballot(pass);
            const uint32_t gm = (uint32_t)(m >> (16 * g)) & 0xFFFFu;
            if (pass) {
              const int slot = cnt_v[v] + __popc(gm & ((1u << (l & 15)) - 1u));
              if (slot < cap) {
                const int r = 4 * g + v;
                L.vals[r * cap + slot] = a;
                L.ids[r * cap + slot] = j;
              }
            }
            cnt_v[v] += __popc(gm);
          }
        }
        wave_sync();
        // compact lists that could overflow on the next tile
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          uint64_t need = ballot(cnt_v[v] > cap - 64) & 0x0001000100010001ull;
          while (need) {
            const int bit = __builtin_ctzll(need);
            need &= need - 1;
            const int gg = bit >> 4;
            const int r = 4 * gg + v;
            const int n = min(__shfl(cnt_v[v], 16 * gg), cap);
            const float beta = __shfl(beta_v[v], 16 * gg);
            const float kth = wave_kth_largest(L.vals + r * cap, n, k, L.hist, L.cv);
            const float thr = f_down((double)kth - 2.0 * (double)beta);
            int nn = compact_list(L.vals + r * cap, L.ids + r * cap, n, thr);
            if (nn > cap - 64) {
              if (l == 0) {
                atomicAdd(p.counters + CNT_OVERFLOW, 1u);
                atomicOr(p.counters + CNT_ERROR, (uint32_t)ERRBIT_OVERFLOW);
              }
              nn = cap - 64;
            }
            if (g == gg) {
              cnt_v[v] = nn;
              thr_v[v] = thr;
            }
          }
        }
      }
    }
  }

  if (p.selall) {
    // combine the online (max, sum, count) of the 16 lanes of each row and write
#pragma unroll
    for (int v = 0; v < 4; ++v) {
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const float m2 = __shfl_xor(om_v[v], off);
        const float s2 = __shfl_xor(os_v[v], off);
        const int c2 = __shfl_xor(oc_v[v], off);
        const float mn = fmaxf(om_v[v], m2);
        const float a1 = om_v[v] == NEG_INF ? 0.0f : os_v[v] * expf(om_v[v] - mn);
        const float a2 = m2 == NEG_INF ? 0.0f : s2 * expf(m2 - mn);
        os_v[v] = a1 + a2;
        om_v[v] = mn;
        oc_v[v] += c2;
      }
      if ((l & 15) == 0 && rv[v]) {
        const int64_t o = (int64_t)p.rho * p.s + oi_v[v];
        p.thr_e[o] = -__builtin_huge_val();
        p.thr_id[o] = -1;
        p.thr_lo[o] = NEG_INF;
        p.thr_hi[o] = NEG_INF;
        p.mshift[o] = om_v[v];
        p.ssum[o] = os_v[v];
        p.nmem[o] = oc_v[v];
        if (p.negs)
          for (int t = cnt_v[v]; t < k; ++t) p.negs[o * k + t] = -1;
      }
    }
    return;
  }

  // publish list counts for the per-row epilogue
#pragma unroll
  for (int v = 0; v < 4; ++v)
    if ((l & 15) == 0) L.rint[(4 * g + v) * 4 + 2] = min(cnt_v[v], cap);
  wave_sync();

  // ---------------------------------------------------------------- epilogue
  const int rho = p.rho;
  const int64_t s = p.s;
  for (int r = 0; r < 16; ++r) {
    const int i = L.rint[r * 4 + 0];
    if (i < 0) continue;
    const int posi = L.rint[r * 4 + 1];
    const int n = L.rint[r * 4 + 2];
    const float beta = L.rflt[r * 2 + 0];
    float* vals = L.vals + r * cap;
    int32_t* ids = L.ids + r * cap;
    const E* xrow = X + (int64_t)i * D;
    const int64_t o = (int64_t)rho * s + i;

    const bool pos_in_win = posi >= 0 && posi < p.C &&
                            in_window(c, chunk_of(p.inv_y[(int64_t)rho * p.C + posi], p.C, n_c), n_c);
    const int64_t ncand = W - (pos_in_win ? 1 : 0);

    double te;
    int tid;
    float tlo, thi;
    if (k == 0) {
      te = __builtin_huge_val();
      tid = -2;
      tlo = thi = __builtin_huge_valf();
    } else if (ncand <= k) {
      te = -__builtin_huge_val();
      tid = -1;
      tlo = thi = NEG_INF;
    } else {
      const float ak = wave_kth_largest(vals, n, k, L.hist, L.cv);
      const float lo = f_down((double)ak - 2.0 * (double)beta);
      const float hi = f_up((double)ak + 2.0 * (double)beta);
      // entries above hi are kept for sure; collect the near-tie set [lo, hi]
      int nabove = 0, na = 0;
      for (int base = 0; base < n; base += WAVE) {
        const int t = base + l;
        const float v = t < n ? vals[t] : NEG_INF;
        nabove += (t < n && v > hi);
        const bool inA = t < n && v >= lo && v <= hi;
        const uint64_t m = ballot(inA);
        if (inA) {
          const int dst = na + popc(m & lanemask_lt());
          if (dst < ALIST) {
            L.ci[dst] = t;
            L.cj[dst] = ids[t];
          }
        }
        na += popc(m);
      }
      nabove = wave_sum(nabove);
      if (na > ALIST) {   // more near-ties than the list holds: flag (never seen on continuous data)
        if (l == 0) {
          atomicAdd(p.counters + CNT_OVERFLOW, 1u);
          atomicOr(p.counters + CNT_ERROR, (uint32_t)ERRBIT_OVERFLOW);
        }
        na = ALIST;
      }
      wave_sync();
      if (l < na) {
        L.ce[l] = exact_dot(xrow, Y + (int64_t)L.cj[l] * D, D);
      }
      wave_sync();
      const int need = k - nabove;   // how many of the near-tie set are kept (>= 1)
      int rank = 0;
      double me = 0.0;
      int mj = 0;
      if (l < na) {
        me = L.ce[l];
        mj = L.cj[l];
        for (int u = 0; u < na; ++u) {
          const double eu = L.ce[u];
          const int ju = L.cj[u];
          rank += (eu > me) || (eu == me && ju < mj);
        }
      }
      const uint64_t tm = ballot(l < na && rank == need - 1);
      const int tl = tm ? __builtin_ctzll(tm) : 0;
      te = __shfl(me, tl);
      tid = __shfl(mj, tl);
      // drop the near-ties that rank below the threshold
      if (l < na && rank >= need) vals[L.ci[l]] = NEG_INF;
      wave_sync();
      if (l == 0) {
        atomicAdd(p.counters + CNT_LOGIT_EXACT, (uint32_t)na);
        if (na > 1) atomicAdd(p.counters + CNT_TOPK_EXACT, 1u);
      }
      const double b2 = (double)beta * (1.0 + 1e-6);
      tlo = f_down(te - b2);
      thi = f_up(te + b2);
      // keep exactly the members: above hi, or near-ties that ranked in
      const float lim = lo;
      int nn = 0;
      for (int base = 0; base < n; base += WAVE) {
        const int t = base + l;
        float v = 0.f;
        int32_t id = 0;
        bool keep = false;
        if (t < n) {
          v = vals[t];
          id = ids[t];
          keep = v >= lim;
        }
        wave_sync();
        const uint64_t m = ballot(keep);
        if (keep) {
          const int dst = nn + popc(m & lanemask_lt());
          vals[dst] = v;
          ids[dst] = id;
        }
        nn += popc(m);
        wave_sync();
      }
      (void)nn;
    }
    // member count after the pass above
    int nm;
    if (k == 0) {
      nm = 0;
    } else if (ncand <= k) {
      nm = n;
    } else {
      nm = k;
    }
    // skip pairs kept in earlier rounds; sum exp over the new ones
    float mx = NEG_INF;
    for (int t = l; t < nm; t += WAVE) mx = fmaxf(mx, vals[t]);
    mx = wave_max(mx);
    float se = 0.0f;
    int cntnew = 0;
    for (int t = l; t < nm; t += WAVE) {
      const float a = vals[t];
      const int j = ids[t];
      bool dup = false;
      for (int r2 = 0; r2 < rho && !dup; ++r2) {
        const int64_t o2 = (int64_t)r2 * s + i;
        const int cx2 = chunk_of(p.inv_x[o2], s, n_c);
        const int cy2 = chunk_of(p.inv_y[(int64_t)r2 * p.C + j], p.C, n_c);
        if (!in_window(cx2, cy2, n_c)) continue;
        dup = beats<E, D>(a, p.thr_lo[o2], p.thr_hi[o2], p.thr_e[o2], p.thr_id[o2], xrow, Y, j, p.counters);
      }
      if (!dup) {
        se += expf(a - mx);
        ++cntnew;
      }
      if (p.negs) p.negs[o * k + t] = j;
    }
    if (p.negs)
      for (int t = nm + l; t < k; t += WAVE) p.negs[o * k + t] = -1;
    se = wave_sumf(se);
    cntnew = wave_sum(cntnew);
    if (l == 0) {
      p.thr_e[o] = te;
      p.thr_id[o] = tid;
      p.thr_lo[o] = tlo;
      p.thr_hi[o] = thi;
      p.mshift[o] = mx;
      p.ssum[o] = se;
      p.nmem[o] = cntnew;
    }
    wave_sync();
  }
}

size_t select_lds_bytes(bool bf16v, int d, int waves, int cap) {
  const size_t esz = bf16v ? 2 : 4;
  const size_t pitch = bf16v ? d + 8 : d + 4;
  return 64 * pitch * esz + 64 * 4 + (size_t)waves * wave_lds_bytes(cap);
}

template <class E, int D, int NW>
static hipError_t launch_sel(const SelectArgs& a, hipStream_t st) {
  const size_t lds = select_lds_bytes(sizeof(E) == 2, D, NW, a.cap);
  auto kern = k_select<E, D, NW>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const unsigned blocks = (unsigned)((int64_t)a.n_c * a.tiles_per_chunk);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * NW), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_select(bool bf16v, int d, int waves, const SelectArgs& a, hipStream_t st) {
#define RECE_SEL(E, DD, NW) \
  if (d == DD && waves == NW) return launch_sel<E, DD, NW>(a, st);
#define RECE_SEL_D(E, DD) RECE_SEL(E, DD, 1) RECE_SEL(E, DD, 2) RECE_SEL(E, DD, 4)
  if (bf16v) {
    RECE_SEL_D(bf16, 32) RECE_SEL_D(bf16, 64) RECE_SEL_D(bf16, 128) RECE_SEL_D(bf16, 256)
  } else {
    RECE_SEL_D(float, 32) RECE_SEL_D(float, 64) RECE_SEL_D(float, 128) RECE_SEL_D(float, 256)
  }
#undef RECE_SEL_D
#undef RECE_SEL
  return hipErrorInvalidValue;
}

}  // namespace rece
