// In-chunk logits and per-position top-k negatives (RECE page, Section 3,
// Algorithm 1: the chunk, window and "logits for wrong classes" lines, repeated
// over rounds; the top-k keeps the largest logits, which Section 3 argues carry
// the largest gradients).
//
// Grid: one workgroup per (X-chunk c, tile of 16*NW sorted positions).  Each wave
// owns 16 positions and keeps their fragments in registers.  The window (item
// chunks c, c-1, c+1 of the round's sorted order, cyclic) streams through LDS 64
// items at a time, double-buffered and prefetched one tile ahead; the 16x64 logit
// block of a wave comes from the matrix cores and never leaves the chip.
//
// Selection, two passes over the window per position:
//   pass 1: a 256-bin histogram of the float32 logits over [-b_i, b_i]
//           (b_i >= every |logit| of the row) locates the bin of the k-th largest;
//           a bin too full for the candidate list is split by further passes;
//   pass 2: the logits are recomputed; a logit above the bin (plus 2*beta, beta
//           bounding |float32 - float64 logit|) is kept for sure and summed on the
//           fly; logits within the bin +- 2*beta go to an LDS candidate list.
// The list then gives the float32 k-th value a_k; the few entries within 2*beta of
// a_k are recomputed in float64 and ranked (logit desc, id asc).  The k-th kept
// element (float64 logit, id) is the position's threshold: membership of any
// later pair is decided against it, so no list of kept pairs is stored.
//
// Rounds: a pair already kept in an earlier round is skipped (the page's
// minus-ln(count) rule makes the multiset of copies a set).  Outputs per position
// and round: the threshold and the sum of exp(logit - shift) over the new pairs.
#include "rece_device.h"
#include "rece_internal.h"

namespace rece {

constexpr int NBINS = 256;
constexpr int SEL_CAP = 128;     // candidate-list capacity per position
constexpr int SEL_SLACK = 32;    // room kept for entries within 2*beta outside the k-th bin
constexpr int MAX_REFINE = 3;    // histogram passes that may split a crowded bin

__device__ __forceinline__ int bin_of(float v, float lo, float scale) {
  const float x = fminf(fmaxf((v - lo) * scale, 0.0f), (float)(NBINS - 1));
  return (int)x;
}

// Exact k-th largest (1-based) of vals[0..n), 1 <= k <= n.  Histogram refinement
// until at most 64 values remain in range, then one value per lane, ranked by
// broadcasting each lane's value in turn.
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
    const float scale = (float)NBINS / (hi - lo);
    for (int b = l; b < NBINS; b += WAVE) hist[b] = 0u;
    wave_sync();
    for (int t = l; t < n; t += WAVE) {
      const float v = vals[t];
      if (v >= lo && v <= hi) atomicAdd(&hist[bin_of(v, lo, scale)], 1u);
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
      if (v >= lo && v <= hi && bin_of(v, lo, scale) == bstar) {
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

// Per-wave LDS region.
struct WaveLds {
  PrevRow* prev;    // [16][MAX_ROUNDS]
  double* ce;       // [ALIST]
  uint32_t* hist;   // [16][NBINS] (histogram passes), aliased by vals/ids (collect pass)
  float* vals;      // [16][SEL_CAP]
  int32_t* ids;     // [16][SEL_CAP]
  uint32_t* khist;  // [NBINS] scratch of wave_kth_largest
  float* cv;        // [ALIST]
  int32_t* ci;      // [ALIST]
  int32_t* cj;      // [ALIST]
  float* rf;        // [16][8] per-row floats
  int32_t* ri;      // [16][4] per-row ints
};
constexpr size_t WAVE_UNION = (size_t)16 * NBINS * 4 > (size_t)16 * SEL_CAP * 8 ? (size_t)16 * NBINS * 4
                                                                                    : (size_t)16 * SEL_CAP * 8;
constexpr size_t WAVE_LDS = 16 * MAX_ROUNDS * sizeof(PrevRow) + ALIST * 8 + WAVE_UNION + NBINS * 4 +
                            ALIST * (4 + 4 + 4) + 16 * 8 * 4 + 16 * 4 * 4;

__device__ inline WaveLds carve(char* base) {
  WaveLds L;
  char* p = base;
  L.prev = reinterpret_cast<PrevRow*>(p);
  p += 16 * MAX_ROUNDS * sizeof(PrevRow);
  L.ce = reinterpret_cast<double*>(p);
  p += ALIST * 8;
  L.hist = reinterpret_cast<uint32_t*>(p);
  L.vals = reinterpret_cast<float*>(p);
  L.ids = reinterpret_cast<int32_t*>(p + 16 * SEL_CAP * 4);
  p += WAVE_UNION;
  L.khist = reinterpret_cast<uint32_t*>(p);
  p += NBINS * 4;
  L.cv = reinterpret_cast<float*>(p);
  p += ALIST * 4;
  L.ci = reinterpret_cast<int32_t*>(p);
  p += ALIST * 4;
  L.cj = reinterpret_cast<int32_t*>(p);
  p += ALIST * 4;
  L.rf = reinterpret_cast<float*>(p);
  p += 16 * 8 * 4;
  L.ri = reinterpret_cast<int32_t*>(p);
  return L;
}

enum { RF_BETA = 0, RF_MX = 1, RF_SEXP = 2, RF_THI = 3, RF_NBUF = 4 };
enum { RI_I = 0, RI_POS = 1, RI_NSURE = 2, RI_NNEW = 3 };

__host__ __device__ constexpr size_t sel_common_lds(size_t pitch, size_t esz) {
  return 2 * 64 * pitch * esz + 3 * 64 * 4 + 2 * (size_t)MAX_ROUNDS * 64 * 4 + 16;
}

template <class E, int D, int NW>
__global__ __launch_bounds__(64 * NW) void k_select(SelectArgs p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int P = Pitch<E, D>::value;
  constexpr int TR = 16 * NW;
  constexpr int NT = 64 * NW;                 // threads
  constexpr int EPP = 16 / (int)sizeof(E);    // elements per 16-byte piece
  constexpr int PIECES = D / EPP;             // pieces per vector
  constexpr int NPT = 64 * PIECES / NT;       // pieces per thread per tile
  static_assert(NPT * NT == 64 * PIECES, "tile pieces must split evenly over the threads");
  const E* __restrict__ X = reinterpret_cast<const E*>(p.X);
  const E* __restrict__ Y = reinterpret_cast<const E*>(p.Y);
  E* ytile0 = reinterpret_cast<E*>(smem);
  E* ytile1 = ytile0 + 64 * P;
  int32_t* yidb = reinterpret_cast<int32_t*>(ytile1 + 64 * P);       // [3][64]
  int32_t* ycyb = yidb + 3 * 64;                                      // [2][MAX_ROUNDS][64]
  int32_t* wg_flag = ycyb + 2 * MAX_ROUNDS * 64;                      // [1]
  const int w = threadIdx.x >> 6, l = lane_id(), g = l >> 4;
  WaveLds L = carve(smem + sel_common_lds(P, sizeof(E)) + (size_t)w * WAVE_LDS);
  const int k = p.k, n_c = p.n_c, rho = p.rho;
  const int64_t s = p.s, C = p.C;

  const int c = blockIdx.x / p.tiles_per_chunk;
  const int tile = blockIdx.x % p.tiles_per_chunk;
  const int64_t x0 = chunk_start(c, s, n_c), x1 = chunk_start(c + 1, s, n_c);
  const int64_t tile0 = x0 + (int64_t)tile * TR;
  if (tile0 >= x1) return;   // whole workgroup leaves together
  const int64_t wrow0 = tile0 + 16 * w;

  // window ranges (own chunk first), in tiles of 64 items
  int64_t rs[3], re[3];
  int ct[4];
  {
    int wc[3];
    int nwc = 0;
    wc[nwc++] = c;
    if (n_c >= 2) wc[nwc++] = (c + n_c - 1) % n_c;
    if (n_c >= 3) wc[nwc++] = (c + 1) % n_c;
    ct[0] = 0;
    for (int q = 0; q < 3; ++q) {
      if (q < nwc) {
        rs[q] = chunk_start(wc[q], C, n_c);
        re[q] = chunk_start(wc[q] + 1, C, n_c);
      } else {
        rs[q] = re[q] = 0;
      }
      ct[q + 1] = ct[q] + (int)((re[q] - rs[q] + 63) / 64);
    }
  }
  const int ntiles = ct[3];

  // fragments of this wave's 16 positions
  const int64_t pA = wrow0 + (l & 15);
  const int iA = pA < x1 ? p.perm_x[pA] : -1;
  Frag<E, D> afr;
  afr.load_global(iA >= 0 ? X + (int64_t)iA * D : nullptr);
  if (l < 16) {
    for (int r2 = 0; r2 < rho; ++r2) {
      PrevRow pr{0.0, 0.f, 0.f, 0, 0};
      if (iA >= 0) {
        const int64_t o2 = (int64_t)r2 * s + iA;
        pr.te = p.thr_e[o2];
        pr.lo = p.thr_lo[o2];
        pr.hi = p.thr_hi[o2];
        pr.tid = p.thr_id[o2];
        pr.cx = chunk_of(p.inv_x[o2], s, n_c);
      }
      L.prev[l * MAX_ROUNDS + r2] = pr;
    }
  }

  const float ymax = p.ynorm_max[0];
  const bool selall = p.selall != 0;
  // per-lane copies of the state of output rows r = 4g + v
  int pos_v[4], i_v[4], kk_v[4];
  bool rv[4];
  float beta_v[4], rlo_v[4], rhi_v[4], rsc_v[4], tlo_v[4], thi_v[4], mx_v[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t pr = wrow0 + 4 * g + v;
    rv[v] = pr < x1;
    i_v[v] = rv[v] ? p.perm_x[pr] : 0;
    pos_v[v] = rv[v] ? p.pos[i_v[v]] : -1;
    const float xn = rv[v] ? p.xnorm[i_v[v]] : 0.0f;
    beta_v[v] = p.beta_coef * xn * ymax;
    // every float32 logit of the row lies in [-bnd, bnd]
    const float bnd = f_up((double)xn * (double)ymax * (1.0 + 1e-5) + 2.0 * (double)beta_v[v]) + 1e-30f;
    rlo_v[v] = -bnd;
    rhi_v[v] = bnd;
    rsc_v[v] = (float)NBINS / (2.0f * bnd);
    kk_v[v] = k;
    tlo_v[v] = thi_v[v] = selall ? NEG_INF : __builtin_huge_valf();
    mx_v[v] = NEG_INF;
    if ((l & 15) == 0) {
      const int r = 4 * g + v;
      L.ri[r * 4 + RI_I] = rv[v] ? i_v[v] : -1;
      L.ri[r * 4 + RI_POS] = pos_v[v];
      L.rf[r * 8 + RF_BETA] = beta_v[v];
    }
  }

  // mode 0: histogram pass; 1: collect pass; 2: nothing to do (k = 0)
  int mode = k == 0 ? 2 : (selall ? 1 : 0);
  float sexp_v[4] = {0.f, 0.f, 0.f, 0.f};
  int nnew_v[4] = {0, 0, 0, 0}, nsure_v[4] = {0, 0, 0, 0}, bcnt_v[4] = {0, 0, 0, 0};

  auto tile_base = [&](int t, int64_t& q0, int64_t& q1) {
    int q = 0;
    while (q < 2 && t >= ct[q + 1]) ++q;
    q0 = rs[q] + (int64_t)(t - ct[q]) * 64;
    q1 = re[q];
  };
  auto load_ids = [&](int t, int slot) {
    if (threadIdx.x < 64) {
      int j = -1;
      if (t < ntiles) {
        int64_t q0, q1;
        tile_base(t, q0, q1);
        if (q0 + threadIdx.x < q1) j = p.perm_y[q0 + threadIdx.x];
      }
      yidb[slot * 64 + threadIdx.x] = j;
    }
  };
  u32x4 pf[NPT];
  int pfcy[MAX_ROUNDS];
  auto fetch_rows = [&](int slot) {
#pragma unroll
    for (int it = 0; it < NPT; ++it) {
      const int pc = threadIdx.x + NT * it;
      const int nb = pc / PIECES, part = pc % PIECES;
      const int j = yidb[slot * 64 + nb];
      pf[it] = j >= 0 ? *reinterpret_cast<const u32x4*>(Y + (int64_t)j * D + part * EPP) : u32x4{0u, 0u, 0u, 0u};
    }
    if (threadIdx.x < 64) {
      const int j = yidb[slot * 64 + threadIdx.x];
#pragma unroll
      for (int r2 = 0; r2 < MAX_ROUNDS; ++r2)
        if (r2 < rho) pfcy[r2] = j >= 0 ? chunk_of(p.inv_y[(int64_t)r2 * C + j], C, n_c) : 0;
    }
  };
  auto store_rows = [&](int buf) {
    E* yt = buf ? ytile1 : ytile0;
#pragma unroll
    for (int it = 0; it < NPT; ++it) {
      const int pc = threadIdx.x + NT * it;
      const int nb = pc / PIECES, part = pc % PIECES;
      *reinterpret_cast<u32x4*>(yt + nb * P + part * EPP) = pf[it];
    }
    if (threadIdx.x < 64) {
#pragma unroll
      for (int r2 = 0; r2 < MAX_ROUNDS; ++r2)
        if (r2 < rho) ycyb[(buf * MAX_ROUNDS + r2) * 64 + threadIdx.x] = pfcy[r2];
    }
  };

  for (int pass = 0; mode < 2; ++pass) {
    if (mode == 0)
      for (int b = l; b < 16 * NBINS; b += WAVE) L.hist[b] = 0u;
    // prologue: ids of tiles 0 and 1, rows of tile 0
    __syncthreads();
    load_ids(0, 0);
    load_ids(1, 1);
    __syncthreads();
    fetch_rows(0);
    store_rows(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
      const int buf = t & 1;
      const int idslot = t % 3;
      if (t + 1 < ntiles) fetch_rows((t + 1) % 3);   // rows of the next tile, in flight during this one
      load_ids(t + 2, (t + 2) % 3);
      const E* yt = buf ? ytile1 : ytile0;
      f32x4 acc[4];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        Frag<E, D> bf;
        bf.load_lds(yt + (cb * 16 + (l & 15)) * P);
        acc[cb] = mma_block(afr, bf, f32x4{0.f, 0.f, 0.f, 0.f});
      }
      if (mode == 0) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int j = yidb[idslot * 64 + cb * 16 + (l & 15)];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float a = acc[cb][v];
            const bool cand = rv[v] && j >= 0 && j != pos_v[v];
            if (cand) {
              mx_v[v] = fmaxf(mx_v[v], a);
              if (a >= rlo_v[v] && a <= rhi_v[v])
                atomicAdd(&L.hist[(4 * g + v) * NBINS + bin_of(a, rlo_v[v], rsc_v[v])], 1u);
            }
          }
        }
      } else {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int n = cb * 16 + (l & 15);
          const int j = yidb[idslot * 64 + n];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float a = acc[cb][v];
            const int r = 4 * g + v;
            const bool cand = rv[v] && j >= 0 && j != pos_v[v];
            const bool sure = cand && a > thi_v[v];
            if (sure) {
              bool dup = false;
              const E* xrow = X + (int64_t)i_v[v] * D;
              for (int r2 = 0; r2 < rho && !dup; ++r2) {
                const PrevRow pr = L.prev[r * MAX_ROUNDS + r2];
                if (!in_window(pr.cx, ycyb[(buf * MAX_ROUNDS + r2) * 64 + n], n_c)) continue;
                dup = beats<E, D>(a, pr.lo, pr.hi, pr.te, pr.tid, xrow, Y, j, p.counters);
              }
              if (!dup) {
                if (a > mx_v[v]) {   // only when the row max is not known in advance (select-all)
                  sexp_v[v] = mx_v[v] == NEG_INF ? 0.0f : sexp_v[v] * expf(mx_v[v] - a);
                  mx_v[v] = a;
                }
                sexp_v[v] += expf(a - mx_v[v]);
                nnew_v[v] += 1;
              }
            }
            if (p.negs) {
              const uint64_t m = ballot(sure);
              const uint32_t gm = (uint32_t)(m >> (16 * g)) & 0xFFFFu;
              if (sure) {
                const int slot = nsure_v[v] + __popc(gm & ((1u << (l & 15)) - 1u));
                if (slot < k) p.negs[((int64_t)rho * s + i_v[v]) * k + slot] = j;
              }
              nsure_v[v] += __popc(gm);
            } else {
              nsure_v[v] += sure ? 1 : 0;
            }
            const bool inb = cand && a >= tlo_v[v] && a <= thi_v[v];
            const uint64_t m2 = ballot(inb);
            const uint32_t gm2 = (uint32_t)(m2 >> (16 * g)) & 0xFFFFu;
            if (inb) {
              const int slot = bcnt_v[v] + __popc(gm2 & ((1u << (l & 15)) - 1u));
              if (slot < SEL_CAP) {
                L.vals[r * SEL_CAP + slot] = a;
                L.ids[r * SEL_CAP + slot] = j;
              }
            }
            bcnt_v[v] += __popc(gm2);
          }
        }
      }
      if (t + 1 < ntiles) store_rows(buf ^ 1);
      __syncthreads();
    }

    if (mode == 1) break;   // collected

    // ---- after a histogram pass: locate the bin of the kk-th largest of each row
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) mx_v[v] = fmaxf(mx_v[v], __shfl_xor(mx_v[v], o));
    bool more = false;
    for (int r = 0; r < 16; ++r) {
      const int gl = 16 * (r >> 2), vv = r & 3;
      int kkr = 0;
      float rlo = 0.f, rsc = 0.f, beta = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (v == vv) {
          kkr = __shfl(kk_v[v], gl);
          rlo = __shfl(rlo_v[v], gl);
          rsc = __shfl(rsc_v[v], gl);
          beta = __shfl(beta_v[v], gl);
        }
      if (kkr <= 0) continue;   // row settled in an earlier pass
      uint32_t h[4];
      uint32_t own = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        h[q] = L.hist[r * NBINS + 4 * l + q];
        own += h[q];
      }
      uint32_t suf = own;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_down(suf, o);
        if (l + o < 64) suf += y;
      }
      const uint32_t total = __shfl(suf, 0);
      int myb = -1;
      uint32_t my_above = 0, my_cnt = 0;
      {
        uint32_t acc = suf - own;
#pragma unroll
        for (int q = 3; q >= 0; --q) {
          if (myb < 0 && acc + h[q] >= (uint32_t)kkr) {
            myb = 4 * l + q;
            my_above = acc;
            my_cnt = h[q];
          }
          acc += h[q];
        }
      }
      const uint64_t hit = ballot(myb >= 0);
      float ntlo, nthi, nrlo = rlo, nrhi = rlo, nrsc = rsc;
      int nkk = 0;
      bool refine = false;
      if ((int)total < kkr || !hit) {
        // the whole window has at most k candidates (first pass only): keep them all
        ntlo = nthi = NEG_INF;
      } else {
        const int src = 63 - __builtin_clzll(hit);
        const int bstar = __shfl(myb, src);
        const int above = (int)__shfl(my_above, src);
        const int cnt = (int)__shfl(my_cnt, src);
        const float elo = rlo + (float)bstar / rsc;
        const float ehi = rlo + (float)(bstar + 1) / rsc;
        const float pad = (fabsf(elo) + fabsf(ehi)) * 1e-6f + 1e-30f;
        ntlo = f_down((double)elo - 2.0 * (double)beta - (double)pad);
        nthi = f_up((double)ehi + 2.0 * (double)beta + (double)pad);
        if (cnt > SEL_CAP - SEL_SLACK && pass < MAX_REFINE && ehi - elo > 4.0f * beta) {
          // crowded bin: split it by another histogram pass over [elo - pad, ehi + pad]
          refine = true;
          nkk = kkr - above;
          nrlo = elo - pad;
          nrhi = ehi + pad;
          nrsc = (float)NBINS / (nrhi - nrlo);
        }
      }
      if (g == (r >> 2)) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (v == vv) {
            tlo_v[v] = ntlo;
            thi_v[v] = nthi;
            kk_v[v] = refine ? nkk : 0;
            rlo_v[v] = refine ? nrlo : __builtin_huge_valf();   // settled rows count nothing more
            rhi_v[v] = refine ? nrhi : -__builtin_huge_valf();
            rsc_v[v] = nrsc;
          }
      }
      more |= refine;
    }
    if (threadIdx.x == 0) *wg_flag = 0;
    __syncthreads();
    if (l == 0 && more) atomicOr(wg_flag, 1);
    __syncthreads();
    mode = *wg_flag ? 0 : 1;
  }

  // ---- publish the per-row sums of the sure members (combine the 16 lanes of each row)
#pragma unroll
  for (int v = 0; v < 4; ++v) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const float m2 = __shfl_xor(mx_v[v], o);
      const float s2 = __shfl_xor(sexp_v[v], o);
      const float mn = fmaxf(mx_v[v], m2);
      const float a1 = mx_v[v] == NEG_INF ? 0.0f : sexp_v[v] * expf(mx_v[v] - mn);
      const float a2 = m2 == NEG_INF ? 0.0f : s2 * expf(m2 - mn);
      sexp_v[v] = a1 + a2;
      mx_v[v] = mn;
      nnew_v[v] += __shfl_xor(nnew_v[v], o);
      if (!p.negs) nsure_v[v] += __shfl_xor(nsure_v[v], o);
    }
    if ((l & 15) == 0) {
      const int r = 4 * g + v;
      L.rf[r * 8 + RF_MX] = mx_v[v];
      L.rf[r * 8 + RF_SEXP] = sexp_v[v];
      L.rf[r * 8 + RF_THI] = thi_v[v];
      L.rf[r * 8 + RF_NBUF] = __int_as_float(bcnt_v[v]);
      L.ri[r * 4 + RI_NSURE] = nsure_v[v];
      L.ri[r * 4 + RI_NNEW] = nnew_v[v];
    }
  }
  wave_sync();

  // ---------------------------------------------------------------- epilogue
  for (int r = 0; r < 16; ++r) {
    const int i = L.ri[r * 4 + RI_I];
    if (i < 0) continue;
    const float beta = L.rf[r * 8 + RF_BETA];
    const float mx = L.rf[r * 8 + RF_MX];
    float se = L.rf[r * 8 + RF_SEXP];
    int nnew = L.ri[r * 4 + RI_NNEW];
    const int nsure = L.ri[r * 4 + RI_NSURE];
    const int nb_all = __float_as_int(L.rf[r * 8 + RF_NBUF]);
    const float thi_r = L.rf[r * 8 + RF_THI];
    const E* xrow = X + (int64_t)i * D;
    const int64_t o = (int64_t)rho * s + i;
    float* vals = L.vals + r * SEL_CAP;
    int32_t* ids = L.ids + r * SEL_CAP;

    double te;
    int tid;
    float tlo, thi;
    int listed = 0;   // kept negatives written to the stage list so far
    if (k == 0) {
      te = __builtin_huge_val();
      tid = -2;
      tlo = thi = __builtin_huge_valf();
    } else if (thi_r == NEG_INF) {
      te = -__builtin_huge_val();   // every candidate kept (all summed as sure members)
      tid = -1;
      tlo = thi = NEG_INF;
      listed = nsure;
    } else {
      const int n = min(nb_all, SEL_CAP);
      const int kk = k - nsure;
      if (nb_all > SEL_CAP || kk < 1 || kk > n) {
        if (l == 0) {
          atomicAdd(p.counters + CNT_OVERFLOW, 1u);
          atomicOr(p.counters + CNT_ERROR, (uint32_t)ERRBIT_OVERFLOW);
        }
      }
      const float ak = n > 0 ? wave_kth_largest(vals, n, max(1, min(kk, n)), L.khist, L.cv) : 0.0f;
      const float lo = f_down((double)ak - 2.0 * (double)beta);
      const float hi = f_up((double)ak + 2.0 * (double)beta);
      int nabove = 0, na = 0;
      for (int base = 0; base < n; base += WAVE) {
        const int t = base + l;
        const float v = t < n ? vals[t] : NEG_INF;
        nabove += (t < n && v > hi) ? 1 : 0;
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
      if (na > ALIST) {
        if (l == 0) {
          atomicAdd(p.counters + CNT_OVERFLOW, 1u);
          atomicOr(p.counters + CNT_ERROR, (uint32_t)ERRBIT_OVERFLOW);
        }
        na = ALIST;
      }
      wave_sync();
      if (l < na) L.ce[l] = exact_dot(xrow, Y + (int64_t)L.cj[l] * D, D);
      wave_sync();
      const int need = k - nsure - nabove;   // near-ties that are kept (>= 1)
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
      if (l < na && rank >= need) vals[L.ci[l]] = NEG_INF;
      wave_sync();
      if (l == 0) {
        atomicAdd(p.counters + CNT_LOGIT_EXACT, (uint32_t)na);
        if (na > 1) atomicAdd(p.counters + CNT_TOPK_EXACT, 1u);
      }
      const double b2 = (double)beta * (1.0 + 1e-6);
      tlo = f_down(te - b2);
      thi = f_up(te + b2);
      // kept list entries: >= lo once the near-ties that ranked out are dropped
      float sl = 0.0f;
      int cl = 0, nk = 0;
      for (int base = 0; base < n; base += WAVE) {
        const int t = base + l;
        const float a = t < n ? vals[t] : NEG_INF;
        const int j = t < n ? ids[t] : -1;
        const bool kept = t < n && a >= lo;
        if (kept) {
          bool dup = false;
          for (int r2 = 0; r2 < rho && !dup; ++r2) {
            const PrevRow pr = L.prev[r * MAX_ROUNDS + r2];
            const int cy2 = chunk_of(p.inv_y[(int64_t)r2 * C + j], C, n_c);
            if (!in_window(pr.cx, cy2, n_c)) continue;
            dup = beats<E, D>(a, pr.lo, pr.hi, pr.te, pr.tid, xrow, Y, j, p.counters);
          }
          if (!dup) {
            sl += expf(a - mx);
            ++cl;
          }
        }
        if (p.negs) {
          const uint64_t km = ballot(kept);
          if (kept) {
            const int slot = nsure + nk + popc(km & lanemask_lt());
            if (slot < k) p.negs[o * k + slot] = j;
          }
          nk += popc(km);
        }
      }
      se += wave_sumf(sl);
      nnew += wave_sum(cl);
      listed = nsure + nk;
    }
    if (p.negs)
      for (int t = listed + l; t < k; t += WAVE) p.negs[o * k + t] = -1;
    if (l == 0) {
      p.thr_e[o] = te;
      p.thr_id[o] = tid;
      p.thr_lo[o] = tlo;
      p.thr_hi[o] = thi;
      p.mshift[o] = mx;
      p.ssum[o] = se;
      p.nmem[o] = nnew;
    }
    wave_sync();
  }
}

size_t select_lds_bytes(bool is_bf16, int d, int waves, int cap) {
  (void)cap;
  const size_t esz = is_bf16 ? 2 : 4;
  const size_t pitch = is_bf16 ? d + 8 : d + 4;
  return sel_common_lds(pitch, esz) + (size_t)waves * WAVE_LDS;
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

hipError_t launch_select(bool is_bf16, int d, int waves, const SelectArgs& a, hipStream_t st) {
#define RECE_SEL(E, DD, NW) \
  if (d == DD && waves == NW) return launch_sel<E, DD, NW>(a, st);
#define RECE_SEL_D(E, DD) RECE_SEL(E, DD, 1) RECE_SEL(E, DD, 2) RECE_SEL(E, DD, 4)
  if (is_bf16) {
    RECE_SEL_D(bf16, 32) RECE_SEL_D(bf16, 64) RECE_SEL_D(bf16, 128) RECE_SEL_D(bf16, 256)
  } else {
    RECE_SEL_D(float, 32) RECE_SEL_D(float, 64) RECE_SEL_D(float, 128) RECE_SEL_D(float, 256)
  }
#undef RECE_SEL_D
#undef RECE_SEL
  return hipErrorInvalidValue;
}

}  // namespace rece
