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
#include "rece_stream.h"
#include "rece_kth.h"

namespace rece {

constexpr int NBINS = 256;
constexpr int SEL_CAP = 64;      // candidate-list capacity per position
constexpr int SEL_SLACK = 16;    // room kept for entries within 2*beta outside the k-th bin
constexpr int MAX_REFINE = 2;    // histogram passes that may split a crowded bin
constexpr float X_TOP = 255.99998f;   // largest histogram coordinate (below 256)

// Per-wave LDS region.
constexpr int WLIST = 128;   // near-tie entries of one wave awaiting float64 values

struct WaveLds {
  PrevRow* prev;    // [16][rounds - 1]
  double* ce;       // [WLIST]
  uint32_t* hist;   // [16][NBINS / 2] two 16-bit counts per word (histogram passes),
                    // aliased by vals/ids (collect pass)
  float* vals;      // [16][SEL_CAP]
  int32_t* ids;     // [16][SEL_CAP]
  uint32_t* khist;  // [NBINS] scratch of wave_kth_largest
  float* cv;        // [64] scratch of wave_kth_largest
  int32_t* ci;      // [WLIST] list index in the row's candidate list
  int32_t* cj;      // [WLIST] item id
  int32_t* cr;      // [WLIST] row
  float* rf;        // [16][8] per-row floats
  int32_t* ri;      // [16][8] per-row ints
};
constexpr size_t WAVE_UNION = (size_t)16 * NBINS * 2 > (size_t)16 * SEL_CAP * 8 ? (size_t)16 * NBINS * 2
                                                                                    : (size_t)16 * SEL_CAP * 8;
// earlier-round thresholds cached per row: rounds - 1 of them (at least one slot)
__host__ __device__ constexpr int nprev_of(int rounds) { return rounds > 1 ? rounds - 1 : 1; }
__host__ __device__ constexpr size_t wave_lds_bytes(int rounds) {
  return 16 * (size_t)nprev_of(rounds) * sizeof(PrevRow) + WLIST * 8 + WAVE_UNION + NBINS * 4 + 64 * 4 +
         WLIST * (4 + 4 + 4) + 16 * 8 * 4 + 16 * 8 * 4;
}

__device__ inline WaveLds carve(char* base, int rounds) {
  WaveLds L;
  char* p = base;
  L.prev = reinterpret_cast<PrevRow*>(p);
  p += 16 * (size_t)nprev_of(rounds) * sizeof(PrevRow);
  L.ce = reinterpret_cast<double*>(p);
  p += WLIST * 8;
  L.hist = reinterpret_cast<uint32_t*>(p);
  L.vals = reinterpret_cast<float*>(p);
  L.ids = reinterpret_cast<int32_t*>(p + 16 * SEL_CAP * 4);
  p += WAVE_UNION;
  L.khist = reinterpret_cast<uint32_t*>(p);
  p += NBINS * 4;
  L.cv = reinterpret_cast<float*>(p);
  p += 64 * 4;
  L.ci = reinterpret_cast<int32_t*>(p);
  p += WLIST * 4;
  L.cj = reinterpret_cast<int32_t*>(p);
  p += WLIST * 4;
  L.cr = reinterpret_cast<int32_t*>(p);
  p += WLIST * 4;
  L.rf = reinterpret_cast<float*>(p);
  p += 16 * 8 * 4;
  L.ri = reinterpret_cast<int32_t*>(p);
  return L;
}

enum { RF_BETA = 0, RF_MX = 1, RF_SEXP = 2, RF_THI = 3, RF_NBUF = 4, RF_ALO = 5, RF_AHI = 6 };
enum { RI_I = 0, RI_POS = 1, RI_NSURE = 2, RI_NNEW = 3, RI_NABOVE = 4, RI_AOFF = 5, RI_NA = 6, RI_MODE = 7 };

// One ring slot: the tile's rows, then 64 item ids, then for each earlier round
// 64 chunk indices of those items in that round.
__host__ __device__ constexpr size_t sel_slot_bytes(size_t row_bytes, int rounds) {
  return row_bytes + 256 * (size_t)rounds;
}
__host__ __device__ constexpr size_t sel_common_lds(size_t row_bytes, int rounds) {
  return 3 * sel_slot_bytes(row_bytes, rounds) + 16;
}

template <class E, int D, int NW>
__global__ __launch_bounds__(64 * NW, (D * sizeof(E) <= 128) ? 2 : 1) void k_select(SelectArgs p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  using G = TileGeom<E, D>;
  constexpr int TI = G::TI;
  constexpr int NCB = TI / 16;                // 16-column blocks per tile
  constexpr int TR = 16 * NW;
  const E* __restrict__ X = reinterpret_cast<const E*>(p.X);
  const E* __restrict__ Y = reinterpret_cast<const E*>(p.Y);
  const E* __restrict__ Xs = reinterpret_cast<const E*>(p.Xs);
  const E* __restrict__ Ys = reinterpret_cast<const E*>(p.Ys);
  const int k = p.k, n_c = p.n_c, rho = p.rho;
  const int64_t s = p.s, C = p.C;
  const size_t slot_bytes = sel_slot_bytes(G::ROW_BYTES, p.rounds);
  char* ring = smem;
  int32_t* wg_flag = reinterpret_cast<int32_t*>(smem + 3 * slot_bytes);
  const int w = threadIdx.x >> 6, l = lane_id(), g = l >> 4;
  WaveLds L = carve(smem + sel_common_lds(G::ROW_BYTES, p.rounds) + (size_t)w * wave_lds_bytes(p.rounds),
                    p.rounds);
  const int NP = nprev_of(p.rounds);
  (void)X;
  uint32_t nexact = 0;   // float64 logits computed by this lane

  const int lb = xcd_block(blockIdx.x, gridDim.x);
  const int c = lb / p.tiles_per_chunk;
  const int tile = lb % p.tiles_per_chunk;
  const int64_t x0 = chunk_start(c, s, n_c), x1 = chunk_start(c + 1, s, n_c);
  const int64_t tile0 = x0 + (int64_t)tile * TR;
  if (tile0 >= x1) return;   // whole workgroup leaves together
  const int64_t wrow0 = tile0 + 16 * w;

  // window ranges (own chunk first), in tiles of TI items
  Ranges win;
  win.init(c, n_c, C, TI, p.nwin);
  const int ntiles = win.ntiles();

  // fragments of this wave's 16 positions (sorted copy: contiguous rows)
  const int64_t pA = wrow0 + (l & 15);
  const int iA = pA < x1 ? p.perm_x[pA] : -1;
  Frag<E, D> afr;
  afr.load_global(pA < x1 ? Xs + pA * D : nullptr);
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
      L.prev[l * NP + r2] = pr;
    }
  }

  const float ymax = p.ynorm_max[0];
  const bool selall = p.selall != 0;
  // per-lane copies of the state of output rows r = 4g + v
  int pos_v[4], i_v[4], kk_v[4];
  bool rv[4];
  // histogram coordinates: x = clamp((a - lo0) * sc0, 0, 256^-) maps the row's logits to
  // [0, 256); a pass at refinement level L counts y = (x - xa) * mul (mul = 256^L) when
  // 0 <= y < 256.  Both steps are exact in float for the values that matter, so every
  // level bins exactly the values whose x lies in the interval chosen one level up.
  float beta_v[4], lo0_v[4], sc0_v[4], xa_v[4], mul_v[4], tlo_v[4], thi_v[4], mx_v[4];
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
    lo0_v[v] = -bnd;
    sc0_v[v] = (float)NBINS / (2.0f * bnd);
    xa_v[v] = rv[v] ? 0.0f : __builtin_huge_valf();   // rows past the chunk count nothing
    mul_v[v] = 1.0f;
    kk_v[v] = rv[v] ? k : 0;
    tlo_v[v] = thi_v[v] = selall ? NEG_INF : __builtin_huge_valf();
    mx_v[v] = NEG_INF;   // row maximum (the exp shift), from the histogram pass
    if ((l & 15) == 0) {
      const int r = 4 * g + v;
      // output row: the position id, or the sorted slot when outputs are per slot
      L.ri[r * 8 + RI_I] = rv[v] ? (p.slot_out ? (int)pr : i_v[v]) : -1;
      L.ri[r * 8 + RI_POS] = pos_v[v];
      L.rf[r * 8 + RF_BETA] = beta_v[v];
    }
  }

  // mode 0: histogram pass; 1: collect pass; 2: nothing to do (k = 0)
  int mode = k == 0 ? 2 : (selall ? 1 : 0);
  float sexp_v[4] = {0.f, 0.f, 0.f, 0.f};
  int nnew_v[4] = {0, 0, 0, 0}, nsure_v[4] = {0, 0, 0, 0}, bcnt_v[4] = {0, 0, 0, 0};

  // copies of one tile: G::ROW_DMA row copies, then ids, then one chunk map per earlier round
  const int ncopies = G::ROW_DMA + 1 + rho;
  int my_copies = 0;
  for (int u = w; u < ncopies; u += NW) ++my_copies;

  for (int pass = 0; mode < 2; ++pass) {
    if (mode == 0)
      for (int b = l; b < 16 * NBINS / 2; b += WAVE) L.hist[b] = 0u;
    __syncthreads();
    issue_window_tile<E, D>(ring, slot_bytes, win, 0, Ys, p.perm_y, p.cyp, C, rho, w, NW);
    if (ntiles > 1) issue_window_tile<E, D>(ring, slot_bytes, win, 1, Ys, p.perm_y, p.cyp, C, rho, w, NW);

    for (int t = 0; t < ntiles; ++t) {
      wait_vmcnt(t + 1 < ntiles ? my_copies : 0);
      raw_barrier();
      if (t + 2 < ntiles) issue_window_tile<E, D>(ring, slot_bytes, win, t + 2, Ys, p.perm_y, p.cyp, C, rho, w, NW);
      const int64_t q0 = range_tile_start(win, t, TI), q1 = range_tile_end(win, t);
      const char* slot = ring + (size_t)(t % 3) * slot_bytes;
      const int32_t* tid_ = reinterpret_cast<const int32_t*>(slot + G::ROW_BYTES);
      const int32_t* tcy = tid_ + 64;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int n = cb * 16 + (l & 15);
        Frag<E, D> bf;
        TileFrag<E, D>::load(bf, slot, n);
        const f32x4 acc = mma_block(afr, bf, f32x4{0.f, 0.f, 0.f, 0.f});
        const bool nvalid = q0 + n < q1;
        const int j = tid_[n];
        if (mode == 0) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float a = acc[v];
            if (nvalid && j != pos_v[v]) {
              mx_v[v] = fmaxf(mx_v[v], a);
              const float x = fminf(fmaxf((a - lo0_v[v]) * sc0_v[v], 0.0f), X_TOP);
              const float y = (x - xa_v[v]) * mul_v[v];
              if (y >= 0.0f && y < (float)NBINS) {
                const int b = (int)y;
                atomicAdd(&L.hist[(4 * g + v) * (NBINS / 2) + (b >> 1)], 1u << (16 * (b & 1)));
              }
            }
          }
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float a = acc[v];
            const int r = 4 * g + v;
            const bool cand = rv[v] && nvalid && j != pos_v[v];
            const bool sure = cand && a > thi_v[v];
            if (sure) {
              bool dup = false;
              const E* xrow = Xs + (wrow0 + r) * D;
              for (int r2 = 0; r2 < rho && !dup; ++r2) {
                const PrevRow pr = L.prev[r * NP + r2];
                if (!in_window(pr.cx, tcy[64 * r2 + n], n_c)) continue;
                dup = beats<E, D>(a, pr.lo, pr.hi, pr.te, pr.tid, xrow, Y, j, nexact);
              }
              if (!dup) {
                if (selall && a > mx_v[v]) {   // no histogram pass ran: keep the shift at the maximum
                  sexp_v[v] = mx_v[v] == NEG_INF ? 0.0f : sexp_v[v] * __expf(mx_v[v] - a);
                  mx_v[v] = a;
                }
                sexp_v[v] += __expf(a - mx_v[v]);
                nnew_v[v] += 1;
              }
            }
            if (p.negs) {
              const uint64_t m = ballot(sure);
              const uint32_t gm = (uint32_t)(m >> (16 * g)) & 0xFFFFu;
              if (sure) {
                const int slotn = nsure_v[v] + __popc(gm & ((1u << (l & 15)) - 1u));
                const int64_t orow = p.slot_out ? (wrow0 + r) : (int64_t)rho * s + i_v[v];
                if (slotn < k) {
                  p.negs[orow * k + slotn] = j;
                  if (p.negl) p.negl[orow * k + slotn] = a;
                }
              }
              nsure_v[v] += __popc(gm);
            } else {
              nsure_v[v] += sure ? 1 : 0;
            }
            const bool inb = cand && a >= tlo_v[v] && a <= thi_v[v];
            const uint64_t m2 = ballot(inb);
            const uint32_t gm2 = (uint32_t)(m2 >> (16 * g)) & 0xFFFFu;
            if (inb) {
              const int slotn = bcnt_v[v] + __popc(gm2 & ((1u << (l & 15)) - 1u));
              if (slotn < SEL_CAP) {
                L.vals[r * SEL_CAP + slotn] = a;
                L.ids[r * SEL_CAP + slotn] = j;
              }
            }
            bcnt_v[v] += __popc(gm2);
          }
        }
      }
    }

    if (mode == 1) break;   // collected

    // ---- after a histogram pass: locate the bin of the kk-th largest of each row
    wave_sync();
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) mx_v[v] = fmaxf(mx_v[v], __shfl_xor(mx_v[v], o));
    bool more = false;
    for (int r = 0; r < 16; ++r) {
      const int gl = 16 * (r >> 2), vv = r & 3;
      int kkr = 0;
      float lo0 = 0.f, sc0 = 0.f, xa = 0.f, mul = 0.f, beta = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (v == vv) {
          kkr = __shfl(kk_v[v], gl);
          lo0 = __shfl(lo0_v[v], gl);
          sc0 = __shfl(sc0_v[v], gl);
          xa = __shfl(xa_v[v], gl);
          mul = __shfl(mul_v[v], gl);
          beta = __shfl(beta_v[v], gl);
        }
      if (kkr <= 0) continue;   // row settled in an earlier pass
      uint32_t h[4];
      {
        const uint32_t w0 = L.hist[r * (NBINS / 2) + 2 * l], w1 = L.hist[r * (NBINS / 2) + 2 * l + 1];
        h[0] = w0 & 0xFFFFu;
        h[1] = w0 >> 16;
        h[2] = w1 & 0xFFFFu;
        h[3] = w1 >> 16;
      }
      const uint32_t own = h[0] + h[1] + h[2] + h[3];
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
      float ntlo, nthi, nxa = xa, nmul = mul;
      int nkk = 0;
      bool refine = false;
      if ((pass == 0 && (int)total <= kkr) || !hit) {
        // the whole window has at most k candidates (first pass only): keep them all
        ntlo = nthi = NEG_INF;
      } else {
        const int src = 63 - __builtin_clzll(hit);
        const int bstar = __shfl(myb, src);
        const int above = (int)__shfl(my_above, src);
        const int cnt = (int)__shfl(my_cnt, src);
        nxa = xa + (float)bstar / mul;   // exact: a multiple of 256^-L below 256
        nmul = mul * (float)NBINS;
        // the bin is x in [nxa, nxa + 1/mul): its logit interval, padded for the rounding of x
        const double vlo = (double)lo0 + (double)nxa / (double)sc0;
        const double vhi = (double)lo0 + ((double)nxa + 1.0 / (double)mul) / (double)sc0;
        const double pad = (fabs(vlo) + fabs(vhi) + fabs((double)lo0)) * 1e-6 + 1e-30;
        ntlo = f_down(vlo - 2.0 * (double)beta - pad);
        nthi = f_up(vhi + 2.0 * (double)beta + pad);
        if (cnt > SEL_CAP - SEL_SLACK && pass < MAX_REFINE && vhi - vlo > 4.0 * (double)beta) {
          refine = true;   // crowded bin: split it by another histogram pass
          nkk = kkr - above;
        }
      }
      if (g == (r >> 2)) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (v == vv) {
            tlo_v[v] = ntlo;
            thi_v[v] = nthi;
            kk_v[v] = refine ? nkk : 0;
            xa_v[v] = refine ? nxa : __builtin_huge_valf();   // settled rows count nothing more
            mul_v[v] = refine ? nmul : 1.0f;
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
      if (selall) {   // lanes saw different maxima: rescale before adding
        const float mn = fmaxf(mx_v[v], m2);
        const float a1 = mx_v[v] == NEG_INF ? 0.0f : sexp_v[v] * __expf(mx_v[v] - mn);
        const float a2 = m2 == NEG_INF ? 0.0f : s2 * __expf(m2 - mn);
        sexp_v[v] = a1 + a2;
        mx_v[v] = mn;
      } else {
        sexp_v[v] += s2;
      }
      nnew_v[v] += __shfl_xor(nnew_v[v], o);
      if (!p.negs) nsure_v[v] += __shfl_xor(nsure_v[v], o);
    }
    if ((l & 15) == 0) {
      const int r = 4 * g + v;
      L.rf[r * 8 + RF_MX] = mx_v[v];
      L.rf[r * 8 + RF_SEXP] = sexp_v[v];
      L.rf[r * 8 + RF_THI] = thi_v[v];
      L.rf[r * 8 + RF_NBUF] = __int_as_float(bcnt_v[v]);
      L.ri[r * 8 + RI_NSURE] = nsure_v[v];
      L.ri[r * 8 + RI_NNEW] = nnew_v[v];
    }
  }
  wave_sync();

  // ---------------------------------------------------------------- epilogue
  // Rows go through three steps in groups: (A) per row, the float32 k-th value a_k
  // of its list and the near-tie entries within 2*beta of a_k, appended to the
  // wave's list; (B) float64 logits of the whole list, one entry per lane;
  // (C) per row, rank the near-ties, set the threshold, sum the kept entries.
  int r_next = 0;
  while (r_next < 16) {
    int tot = 0;
    int r_end = r_next;
    for (int r = r_next; r < 16; ++r) {
      const int i = L.ri[r * 8 + RI_I];
      int mode_r = 0;   // 0: skip, 1: no near-ties (k == 0 or all kept), 2: near-tie list
      if (i >= 0) mode_r = (k == 0 || L.rf[r * 8 + RF_THI] == NEG_INF) ? 1 : 2;
      if (mode_r == 2) {
        const int nb_all = __float_as_int(L.rf[r * 8 + RF_NBUF]);
        const int nsure = L.ri[r * 8 + RI_NSURE];
        const float beta = L.rf[r * 8 + RF_BETA];
        const int n = min(nb_all, SEL_CAP);
        const int kk = k - nsure;
        if (nb_all > SEL_CAP || kk < 1 || kk > n) {
          if (l == 0) {
            atomicAdd(p.counters + CNT_OVERFLOW, 1u);
            atomicOr(p.counters + CNT_ERROR, (uint32_t)ERRBIT_OVERFLOW);
          }
        }
        const float* vals = L.vals + r * SEL_CAP;
        const float ak = n > 0 ? wave_kth_largest(vals, n, max(1, min(kk, n)), L.khist, L.cv) : 0.0f;
        const float lo = f_down((double)ak - 2.0 * (double)beta);
        const float hi = f_up((double)ak + 2.0 * (double)beta);
        int nabove = 0, na = 0;
        for (int base = 0; base < n; base += WAVE) {
          const int t = base + l;
          const float v = t < n ? vals[t] : NEG_INF;
          nabove += (t < n && v > hi) ? 1 : 0;
          na += popc(ballot(t < n && v >= lo && v <= hi));
        }
        nabove = wave_sum(nabove);
        if (tot + na > WLIST && r > r_next) break;   // next group
        if (na > WLIST) {   // cannot rank more near-ties than the list holds
          if (l == 0) {
            atomicAdd(p.counters + CNT_OVERFLOW, 1u);
            atomicOr(p.counters + CNT_ERROR, (uint32_t)ERRBIT_OVERFLOW);
          }
          na = WLIST;
        }
        int w0 = 0;
        for (int base = 0; base < n; base += WAVE) {
          const int t = base + l;
          const float v = t < n ? vals[t] : NEG_INF;
          const bool inA = t < n && v >= lo && v <= hi;
          const uint64_t m = ballot(inA);
          if (inA) {
            const int dst = w0 + popc(m & lanemask_lt());
            if (dst < na) {
              L.ci[tot + dst] = t;
              L.cj[tot + dst] = L.ids[r * SEL_CAP + t];
              L.cr[tot + dst] = r;
            }
          }
          w0 += popc(m);
        }
        if (l == 0) {
          L.rf[r * 8 + RF_ALO] = lo;
          L.rf[r * 8 + RF_AHI] = hi;
          L.ri[r * 8 + RI_NABOVE] = nabove;
          L.ri[r * 8 + RI_AOFF] = tot;
          L.ri[r * 8 + RI_NA] = na;
        }
        tot += na;
      }
      if (l == 0) L.ri[r * 8 + RI_MODE] = mode_r;
      r_end = r + 1;
    }
    wave_sync();
    // (B) float64 logits of the group's near-ties
    for (int e0 = 0; e0 < tot; e0 += WAVE)
      if (e0 + l < tot)
        L.ce[e0 + l] = exact_dot<E, D>(Xs + (wrow0 + L.cr[e0 + l]) * D, Y + (int64_t)L.cj[e0 + l] * D);
    if (l == 0) nexact += (uint32_t)tot;
    wave_sync();
    // (C) thresholds and sums
    for (int r = r_next; r < r_end; ++r) {
      const int mode_r = L.ri[r * 8 + RI_MODE];
      if (mode_r == 0) continue;
      const int i = L.ri[r * 8 + RI_I];
      const float beta = L.rf[r * 8 + RF_BETA];
      const float mx = L.rf[r * 8 + RF_MX];
      float se = L.rf[r * 8 + RF_SEXP];
      int nnew = L.ri[r * 8 + RI_NNEW];
      const int nsure = L.ri[r * 8 + RI_NSURE];
      const E* xrow = Xs + (wrow0 + r) * D;
      const int64_t o = p.slot_out ? (int64_t)i : (int64_t)rho * s + i;
      double te;
      int tid;
      float tlo, thi;
      int listed = 0;
      if (k == 0) {
        te = __builtin_huge_val();
        tid = -2;
        tlo = thi = __builtin_huge_valf();
      } else if (mode_r == 1) {
        te = -__builtin_huge_val();   // every candidate kept (all summed as sure members)
        tid = -1;
        tlo = thi = NEG_INF;
        listed = nsure;
      } else {
        float* vals = L.vals + r * SEL_CAP;
        const int32_t* ids = L.ids + r * SEL_CAP;
        const int n = min(__float_as_int(L.rf[r * 8 + RF_NBUF]), SEL_CAP);
        const float lo = L.rf[r * 8 + RF_ALO];
        const int nabove = L.ri[r * 8 + RI_NABOVE];
        const int aoff = L.ri[r * 8 + RI_AOFF];
        const int na = L.ri[r * 8 + RI_NA];
        const int need = k - nsure - nabove;   // near-ties that are kept (>= 1)
        // rank the row's near-ties (order: float64 logit desc, id asc); na may exceed 64
        te = 0.0;
        tid = 0;
        for (int a0 = 0; a0 < na; a0 += WAVE) {
          const int ea = a0 + l;
          int rank = 0;
          double me = 0.0;
          int mj = 0;
          if (ea < na) {
            me = L.ce[aoff + ea];
            mj = L.cj[aoff + ea];
            for (int u = 0; u < na; ++u) {
              const double eu = L.ce[aoff + u];
              const int ju = L.cj[aoff + u];
              rank += (eu > me) || (eu == me && ju < mj);
            }
          }
          const uint64_t tm = ballot(ea < na && rank == need - 1);
          if (tm) {
            const int tl = __builtin_ctzll(tm);
            te = __shfl(me, tl);
            tid = __shfl(mj, tl);
          }
          if (ea < na && rank >= need) vals[L.ci[aoff + ea]] = NEG_INF;
        }
        wave_sync();
        if (l == 0 && na > 1) atomicAdd(p.counters + CNT_TOPK_EXACT, 1u);
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
              const PrevRow pr = L.prev[r * NP + r2];
              const int cy2 = chunk_of(p.inv_y[(int64_t)r2 * C + j], C, n_c);
              if (!in_window(pr.cx, cy2, n_c)) continue;
              dup = beats<E, D>(a, pr.lo, pr.hi, pr.te, pr.tid, xrow, Y, j, nexact);
            }
            if (!dup) {
              sl += __expf(a - mx);
              ++cl;
            }
          }
          if (p.negs) {
            const uint64_t km = ballot(kept);
            if (kept) {
              const int slotn = nsure + nk + popc(km & lanemask_lt());
              if (slotn < k) {
                p.negs[o * k + slotn] = j;
                if (p.negl) p.negl[o * k + slotn] = a;
              }
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
    r_next = r_end;
  }
  flush_count(p.counters + CNT_LOGIT_EXACT, nexact);
}

size_t select_lds_bytes(bool is_bf16, int d, int waves, int rounds) {
  const size_t rb = (size_t)d * (is_bf16 ? 2 : 4);
  const size_t ti = rb <= 256 ? 64 : (rb == 512 ? 32 : 16);
  return sel_common_lds(ti * rb, rounds) + (size_t)waves * wave_lds_bytes(rounds);
}

template <class E, int D, int NW>
static hipError_t launch_sel(const SelectArgs& a, hipStream_t st) {
  const size_t lds = select_lds_bytes(sizeof(E) == 2, D, NW, a.rounds);
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
