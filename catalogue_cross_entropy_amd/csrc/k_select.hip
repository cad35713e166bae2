// In-chunk logits and per-position top-k negatives (RECE page, Section 3,
// Algorithm 1: the chunk, window and wrong-class logit lines, repeated over
// rounds; the top-k keeps the largest logits, which Section 3 argues carry the
// largest gradients).
//
// Grid: one workgroup per (X-chunk c, tile of 16*NW sorted positions).  Each wave
// owns 16 positions and keeps their fragments in registers.  The window (item
// chunks c - n_ec .. c + n_ec of the round's sorted order, cyclic or clipped; at
// most two slot ranges) streams through LDS 64 items at a time, double-buffered
// and prefetched one tile ahead; the 16x64 logit block of a wave comes from the
// matrix cores and never leaves the chip.
//
// Selection, two passes over the window per position:
//   pass 1: a 256-bin histogram of the float32 logits over [-b_i, b_i]
//           (b_i >= every |logit| of the row) locates the bin of the k-th largest;
//           a bin too full for the candidate list is split by further passes;
//           the counts are 16 bits, two to an LDS word, unless a window can hold
//           more than 65535 items (WIDE: one 32-bit count per word);
//   pass 2: the logits are recomputed; a logit above the bin (plus 2*beta, beta
//           bounding |float32 - float64 logit|) is kept for sure and summed on the
//           fly; logits within the bin +- 2*beta go to an LDS candidate list.
// The list then gives the float32 k-th value a_k; the few entries within 2*beta of
// a_k are recomputed in float64 and ranked (logit desc, id asc).  The k-th kept
// element (float64 logit, id) is the position's threshold; the kept ids are
// written out, unordered and -1 padded, with their float32 logits when asked
// (negl).
//
// Rounds: every round selects on its own window; which of its kept pairs were
// already kept in an earlier round (the page's minus-ln(count) rule makes the
// multiset of copies a set) does not change its selection, only which pairs its
// sum counts, so that is settled afterwards from the kept lists (k_round_dedup)
// and the rounds need not wait for one another.  Outputs per position and round:
// the threshold and the sum of exp(logit - shift) over the kept pairs.
#include <type_traits>

#include "rece_device.h"
#include "rece_internal.h"
#include "rece_stream.h"

namespace rece {

constexpr int NBINS = 256;
constexpr int SEL_CAP = 64;      // candidate-list capacity per position
constexpr int SEL_SLACK = 16;    // room kept for entries within 2*beta outside the k-th bin
constexpr int MAX_REFINE = 2;    // histogram passes that may split a crowded bin
constexpr float X_TOP = 255.99998f;   // largest histogram coordinate (below 256)
constexpr float LOG2E_F = 1.44269504088896341f;

// Per-wave LDS: the row histograms / candidate lists, and the batch of WL near-tie
// entries awaiting float64 values.  The batch is used only after the streaming
// passes, so it lives in the window ring, which is idle by then.

struct WaveLds {
  double* ce;       // [WL] (in the ring)
  uint32_t* hist;   // [16][HistGeom::STRIDE] two 16-bit counts per word, or one 32-bit count
                    // (WIDE), in the histogram passes; aliased by vals/ids (collect pass)
  float* vals;      // [16][LIST_STRIDE] (SEL_CAP used)
  int32_t* ids;     // [16][LIST_STRIDE]
  int32_t* ci;      // [WL] list index in the row's candidate list (in the ring)
  int32_t* cj;      // [WL] item id (in the ring)
  int32_t* cr;      // [WL] row (in the ring)
};
// Row strides in LDS, padded so that the 16 rows of a wave start in different
// banks (histogram: 129 words, 257 when WIDE; lists: 68 entries, a multiple of
// four for the 16-byte reads of the epilogue).
constexpr int LIST_STRIDE = SEL_CAP + 4;
template <bool WIDE> struct HistGeom {
  static constexpr int STRIDE = WIDE ? NBINS + 1 : NBINS / 2 + 1;
  static constexpr size_t WAVE_LDS = (size_t)16 * STRIDE * 4 > (size_t)16 * LIST_STRIDE * 8
                                         ? (size_t)16 * STRIDE * 4
                                         : (size_t)16 * LIST_STRIDE * 8;
};
constexpr size_t BATCH_ENTRY = 8 + 4 + 4 + 4;   // ce, ci, cj, cr

// base: the wave's histogram/list region; batch: the wave's part of the ring
__device__ inline WaveLds carve(char* base, char* batch, int wl) {
  WaveLds L;
  L.hist = reinterpret_cast<uint32_t*>(base);
  L.vals = reinterpret_cast<float*>(base);
  L.ids = reinterpret_cast<int32_t*>(base + 16 * LIST_STRIDE * 4);
  char* p = batch;
  L.ce = reinterpret_cast<double*>(p);
  p += (size_t)wl * 8;
  L.ci = reinterpret_cast<int32_t*>(p);
  p += (size_t)wl * 4;
  L.cj = reinterpret_cast<int32_t*>(p);
  p += (size_t)wl * 4;
  L.cr = reinterpret_cast<int32_t*>(p);
  return L;
}


// One ring slot: the tile's rows, then 64 item ids.
__host__ __device__ constexpr size_t sel_slot_bytes(size_t row_bytes) { return row_bytes + 256; }
__host__ __device__ constexpr size_t sel_common_lds(size_t row_bytes, int ring) {
  return (size_t)ring * sel_slot_bytes(row_bytes) + 16;
}

// Ring slots (one tile in flight while the other is read) and the near-tie batch
// per wave: 128 entries where NW waves' batches fit in the ring, else 64.  Up to
// 256-byte vectors a workgroup of four waves then takes 51.7 KB of LDS, so three
// share a CU (a third wave per SIMD hides more of the copy and LDS latency than a
// third ring slot did).
template <class E, int D, int NW> struct SelGeom {
  static constexpr int RING = 2;
  static constexpr size_t RING_BYTES = (size_t)RING * sel_slot_bytes(TileGeom<E, D>::ROW_BYTES);
  static constexpr int WL = (size_t)NW * 128 * BATCH_ENTRY <= RING_BYTES ? 128 : 64;
  static_assert((size_t)NW * WL * BATCH_ENTRY <= RING_BYTES, "near-tie batches must fit in the ring");
};

// NEGS: the kept ids are written out (p.negs set); a template flag keeps that
// code out of the streaming loop when they are not.
template <class E, int D, int NW, bool NEGS, bool WIDE>
__global__ __launch_bounds__(64 * NW, (D * sizeof(E) <= 256) ? 3 : ((D * sizeof(E) <= 512) ? 2 : 1)) void k_select(SelectArgs p) {
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
  const size_t slot_bytes = sel_slot_bytes(G::ROW_BYTES);
  char* ring = smem;
  constexpr int RING = SelGeom<E, D, NW>::RING, WLIST = SelGeom<E, D, NW>::WL;
  int32_t* wg_flag = reinterpret_cast<int32_t*>(smem + RING * slot_bytes);
  const int w = threadIdx.x >> 6, l = lane_id(), g = l >> 4;
  constexpr int HIST_STRIDE = HistGeom<WIDE>::STRIDE;
  WaveLds L = carve(smem + sel_common_lds(G::ROW_BYTES, RING) + (size_t)w * HistGeom<WIDE>::WAVE_LDS,
                    smem + (size_t)w * WLIST * BATCH_ENTRY, WLIST);
  (void)X;
  (void)n_c;
  uint32_t nexact = 0;   // float64 logits computed by this lane
  uint32_t ntopk = 0;    // rows whose k-th element needed a float64 ranking (same in every lane)

  const int lb = xcd_block(blockIdx.x, gridDim.x);
  const int c = lb / p.tiles_per_chunk;
  const int tile = lb % p.tiles_per_chunk;
  const int64_t x0 = chunk_start(c, s, n_c), x1 = chunk_start(c + 1, s, n_c);
  const int64_t tile0 = x0 + (int64_t)tile * TR;
  if (tile0 >= x1) return;   // whole workgroup leaves together
  const int64_t wrow0 = tile0 + 16 * w;

  // window ranges (own chunk first), in tiles of TI items
  Ranges win;
  win.init(c, n_c, C, TI, p.n_ec, p.wrap);
  const int ntiles = win.ntiles();

  // fragments of this wave's 16 positions (sorted copy: contiguous rows)
  const int64_t pA = wrow0 + (l & 15);
  const int iA = pA < x1 ? p.perm_x[pA] : -1;
  Frag<E, D> afr;
  afr.load_global(pA < x1 ? Xs + pA * D : nullptr);

  // Layout: logit blocks are computed transposed (items x positions), so lane l
  // works for row r = l % 16 (its position) on items 4*(l/16) + v of every
  // 16-item block; a row's four lanes are r, r+16, r+32, r+48.  Row state is
  // one scalar per lane, kept equal in the row's four lanes.
  const int r = l & 15;
  const bool rv = pA < x1;
  const uint64_t rowbits = 0x0001000100010001ull << r;   // the row's lanes
  const uint64_t row_lt = rowbits & lanemask_lt();      // the row's lanes below this one
  const float ymax = p.ynorm_max[0];
  const bool selall = p.selall != 0;
  const int pos = rv ? p.pos[iA] : -1;
  const float xn = rv ? p.xnorm[iA] : 0.0f;
  const float beta = p.beta_coef * xn * ymax;
  // histogram coordinates: x = clamp(a * sc0 + off0, 0, 256^-) maps the row's logits to
  // [0, 256); a pass at refinement level L counts y = (x - xa) * mul (mul = 256^L) when
  // 0 <= y < 256.  Both steps are exact in float for the values that matter, so every
  // level bins exactly the values whose x lies in the interval chosen one level up.
  // Every float32 logit of the row lies in [-bnd, bnd].
  const float bnd = f_up((double)xn * (double)ymax * (1.0 + 1e-5) + 2.0 * (double)beta) + 1e-30f;
  const float lo0 = -bnd, sc0 = (float)NBINS / (2.0f * bnd);
  // bin coordinate x = med3(a * sc0 + off0, 0, 256^-), the same expression in every pass
  const float off0 = -lo0 * sc0;
  char* hist_row = reinterpret_cast<char*>(L.hist + r * HIST_STRIDE);
  float xa = rv ? 0.0f : __builtin_huge_valf();   // rows past the chunk count nothing
  float mul = 1.0f;
  int kk = rv ? k : 0;
  float tlo = (selall && rv) ? NEG_INF : __builtin_huge_valf(), thi = tlo;   // rows past the chunk keep +inf
  float mx = NEG_INF;   // row maximum (the exp shift), from the histogram pass
  // output row: the position id, or the sorted slot when outputs are per slot
  const int rowid = rv ? (p.slot_out ? (int)pA : iA) : -1;
  const int64_t orow = p.slot_out ? pA : (int64_t)rho * s + iA;   // negs row (valid rows only)
  const int64_t lrow = p.slot_out ? pA : (int64_t)iA;              // negl row (one round's lists)

  // mode 0: histogram pass; 1: collect pass; 2: nothing to do (k = 0)
  int mode = k == 0 ? 2 : (selall ? 1 : 0);
  float sexp = 0.0f;
  int nnew = 0, nsure = 0, bcnt = 0;

  // copies of one tile: G::ROW_DMA row copies, then the ids
  const int ncopies = G::ROW_DMA + 1;
  int my_copies = 0;
  for (int u = w; u < ncopies; u += NW) ++my_copies;

  for (int pass = 0; mode < 2; ++pass) {
    if (mode == 0)
      for (int b = l; b < 16 * HIST_STRIDE; b += WAVE) L.hist[b] = 0u;
    __syncthreads();
    issue_window_tile<E, D, NW, RING>(ring, slot_bytes, win, 0, Ys, p.perm_y, nullptr, C, 0, w);
    if (RING == 3 && ntiles > 1)
      issue_window_tile<E, D, NW, RING>(ring, slot_bytes, win, 1, Ys, p.perm_y, nullptr, C, 0, w);

    for (int t = 0; t < ntiles; ++t) {
      // tile t's copies are complete once only those of later tiles remain outstanding
      wait_vmcnt(RING == 3 && t + 1 < ntiles ? my_copies : 0);
      raw_barrier();   // every wave's copies of tile t landed; slot (t + RING - 1) % RING is free
      if (t + RING - 1 < ntiles)
        issue_window_tile<E, D, NW, RING>(ring, slot_bytes, win, t + RING - 1, Ys, p.perm_y, nullptr, C, 0, w);
      const int64_t q0 = range_tile_start(win, t, TI), q1 = range_tile_end(win, t);
      const char* slot = ring + (size_t)(t % RING) * slot_bytes;
      const int32_t* tid_ = reinterpret_cast<const int32_t*>(slot + G::ROW_BYTES);
      const int nlim = (int)(q1 - q0);   // valid items of this tile
      f32x4 acc[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        Frag<E, D> bf;
        TileFrag<E, D>::load(bf, slot, cb * 16 + r);
        acc[cb] = mma_block(bf, afr, f32x4{0.f, 0.f, 0.f, 0.f});   // [item 4g+v][row r]
      }
      const bool full = nlim >= TI;   // no item beyond the range end in this tile
      if (mode == 0) {
        if (pass == 0 && full) {
          // level 0 over a full tile: every value is binned; only the positive adds 0
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const u32x4 jj = *reinterpret_cast<const u32x4*>(tid_ + cb * 16 + 4 * g);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int b = (int)__builtin_amdgcn_fmed3f(fmaf(acc[cb][v], sc0, off0), 0.0f, X_TOP);
              if (WIDE)
                lds_add_u32(hist_row + (b << 2), (int)jj[v] != pos ? 1u : 0u);
              else
                lds_add_u32(hist_row + ((b >> 1) << 2), (int)jj[v] != pos ? 1u << ((b & 1) << 4) : 0u);
            }
          }
        } else {
          // refinement levels and the last tile of a range: branch-free, every lane adds
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const u32x4 jj = *reinterpret_cast<const u32x4*>(tid_ + cb * 16 + 4 * g);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const bool valid = cb * 16 + 4 * g + v < nlim && (int)jj[v] != pos;
              const float x = __builtin_amdgcn_fmed3f(fmaf(acc[cb][v], sc0, off0), 0.0f, X_TOP);
              const float y = (x - xa) * mul;
              const bool hit = valid && y >= 0.0f && y < (float)NBINS;
              const int b = hit ? (int)y : 0;
              if (WIDE)
                lds_add_u32(hist_row + (b << 2), hit ? 1u : 0u);
              else
                lds_add_u32(hist_row + ((b >> 1) << 2), hit ? 1u << ((b & 1) << 4) : 0u);
            }
          }
        }
      } else {
        // collect: sure members (above thi) are counted and summed; the band [tlo, thi]
        // goes to the row's list.  Rows past the chunk have tlo = thi = +inf.
        float mxl = mx * LOG2E_F;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const u32x4 jj = *reinterpret_cast<const u32x4*>(tid_ + cb * 16 + 4 * g);
          bool inb[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int n = cb * 16 + 4 * g + v;
            const int j = (int)jj[v];
            const float a = acc[cb][v];
            const bool cand = (full || n < nlim) && j != pos;
            const bool sure = cand && a > thi;
            inb[v] = cand && a >= tlo && a <= thi;
            if (selall && sure && a > mx) {   // no histogram pass ran: keep the shift at the maximum
              sexp = mx == NEG_INF ? 0.0f : sexp * __expf(mx - a);
              mx = a;
              mxl = mx * LOG2E_F;
            }
            // exp(a - mx) as 2^(a log2 e - mx log2 e), one fma before the exponential
            sexp += sure ? __builtin_amdgcn_exp2f(fmaf(a, LOG2E_F, -mxl)) : 0.0f;
            if (NEGS) {
              const uint64_t ms = ballot(sure);
              if (sure) {
                const int slotn = nsure + popc(ms & row_lt);
                if (slotn < k) {
                  p.negs[orow * k + slotn] = j;
                  if (p.negl) p.negl[lrow * k + slotn] = a;
                }
              }
              nsure += popc(ms & rowbits);
            } else {
              nsure += sure ? 1 : 0;
            }
          }
          if (ballot(inb[0] || inb[1] || inb[2] || inb[3])) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const uint64_t m2 = ballot(inb[v]);
              if (inb[v]) {
                const int slotn = bcnt + popc(m2 & row_lt);
                if (slotn < SEL_CAP) {
                  lds_store_u32(&L.vals[r * LIST_STRIDE + slotn], __float_as_uint(acc[cb][v]));
                  lds_store_u32(&L.ids[r * LIST_STRIDE + slotn], jj[v]);
                }
              }
              bcnt += popc(m2 & rowbits);
            }
          }
        }
      }
    }

    if (mode == 1) break;   // collected

    // ---- after a histogram pass: locate the bin of the kk-th largest of each row
    wave_sync();
    bool more = false;
    for (int rr = 0; rr < 16; ++rr) {
      const int kkr = lane_val(kk, rr);
      if (kkr <= 0) continue;   // row settled in an earlier pass
      const float xar = lane_val(xa, rr), mulr = lane_val(mul, rr), lo0r = lane_val(lo0, rr);
      const float sc0r = lane_val(sc0, rr), off0r = lane_val(off0, rr), betar = lane_val(beta, rr);
      uint32_t h[4];
      if (WIDE) {
#pragma unroll
        for (int q = 0; q < 4; ++q) h[q] = L.hist[rr * HIST_STRIDE + 4 * l + q];
      } else {
        const uint32_t w0 = L.hist[rr * HIST_STRIDE + 2 * l], w1 = L.hist[rr * HIST_STRIDE + 2 * l + 1];
        h[0] = w0 & 0xFFFFu;
        h[1] = w0 >> 16;
        h[2] = w1 & 0xFFFFu;
        h[3] = w1 >> 16;
      }
      const uint32_t own = h[0] + h[1] + h[2] + h[3];
      // suffix sum (bins at or above this lane's four), from the prefix sum
      const uint32_t pre = wave_prefix_incl(own);
      const uint32_t total = lane_val(pre, 63);
      const uint32_t suf = total - pre + own;
      int myb = -1;
      uint32_t my_above = 0, my_cnt = 0;
      {
        uint32_t a2 = suf - own;
#pragma unroll
        for (int q = 3; q >= 0; --q) {
          if (myb < 0 && a2 + h[q] >= (uint32_t)kkr) {
            myb = 4 * l + q;
            my_above = a2;
            my_cnt = h[q];
          }
          a2 += h[q];
        }
      }
      const uint64_t hit = ballot(myb >= 0);
      float mxr = NEG_INF;   // exp shift: the top edge of the highest non-empty level-0 bin
      if (pass == 0) {
        const uint64_t nz = ballot(own > 0);
        if (nz) {
          const int tl = 63 - __builtin_clzll(nz);
          const int hq = h[3] ? 3 : (h[2] ? 2 : (h[1] ? 1 : 0));
          const int btop = 4 * tl + lane_val(hq, tl);
          const double top = ((double)(btop + 1) - (double)off0r) / (double)sc0r;
          mxr = f_up(top + (fabs(top) + fabs((double)lo0r)) * 1e-6 + 1e-30);
        }
      }
      float ntlo, nthi, nxa = xar, nmul = mulr;
      int nkk = 0;
      bool refine = false;
      if ((pass == 0 && (int)total <= kkr) || !hit) {
        // the whole window has at most k candidates (first pass only): keep them all
        ntlo = nthi = NEG_INF;
      } else {
        const int src = 63 - __builtin_clzll(hit);
        const int bstar = lane_val(myb, src);
        const int above = (int)lane_val(my_above, src);
        const int cnt = (int)lane_val(my_cnt, src);
        nxa = xar + (float)bstar / mulr;   // exact: a multiple of 256^-L below 256
        nmul = mulr * (float)NBINS;
        // the bin is x in [nxa, nxa + 1/mul): its logit interval, padded for the rounding of x
        const double vlo = ((double)nxa - (double)off0r) / (double)sc0r;
        const double vhi = ((double)nxa + 1.0 / (double)mulr - (double)off0r) / (double)sc0r;
        const double pad = (fabs(vlo) + fabs(vhi) + fabs((double)lo0r)) * 1e-6 + 1e-30;
        ntlo = f_down(vlo - 2.0 * (double)betar - pad);
        nthi = f_up(vhi + 2.0 * (double)betar + pad);
        if (cnt > SEL_CAP - SEL_SLACK && pass < MAX_REFINE && vhi - vlo > 4.0 * (double)betar) {
          refine = true;   // crowded bin: split it by another histogram pass
          nkk = kkr - above;
        }
      }
      if (r == rr) {
        if (pass == 0) mx = mxr;
        tlo = ntlo;
        thi = nthi;
        kk = refine ? nkk : 0;
        xa = refine ? nxa : __builtin_huge_valf();   // settled rows count nothing more
        mul = refine ? nmul : 1.0f;
      }
      more |= refine;
    }
    if (threadIdx.x == 0) *wg_flag = 0;
    __syncthreads();
    if (l == 0 && more) atomicOr(wg_flag, 1);
    __syncthreads();
    mode = *wg_flag ? 0 : 1;
  }

  // every wave has read its last ring tile and no copy is in flight: the ring now
  // holds the near-tie batches
  __syncthreads();

  // ---- publish the per-row sums of the sure members (combine the row's four lanes)
#pragma unroll
  for (int o = 16; o < 64; o <<= 1) {
    const float m2 = __shfl_xor(mx, o);
    const float s2 = __shfl_xor(sexp, o);
    if (selall) {   // lanes saw different maxima: rescale before adding
      const float mn = fmaxf(mx, m2);
      const float a1 = mx == NEG_INF ? 0.0f : sexp * __expf(mx - mn);
      const float a2 = m2 == NEG_INF ? 0.0f : s2 * __expf(m2 - mn);
      sexp = a1 + a2;
      mx = mn;
    } else {
      sexp += s2;
    }
    if (!NEGS) nsure += __shfl_xor(nsure, o);
  }
  nnew = nsure;

  // ---------------------------------------------------------------- epilogue
  // Rows go through three steps in groups.  (A) Per row: the float32 k-th value
  // a_k of its list (at most 64 entries, one per lane; kk = k minus the sure
  // members) by counting the entries above and at or above each one; the
  // near-ties, the entries within 2*beta of a_k, join the wave's float64 batch.
  // (B) Float64 logits of the batch, one entry per lane.  (C) Per row: rank the
  // near-ties by (float64 logit desc, id asc); the k-th kept element is the row's
  // threshold; the kept list entries are those above the near-ties plus the
  // near-ties ranked within the count still missing.
  // A row's state is the same in its four lanes (r, r + 16, r + 32, r + 48), so
  // the steps read it with readlane from lane r; what (A) hands to (C) is kept in
  // lane r of the ep_* registers.
  int ep_mode = 0, ep_nabove = 0, ep_aoff = 0, ep_na = 0, ep_kk = 0;
  float ep_lo = 0.0f, ep_hi = 0.0f;
  int r_next = 0;
  while (r_next < 16) {
    int tot = 0;
    int r_end = r_next;
    for (int r = r_next; r < 16; ++r) {
      const int i = lane_val(rowid, r);
      int mode_r = 0;   // 0: skip, 1: no near-ties (k == 0 or all kept), 2: near-tie list
      if (i >= 0) mode_r = (k == 0 || lane_val(thi, r) == NEG_INF) ? 1 : 2;
      if (mode_r == 2) {
        const int nb_all = lane_val(bcnt, r);
        const int nsure_r = lane_val(nsure, r);
        const float beta_r = lane_val(beta, r);
        const int n = min(nb_all, SEL_CAP);
        int kk = k - nsure_r;
        if (nb_all > SEL_CAP || kk < 1 || kk > n) {
          if (l == 0) {
            atomicAdd(p.counters + CNT_OVERFLOW, 1u);
            atomicOr(p.counters + CNT_ERROR, (uint32_t)ERRBIT_OVERFLOW);
          }
          kk = max(1, min(kk, max(n, 1)));
        }
        const float v = l < n ? L.vals[r * LIST_STRIDE + l] : NEG_INF;
        const int id = l < n ? L.ids[r * LIST_STRIDE + l] : 0x7FFFFFFF;
        // a_k, the kk-th largest float value of the list: the value v of the lane with
        // (#entries above v) < kk <= (#entries at or above v); every lane counts against
        // each list entry, taken from the lane that holds it (readlane: no memory trip)
        int cgt = 0, cge = 0;
        for (int u = 0; u < n; ++u) {
          const float q = lane_val(v, u);
          cgt += q > v;
          cge += q >= v;
        }
        const uint64_t at_k = ballot(l < n && cgt < kk && cge >= kk);
        const float ak = lane_val(v, at_k ? (int)__builtin_ctzll(at_k) : 0);
        const float lo = f_down((double)ak - 2.0 * (double)beta_r);
        const float hi = f_up((double)ak + 2.0 * (double)beta_r);
        const int nabove = popc(ballot(l < n && v > hi));
        const bool inb = l < n && v >= lo && v <= hi;
        const uint64_t inbm = ballot(inb);
        int na = popc(inbm);
        if (tot + na > WLIST && r > r_next) break;   // next group
        if (na > WLIST) {   // cannot rank more near-ties than the batch holds
          if (l == 0) {
            atomicAdd(p.counters + CNT_OVERFLOW, 1u);
            atomicOr(p.counters + CNT_ERROR, (uint32_t)ERRBIT_OVERFLOW);
          }
          na = WLIST;
        }
        const int e = popc(inbm & lanemask_lt());   // near-tie e (list order)
        if (inb && e < na) {
          L.ci[tot + e] = l;
          L.cj[tot + e] = id & 0x7FFFFFFF;
          L.cr[tot + e] = r;
        }
        if (l == r) {
          ep_hi = hi;
          ep_lo = lo;
          ep_nabove = nabove;
          ep_aoff = tot;
          ep_na = na;
          ep_kk = kk;
        }
        tot += na;
      }
      if (l == r) ep_mode = mode_r;
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
      const int mode_r = lane_val(ep_mode, r);
      if (mode_r == 0) continue;
      const int i = lane_val(rowid, r);
      const float beta_r = lane_val(beta, r);
      const float mx_r = lane_val(mx, r);
      float se = lane_val(sexp, r);
      int nnew_r = lane_val(nnew, r);
      const int nsure_r = lane_val(nsure, r);
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
        listed = nsure_r;
      } else {
        const int n = min(lane_val(bcnt, r), SEL_CAP);
        const int nabove = lane_val(ep_nabove, r);
        const int aoff = lane_val(ep_aoff, r);
        const int na = lane_val(ep_na, r);
        const int need = lane_val(ep_kk, r) - nabove;   // near-ties that are kept (>= 1)
        // rank of this lane's near-tie (the e-th list entry within [lo, hi])
        const float lo = lane_val(ep_lo, r), hi = lane_val(ep_hi, r);
        const float a = l < n ? L.vals[r * LIST_STRIDE + l] : NEG_INF;
        const int jraw = l < n ? L.ids[r * LIST_STRIDE + l] : 0;
        const bool inb = l < n && a >= lo && a <= hi;
        const int e = popc(ballot(inb) & lanemask_lt());
        int rank = WAVE;
        double me = 0.0;
        int mj = 0;
        if (inb && e < na) {
          me = L.ce[aoff + e];
          mj = L.cj[aoff + e];
          rank = 0;
          for (int u = 0; u < na; ++u) {
            const double eu = L.ce[aoff + u];
            const int ju = L.cj[aoff + u];
            rank += (eu > me) || (eu == me && ju < mj);
          }
        }
        const uint64_t tm = ballot(rank == need - 1);
        te = 0.0;
        tid = 0;
        if (tm) {
          const int tl = __builtin_ctzll(tm);
          te = lane_val(me, tl);
          tid = lane_val(mj, tl);
        }
        if (na > 1) ++ntopk;
        const double b2 = (double)beta_r * (1.0 + 1e-6);
        tlo = f_down(te - b2);
        thi = f_up(te + b2);
        // kept list entries: those above the near-ties and the near-ties ranked in
        const bool kept = l < n && (a > hi || rank < need);
        se += wave_sum_dpp(kept ? __expf(a - mx_r) : 0.0f);
        nnew_r += popc(ballot(kept));
        if (NEGS) {
          const uint64_t km = ballot(kept);
          if (kept) {
            const int slotn = nsure_r + popc(km & lanemask_lt());
            if (slotn < k) {
              p.negs[o * k + slotn] = jraw;
              if (p.negl) p.negl[(int64_t)i * k + slotn] = a;
            }
          }
          listed = nsure_r + popc(km);
        }
      }
      if (NEGS)
        for (int t = listed + l; t < k; t += WAVE) p.negs[o * k + t] = -1;
      if (l == 0) {
        p.thr_e[o] = te;
        p.thr_id[o] = tid;
        p.thr_lo[o] = tlo;
        p.thr_hi[o] = thi;
        p.mshift[o] = mx_r;
        p.ssum[o] = se;
        p.nmem[o] = nnew_r;
      }
    }
    wave_sync();
    r_next = r_end;
  }
  flush_count(p.counters + CNT_LOGIT_EXACT, nexact);
  if (lane_id() == 0 && ntopk) atomicAdd(p.counters + CNT_TOPK_EXACT, ntopk);
}

template <class E, int D>
static size_t select_lds_bytes_t(int waves, bool wide) {
  return sel_common_lds(TileGeom<E, D>::ROW_BYTES, SelGeom<E, D, 4>::RING) +
         (size_t)waves * (wide ? HistGeom<true>::WAVE_LDS : HistGeom<false>::WAVE_LDS);
}
size_t select_lds_bytes(bool is_bf16, int d, int waves, bool wide) {
#define RECE_L(E, DD) \
  if (d == DD) return select_lds_bytes_t<E, DD>(waves, wide);
  if (is_bf16) {
    RECE_L(bf16, 32) RECE_L(bf16, 64) RECE_L(bf16, 128) RECE_L(bf16, 256)
  } else {
    RECE_L(float, 32) RECE_L(float, 64) RECE_L(float, 128) RECE_L(float, 256)
  }
#undef RECE_L
  return 0;
}

template <class E, int D, int NW>
static hipError_t launch_sel(const SelectArgs& a, hipStream_t st) {
  const bool wide = a.wide != 0;
  const size_t lds = select_lds_bytes(sizeof(E) == 2, D, NW, wide);
  auto kern = wide ? (a.negs ? k_select<E, D, NW, true, true> : k_select<E, D, NW, false, true>)
                   : (a.negs ? k_select<E, D, NW, true, false> : k_select<E, D, NW, false, false>);
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
