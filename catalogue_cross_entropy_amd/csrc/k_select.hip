// In-chunk logits and per-position top-k negatives (RECE page, Section 3,
// Algorithm 1: the chunk, window and wrong-class logit steps, repeated over
// rounds; the top-k keeps the largest logits, which Section 3 argues carry the
// largest gradients).  Also the per-bucket step of the bucket variant (one
// "chunk" per bucket, its window the bucket's own items).
//
// Kernels per round:
//
// k_sel_stream: one workgroup per (X-chunk c, tile of 16*NW sorted positions).
//   Each wave owns 16 positions and keeps their matrix-core fragments in
//   registers.  The window (item chunks c - n_ec .. c + n_ec of the round's
//   sorted order, cyclic or clipped; at most two slot ranges) streams through LDS
//   once, a tile of items at a time, two tiles in flight; the 16 x TI logit block
//   of a wave comes from the matrix cores and never leaves the chip.  Every logit
//   is compared with its row's running threshold; those that pass (item id,
//   float32 logit) are appended to the row's candidate list in scratch memory.
//   The threshold starts at -inf.  When a row's list is nearly full, the lists of
//   the wave's rows are compacted together by histogram (compact_hist): a value T
//   with at least k entries at or above it raises the threshold to T - 2*beta
//   (beta bounds |float32 - float64 logit|), and the list keeps what is above the
//   threshold.  No entry of the final top-k is dropped: k others beat what falls
//   below.  Near-ties stay in; the finishing kernel ranks them exactly.
//   A row whose list the bins cannot shrink (hundreds of ties) is flagged; a
//   second launch of the kernel streams the windows of the flagged rows only, with
//   an exact compaction (compact_exact) that ranks ties in float64 and by id.
//
// k_sel_finish: one wave per row.  The row's list is loaded into LDS; if it
//   holds more than k entries (or was ever compacted) the exact top-k in the
//   order (float64 logit descending, item id ascending) is taken: the float32
//   k-th value decides every entry farther than 2*beta from it, the rest are
//   recomputed in float64 (coordinate-order scalar products) and ranked.  The
//   row's outputs: the k-th kept element (float64 logit, id) as its threshold,
//   the kept ids (and, when asked, their float32 logits), the exp shift and the
//   sum of exp(logit - shift) over the kept set.
//
// Rounds: every round selects on its own window; which of its kept pairs were
// already kept in an earlier round (the page's minus-ln(count) rule makes the
// multiset of copies a set) does not change its selection, only which pairs its
// sum counts, so that is settled afterwards from the kept lists (k_round_dedup)
// and the rounds need not wait for one another.
#include <algorithm>

#include "rece_device.h"
#include "rece_internal.h"
#include "rece_kth.h"
#include "rece_stream.h"

namespace rece {

// The row ring: SEL_RING slots of a tile's rows, gathered from the item table by
// id.  The id ring: SEL_IDS slots of 64 item ids, filled one tile further ahead
// (the row copies of a tile read its ids from LDS).
constexpr int SEL_RING = 3;   // tiles t+1 and t+2 in flight while tile t is scored
constexpr int SEL_IDS = 4;    // ids of tiles t .. t+3
constexpr size_t SEL_IDS_BYTES = SEL_IDS * 256;
constexpr int SEL_NB = 64;    // histogram bins of a row's list compaction
// Per wave: the 16 rows' compaction histograms; for the exact fallback (one row at
// a time) the float32 values of the row's list and the k-th search's histogram and
// candidates.  The two uses never overlap in time.
__host__ __device__ constexpr size_t sel_wave_bytes(int cap) {
  return (16 * SEL_NB * 4) > (((size_t)cap * 4 + 1024 + 256 + 15) / 16 * 16)
             ? (size_t)(16 * SEL_NB * 4)
             : (((size_t)cap * 4 + 1024 + 256 + 15) / 16 * 16);
}
// Capacity of a row's candidate list: room for 3k entries plus two tiles.
int select_list_cap(int k, int d, bool bf16) {
  const int rb = d * (bf16 ? 2 : 4);
  const int ti = rb <= 128 ? 64 : (rb <= 512 ? 32 : 16);
  return 3 * k + 2 * ti;
}

// Entry t of a row's list, read past the (non-coherent) vector L1 cache: the
// wave itself wrote it earlier in this kernel.
__device__ __forceinline__ uint64_t list_load(const int2* list, int t) {
  return __hip_atomic_load(reinterpret_cast<const uint64_t*>(list) + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double dbl_load(const double* p, int t) {
  return __longlong_as_double((long long)__hip_atomic_load(reinterpret_cast<const uint64_t*>(p) + t, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ int entry_id(uint64_t e) { return (int)(uint32_t)e; }
__device__ __forceinline__ float entry_val(uint64_t e) { return __int_as_float((int)(e >> 32)); }

// Reduce a row's list (n > k entries, in scratch memory) to its exact top-k in the
// order (float64 logit descending, item id ascending), in place and in list order.
// Every entry of the row's final top-k is in the list, so no kept entry can leave
// it: an entry that k others beat is beaten in the whole window too.  The float32
// k-th value a_k decides every entry more than 2*beta from it; the band within
// 2*beta is recomputed in float64 (values in `dbuf`, the wave's scratch) and ranked.
// Returns the k-th kept element (te, tid).  Called by the whole wave with every
// argument uniform.
template <class E, int D>
__device__ __attribute__((noinline)) void compact_exact(int2* list, int n, int k, float beta, const E* xrow, const E* Y, float* sv,
                              uint32_t* khist, float* kcand, double* dbuf, double& te_out, int& tid_out,
                              uint32_t& nexact) {
  const int l = lane_id();
  for (int t = l; t < n; t += WAVE) sv[t] = entry_val(list_load(list, t));
  wave_sync();
  const float ak = wave_kth_largest(sv, n, k, khist, kcand);
  const float lo = f_down((double)ak - 2.0 * (double)beta);
  const float hi = f_up((double)ak + 2.0 * (double)beta);
  // the band, in list order: its list indices go to sv (as ints, index <= entry),
  // its float64 logits to dbuf
  int32_t* bidx = reinterpret_cast<int32_t*>(sv);
  int nabove = 0, nb = 0;
  for (int base = 0; base < n; base += WAVE) {
    const int t = base + l;
    const float a = t < n ? sv[t] : NEG_INF;
    const bool inb = t < n && a >= lo && a <= hi;
    nabove += popc(ballot(t < n && a > hi));
    const uint64_t mk = ballot(inb);
    if (inb) {
      const int b = nb + popc(mk & lanemask_lt());
      bidx[b] = t;
      dbuf[b] = exact_dot<E, D, 2>(xrow, Y + (int64_t)entry_id(list_load(list, t)) * D);
    }
    nb += popc(mk);
  }
  if (l == 0) nexact += (uint32_t)nb;   // lane 0 keeps the wave's count
  wave_sync();
  const int need = k - nabove;   // band entries kept (>= 1)
  double te = 0.0;
  int tid = 0;
  for (int b0 = 0; b0 < nb; b0 += WAVE) {
    const int b = b0 + l;
    const bool mine = b < nb;
    const int t = mine ? bidx[b] : 0;
    const double me = mine ? dbl_load(dbuf, b) : 0.0;
    const int mj = mine ? entry_id(list_load(list, t)) : 0;
    int rank = 0;
    for (int c0 = 0; c0 < nb; c0 += WAVE) {   // the band 64 entries at a time, read from the lanes
      const int cb = c0 + l;
      const double ce = cb < nb ? dbl_load(dbuf, cb) : 0.0;
      const int cj = cb < nb ? entry_id(list_load(list, bidx[cb])) : 0;
      const int m = nb - c0 < WAVE ? nb - c0 : WAVE;
      for (int u = 0; u < m; ++u) {
        const double eu = lane_val(ce, u);
        const int ju = lane_val(cj, u);
        rank += (eu > me) || (eu == me && ju < mj);
      }
    }
    const uint64_t tm = ballot(mine && rank == need - 1);
    if (tm) {
      const int tl = __builtin_ctzll(tm);
      te = lane_val(me, tl);
      tid = lane_val(mj, tl);
    }
    if (mine && rank >= need)   // ranked out: dropped below
      *reinterpret_cast<uint64_t*>(list + t) = ((uint64_t)(uint32_t)__float_as_int(NEG_INF) << 32) | (uint32_t)mj;
  }
  wave_sync();
  int m = 0;
  for (int base = 0; base < n; base += WAVE) {
    const int t = base + l;
    const uint64_t e = t < n ? list_load(list, t) : 0ull;
    const bool keep = t < n && entry_val(e) >= lo;
    const uint64_t mk = ballot(keep);
    if (keep) *reinterpret_cast<uint64_t*>(list + m + popc(mk & lanemask_lt())) = e;
    m += popc(mk);
  }
  wave_sync();
  te_out = te;
  tid_out = tid;
}

// Row histograms.  Each row of the wave keeps SEL_NB counts in LDS, one per bin of
// the map b(v) = clamp((v - hlo) * hsc, 0, SEL_NB - 1), over every entry of its
// list.  No list value lies below hlo (hlo is -||x|| max||y||, a bound of every
// logit, until the first compaction, then the row's threshold), so every entry in
// a bin b >= 1 is at least bin b's lower edge; values above the top edge count in
// the top bin.
__device__ __forceinline__ int sel_bin(float v, float hlo, float hsc) {
  return (int)fminf(fmaxf((v - hlo) * hsc, 0.0f), (float)(SEL_NB - 1));
}

// Bin of the row's k-th largest list value (the highest bin whose count from the
// top reaches k), or -1 if the list has fewer than k entries.  Lane g of the row
// reads bins 16 g .. 16 g + 15.  Uniform over the row's lanes.
__device__ __forceinline__ int row_kth_bin(const uint32_t* hist_r, int g, int r, int k) {
  constexpr int NB4 = SEL_NB / 4;
  static_assert(NB4 == 16, "four 16-byte reads per lane");
  u32x4 hv[4];
  uint32_t ha[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) ha[q] = lds_addr(hist_r + g * NB4 + 4 * q);
  LdsRead128<4>::run(ha, hv);   // no wait for the tile copies in flight
  uint32_t h[NB4];
  uint32_t own = 0;
#pragma unroll
  for (int b = 0; b < NB4; ++b) {
    h[b] = hv[b / 4][b % 4];
    own += h[b];
  }
  uint32_t above = 0;
#pragma unroll
  for (int q = 1; q < 4; ++q) {
    const uint32_t sq = __shfl(own, r + 16 * q);
    above += q > g ? sq : 0u;
  }
  int found = -1;
  uint32_t acc = above;
#pragma unroll
  for (int b = NB4 - 1; b >= 0; --b) {
    if (found < 0 && acc + h[b] >= (uint32_t)k) found = g * NB4 + b;
    acc += h[b];
  }
  found = max(found, __shfl_xor(found, 16));
  return max(found, __shfl_xor(found, 32));
}

// Raise the row's threshold from its histogram: at least k list entries lie at or
// above the lower edge T of bin `found` >= 1, so at least k window entries have a
// float64 logit >= T - beta and anything whose float32 logit is below T - 2*beta
// is beaten by k others.  The edge is taken a few rounding units low.
__device__ __forceinline__ void raise_from_bin(int found, float hlo, float hsc, float beta, float& lo) {
  if (found < 1) return;
  const double e = (double)hlo + (double)found / (double)hsc;
  const double T = e - (fabs((double)hlo) + fabs(e)) * 0x1p-21;
  lo = fmaxf(lo, f_down(T - 2.0 * (double)beta * (1.0 + 1e-6)));
}

// Compaction of the lists of the rows with `act` set, each row by its own four
// lanes, all rows at once: the threshold is raised from the histogram, the list
// keeps the entries at or above it (in list order), and the histogram is rebuilt on
// a new map from the threshold to the row's largest value.  Called by the whole
// wave; `act` is uniform over a row's lanes.
__device__ __forceinline__ void compact_hist(int2* list, bool act, int& cnt, int k, float beta, float& lo, float& hlo,
                                             float& hsc, float& vmx, uint32_t* hist_r) {
  const int l = lane_id(), g = l >> 4, r = l & 15;
  const uint64_t rowbits = 0x0001000100010001ull << r;
  const uint64_t row_lt = rowbits & lanemask_lt();
  constexpr int NB4 = SEL_NB / 4;
  const int found = row_kth_bin(hist_r, g, r, k);
  if (act) raise_from_bin(found, hlo, hsc, beta, lo);
  float rmx = fmaxf(vmx, __shfl_xor(vmx, 16));
  rmx = fmaxf(rmx, __shfl_xor(rmx, 32));
  if (act && lo > NEG_INF) {   // new map: [lo, largest value]
    hlo = lo;
    hsc = rmx > lo ? (float)SEL_NB / (rmx - lo) : 0.0f;
  }
  wave_sync();
  if (act) {
#pragma unroll
    for (int b = 0; b < NB4; ++b) hist_r[g * NB4 + b] = 0u;
  }
  wave_sync();
  const int cmax = wave_max_i(act ? cnt : 0);
  constexpr int BATCH = 8;
  int m = 0;
  for (int u0 = 0; u0 < cmax; u0 += 4 * BATCH) {
    uint64_t e[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int u = u0 + 4 * j + g;
      e[j] = act && u < cnt ? list_load(list, u) : 0ull;
    }
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int u = u0 + 4 * j + g;
      const float a = entry_val(e[j]);
      const bool keep = act && u < cnt && a >= lo;
      const uint64_t mk = ballot(keep);
      if (keep) {
        *reinterpret_cast<uint64_t*>(list + m + popc(mk & row_lt)) = e[j];
        atomicAdd(hist_r + sel_bin(a, hlo, hsc), 1u);
      }
      m += popc(mk & rowbits);
    }
  }
  wave_sync();
  if (act) cnt = m;
}

// clist_n flags: the list was compacted or its threshold raised, which happens
// only with more than k candidates; the row is left for the exact pass (its list
// is not valid).
constexpr uint32_t LIST_COMPACTED = 0x80000000u;
constexpr uint32_t LIST_REDO = 0x40000000u;
constexpr int SEL_RAISE_EVERY = 32;   // insertions between two threshold raises of a row

// EXACT = false: every row of the tile; thresholds raised and lists compacted by
//   histogram only; a row whose list the bins cannot shrink stops taking
//   candidates and is flagged LIST_REDO.
// EXACT = true: only the flagged rows (a workgroup without one leaves at once), from
//   the start of the window, with the exact compaction; rare (ties by the hundred).
template <class E, int D, int NW, bool EXACT>
__global__ __launch_bounds__(64 * NW, 2) void k_sel_stream(SelectArgs p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  using G = TileGeom<E, D>;
  constexpr int TI = G::TI;
  constexpr int NCB = TI / 16;                // 16-column blocks per tile
  constexpr int TR = 16 * NW;
  const E* __restrict__ X = reinterpret_cast<const E*>(p.X);
  const E* __restrict__ Y = reinterpret_cast<const E*>(p.Y);
  const int k = p.k, n_c = p.n_c, cap = p.cap;
  const int64_t s = p.s, C = p.C;
  // The exact pass: nothing to do unless some list went there (the counter counts
  // the flagged rows of every launch since the counters were cleared; the histogram
  // pass of this launch's rows completed before this kernel started).
  if constexpr (EXACT) {
    if (p.counters[CNT_SEL_REDO] == 0u) return;
  }
  constexpr size_t slot_bytes = G::ROW_BYTES;
  char* ring = smem;
  int32_t* idring = reinterpret_cast<int32_t*>(smem + SEL_RING * slot_bytes);
  const int w = threadIdx.x >> 6, l = lane_id(), g = l >> 4, r = l & 15;
  char* wscr = smem + SEL_RING * slot_bytes + SEL_IDS_BYTES + (size_t)w * sel_wave_bytes(p.selall ? 0 : cap);
  uint32_t* hist_r = reinterpret_cast<uint32_t*>(wscr) + r * SEL_NB;
  float* cvals = reinterpret_cast<float*>(wscr);
  uint32_t* khist = reinterpret_cast<uint32_t*>(wscr + (size_t)cap * 4);
  float* kcand = reinterpret_cast<float*>(wscr + (size_t)cap * 4 + 1024);

  const int lb = xcd_block(blockIdx.x, gridDim.x);
  const int c = lb / p.tiles_per_chunk;
  const int tile = lb % p.tiles_per_chunk;
  const int64_t x0 = chunk_start(c, s, n_c), x1 = chunk_start(c + 1, s, n_c);
  const int64_t tile0 = x0 + (int64_t)tile * TR;
  if (tile0 >= x1) return;   // whole workgroup leaves together
  const int64_t wrow0 = tile0 + 16 * w;

  Ranges win;
  win.init(c, n_c, C, TI, p.n_ec, p.wrap, window_rotation(p.win_order, c, p.n_ec));
  const int ntiles = win.ntiles();

  // fragments of this wave's 16 positions (sorted copy: contiguous rows)
  const int64_t pA = wrow0 + r;
  const bool rv = pA < x1;
  const int iA = settled(rv ? p.perm_x[pA] : -1);
  Frag<E, D> afr;
  afr.load_global(rv ? X + (int64_t)iA * D : nullptr);
  afr.settle();

  // Layout: logit blocks are computed transposed (items x positions), so lane l
  // works for row r = l % 16 (its position) on items 4*(l/16) + v of every
  // 16-item block; a row's four lanes are r, r+16, r+32, r+48.  Row state is one
  // scalar per lane, kept equal in the row's four lanes (vmx, the largest value
  // listed, is per lane: each covers the entries its lane wrote).
  const int pos = settled(rv ? p.pos[iA] : -1);
  const float bnd = settled(rv ? p.xnorm[iA] * p.ynorm_max[0] : 0.0f);   // every |logit| of the row is below
  const float beta = p.beta_coef * bnd;
  const int64_t lrow = p.slot_out ? pA : (int64_t)iA;   // list row (position id, or slot)
  int2* list = p.clist + (rv ? lrow : 0) * cap;
  double* dbuf = p.cdbl + ((int64_t)blockIdx.x * NW + w) * cap;   // this wave's float64 scratch
  bool take = rv;   // rows past the chunk (and, in the exact pass, unflagged rows) take nothing
  if constexpr (EXACT) {
    take = rv && ((uint32_t)p.clist_n[lrow] & LIST_REDO) != 0u;
    if (!__syncthreads_or(take)) return;   // whole workgroup leaves together
  }
  // Row state: a logit below lo cannot enter the row's top-k (-inf until the first
  // raise); every other candidate goes in, near-ties included (the finishing kernel
  // ranks them exactly).
  float lo = take ? NEG_INF : __builtin_huge_valf();
  int cnt = 0, last_raise = 0;
  int compacted = 0, redo = 0;
  int fine = 0;   // the row's histogram map has been rebuilt around its k-th value
  uint32_t nlisted = 0;   // entries this lane appended to lists
  float vmx = NEG_INF;
  float hlo = -bnd, hsc = bnd > 0.0f ? (float)SEL_NB / (2.0f * bnd) : 0.0f;
  uint32_t nexact = 0;
  // Copies per tile: each wave its ROW_DMA / NW row copies, wave 0 also the ids
  // of the tile three ahead, issued before the rows of the tile two ahead.  Once
  // only the row copies of tile t+1 remain outstanding, tile t's rows and the ids
  // of tile t+2 have landed (loads complete in order).
  constexpr int MINC = G::ROW_DMA / NW;
  auto issue_ids = [&](int tt) {
    if (w == 0)
      dma_ints(idring + (tt % SEL_IDS) * 64, p.perm_y, range_tile_start(win, tt, TI), range_tile_end(win, tt));
  };
  auto issue_rows = [&](int tt) {
    dma_rows_gather<E, D, NW>(ring + (size_t)(tt % SEL_RING) * slot_bytes, Y, idring + (tt % SEL_IDS) * 64, w);
  };
  if constexpr (!EXACT) {
#pragma unroll
    for (int b = 0; b < SEL_NB / 4; ++b) hist_r[g * (SEL_NB / 4) + b] = 0u;
    wave_sync();
  }

  if constexpr (!EXACT) {
    if (p.prepass && k > 0 && !p.selall) {
      // Pass 0 (windows of a few k): every logit of the row's window, the positive
      // included and items past a range's end left out, into the row's histogram
      // on [0, bound].  The bin of the (k+1)-th largest then bounds the k-th
      // largest negative from below, and the listing pass starts with its
      // threshold there instead of at -inf (far fewer entries listed).
      hlo = 0.0f;
      hsc = bnd > 0.0f ? (float)SEL_NB / bnd : 0.0f;
      for (int t0 = 0; t0 < SEL_RING && t0 < ntiles; ++t0) issue_ids(t0);
      wait_vmcnt_c<0>();
      raw_barrier();
      for (int t0 = 0; t0 < SEL_RING - 1 && t0 < ntiles; ++t0) issue_rows(t0);
      for (int t = 0; t < ntiles; ++t) {
        if (t + 1 < ntiles)
          wait_vmcnt_c<MINC>();
        else
          wait_vmcnt_c<0>();
        raw_barrier();
        if (t + SEL_RING < ntiles) issue_ids(t + SEL_RING);
        if (t + SEL_RING - 1 < ntiles) issue_rows(t + SEL_RING - 1);
        const int64_t q0 = range_tile_start(win, t, TI), q1 = range_tile_end(win, t);
        const char* slot = ring + (size_t)(t % SEL_RING) * slot_bytes;
        const int nlim = (int)(q1 - q0);
        const bool full = nlim >= TI;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          Frag<E, D> bf;
          TileFrag<E, D>::load(bf, slot, cb * 16 + r);
          const f32x4 a4 = mma_block(bf, afr, f32x4{0.f, 0.f, 0.f, 0.f});   // [item 4g+v][row r]
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            if (take && (full || cb * 16 + 4 * g + v < nlim)) {
              vmx = __builtin_amdgcn_fmed3f(vmx, a4[v], __builtin_huge_valf());
              lds_add_u32(hist_r + sel_bin(a4[v], hlo, hsc), 1u);
            }
          }
        }
      }
      raw_barrier();   // every wave is done with the ring before the listing pass refills it
      const int found = row_kth_bin(hist_r, g, r, k + 1);
      if (take) raise_from_bin(found, hlo, hsc, beta, lo);
      float rmx = fmaxf(vmx, __shfl_xor(vmx, 16));
      rmx = fmaxf(rmx, __shfl_xor(rmx, 32));
      if (take && lo > NEG_INF) {   // a fine map from the threshold to the row's largest logit
        hlo = lo;
        hsc = rmx > lo ? (float)SEL_NB / (rmx - lo) : 0.0f;
        fine = 1;
        compacted = 1;   // the list leaves out entries below a threshold: the finish ranks it
      } else {   // no threshold: the listing pass as without this pass
        hlo = -bnd;
        hsc = bnd > 0.0f ? (float)SEL_NB / (2.0f * bnd) : 0.0f;
      }
      wave_sync();
#pragma unroll
      for (int b = 0; b < SEL_NB / 4; ++b) hist_r[g * (SEL_NB / 4) + b] = 0u;
      wave_sync();
      vmx = NEG_INF;
    }
  }

  if (k > 0) {
    // the ids of tiles 0 .. 2, then the rows of tiles 0 and 1
    for (int t0 = 0; t0 < SEL_RING && t0 < ntiles; ++t0) issue_ids(t0);
    wait_vmcnt_c<0>();
    raw_barrier();
    for (int t0 = 0; t0 < SEL_RING - 1 && t0 < ntiles; ++t0) issue_rows(t0);
    for (int t = 0; t < ntiles; ++t) {
      static_assert(SEL_RING == 3 && SEL_IDS == 4, "rows two tiles ahead, ids three");
      if (t + 1 < ntiles)
        wait_vmcnt_c<MINC>();
      else
        wait_vmcnt_c<0>();
      // every wave's copies of tile t and the ids of tile t+2 landed; row slot
      // (t - 1) % RING and id slot (t - 1) % IDS are free
      raw_barrier();
      if (t + SEL_RING < ntiles) issue_ids(t + SEL_RING);
      if (t + SEL_RING - 1 < ntiles) issue_rows(t + SEL_RING - 1);
      const int64_t q0 = range_tile_start(win, t, TI), q1 = range_tile_end(win, t);
      const char* slot = ring + (size_t)(t % SEL_RING) * slot_bytes;
      const int32_t* tid_ = idring + (t % SEL_IDS) * 64;
      const int nlim = (int)(q1 - q0);   // valid items of this tile
      const bool full = nlim >= TI;

      if constexpr (!EXACT) {
        // The first raise of a row compacts its list, which rebuilds the histogram
        // on [threshold, largest value]: the initial map spans every possible logit
        // and its bins are far too coarse to follow the k-th value, so the threshold
        // would lag behind it and let through several times the candidates.
        if (!p.selall && ballot(take && !fine && cnt > k)) {
          wait_vmcnt(0);   // this wave's list stores have reached memory
          const bool act = take && !fine && cnt > k;
          compact_hist(list, act, cnt, k, beta, lo, hlo, hsc, vmx, hist_r);
          if (act) {
            fine = 1;
            last_raise = cnt;
            compacted = 1;
          }
        } else if (!p.selall && ballot(cnt > k && cnt - last_raise >= SEL_RAISE_EVERY)) {
          // threshold raises, from the histograms (no list traffic)
          const int found = row_kth_bin(hist_r, g, r, k);
          if (take && cnt > k && cnt - last_raise >= SEL_RAISE_EVERY) {
            raise_from_bin(found, hlo, hsc, beta, lo);
            last_raise = cnt;
            compacted = 1;
          }
        }
      }
      // a row takes at most TI entries from this tile: make room first (a list that
      // holds whole windows never needs it)
      if (!p.selall && ballot(cnt > cap - TI)) {
        wait_vmcnt(0);   // this wave's list stores have reached memory
        if constexpr (!EXACT) {
          const bool act = take && cnt > (cap - TI) / 2;   // more than k candidates
          compact_hist(list, act, cnt, k, beta, lo, hlo, hsc, vmx, hist_r);
          last_raise = cnt;
          compacted = compacted | (act ? 1 : 0);
          if (cnt > cap - TI) {   // the bins could not shrink the list: the exact pass redoes the row
            redo = 1;
            take = false;
            lo = __builtin_huge_valf();
            cnt = 0;
          }
        } else {
          for (int rr = 0; rr < 16; ++rr) {
            if (lane_val(cnt, rr) <= cap - TI) continue;
            int2* lrr = p.clist + (int64_t)lane_val((int)lrow, rr) * cap;
            const E* xrr = X + (int64_t)lane_val(iA, rr) * D;
            double te_n;
            int tid_n;
            compact_exact<E, D>(lrr, lane_val(cnt, rr), k, lane_val(beta, rr), xrr,
                                reinterpret_cast<const E*>(p.Y), cvals, khist, kcand, dbuf, te_n, tid_n, nexact);
            if (r == rr) {
              cnt = k;
              lo = fmaxf(lo, f_down(te_n - (double)beta * (1.0 + 1e-6)));
              compacted = 1;
            }
          }
        }
      }

      f32x4 acc[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        Frag<E, D> bf;
        TileFrag<E, D>::load(bf, slot, cb * 16 + r);
        acc[cb] = mma_block(bf, afr, f32x4{0.f, 0.f, 0.f, 0.f});   // [item 4g+v][row r]
      }
      bool any = false;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int v = 0; v < 4; ++v) any |= acc[cb][v] >= lo;
      if (ballot(any)) {
        // this lane's candidates of the tile (bit 4 cb + v), counted once; the row's
        // lanes then write to consecutive slots, lane g after lanes 0 .. g-1 of the
        // row, each in (block, v) order
        uint32_t cm = 0;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          u32x4 jj;
          const uint32_t ja = lds_addr(tid_ + cb * 16 + 4 * g);
          LdsRead128<1>::run(&ja, &jj);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int n = cb * 16 + 4 * g + v;
            const bool cand = acc[cb][v] >= lo && (full || n < nlim) && (int)jj[v] != pos;
            cm |= (uint32_t)cand << (4 * cb + v);
          }
        }
        const int c0 = popc(cm);
        const int c1 = __shfl_xor(c0, 16), c2 = __shfl_xor(c0, 32), c3 = __shfl_xor(c0, 48);   // lanes g^1, g^2, g^3
        int slotn = cnt + ((g & 1) ? c1 : 0) + ((g & 2) ? c2 + c3 : 0);
        cnt += c0 + c1 + c2 + c3;
        nlisted += (uint32_t)c0;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          if (!((cm >> (4 * cb)) & 15u)) continue;
          u32x4 jj;
          const uint32_t ja = lds_addr(tid_ + cb * 16 + 4 * g);
          LdsRead128<1>::run(&ja, &jj);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            if ((cm >> (4 * cb + v)) & 1u) {
              const float a = acc[cb][v];
              if (slotn < cap) list[slotn] = int2{(int)jj[v], __float_as_int(a)};
              ++slotn;
              if constexpr (!EXACT) {
                vmx = fmaxf(vmx, a);
                lds_add_u32(hist_r + sel_bin(a, hlo, hsc), 1u);
              }
            }
          }
        }
      }
    }
  }
  flush_count(p.counters + CNT_LOGIT_EXACT, nexact);
  flush_count(p.counters + CNT_LISTED, nlisted);
  if constexpr (!EXACT) {
    // the tightest threshold for the finishing kernel's filter
    if (!p.selall && ballot(take && cnt > k && cnt > last_raise)) {
      const int found = row_kth_bin(hist_r, g, r, k);
      if (take && cnt > k && cnt > last_raise) {
        raise_from_bin(found, hlo, hsc, beta, lo);
        compacted = 1;
      }
    }
  }
  if (rv && g == 0 && (!EXACT || take)) {
    p.clist_n[lrow] = (int)(redo ? LIST_REDO : ((uint32_t)(cnt < cap ? cnt : cap) | (compacted ? LIST_COMPACTED : 0u)));
    p.clist_lo[lrow] = redo ? NEG_INF : lo;
  }
  if constexpr (!EXACT) {
    const uint32_t nredo = (uint32_t)popc(ballot(rv && g == 0 && redo));
    if (nredo && l == 0) atomicAdd(p.counters + CNT_SEL_REDO, nredo);
  }
}

template <class E, int D>
__device__ __forceinline__ void sel_finish_row(const SelectArgs& p, char* smem, int w, int64_t row, uint32_t& nexact,
                                               uint32_t& nnear) {
  const int l = lane_id();
  const int k = p.k, cap = p.cap;
  const int64_t i = p.slot_out ? (int64_t)p.perm_x[row] : row;   // position id
  const E* X = reinterpret_cast<const E*>(p.X);
  const E* Y = reinterpret_cast<const E*>(p.Y);
  const E* xrow = X + i * D;
  const float beta = p.beta_coef * p.xnorm[i] * p.ynorm_max[0];
  const int64_t o = p.slot_out ? row : (int64_t)p.rho * p.s + row;   // output row

  const uint32_t nf = k > 0 ? (uint32_t)p.clist_n[row] : 0u;
  const int n = (int)(nf & ~(LIST_COMPACTED | LIST_REDO));
  const bool compacted = (nf & LIST_COMPACTED) != 0u;
  const int2* list = p.clist + row * (int64_t)cap;
  double te;
  int tid;
  int kept;
  float mx = NEG_INF, se = 0.0f;
  if (k == 0) {   // nothing is kept
    te = __builtin_huge_val();
    tid = -2;
    kept = 0;
  } else if (!compacted && n <= k) {   // the whole window is at most k candidates: all kept
    te = -__builtin_huge_val();
    tid = -1;
    kept = n;
    for (int t = l; t < n; t += WAVE) mx = fmaxf(mx, __int_as_float(list[t].y));
    mx = wave_max(mx);
    for (int t = l; t < n; t += WAVE) {
      const int2 e = list[t];
      se += __expf(__int_as_float(e.y) - mx);
      p.negs[o * k + t] = e.x;
      if (p.negl) p.negl[row * k + t] = __int_as_float(e.y);
    }
    se = wave_sumf(se);
  } else {
    const MergeLds L = carve_topk(smem + (size_t)w * ((topk_wave_bytes(cap) + 15) / 16 * 16), cap);
    // the entries below the row's final threshold cannot be kept: at least k others
    // beat each of them (at least k entries remain)
    const float flo = p.clist_lo[row];
    int nk = 0;
    constexpr int LB = 4;
    for (int base = 0; base < n; base += LB * WAVE) {
      int2 e[LB];
#pragma unroll
      for (int q = 0; q < LB; ++q) {
        const int t = base + q * WAVE + l;
        e[q] = t < n ? list[t] : int2{0, 0};
      }
#pragma unroll
      for (int q = 0; q < LB; ++q) {
        const int t = base + q * WAVE + l;
        const bool keep = t < n && __int_as_float(e[q].y) >= flo;
        const uint64_t mk = ballot(keep);
        if (keep) {
          const int dst = nk + popc(mk & lanemask_lt());
          L.ids[dst] = e[q].x;
          L.vals[dst] = __int_as_float(e[q].y);
        }
        nk += popc(mk);
      }
    }
    wave_sync();
    const uint32_t before = nexact;
    reduce_to_k<E, D>(L, nk, k, beta, xrow, Y, te, tid, nexact, p.counters);
    kept = k;
    if (nexact - before > 1) ++nnear;   // lane 0 holds the counts
    for (int t = l; t < kept; t += WAVE) mx = fmaxf(mx, L.vals[t]);
    mx = wave_max(mx);
    for (int t = l; t < kept; t += WAVE) {
      se += __expf(L.vals[t] - mx);
      p.negs[o * k + t] = L.ids[t];
      if (p.negl) p.negl[row * k + t] = L.vals[t];
    }
    se = wave_sumf(se);
  }
  for (int t = kept + l; t < k; t += WAVE) p.negs[o * k + t] = -1;
  if (l == 0) {
    float tlo, thi;
    if (k == 0) {
      tlo = thi = __builtin_huge_valf();
    } else if (tid == -1) {
      tlo = thi = NEG_INF;
    } else {
      const double b2 = (double)beta * (1.0 + 1e-6);
      tlo = f_down(te - b2);
      thi = f_up(te + b2);
    }
    p.thr_e[o] = te;
    p.thr_id[o] = tid;
    p.thr_lo[o] = tlo;
    p.thr_hi[o] = thi;
    p.mshift[o] = kept > 0 ? mx : 0.0f;
    p.ssum[o] = kept > 0 ? se : 0.0f;
    p.nmem[o] = kept;
  }
}

template <class E, int D>
__global__ __launch_bounds__(256, 4) void k_sel_finish(SelectArgs p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int nw = blockDim.x >> 6;
  const int w = threadIdx.x >> 6;
  // a fixed grid: each wave takes rows w0, w0 + waves, ... (no block barrier in
  // this kernel, so the waves of a workgroup run their rows independently)
  const int64_t waves = (int64_t)gridDim.x * nw;
  // counts flushed once per wave (one address shared by every wave)
  uint32_t nexact = 0, nnear = 0;
  for (int64_t row = (int64_t)blockIdx.x * nw + w; row < p.s; row += waves)
    sel_finish_row<E, D>(p, smem, w, row, nexact, nnear);
  flush_count(p.counters + CNT_LOGIT_EXACT, nexact);
  flush_count(p.counters + CNT_TOPK_EXACT, nnear);
}

template <class E, int D, int NW>
static size_t stream_lds_bytes(int cap_lds) {
  return (size_t)SEL_RING * TileGeom<E, D>::ROW_BYTES + SEL_IDS_BYTES + (size_t)NW * sel_wave_bytes(cap_lds);
}

// Waves per workgroup of the finishing kernel (LDS holds each wave's list), 0 if
// one list does not fit.
int select_finish_waves(int cap_lds) {
  const size_t per = (topk_wave_bytes(cap_lds) + 15) / 16 * 16;
  for (int nw : {4, 2, 1})
    if ((size_t)nw * per <= 160 * 1024) return nw;
  return 0;
}

size_t select_lds_bytes(bool is_bf16, int d, int waves, int cap_lds) {
#define RECE_L(E, DD)                                                   \
  if (d == DD) {                                                        \
    if (waves == 1) return stream_lds_bytes<E, DD, 1>(cap_lds);         \
    if (waves == 2) return stream_lds_bytes<E, DD, 2>(cap_lds);         \
    return stream_lds_bytes<E, DD, 4>(cap_lds);                         \
  }
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
  const int cap_lds = a.selall ? 0 : a.cap;
  if (a.k > 0) {
    const size_t lds = stream_lds_bytes<E, D, NW>(cap_lds);
    const unsigned blocks = (unsigned)((int64_t)a.n_c * a.tiles_per_chunk);
    // the histogram pass, then (lists that can be compacted only) the exact pass over
    // the rows it flagged
    for (int exact = 0; exact < (a.selall ? 1 : 2); ++exact) {
      auto kern = exact ? k_sel_stream<E, D, NW, true> : k_sel_stream<E, D, NW, false>;
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * NW), lds, st, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  const int nwf = a.selall ? 4 : select_finish_waves(cap_lds);
  if (nwf == 0) return hipErrorInvalidValue;
  const size_t lds = a.selall ? 0 : (size_t)nwf * ((topk_wave_bytes(cap_lds) + 15) / 16 * 16);
  auto fin = k_sel_finish<E, D>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fin),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  // as many workgroups as fit on the device at once (each wave loops over rows)
  int64_t fit = 0;
  e = resident_blocks(reinterpret_cast<const void*>(fin), 64 * nwf, lds, &fit);
  if (e != hipSuccess) return e;
  const int64_t want = (a.s + nwf - 1) / nwf;
  hipLaunchKernelGGL(fin, dim3((unsigned)std::max<int64_t>(1, std::min(want, fit))), dim3(64 * nwf), lds, st, a);
  return hipGetLastError();
}

hipError_t resident_blocks(const void* kernel, int threads, size_t lds, int64_t* out) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds);
  if (e != hipSuccess) return e;
  *out = (int64_t)std::max(cus, 1) * std::max(per_cu, 1);
  return hipSuccess;
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
