// Backward pass: d loss / d X and d loss / d Y with the selection held fixed
// (RECE page, Section 3, Eq. 4: softmax minus one-hot, restricted to the scored
// set {positive} u kept negatives; chained through logit = x . y).
//
// The position side reads the forward pass's kept lists; the item side has no
// list by item, so it walks the same chunk windows as the forward pass,
// recomputes the logits on the matrix cores, and decides membership of a pair
// against the per-position thresholds saved by the forward pass (float32 bounds
// first, float64 recomputation inside the bounds).  A pair already kept in an
// earlier round is skipped, so every kept pair counts once.
//   * k_dx_lists (RECE): per position, dX = sum over its listed pairs of
//     gbar exp(logit - lse) y_j plus the positive term: one gathered row per pair;
//   * k_bwd_rows (bucket variant): per (bucket, position tile), G . Y_window, G the 16x64
//     gradient block of the tile, kept in registers in the operand layout of the
//     product (bf16 hi+lo split for bf16 inputs, so G keeps ~16 significant bits;
//     float32 matrix cores for float32 inputs);
//   * k_bwd_items: per (item chunk, item tile), dY += G^T . X over the positions
//     of the three X-chunks whose windows hold the tile - a reduction grouped by
//     item in sorted order, no atomics;
//   * positives: positions sorted by positive id (LSD counting sort), then a
//     segmented reduction in fixed-size pieces plus an in-order combine of the
//     pieces of long segments.
// Rounds run one after the other on the stream; round 0 writes dX and dY, later
// rounds add, so every sum has a fixed order (bit-reproducible).
#include "rece_device.h"
#include "rece_internal.h"
#include "rece_stream.h"

namespace rece {

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Upstream gradient of position i's loss.
__device__ __forceinline__ float gbar_of(const BwdArgs& p, int64_t i) {
  return p.dloss_pp ? p.dloss_pp[i] : p.dloss[0] / (float)p.npos;
}

// Bucket variant: a pair (position, item) met in a bucket counts there only if no
// earlier bucket of the position (the first m entries of its group, starting at
// `start` in sce_sorted) also took the item.
__device__ __forceinline__ bool sce_seen_before(const BwdArgs& p, int start, int m, int j) {
  for (int e = 0; e < m; ++e) {
    const int b2 = p.sce_sorted[start + e] / p.b_x;
    if ((p.qbits[(int64_t)b2 * p.qwords + (j >> 5)] >> (j & 31)) & 1u) return true;
  }
  return false;
}

// LDS address of the transpose read giving four 16-bit values of coordinate
// 16*nb + (l % 16) for items r0 .. r0 + 3 of a swizzled bf16 tile, r0 = base +
// 4*(l/16) (ds_read_b64_tr_b16).  Within each 16-lane group, source lane j names
// 4 coordinates of one item (item r0 + j/4, coordinates 16*nb + 4*(j%4) .. +3);
// the read hands lane i coordinate i of the group's 4 items.
template <int D>
__device__ __forceinline__ const char* tile_tr4_addr(const char* rows, int base, int nb) {
  using G = TileGeom<bf16, D>;
  const int l = lane_id(), j = l & 15;
  const int row = base + 4 * (l >> 4) + (j >> 2);
  const int dim0 = 16 * nb + 4 * (j & 3);
  const int ch = (dim0 >> 3) ^ (row & G::SWM);
  return rows + row * G::RB + ch * 16 + ((dim0 >> 2) & 1) * 8;
}

// acc[nb] += G[16 positions][TI items] . tile[TI items][D] where lane l holds
// G[position l % 16][item 16*cb + 4*(l/16) + v] in gv[cb][v].  bf16: G split into
// bf16 hi + lo (~16 significant bits), k = 32 items per step, item order
// (4 of block 2ks, 4 of block 2ks+1) on both operands; f32: k = 4 items per step.
template <class E, int D>
__device__ __forceinline__ void accumulate_rows(f32x4 (&acc)[D / 16], const float (&gv)[TileGeom<E, D>::TI / 16][4],
                                                const char* rows) {
  using G = TileGeom<E, D>;
  const int l = lane_id();
  if constexpr (sizeof(E) == 2) {
#pragma unroll
    for (int ks = 0; ks < G::TI / 32; ++ks) {
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float g0 = gv[2 * ks + (e >> 2)][e & 3], g1 = gv[2 * ks + (e >> 2)][(e & 3) + 1];
        const uint32_t h0 = bf16_rne(g0), h1 = bf16_rne(g1);
        const uint32_t l0 = bf16_rne(g0 - __uint_as_float(h0 << 16)), l1 = bf16_rne(g1 - __uint_as_float(h1 << 16));
        ph[e / 2] = h0 | (h1 << 16);
        pl[e / 2] = l0 | (l1 << 16);
      }
      const bf16x8 ahi = __builtin_bit_cast(bf16x8, u32x4{ph[0], ph[1], ph[2], ph[3]});
      const bf16x8 alo = __builtin_bit_cast(bf16x8, u32x4{pl[0], pl[1], pl[2], pl[3]});
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) {
        short4v b0, b1;
        lds_tr16_pair(tile_tr4_addr<D>(rows, 32 * ks, nb), tile_tr4_addr<D>(rows, 32 * ks + 16, nb), b0, b1);
        const short4v b8[2] = {b0, b1};
        const bf16x8 b = __builtin_bit_cast(bf16x8, b8);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b, acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, b, acc[nb], 0, 0, 0);
      }
    }
  } else {
    const int g = l >> 4;
#pragma unroll
    for (int cb = 0; cb < G::TI / 16; ++cb)
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb)
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(
              gv[cb][v], tile_elem<float, D>(rows, 16 * cb + 4 * g + v, 16 * nb + (l & 15)), acc[nb], 0, 0, 0);
  }
}

// ------------------------------------------------------------------ dX
__host__ __device__ constexpr size_t rows_slot_bytes(size_t row_bytes, int rounds) {
  return row_bytes + 256 * (size_t)rounds;
}
constexpr size_t ROWS_WAVE_LDS = 16 * MAX_ROUNDS * sizeof(PrevRow);

// SCE = true: bucket variant (rows are (bucket, position) slots, window = the
// bucket's items, output = one partial row per slot, no positive term).
//
// Layout: the logit block is computed transposed (items x positions), so lane l
// holds position l % 16 for items 4*(l/16) + v of every 16-item block.  Those
// are exactly the values the G . Y product needs as its A operand (k = items,
// permuted identically on both sides), so G never goes through LDS; the B
// operand (Y transposed) comes from the row tile with the LDS transpose read.
template <class E, int D, int NW, bool SCE>
__global__ __launch_bounds__(64 * NW, (D * sizeof(E) <= 512) ? 2 : 1) void k_bwd_rows(BwdArgs p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  using G = TileGeom<E, D>;
  constexpr int TI = G::TI;
  constexpr int NCB = TI / 16;
  constexpr int TR = 16 * NW;
  const E* __restrict__ Y = reinterpret_cast<const E*>(p.Y);
  const E* __restrict__ Xs = reinterpret_cast<const E*>(p.Xs);
  const E* __restrict__ Ys = reinterpret_cast<const E*>(p.Ys);
  const int n_c = p.n_c, rho = p.rho;
  const int64_t s = p.s, C = p.C;
  const size_t slot_bytes = rows_slot_bytes(G::ROW_BYTES, p.rounds);
  char* ring = smem;
  const int w = threadIdx.x >> 6, l = lane_id(), g = l >> 4;
  PrevRow* prev = reinterpret_cast<PrevRow*>(smem + 3 * slot_bytes + (size_t)w * ROWS_WAVE_LDS);

  const int lb = xcd_block(blockIdx.x, gridDim.x);
  const int c = lb / p.tiles_per_chunk;
  const int tile_i = lb % p.tiles_per_chunk;
  const int64_t x0 = chunk_start(c, s, n_c), x1 = chunk_start(c + 1, s, n_c);
  const int64_t tile0 = x0 + (int64_t)tile_i * TR;
  if (tile0 >= x1) return;
  uint32_t nexact = 0;   // float64 logits computed by this lane
  const int64_t wrow0 = tile0 + 16 * w;
  Ranges win;
  win.init(c, n_c, C, TI, p.nwin);
  const int ntiles = win.ntiles();

  // this lane's position: row l % 16 of the wave
  const int64_t pA = wrow0 + (l & 15);
  const bool rvA = pA < x1;
  Frag<E, D> afr;
  afr.load_global(rvA ? Xs + pA * D : nullptr);
  if (l < 16)
    for (int r2 = 0; r2 < rho; ++r2) prev[l * MAX_ROUNDS + r2] = rvA ? p.prev[(int64_t)r2 * s + pA] : PrevRow{};
  const PosRec rc = p.rec[rvA ? pA : x0];
  const int posA = rvA ? rc.pos : -1;
  const float lseA = rc.lse, gbA = rc.gb, loA = rc.lo, hiA = rc.hi;
  const double teA = rc.te;
  const int tidA = rc.tid, gstA = rc.pad0, gmA = rc.pad1;
  const E* xrowA = Xs + (rvA ? pA : x0) * D;
  const PrevRow p0 = rho > 0 ? p.prev[rvA ? pA : x0] : PrevRow{};   // round 0's set of this position

  f32x4 dacc[D / 16];
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) dacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ncopies = G::ROW_DMA + 1 + rho;
  int my_copies = 0;
  for (int u = w; u < ncopies; u += NW) ++my_copies;
  __syncthreads();
  issue_window_tile<E, D, NW>(ring, slot_bytes, win, 0, Ys, p.perm_y, p.cyp, C, rho, w);
  if (ntiles > 1) issue_window_tile<E, D, NW>(ring, slot_bytes, win, 1, Ys, p.perm_y, p.cyp, C, rho, w);
  for (int t = 0; t < ntiles; ++t) {
    wait_vmcnt(t + 1 < ntiles ? my_copies : 0);
    raw_barrier();
    if (t + 2 < ntiles) issue_window_tile<E, D, NW>(ring, slot_bytes, win, t + 2, Ys, p.perm_y, p.cyp, C, rho, w);
    const int64_t q0 = range_tile_start(win, t, TI), q1 = range_tile_end(win, t);
    const char* slot = ring + (size_t)(t % 3) * slot_bytes;
    const int32_t* tid_ = reinterpret_cast<const int32_t*>(slot + G::ROW_BYTES);
    const int32_t* tcy = tid_ + 64;
    const int nlim = (int)(q1 - q0);   // valid rows of this tile
    f32x4 acc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      Frag<E, D> bf;
      TileFrag<E, D>::load(bf, slot, cb * 16 + (l & 15));
      acc[cb] = mma_block(bf, afr, f32x4{0.f, 0.f, 0.f, 0.f});   // [item 4g+v][position l%16]
    }
    float gv[NCB][4];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int n0 = cb * 16 + 4 * g;
      const u32x4 jj = *reinterpret_cast<const u32x4*>(tid_ + n0);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int n = n0 + v;
        const int j = (int)jj[v];
        const float a = acc[cb][v];
        const bool cand = rvA && n < nlim && j != posA;
        bool mem = cand && a > hiA;
        if (cand && !mem && a >= loA)   // inside the float32 bounds: float64 decides (rare)
          mem = beats<E, D>(a, loA, hiA, teA, tidA, xrowA, Y, j, nexact);
        if ((SCE || rho > 0) && mem) {
          if (SCE && gmA > 0 && sce_seen_before(p, gstA, gmA, j)) mem = false;
          if (rho > 0 && mem && in_window(p0.cx, tcy[n], n_c) &&
              beats<E, D>(a, p0.lo, p0.hi, p0.te, p0.tid, xrowA, Y, j, nexact))
            mem = false;   // kept in round 0 (registers); rounds 1 .. rho-1 below
          for (int r2 = 1; r2 < rho && mem; ++r2) {
            const PrevRow pr = prev[(l & 15) * MAX_ROUNDS + r2];
            if (!in_window(pr.cx, tcy[64 * r2 + n], n_c)) continue;
            if (beats<E, D>(a, pr.lo, pr.hi, pr.te, pr.tid, xrowA, Y, j, nexact)) mem = false;
          }
        }
        gv[cb][v] = mem ? __expf(a - lseA) * gbA : 0.0f;
      }
    }
    accumulate_rows<E, D>(dacc, gv, slot);
  }

  // write: rows 4g+v, coordinates 16nb + (l & 15); round 0 adds the positive term
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t pr = wrow0 + 4 * g + v;
    if (pr >= x1) continue;
    if (SCE) {   // partial row of this slot
      float* dst = p.dX + pr * D;
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) dst[16 * nb + (l & 15)] = dacc[nb][v];
      continue;
    }
    const PosRec rv = p.rec[pr];
    float* dst = p.dX + (int64_t)rv.i * D;
    float gpos = 0.0f;
    const int pclamp = rv.pos < 0 ? 0 : (rv.pos >= p.C ? (int)(p.C - 1) : rv.pos);
    const E* ypos = Y + (int64_t)pclamp * D;
    if (rho == 0) gpos = (expf(rv.lpos - rv.lse) - 1.0f) * rv.gb;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) {
      const int t = 16 * nb + (l & 15);
      float val = dacc[nb][v];
      if (rho == 0)
        val += gpos * to_f32(ypos[t]);
      else
        val += dst[t];
      dst[t] = val;
    }
  }
  flush_count(p.counters + CNT_LOGIT_EXACT, nexact);
}

// ------------------------------------------------------------------ dY (negatives)
template <class E, int D>
struct ItemsLayout {
  using G = TileGeom<E, D>;
  using RC = RecCopy<sizeof(PosRec), G::TI>;
  using PC = RecCopy<sizeof(PrevRow), G::TI>;
  static __host__ __device__ constexpr size_t slot_bytes(int rounds) {
    return (size_t)G::ROW_BYTES + RC::LDS_BYTES + (size_t)(rounds > 1 ? rounds - 1 : 0) * PC::LDS_BYTES;
  }
};
constexpr size_t ITEMS_WAVE_LDS = 16 * MAX_ROUNDS * 4;

// Copies of position tile t: rows of the sorted positions, their records, and their
// records of each earlier round, into ring slot t % 3.
template <class E, int D, int NW>
__device__ __forceinline__ void issue_items_tile(char* ring, size_t slot_bytes, Ranges r, int t, const E* xs,
                                                 const PosRec* rec, const PrevRow* prev, int64_t s, int rho,
                                                 int wave) {
  using G = TileGeom<E, D>;
  using LY = ItemsLayout<E, D>;
  const int64_t q0 = range_tile_start(r, t, G::TI), q1 = range_tile_end(r, t);
  char* slot = ring + (size_t)(t % 3) * slot_bytes;
  dma_rows<E, D, NW>(slot, xs, q0, q1, wave);
  char* rb = slot + G::ROW_BYTES;
  LY::RC::template issue<NW>(rb, rec, q0, q1, G::ROW_DMA, wave);
  for (int r2 = 0; r2 < rho; ++r2)
    LY::PC::template issue<NW>(rb + LY::RC::LDS_BYTES + (size_t)r2 * LY::PC::LDS_BYTES, prev + (int64_t)r2 * s, q0,
                               q1, G::ROW_DMA + LY::RC::COPIES + r2 * LY::PC::COPIES, wave);
}

// Transposed logit block as in k_bwd_rows: lane l holds item l % 16 of the wave
// and positions 4*(l/16) + v of every 16-position block of the tile, the A
// operand of dY = G^T . X; X transposed comes from the tile by transpose reads.
template <class E, int D, int NW, bool SCE>
__global__ __launch_bounds__(64 * NW, (D * sizeof(E) <= 512) ? 2 : 1) void k_bwd_items(BwdArgs p, int itiles) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  using G = TileGeom<E, D>;
  using LY = ItemsLayout<E, D>;
  constexpr int TI = G::TI;
  constexpr int NCB = TI / 16;
  constexpr int TR = 16 * NW;
  const E* __restrict__ Y = reinterpret_cast<const E*>(p.Y);
  const E* __restrict__ Xs = reinterpret_cast<const E*>(p.Xs);
  const E* __restrict__ Ys = reinterpret_cast<const E*>(p.Ys);
  const int n_c = p.n_c, rho = p.rho;
  const int64_t s = p.s, C = p.C;
  const size_t slot_bytes = LY::slot_bytes(p.rounds);
  char* ring = smem;
  const int w = threadIdx.x >> 6, l = lane_id(), g = l >> 4;
  int32_t* cy2w = reinterpret_cast<int32_t*>(smem + 3 * slot_bytes + (size_t)w * ITEMS_WAVE_LDS);   // [16][MAX_ROUNDS]

  const int lb = xcd_block(blockIdx.x, gridDim.x);
  const int c = lb / itiles;
  const int it = lb % itiles;
  const int64_t y0 = chunk_start(c, C, n_c), y1 = chunk_start(c + 1, C, n_c);
  const int64_t tile0 = y0 + (int64_t)it * TR;
  if (tile0 >= y1) return;
  uint32_t nexact = 0;   // float64 logits computed by this lane
  const int64_t wq0 = tile0 + 16 * w;
  Ranges xr;
  xr.init(c, n_c, s, TI, p.nwin);   // X-chunks whose window holds item chunk c (the relation is symmetric)
  const int ntiles = xr.ntiles();

  // this lane's item: row l % 16 of the wave
  const int64_t qA = wq0 + (l & 15);
  const bool rvA = qA < y1;
  const int jA = rvA ? p.perm_y[qA] : -1;
  const int cy0 = (rho > 0 && rvA) ? p.cyp[qA] : 0;   // this item's chunk in round 0
  Frag<E, D> afr;
  afr.load_global(rvA ? Ys + qA * D : nullptr);
  if (l < 16)
    for (int r2 = 0; r2 < rho; ++r2) cy2w[l * MAX_ROUNDS + r2] = rvA ? p.cyp[(int64_t)r2 * C + qA] : 0;
  f32x4 dacc[D / 16];
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) dacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ncopies = G::ROW_DMA + LY::RC::COPIES + rho * LY::PC::COPIES;
  int my_copies = 0;
  for (int u = w; u < ncopies; u += NW) ++my_copies;

  __syncthreads();
  issue_items_tile<E, D, NW>(ring, slot_bytes, xr, 0, Xs, p.rec, p.prev, s, rho, w);
  if (ntiles > 1) issue_items_tile<E, D, NW>(ring, slot_bytes, xr, 1, Xs, p.rec, p.prev, s, rho, w);
  for (int t = 0; t < ntiles; ++t) {
    wait_vmcnt(t + 1 < ntiles ? my_copies : 0);
    raw_barrier();
    if (t + 2 < ntiles) issue_items_tile<E, D, NW>(ring, slot_bytes, xr, t + 2, Xs, p.rec, p.prev, s, rho, w);
    const int64_t q0 = range_tile_start(xr, t, TI), q1 = range_tile_end(xr, t);
    const char* slot = ring + (size_t)(t % 3) * slot_bytes;
    const PosRec* recs = reinterpret_cast<const PosRec*>(slot + G::ROW_BYTES);
    const PrevRow* prevs = reinterpret_cast<const PrevRow*>(slot + G::ROW_BYTES + LY::RC::LDS_BYTES);
    const int nlim = (int)(q1 - q0);   // valid rows of this tile
    f32x4 acc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      Frag<E, D> bf;
      TileFrag<E, D>::load(bf, slot, cb * 16 + (l & 15));
      acc[cb] = mma_block(bf, afr, f32x4{0.f, 0.f, 0.f, 0.f});   // [position 4g+v][item l%16]
    }
    float gv[NCB][4];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int n = cb * 16 + 4 * g + v;
        const f32x4 hot = *reinterpret_cast<const f32x4*>(&recs[n].lse);   // lse, gb, lo, hi
        const int pos_n = recs[n].pos;
        const float a = acc[cb][v];
        const bool cand = rvA && n < nlim && jA != pos_n;
        bool mem = cand && a > hot[3];
        if (cand && !mem && a >= hot[2])   // inside the float32 bounds: float64 decides (rare)
          mem = beats<E, D>(a, hot[2], hot[3], recs[n].te, recs[n].tid, Xs + (q0 + n) * D, Y, jA, nexact);
        if ((SCE || rho > 0) && mem) {
          if (SCE && recs[n].pad1 > 0 && sce_seen_before(p, recs[n].pad0, recs[n].pad1, jA)) mem = false;
          for (int r2 = 0; r2 < rho && mem; ++r2) {
            const int cyr = r2 == 0 ? cy0 : cy2w[(l & 15) * MAX_ROUNDS + r2];
            if (!in_window(prevs[(size_t)r2 * (LY::PC::LDS_BYTES / sizeof(PrevRow)) + n].cx, cyr, n_c)) continue;
            const PrevRow pr = prevs[(size_t)r2 * (LY::PC::LDS_BYTES / sizeof(PrevRow)) + n];
            if (beats<E, D>(a, pr.lo, pr.hi, pr.te, pr.tid, Xs + (q0 + n) * D, Y, jA, nexact)) mem = false;
          }
        }
        gv[cb][v] = mem ? __expf(a - hot[0]) * hot[1] : 0.0f;
      }
    }
    accumulate_rows<E, D>(dacc, gv, slot);
  }

#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t qr = wq0 + 4 * g + v;
    if (qr >= y1) continue;
    float* dst = p.dY + (SCE ? qr : (int64_t)p.perm_y[qr]) * D;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) {
      const int t = 16 * nb + (l & 15);
      float val = dacc[nb][v];
      if (rho > 0) val += dst[t];
      dst[t] = val;
    }
  }
  flush_count(p.counters + CNT_LOGIT_EXACT, nexact);
}

// ------------------------------------------------------------------ dX from the kept lists
// Sixteen bytes of a row as floats.
__device__ __forceinline__ void load16f(const bf16* ptr, float (&v)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(ptr);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    v[2 * t] = __uint_as_float(w[t] << 16);
    v[2 * t + 1] = __uint_as_float(w[t] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load16f(const float* ptr, float (&v)[4]) {
  const float4 u = *reinterpret_cast<const float4*>(ptr);
  v[0] = u.x;
  v[1] = u.y;
  v[2] = u.z;
  v[3] = u.w;
}

// One wave per position i (RECE page, Eq. 4, the position side):
//   dX_i = sum over the kept pairs (i, j) of every round that no earlier round
//          kept (list ids >= 0) of gbar_i exp(x_i . y_j - lse_i) y_j
//        + (exp(lpos_i - lse_i) - 1) gbar_i y_pos.
// The logit is recomputed in float32 from the two rows the sum reads anyway.
// Lanes work in groups of LPR, each lane on 16 bytes of a row: group q takes list
// entry RPI * step + q, UNR steps in flight; at the end the groups' partial rows
// are added in a fixed order, so the result is bit-reproducible.
template <class E, int D>
__global__ __launch_bounds__(256) void k_dx_lists(BwdArgs p) {
  constexpr int EPL = 16 / (int)sizeof(E);   // elements per lane
  constexpr int LPR = D / EPL;               // lanes per row
  constexpr int RPI = WAVE / LPR;            // rows per step
  constexpr int UNR = RPI >= 4 ? 4 : 8;      // steps in flight
  static_assert(LPR >= 1 && LPR <= WAVE && (LPR & (LPR - 1)) == 0, "row split");
  const E* __restrict__ X = reinterpret_cast<const E*>(p.X);
  const E* __restrict__ Y = reinterpret_cast<const E*>(p.Y);
  const int l = lane_id();
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= p.s) return;
  const int q = l / LPR, sub = l % LPR;
  float x[EPL];
  load16f(X + i * D + sub * EPL, x);
  const float lse = p.lse[i];
  const float gb = gbar_of(p, i);
  float acc[EPL];
#pragma unroll
  for (int t = 0; t < EPL; ++t) acc[t] = 0.0f;
  const int k = p.k;
  for (int rho = 0; rho < p.rounds; ++rho) {
    const int32_t* list = p.negs + ((int64_t)rho * p.s + i) * k;
    for (int e0 = 0; e0 < k; e0 += WAVE) {
      const int ent = e0 + l < k ? list[e0 + l] : -1;
      const uint64_t vm = ballot(ent >= 0);
      if (!vm) continue;
      const int nstep = (64 - __builtin_clzll(vm) + RPI - 1) / RPI;   // steps up to the last listed entry
      for (int t0 = 0; t0 < nstep; t0 += UNR) {
        float y[UNR][EPL];
        int jj[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int e = (t0 + u) * RPI + q;
          const int j = __shfl(ent, e < WAVE ? e : 0);
          jj[u] = (t0 + u < nstep && e < WAVE) ? j : -1;
          if (jj[u] >= 0) {
            load16f(Y + (int64_t)jj[u] * D + sub * EPL, y[u]);
          } else {
#pragma unroll
            for (int t = 0; t < EPL; ++t) y[u][t] = 0.0f;
          }
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          float dot = 0.0f;
#pragma unroll
          for (int t = 0; t < EPL; ++t) dot = fmaf(x[t], y[u][t], dot);
#pragma unroll
          for (int o = 1; o < LPR; o <<= 1) dot += __shfl_xor(dot, o);
          const float g = jj[u] >= 0 ? __expf(dot - lse) * gb : 0.0f;
#pragma unroll
          for (int t = 0; t < EPL; ++t) acc[t] = fmaf(g, y[u][t], acc[t]);
        }
      }
    }
  }
  // the positive term, in group 0
  if (q == 0) {
    const int pj = p.pos[i];
    const int pc = pj < 0 ? 0 : (pj >= p.C ? (int)(p.C - 1) : pj);
    const float gpos = (expf(p.lpos[i] - lse) - 1.0f) * gb;
    float yp[EPL];
    load16f(Y + (int64_t)pc * D + sub * EPL, yp);
#pragma unroll
    for (int t = 0; t < EPL; ++t) acc[t] = fmaf(gpos, yp[t], acc[t]);
  }
#pragma unroll
  for (int o = LPR; o < WAVE; o <<= 1)
#pragma unroll
    for (int t = 0; t < EPL; ++t) acc[t] += __shfl_xor(acc[t], o);
  if (q == 0) {
    float4* dst = reinterpret_cast<float4*>(p.dX + i * D + sub * EPL);
#pragma unroll
    for (int t = 0; t < EPL / 4; ++t) dst[t] = float4{acc[4 * t], acc[4 * t + 1], acc[4 * t + 2], acc[4 * t + 3]};
  }
}

__global__ void k_strip_mark(const int32_t* __restrict__ src, int64_t n, int32_t* __restrict__ dst) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) {
    const int v = src[t];
    dst[t] = v == -1 ? -1 : (v & 0x7FFFFFFF);
  }
}

// ------------------------------------------------------------------ dY (positives)
constexpr int PIECE = 64;   // sorted positions per piece (one wave)

// pflag bits per piece: 1 = head run continues from the previous piece,
// 2 = head run continues into the next piece, 4 = a tail run starts here and continues.
// Runs that neither come from the previous piece nor continue into the next are
// staged (item and row) and added to dY by k_pos_combine: the pieces kernel reads
// and writes nothing of dY, so it can run while dY is still being written.
struct PosStage {
  int32_t* n;       // [npieces] staged runs of each piece
  int32_t* items;   // [npieces * PIECE]
  float* rows;      // [npieces * PIECE][D]
};

template <class E, int D>
__global__ __launch_bounds__(256) void k_pos_pieces(BwdArgs p, const int32_t* __restrict__ sorted,
                                                    float* __restrict__ partial, int32_t* __restrict__ pitem,
                                                    int32_t* __restrict__ pflag, PosStage stage, int64_t npieces) {
  constexpr int PER = (D + 63) / 64;   // coordinates per lane
  const E* __restrict__ X = reinterpret_cast<const E*>(p.X);
  const int w = threadIdx.x >> 6, l = lane_id();
  const int64_t piece = (int64_t)blockIdx.x * 4 + w;
  if (piece >= npieces) return;
  const int64_t s = p.s;
  const int64_t t0 = piece * PIECE, t1 = min(s, t0 + PIECE);
  float acc[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) acc[u] = 0.0f;
  int flags = 0;
  int head_item = -1, tail_item = -1;
  int nstage = 0;
  const int prev_item = t0 > 0 ? p.pos[sorted[t0 - 1]] : -1;
  const int next_item = t1 < s ? p.pos[sorted[t1]] : -1;
  // lane e holds sorted position t0 + e: its id, positive item and coefficient (all
  // loads in parallel); the walk below takes them with uniform lane reads
  const int nt = (int)(t1 - t0);
  const int i_l = l < nt ? sorted[t0 + l] : 0;
  const int item_l = l < nt ? p.pos[i_l] : -1;
  const float gp_l = l < nt ? (expf(p.lpos[i_l] - p.lse[i_l]) - 1.0f) * gbar_of(p, i_l) : 0.0f;
  int cur = __builtin_amdgcn_readfirstlane(item_l);
  int64_t run_start = t0;
  constexpr int BATCH = 8;   // rows of X in flight
  for (int tb = 0; tb < nt; tb += BATCH) {
    float xv[BATCH][PER];
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      const int i = __builtin_amdgcn_readlane(i_l, tb + q < nt ? tb + q : 0);
      const E* xr = X + (int64_t)i * D;
#pragma unroll
      for (int u = 0; u < PER; ++u) xv[q][u] = (tb + q < nt && l + 64 * u < D) ? to_f32(xr[l + 64 * u]) : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      if (tb + q >= nt) break;
      const int64_t t = t0 + tb + q;
      const int item = __builtin_amdgcn_readlane(item_l, tb + q);
      if (item != cur) {
        // flush the run [run_start, t) of item cur
        if (run_start == t0 && prev_item == cur) {
          head_item = cur;
          flags |= 1;
#pragma unroll
          for (int u = 0; u < PER; ++u)
            if (l + 64 * u < D) partial[(piece * 2 + 0) * D + l + 64 * u] = acc[u];
        } else if (cur >= 0 && cur < p.C) {
          const int64_t slot = piece * PIECE + nstage++;
          if (l == 0) stage.items[slot] = cur;
#pragma unroll
          for (int u = 0; u < PER; ++u)
            if (l + 64 * u < D) stage.rows[slot * D + l + 64 * u] = acc[u];
        }
#pragma unroll
        for (int u = 0; u < PER; ++u) acc[u] = 0.0f;
        cur = item;
        run_start = t;
      }
      const float gp = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gp_l), tb + q));
#pragma unroll
      for (int u = 0; u < PER; ++u) acc[u] = fmaf(gp, xv[q][u], acc[u]);
    }
  }
  // last run [run_start, t1)
  const bool from_prev = run_start == t0 && prev_item == cur;
  const bool to_next = next_item == cur;
  if (from_prev) {
    head_item = cur;
    flags |= 1;
    if (to_next) flags |= 2;
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (l + 64 * u < D) partial[(piece * 2 + 0) * D + l + 64 * u] = acc[u];
  } else if (to_next) {
    tail_item = (cur >= 0 && cur < p.C) ? cur : -1;
    flags |= 4;
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (l + 64 * u < D) partial[(piece * 2 + 1) * D + l + 64 * u] = acc[u];
  } else if (cur >= 0 && cur < p.C) {
    const int64_t slot = piece * PIECE + nstage++;
    if (l == 0) stage.items[slot] = cur;
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (l + 64 * u < D) stage.rows[slot * D + l + 64 * u] = acc[u];
  }
  if (l == 0) {
    pitem[piece * 2 + 0] = head_item;
    pitem[piece * 2 + 1] = tail_item;
    pflag[piece] = flags;
    stage.n[piece] = nstage;
  }
}

// Per piece: add its staged runs to dY (each item's positions form one run, so
// no other wave writes those rows); then, for a run that starts in this piece and
// continues, add the head partials of the following pieces, in order, until the
// run ends.
template <int D>
__global__ __launch_bounds__(256) void k_pos_combine(float* __restrict__ dY, const float* __restrict__ partial,
                                                     const int32_t* __restrict__ pitem,
                                                     const int32_t* __restrict__ pflag, PosStage stage,
                                                     int64_t npieces) {
  constexpr int PER = (D + 63) / 64;
  const int w = threadIdx.x >> 6, l = lane_id();
  const int64_t piece = (int64_t)blockIdx.x * 4 + w;
  if (piece >= npieces) return;
  {
    // the piece's staged runs, each added once to its item's row: 16 bytes per lane,
    // RPI rows per instruction, BATCH instructions in flight
    static_assert(D % 4 == 0 && D <= 256, "rows of whole 16-byte chunks, at most 64 per row");
    constexpr int LPR = D / 4, RPI = 64 / LPR, BATCH = 8;
    const int q = l / LPR, sub = l % LPR;
    const int ns = stage.n[piece];
    for (int e0 = 0; e0 < ns; e0 += RPI * BATCH) {
      float4 rv[BATCH], yv[BATCH];
      int64_t base[BATCH];
#pragma unroll
      for (int e = 0; e < BATCH; ++e) {
        const int idx = e0 + e * RPI + q;
        const bool in = q < RPI && idx < ns;
        const int64_t slot = piece * PIECE + (in ? idx : 0);
        base[e] = (int64_t)stage.items[slot] * D + 4 * sub;
        rv[e] = in ? *reinterpret_cast<const float4*>(stage.rows + slot * D + 4 * sub) : float4{0.f, 0.f, 0.f, 0.f};
        yv[e] = in ? *reinterpret_cast<const float4*>(dY + base[e]) : float4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int e = 0; e < BATCH; ++e)
        if (q < RPI && e0 + e * RPI + q < ns)
          *reinterpret_cast<float4*>(dY + base[e]) =
              float4{yv[e].x + rv[e].x, yv[e].y + rv[e].y, yv[e].z + rv[e].z, yv[e].w + rv[e].w};
    }
  }
  if (!(pflag[piece] & 4)) return;
  const int item = pitem[piece * 2 + 1];
  if (item < 0) return;
  float acc[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) acc[u] = l + 64 * u < D ? partial[(piece * 2 + 1) * D + l + 64 * u] : 0.0f;
  // the run covers pieces piece+1 .. the first one whose head run does not continue
  // (flag 2 clear) or the last piece; 64 flags are read at once, then the partial
  // rows in order, several loads in flight
  for (int64_t q0 = piece + 1; q0 < npieces; q0 += WAVE) {
    const int64_t qq = q0 + l;
    const int f = qq < npieces ? pflag[qq] : 0;
    const uint64_t stop = ballot(qq >= npieces || !(f & 2));
    const int nin = stop ? (int)min((int64_t)__builtin_ctzll(stop) + 1, npieces - q0) : WAVE;
    constexpr int BATCH = 8;
    for (int e0 = 0; e0 < nin; e0 += BATCH) {
      float pv[BATCH][PER];
#pragma unroll
      for (int e = 0; e < BATCH; ++e)
#pragma unroll
        for (int u = 0; u < PER; ++u)
          pv[e][u] = (e0 + e < nin && l + 64 * u < D) ? partial[((q0 + e0 + e) * 2 + 0) * D + l + 64 * u] : 0.0f;
#pragma unroll
      for (int e = 0; e < BATCH; ++e)
#pragma unroll
        for (int u = 0; u < PER; ++u) acc[u] += pv[e][u];
    }
    if (stop) break;
  }
  float* dst = dY + (int64_t)item * D;
#pragma unroll
  for (int u = 0; u < PER; ++u)
    if (l + 64 * u < D) dst[l + 64 * u] += acc[u];
}

// ------------------------------------------------------------------ launchers
template <class E, int D>
static size_t rows_lds(int NW, int rounds) {
  return 3 * rows_slot_bytes(TileGeom<E, D>::ROW_BYTES, rounds) + (size_t)NW * ROWS_WAVE_LDS;
}
template <class E, int D>
static size_t items_lds(int NW, int rounds) {
  return 3 * ItemsLayout<E, D>::slot_bytes(rounds) + (size_t)NW * ITEMS_WAVE_LDS;
}

template <class E, int D, int NW, bool SCE>
static hipError_t launch_rows_t(const BwdArgs& a, hipStream_t st) {
  const size_t lds = rows_lds<E, D>(NW, a.rounds);
  auto kern = k_bwd_rows<E, D, NW, SCE>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)((int64_t)a.n_c * a.tiles_per_chunk)), dim3(64 * NW), lds, st, a);
  return hipGetLastError();
}
template <class E, int D, int NW, bool SCE>
static hipError_t launch_items_t(const BwdArgs& a, int itiles, hipStream_t st) {
  const size_t lds = items_lds<E, D>(NW, a.rounds);
  auto kern = k_bwd_items<E, D, NW, SCE>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)((int64_t)a.n_c * itiles)), dim3(64 * NW), lds, st, a, itiles);
  return hipGetLastError();
}

hipError_t launch_bwd_rows(bool bf16v, int d, int waves, const BwdArgs& a, hipStream_t st) {
#define RECE_R(E, DD) \
  if (d == DD) return a.sce ? launch_rows_t<E, DD, 4, true>(a, st) : launch_rows_t<E, DD, 4, false>(a, st);
  (void)waves;
  if (bf16v) {
    RECE_R(bf16, 32) RECE_R(bf16, 64) RECE_R(bf16, 128) RECE_R(bf16, 256)
  } else {
    RECE_R(float, 32) RECE_R(float, 64) RECE_R(float, 128) RECE_R(float, 256)
  }
#undef RECE_R
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_items(bool bf16v, int d, int waves, const BwdArgs& a, int itiles, hipStream_t st) {
#define RECE_I(E, DD) \
  if (d == DD)                                                                    \
    return a.sce ? launch_items_t<E, DD, 4, true>(a, itiles, st) : launch_items_t<E, DD, 4, false>(a, itiles, st);
  (void)waves;
  if (bf16v) {
    RECE_I(bf16, 32) RECE_I(bf16, 64) RECE_I(bf16, 128) RECE_I(bf16, 256)
  } else {
    RECE_I(float, 32) RECE_I(float, 64) RECE_I(float, 128) RECE_I(float, 256)
  }
#undef RECE_I
  return hipErrorInvalidValue;
}

// The work area: head/tail partial rows [npieces][2][D] floats, staged rows
// [npieces * PIECE][D] floats, then pitem [npieces][2], pflag [npieces], staged
// counts [npieces] and staged items [npieces * PIECE], all int32.
struct PosArea {
  float* partial;
  int32_t* pitem;
  int32_t* pflag;
  PosStage stage;
  int64_t npieces;
};
static PosArea pos_area(float* base, int64_t s, int d) {
  PosArea a;
  a.npieces = (s + PIECE - 1) / PIECE;
  a.partial = base;
  a.stage.rows = base + a.npieces * 2 * d;
  a.pitem = reinterpret_cast<int32_t*>(a.stage.rows + a.npieces * PIECE * d);
  a.pflag = a.pitem + a.npieces * 2;
  a.stage.n = a.pflag + a.npieces;
  a.stage.items = a.stage.n + a.npieces;
  return a;
}

template <class E, int D>
static hipError_t launch_pieces_t(const BwdArgs& a, const int32_t* sorted, float* area, hipStream_t st) {
  const PosArea w = pos_area(area, a.s, D);
  const unsigned blocks = (unsigned)((w.npieces + 3) / 4);
  hipLaunchKernelGGL((k_pos_pieces<E, D>), dim3(blocks), dim3(256), 0, st, a, sorted, w.partial, w.pitem, w.pflag,
                     w.stage, w.npieces);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_combine_t(int64_t s, float* dY, float* area, hipStream_t st) {
  const PosArea w = pos_area(area, s, D);
  const unsigned blocks = (unsigned)((w.npieces + 3) / 4);
  hipLaunchKernelGGL((k_pos_combine<D>), dim3(blocks), dim3(256), 0, st, dY, w.partial, w.pitem, w.pflag, w.stage,
                     w.npieces);
  return hipGetLastError();
}

hipError_t launch_pos_pieces(bool bf16v, int d, const BwdArgs& a, const int32_t* sorted, float* area,
                             hipStream_t st) {
  if (a.s == 0) return hipSuccess;
#define RECE_P(E, DD) \
  if (d == DD) return launch_pieces_t<E, DD>(a, sorted, area, st);
  if (bf16v) {
    RECE_P(bf16, 32) RECE_P(bf16, 64) RECE_P(bf16, 128) RECE_P(bf16, 256)
  } else {
    RECE_P(float, 32) RECE_P(float, 64) RECE_P(float, 128) RECE_P(float, 256)
  }
#undef RECE_P
  return hipErrorInvalidValue;
}

hipError_t launch_pos_combine(int d, int64_t s, float* dY, float* area, hipStream_t st) {
  if (s == 0) return hipSuccess;
  switch (d) {
    case 32: return launch_combine_t<32>(s, dY, area, st);
    case 64: return launch_combine_t<64>(s, dY, area, st);
    case 128: return launch_combine_t<128>(s, dY, area, st);
    case 256: return launch_combine_t<256>(s, dY, area, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_pos_dy(bool bf16v, int d, const BwdArgs& a, const int32_t* sorted, float* area,
                         hipStream_t st) {
  const hipError_t e = launch_pos_pieces(bf16v, d, a, sorted, area, st);
  if (e != hipSuccess) return e;
  return launch_pos_combine(d, a.s, a.dY, area, st);
}

hipError_t launch_dx_lists(bool bf16v, int d, const BwdArgs& a, hipStream_t st) {
  if (a.s == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((a.s + 3) / 4);
#define RECE_DXL(E, DD) \
  if (d == DD) {        \
    hipLaunchKernelGGL((k_dx_lists<E, DD>), dim3(blocks), dim3(256), 0, st, a); \
    return hipGetLastError(); \
  }
  if (bf16v) {
    RECE_DXL(bf16, 32) RECE_DXL(bf16, 64) RECE_DXL(bf16, 128) RECE_DXL(bf16, 256)
  } else {
    RECE_DXL(float, 32) RECE_DXL(float, 64) RECE_DXL(float, 128) RECE_DXL(float, 256)
  }
#undef RECE_DXL
  return hipErrorInvalidValue;
}

hipError_t launch_strip_mark(const int32_t* src, int64_t n, int32_t* dst, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_strip_mark, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src, n, dst);
  return hipGetLastError();
}

size_t pos_partial_bytes(int64_t s, int d) {
  const int64_t npieces = (s + PIECE - 1) / PIECE;
  return (size_t)npieces * (2 + PIECE) * d * 4 + (size_t)npieces * (4 + PIECE) * 4;
}

}  // namespace rece
