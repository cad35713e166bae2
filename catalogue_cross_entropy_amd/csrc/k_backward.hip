// Backward pass: d loss / d X and d loss / d Y with the selection held fixed
// (RECE page, Section 3, Eq. 4: softmax minus one-hot, restricted to the scored
// set {positive} u kept negatives; chained through logit = x . y).
//
// No list of kept pairs exists: each kernel walks the same chunk windows as the
// forward pass, recomputes the logits on the matrix cores, and decides
// membership of a pair against the per-position thresholds saved by the forward
// pass (float32 bounds first, float64 recomputation inside the bounds).  A pair
// already kept in an earlier round is skipped, so every kept pair counts once.
//   * k_bwd_rows: per (X-chunk, position tile), dX += G . Y_window, G the 16x64
//     gradient block of the tile (bf16 hi+lo split for bf16 inputs, so G keeps
//     ~16 significant bits; float32 matrix cores for float32 inputs);
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

namespace rece {

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Upstream gradient of position i's loss.
__device__ __forceinline__ float gbar_of(const BwdArgs& p, int64_t i) {
  return p.dloss_pp ? p.dloss_pp[i] : p.dloss[0] / (float)p.s;
}

template <class E> struct TPitch;
template <> struct TPitch<bf16> { static constexpr int value = 72; };
template <> struct TPitch<float> { static constexpr int value = 68; };
constexpr int GP = 68;   // pitch of the per-wave gradient block [16][64]

// Stage 64 vectors (ids[n] >= 0, else zeros) as a row-major tile [64][P] and a
// transposed tile [D][TP].
template <class E, int D>
__device__ __forceinline__ void load_tiles(const E* __restrict__ src, const int32_t* ids, E* tile, E* tileT,
                                           int nthreads) {
  constexpr int P = Pitch<E, D>::value;
  constexpr int TP = TPitch<E>::value;
  constexpr int EPP = 16 / (int)sizeof(E);
  constexpr int PIECES = D / EPP;
  for (int pc = threadIdx.x; pc < 64 * PIECES; pc += nthreads) {
    const int nb = pc / PIECES, part = pc % PIECES;
    const int j = ids[nb];
    u32x4 val = {0u, 0u, 0u, 0u};
    if (j >= 0) val = *reinterpret_cast<const u32x4*>(src + (int64_t)j * D + part * EPP);
    *reinterpret_cast<u32x4*>(tile + nb * P + part * EPP) = val;
    const E* ev = reinterpret_cast<const E*>(&val);
#pragma unroll
    for (int t = 0; t < EPP; ++t) tileT[(part * EPP + t) * TP + nb] = ev[t];
  }
}

// acc[nb] += G[16][64] . T[d][64]^T for the wave's 16 rows; G in LDS (float).
template <class E, int D>
__device__ __forceinline__ void accumulate_gt(f32x4 (&acc)[D / 16], const float* G, const E* tileT) {
  constexpr int TP = TPitch<E>::value;
  const int l = lane_id();
  const int q = l >> 4;
  if constexpr (sizeof(E) == 2) {
    bf16x8 ahi[2], alo[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint16_t h[8], lo[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float gv = G[(l & 15) * GP + 32 * ks + 8 * q + t];
        h[t] = bf16_rne(gv);
        lo[t] = bf16_rne(gv - __uint_as_float((uint32_t)h[t] << 16));
      }
      u32x4 ph, pl;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        ph[t] = (uint32_t)h[2 * t] | ((uint32_t)h[2 * t + 1] << 16);
        pl[t] = (uint32_t)lo[2 * t] | ((uint32_t)lo[2 * t + 1] << 16);
      }
      ahi[ks] = __builtin_bit_cast(bf16x8, ph);
      alo[ks] = __builtin_bit_cast(bf16x8, pl);
    }
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) {
      const E* trow = tileT + (16 * nb + (l & 15)) * TP;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(trow + 32 * ks + 8 * q);
        const bf16x8 b = __builtin_bit_cast(bf16x8, raw);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[ks], b, acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[ks], b, acc[nb], 0, 0, 0);
      }
    }
  } else {
    float av[16];
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) av[ks] = G[(l & 15) * GP + 4 * ks + q];
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) {
      const float* trow = reinterpret_cast<const float*>(tileT) + (16 * nb + (l & 15)) * TP;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[ks], trow[4 * ks + q], acc[nb], 0, 0, 0);
    }
  }
}

template <class E, int D>
__host__ __device__ constexpr size_t bwd_common_lds() {
  return (size_t)64 * Pitch<E, D>::value * sizeof(E) + (size_t)D * TPitch<E>::value * sizeof(E) + 64 * 4 +
         (size_t)MAX_ROUNDS * 64 * 4;
}

// ------------------------------------------------------------------ dX
template <class E, int D, int NW>
__global__ __launch_bounds__(64 * NW) void k_bwd_rows(BwdArgs p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int P = Pitch<E, D>::value;
  constexpr int TR = 16 * NW;
  const E* __restrict__ X = reinterpret_cast<const E*>(p.X);
  const E* __restrict__ Y = reinterpret_cast<const E*>(p.Y);
  E* tile = reinterpret_cast<E*>(smem);
  E* tileT = tile + 64 * P;
  int32_t* yid = reinterpret_cast<int32_t*>(tileT + D * TPitch<E>::value);
  int32_t* cy2s = yid + 64;   // [MAX_ROUNDS][64]
  const int w = threadIdx.x >> 6, l = lane_id(), g = l >> 4;
  char* wb = smem + bwd_common_lds<E, D>() + (size_t)w * (16 * GP * 4 + 16 * MAX_ROUNDS * sizeof(PrevRow));
  float* G = reinterpret_cast<float*>(wb);
  PrevRow* prev = reinterpret_cast<PrevRow*>(wb + 16 * GP * 4);
  const int n_c = p.n_c, rho = p.rho;
  const int64_t s = p.s;

  const int c = blockIdx.x / p.tiles_per_chunk;
  const int tile_i = blockIdx.x % p.tiles_per_chunk;
  const int64_t x0 = chunk_start(c, s, n_c), x1 = chunk_start(c + 1, s, n_c);
  const int64_t tile0 = x0 + (int64_t)tile_i * TR;
  if (tile0 >= x1) return;
  const int64_t wrow0 = tile0 + 16 * w;

  int wc[3];
  int nwc = 0;
  wc[nwc++] = c;
  if (n_c >= 2) wc[nwc++] = (c + n_c - 1) % n_c;
  if (n_c >= 3) wc[nwc++] = (c + 1) % n_c;

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
      prev[l * MAX_ROUNDS + r2] = pr;
    }
  }

  int i_v[4], pos_v[4], tid_v[4];
  float lse_v[4], gb_v[4], lo_v[4], hi_v[4];
  double te_v[4];
  bool rv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t pr = wrow0 + 4 * g + v;
    rv[v] = pr < x1;
    const int i = rv[v] ? p.perm_x[pr] : 0;
    const int64_t o = (int64_t)rho * s + i;
    i_v[v] = i;
    pos_v[v] = rv[v] ? p.pos[i] : -1;
    lse_v[v] = p.lse[i];
    gb_v[v] = gbar_of(p, i);
    lo_v[v] = p.thr_lo[o];
    hi_v[v] = p.thr_hi[o];
    te_v[v] = p.thr_e[o];
    tid_v[v] = p.thr_id[o];
  }
  f32x4 dacc[D / 16];
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) dacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int q = 0; q < nwc; ++q) {
    const int64_t y0 = chunk_start(wc[q], p.C, n_c), y1 = chunk_start(wc[q] + 1, p.C, n_c);
    for (int64_t q0 = y0; q0 < y1; q0 += 64) {
      __syncthreads();
      if (threadIdx.x < 64) {
        const int j = q0 + threadIdx.x < y1 ? p.perm_y[q0 + threadIdx.x] : -1;
        yid[threadIdx.x] = j;
        for (int r2 = 0; r2 < rho; ++r2)
          cy2s[r2 * 64 + threadIdx.x] = j >= 0 ? chunk_of(p.inv_y[(int64_t)r2 * p.C + j], p.C, n_c) : 0;
      }
      __syncthreads();
      load_tiles<E, D>(Y, yid, tile, tileT, 64 * NW);
      __syncthreads();
      f32x4 acc[4];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        Frag<E, D> bf;
        bf.load_lds(tile + (cb * 16 + (l & 15)) * P);
        acc[cb] = mma_block(afr, bf, f32x4{0.f, 0.f, 0.f, 0.f});
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int n = cb * 16 + (l & 15);
        const int j = yid[n];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float a = acc[cb][v];
          float gv = 0.0f;
          if (rv[v] && j >= 0 && j != pos_v[v]) {
            const E* xrow = X + (int64_t)i_v[v] * D;
            bool mem = beats<E, D>(a, lo_v[v], hi_v[v], te_v[v], tid_v[v], xrow, Y, j, p.counters);
            for (int r2 = 0; r2 < rho && mem; ++r2) {
              const PrevRow pr = prev[(4 * g + v) * MAX_ROUNDS + r2];
              if (!in_window(pr.cx, cy2s[r2 * 64 + n], n_c)) continue;
              if (beats<E, D>(a, pr.lo, pr.hi, pr.te, pr.tid, xrow, Y, j, p.counters)) mem = false;
            }
            if (mem) gv = expf(a - lse_v[v]) * gb_v[v];
          }
          G[(4 * g + v) * GP + n] = gv;
        }
      }
      wave_sync();
      accumulate_gt<E, D>(dacc, G, tileT);
      wave_sync();
    }
  }

  // write: rows 4g+v, coordinates 16nb + (l & 15); round 0 adds the positive term
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    if (!rv[v]) continue;
    float* dst = p.dX + (int64_t)i_v[v] * D;
    float gpos = 0.0f;
    const int pclamp = pos_v[v] < 0 ? 0 : (pos_v[v] >= p.C ? (int)(p.C - 1) : pos_v[v]);
    const E* ypos = Y + (int64_t)pclamp * D;
    if (rho == 0) gpos = (expf(p.lpos[i_v[v]] - lse_v[v]) - 1.0f) * gb_v[v];
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
}

// ------------------------------------------------------------------ dY (negatives)
struct PosInfo {   // a position's data in the current round, staged per tile
  float lse, gb, lo, hi;
  double te;
  int i, pos, tid, pad;
};

template <class E, int D, int NW>
__global__ __launch_bounds__(64 * NW) void k_bwd_items(BwdArgs p, int itiles) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int P = Pitch<E, D>::value;
  constexpr int TR = 16 * NW;
  const E* __restrict__ X = reinterpret_cast<const E*>(p.X);
  const E* __restrict__ Y = reinterpret_cast<const E*>(p.Y);
  E* tile = reinterpret_cast<E*>(smem);
  E* tileT = tile + 64 * P;
  int32_t* xid = reinterpret_cast<int32_t*>(tileT + D * TPitch<E>::value);
  char* after = smem + bwd_common_lds<E, D>();
  PosInfo* pinfo = reinterpret_cast<PosInfo*>(after);                          // [64]
  PrevRow* pprev = reinterpret_cast<PrevRow*>(after + 64 * sizeof(PosInfo));   // [64][MAX_ROUNDS]
  const int w = threadIdx.x >> 6, l = lane_id(), g = l >> 4;
  char* wbase = after + 64 * sizeof(PosInfo) + 64 * MAX_ROUNDS * sizeof(PrevRow) +
                (size_t)w * (16 * GP * 4 + 16 * MAX_ROUNDS * 4);
  float* G = reinterpret_cast<float*>(wbase);
  int32_t* cy2w = reinterpret_cast<int32_t*>(wbase + 16 * GP * 4);   // [16][MAX_ROUNDS]
  const int n_c = p.n_c, rho = p.rho;
  const int64_t s = p.s, C = p.C;

  const int c = blockIdx.x / itiles;
  const int it = blockIdx.x % itiles;
  const int64_t y0 = chunk_start(c, C, n_c), y1 = chunk_start(c + 1, C, n_c);
  const int64_t tile0 = y0 + (int64_t)it * TR;
  if (tile0 >= y1) return;
  const int64_t wq0 = tile0 + 16 * w;

  const int64_t qA = wq0 + (l & 15);
  const int jA = qA < y1 ? p.perm_y[qA] : -1;
  Frag<E, D> afr;
  afr.load_global(jA >= 0 ? Y + (int64_t)jA * D : nullptr);
  if (l < 16)
    for (int r2 = 0; r2 < rho; ++r2)
      cy2w[l * MAX_ROUNDS + r2] = jA >= 0 ? chunk_of(p.inv_y[(int64_t)r2 * C + jA], C, n_c) : 0;

  int j_v[4];
  bool rv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t qr = wq0 + 4 * g + v;
    rv[v] = qr < y1;
    j_v[v] = rv[v] ? p.perm_y[qr] : -1;
  }
  f32x4 dacc[D / 16];
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) dacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // X-chunks whose window holds item chunk c (the window relation is symmetric)
  int xc[3];
  int nxc = 0;
  xc[nxc++] = c;
  if (n_c >= 2) xc[nxc++] = (c + n_c - 1) % n_c;
  if (n_c >= 3) xc[nxc++] = (c + 1) % n_c;

  for (int q = 0; q < nxc; ++q) {
    const int64_t px0 = chunk_start(xc[q], s, n_c), px1 = chunk_start(xc[q] + 1, s, n_c);
    for (int64_t p0 = px0; p0 < px1; p0 += 64) {
      __syncthreads();
      if (threadIdx.x < 64) {
        const int64_t pp = p0 + threadIdx.x;
        const int i = pp < px1 ? p.perm_x[pp] : -1;
        xid[threadIdx.x] = i;
        PosInfo pi{0.f, 0.f, 0.f, 0.f, 0.0, i, -1, 0, 0};
        if (i >= 0) {
          const int64_t o = (int64_t)rho * s + i;
          pi.lse = p.lse[i];
          pi.gb = gbar_of(p, i);
          pi.lo = p.thr_lo[o];
          pi.hi = p.thr_hi[o];
          pi.te = p.thr_e[o];
          pi.tid = p.thr_id[o];
          pi.pos = p.pos[i];
          for (int r2 = 0; r2 < rho; ++r2) {
            const int64_t o2 = (int64_t)r2 * s + i;
            PrevRow pr;
            pr.te = p.thr_e[o2];
            pr.lo = p.thr_lo[o2];
            pr.hi = p.thr_hi[o2];
            pr.tid = p.thr_id[o2];
            pr.cx = chunk_of(p.inv_x[o2], s, n_c);
            pprev[threadIdx.x * MAX_ROUNDS + r2] = pr;
          }
        }
        pinfo[threadIdx.x] = pi;
      }
      __syncthreads();
      load_tiles<E, D>(X, xid, tile, tileT, 64 * NW);
      __syncthreads();
      f32x4 acc[4];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        Frag<E, D> bf;
        bf.load_lds(tile + (cb * 16 + (l & 15)) * P);
        acc[cb] = mma_block(afr, bf, f32x4{0.f, 0.f, 0.f, 0.f});
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int n = cb * 16 + (l & 15);
        const PosInfo pi = pinfo[n];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float a = acc[cb][v];
          const int j = j_v[v];
          float gv = 0.0f;
          if (rv[v] && pi.i >= 0 && j != pi.pos) {
            const E* xrow = X + (int64_t)pi.i * D;
            bool mem = beats<E, D>(a, pi.lo, pi.hi, pi.te, pi.tid, xrow, Y, j, p.counters);
            for (int r2 = 0; r2 < rho && mem; ++r2) {
              const PrevRow pr = pprev[n * MAX_ROUNDS + r2];
              if (!in_window(pr.cx, cy2w[(4 * g + v) * MAX_ROUNDS + r2], n_c)) continue;
              if (beats<E, D>(a, pr.lo, pr.hi, pr.te, pr.tid, xrow, Y, j, p.counters)) mem = false;
            }
            if (mem) gv = expf(a - pi.lse) * pi.gb;
          }
          G[(4 * g + v) * GP + n] = gv;
        }
      }
      wave_sync();
      accumulate_gt<E, D>(dacc, G, tileT);
      wave_sync();
    }
  }

#pragma unroll
  for (int v = 0; v < 4; ++v) {
    if (!rv[v]) continue;
    float* dst = p.dY + (int64_t)j_v[v] * D;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) {
      const int t = 16 * nb + (l & 15);
      float val = dacc[nb][v];
      if (rho > 0) val += dst[t];
      dst[t] = val;
    }
  }
}

// ------------------------------------------------------------------ dY (positives)
constexpr int PIECE = 64;   // sorted positions per piece (one wave)

// pflag bits per piece: 1 = head run continues from the previous piece,
// 2 = head run continues into the next piece, 4 = a tail run starts here and continues.
template <class E, int D>
__global__ __launch_bounds__(256) void k_pos_pieces(BwdArgs p, const int32_t* __restrict__ sorted,
                                                    float* __restrict__ partial, int32_t* __restrict__ pitem,
                                                    int32_t* __restrict__ pflag, int64_t npieces) {
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
  const int prev_item = t0 > 0 ? p.pos[sorted[t0 - 1]] : -1;
  const int next_item = t1 < s ? p.pos[sorted[t1]] : -1;
  int cur = p.pos[sorted[t0]];
  int64_t run_start = t0;
  for (int64_t t = t0; t < t1; ++t) {
    const int i = sorted[t];
    const int item = p.pos[i];
    if (item != cur) {
      // flush the run [run_start, t) of item cur
      if (run_start == t0 && prev_item == cur) {
        head_item = cur;
        flags |= 1;
#pragma unroll
        for (int u = 0; u < PER; ++u)
          if (l + 64 * u < D) partial[(piece * 2 + 0) * D + l + 64 * u] = acc[u];
      } else if (cur >= 0 && cur < p.C) {
        float* dst = p.dY + (int64_t)cur * D;
#pragma unroll
        for (int u = 0; u < PER; ++u)
          if (l + 64 * u < D) dst[l + 64 * u] += acc[u];
      }
#pragma unroll
      for (int u = 0; u < PER; ++u) acc[u] = 0.0f;
      cur = item;
      run_start = t;
    }
    const float gp = (expf(p.lpos[i] - p.lse[i]) - 1.0f) * gbar_of(p, i);
    const E* xr = X + (int64_t)i * D;
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (l + 64 * u < D) acc[u] = fmaf(gp, to_f32(xr[l + 64 * u]), acc[u]);
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
    float* dst = p.dY + (int64_t)cur * D;
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (l + 64 * u < D) dst[l + 64 * u] += acc[u];
  }
  if (l == 0) {
    pitem[piece * 2 + 0] = head_item;
    pitem[piece * 2 + 1] = tail_item;
    pflag[piece] = flags;
  }
}

// A run that starts in piece q and continues: add the head partials of the
// following pieces, in order, until the run ends.
template <int D>
__global__ __launch_bounds__(256) void k_pos_combine(float* __restrict__ dY, const float* __restrict__ partial,
                                                     const int32_t* __restrict__ pitem,
                                                     const int32_t* __restrict__ pflag, int64_t npieces) {
  constexpr int PER = (D + 63) / 64;
  const int w = threadIdx.x >> 6, l = lane_id();
  const int64_t piece = (int64_t)blockIdx.x * 4 + w;
  if (piece >= npieces) return;
  if (!(pflag[piece] & 4)) return;
  const int item = pitem[piece * 2 + 1];
  if (item < 0) return;
  float acc[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) acc[u] = l + 64 * u < D ? partial[(piece * 2 + 1) * D + l + 64 * u] : 0.0f;
  for (int64_t q = piece + 1; q < npieces; ++q) {
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (l + 64 * u < D) acc[u] += partial[(q * 2 + 0) * D + l + 64 * u];
    if (!(pflag[q] & 2)) break;
  }
  float* dst = dY + (int64_t)item * D;
#pragma unroll
  for (int u = 0; u < PER; ++u)
    if (l + 64 * u < D) dst[l + 64 * u] += acc[u];
}

// ------------------------------------------------------------------ launchers
template <class E, int D>
static size_t rows_lds(int NW) {
  return bwd_common_lds<E, D>() + (size_t)NW * (16 * GP * 4 + 16 * MAX_ROUNDS * sizeof(PrevRow));
}
template <class E, int D>
static size_t items_lds(int NW) {
  return bwd_common_lds<E, D>() + 64 * sizeof(PosInfo) + 64 * MAX_ROUNDS * sizeof(PrevRow) +
         (size_t)NW * (16 * GP * 4 + 16 * MAX_ROUNDS * 4);
}

template <class E, int D, int NW>
static hipError_t launch_rows_t(const BwdArgs& a, hipStream_t st) {
  const size_t lds = rows_lds<E, D>(NW);
  auto kern = k_bwd_rows<E, D, NW>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)((int64_t)a.n_c * a.tiles_per_chunk)), dim3(64 * NW), lds, st, a);
  return hipGetLastError();
}
template <class E, int D, int NW>
static hipError_t launch_items_t(const BwdArgs& a, int itiles, hipStream_t st) {
  const size_t lds = items_lds<E, D>(NW);
  auto kern = k_bwd_items<E, D, NW>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)((int64_t)a.n_c * itiles)), dim3(64 * NW), lds, st, a, itiles);
  return hipGetLastError();
}

hipError_t launch_bwd_rows(bool bf16v, int d, int waves, const BwdArgs& a, hipStream_t st) {
#define RECE_R(E, DD) \
  if (d == DD) return launch_rows_t<E, DD, 4>(a, st);
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
  if (d == DD) return launch_items_t<E, DD, 4>(a, itiles, st);
  (void)waves;
  if (bf16v) {
    RECE_I(bf16, 32) RECE_I(bf16, 64) RECE_I(bf16, 128) RECE_I(bf16, 256)
  } else {
    RECE_I(float, 32) RECE_I(float, 64) RECE_I(float, 128) RECE_I(float, 256)
  }
#undef RECE_I
  return hipErrorInvalidValue;
}

template <class E, int D>
static hipError_t launch_pos_t(const BwdArgs& a, const int32_t* sorted, float* partial, hipStream_t st) {
  const int64_t npieces = (a.s + PIECE - 1) / PIECE;
  int32_t* pitem = reinterpret_cast<int32_t*>(partial + npieces * 2 * D);
  int32_t* pflag = pitem + npieces * 2;
  const unsigned blocks = (unsigned)((npieces + 3) / 4);
  hipLaunchKernelGGL((k_pos_pieces<E, D>), dim3(blocks), dim3(256), 0, st, a, sorted, partial, pitem, pflag,
                     npieces);
  hipLaunchKernelGGL((k_pos_combine<D>), dim3(blocks), dim3(256), 0, st, a.dY, partial, pitem, pflag, npieces);
  return hipGetLastError();
}

hipError_t launch_pos_dy(bool bf16v, int d, const BwdArgs& a, const int32_t* sorted, float* partial,
                         hipStream_t st) {
#define RECE_P(E, DD) \
  if (d == DD) return launch_pos_t<E, DD>(a, sorted, partial, st);
  if (bf16v) {
    RECE_P(bf16, 32) RECE_P(bf16, 64) RECE_P(bf16, 128) RECE_P(bf16, 256)
  } else {
    RECE_P(float, 32) RECE_P(float, 64) RECE_P(float, 128) RECE_P(float, 256)
  }
#undef RECE_P
  return hipErrorInvalidValue;
}

size_t pos_partial_bytes(int64_t s, int d) {
  const int64_t npieces = (s + PIECE - 1) / PIECE;
  return (size_t)npieces * 2 * d * 4 + (size_t)npieces * 3 * 4;
}

}  // namespace rece
