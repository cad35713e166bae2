// Backward pass: d loss / d X and d loss / d Y with the selection held fixed
// (RECE page, Section 3, Eq. 4: softmax minus one-hot, restricted to the scored
// set {positive} u kept negatives, chained through logit = x . y).
//
// Both sides read the kept lists the forward pass wrote, negs[r][s][k] (item
// ids, -1 padded, bit 31 set on a pair an earlier round also kept, so every
// pair counts once), plus lse and the positive logit of each position.  No
// window is revisited and no float atomics are used: every sum has a fixed
// order and two runs give identical bits.
//   * dX (k_dx_lists): one wave per position gathers the Y rows of its list
//     entries and adds g * y_j, then the positive term;
//   * dY: the pairs (item, position) of all lists plus one pair per position
//     for its positive are sorted by item with a stable LSD counting sort of
//     (key, value) records; the sorted array is cut into fixed sub-pieces of
//     DY_SUB pairs, one lane group per sub-piece walks its pairs in order and
//     sums g * x_i per item; an item that spans sub-pieces leaves partial rows
//     that a second kernel adds in sub-piece order.  Every row of dY is
//     written once (items no pair names get zero rows).
#include "rece_device.h"
#include "rece_internal.h"

namespace rece {

// Write (or clear) row j of dY: EPL floats of lane `sub`.
template <int EPL>
__device__ __forceinline__ void store_row(float* dst, const float (&v)[EPL]) {
#pragma unroll
  for (int t = 0; t < EPL / 4; ++t)
    reinterpret_cast<float4*>(dst)[t] = float4{v[4 * t], v[4 * t + 1], v[4 * t + 2], v[4 * t + 3]};
}

// EPL gradient values at element `off` of a float32 or (b16) bf16 output.
template <int EPL>
__device__ __forceinline__ void store_grad(void* base, int64_t off, const float (&v)[EPL], bool b16) {
  if (b16) {
    uint32_t w[EPL / 2];
#pragma unroll
    for (int t = 0; t < EPL / 2; ++t) w[t] = bf16_bits_rne(v[2 * t]) | (bf16_bits_rne(v[2 * t + 1]) << 16);
    uint16_t* d = static_cast<uint16_t*>(base) + off;
    if constexpr (EPL == 8)
      *reinterpret_cast<u32x4*>(d) = u32x4{w[0], w[1], w[2], w[3]};
    else
#pragma unroll
      for (int t = 0; t < EPL / 2; ++t) reinterpret_cast<uint32_t*>(d)[t] = w[t];
  } else {
    store_row<EPL>(static_cast<float*>(base) + off, v);
  }
}

// Upstream gradient of position i's loss (0 for padding under the mask, whose
// mean counts only the other positions).
__device__ __forceinline__ float gbar_of(const BwdArgs& p, int64_t i) {
  if (p.ignore) {
    if (p.pos[i] < 0) return 0.0f;
    return p.dloss_pp ? p.dloss_pp[i] : p.dloss[0] * p.wmean[0];
  }
  return p.dloss_pp ? p.dloss_pp[i] : p.dloss[0] / (float)p.s;
}

// Per position: {lse, upstream gradient, coefficient of the positive (Eq. 4: its
// softmax share minus one, times the upstream gradient), 0}, read by both sides.
__global__ __launch_bounds__(256) void k_pos_coef(BwdArgs p, float4* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= p.s) return;
  const float lse = p.lse[i];
  const float gb = gbar_of(p, i);
  out[i] = float4{lse, gb, (expf(p.lpos[i] - lse) - 1.0f) * gb, 0.0f};
}

// Sixteen bytes of a row as floats.
__device__ __forceinline__ void cvt16f(const u32x4 u, float (&v)[8]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    v[2 * t] = __uint_as_float(u[t] << 16);
    v[2 * t + 1] = __uint_as_float(u[t] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void cvt16f(const u32x4 u, float (&v)[4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) v[t] = __uint_as_float(u[t]);
}
template <class E, int N>
__device__ __forceinline__ void load16f(const E* ptr, float (&v)[N]) {
  cvt16f(*reinterpret_cast<const u32x4*>(ptr), v);
}

// ------------------------------------------------------------------ dX from the kept lists
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
  const float4 pci = reinterpret_cast<const float4*>(p.pcoef)[i];
  const float lse = pci.x, gb = pci.y;
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
    const float gpos = pci.z;
    float yp[EPL];
    load16f(Y + (int64_t)pc * D + sub * EPL, yp);
#pragma unroll
    for (int t = 0; t < EPL; ++t) acc[t] = fmaf(gpos, yp[t], acc[t]);
  }
#pragma unroll
  for (int o = LPR; o < WAVE; o <<= 1)
#pragma unroll
    for (int t = 0; t < EPL; ++t) acc[t] += __shfl_xor(acc[t], o);
  if (q == 0) store_grad<EPL>(p.dX, i * D + sub * EPL, acc, p.grad_bf16 != 0);
}

// ------------------------------------------------------------------ exports
__global__ void k_strip_mark(const int32_t* __restrict__ src, int64_t n, int32_t* __restrict__ dst) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) {
    const int v = src[t];
    dst[t] = v == -1 ? -1 : (v & 0x7FFFFFFF);
  }
}

// One wave per position: the ids of its lists of all rounds that no earlier
// round kept, in (round, list) order, then -1 up to rounds * k entries.
__global__ __launch_bounds__(256) void k_union_ids(const int32_t* __restrict__ negs, int64_t s, int k, int rounds,
                                                   int32_t* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= s) return;
  const int l = lane_id();
  const int64_t width = (int64_t)rounds * k;
  int32_t* out = dst + i * width;
  int64_t n = 0;
  for (int rho = 0; rho < rounds; ++rho) {
    const int32_t* list = negs + ((int64_t)rho * s + i) * k;
    for (int e0 = 0; e0 < k; e0 += WAVE) {
      const int v = e0 + l < k ? list[e0 + l] : -1;
      const uint64_t m = ballot(v >= 0);
      if (v >= 0) out[n + popc(m & lanemask_lt())] = v;
      n += popc(m);
    }
  }
  for (int64_t t = n + l; t < width; t += WAVE) out[t] = -1;
}

// ------------------------------------------------------------------ pair sort by item
// Records (key, value): key = item id, value = position id, bit 31 set on the
// record of a position's positive.  The first pass reads them from the kept
// lists and the positives (entry t < nl: list entry t, value (t / k) mod s;
// entry nl + i: the positive of position i) and drops list entries < 0 and
// ids outside [0, C); later passes read the previous pass's output, whose
// length the previous scatter stored in ntot.
struct PairSrc {
  const int32_t* negs;   // [nl] first pass
  const int32_t* pos;    // [s]  first pass
  const int32_t* kin;    // later passes
  const int32_t* vin;
  const uint32_t* nin;   // later passes: number of records in kin / vin
  int64_t nl, s, C;
  int k;
  double rk, rs;         // 1 / k, 1 / s (first pass)
};

// floor(n / d) for 0 <= n < 2^32 and d >= 1, given rd = 1 / d rounded to double:
// the double product is within 2^-20 of n / d, so its truncation is off by at most
// one either way, which one exact check corrects.  No branch and no integer
// division (a software division per record would make the compiler branch around
// it, and wait for each record's loads at the join).
__device__ __forceinline__ uint32_t udiv_rd(uint32_t n, uint32_t d, double rd) {
  int64_t q = (int64_t)((double)n * rd);
  const int64_t r = (int64_t)n - q * (int64_t)d;
  q += (r >= (int64_t)d ? 1 : 0) - (r < 0 ? 1 : 0);
  return (uint32_t)q;
}

// Record t of the pass's input (t < n), loaded without branches so that the loads
// of many records can be in flight at once: addresses are clamped into range and
// the choice between a list entry and a positive is a select.  n >= 1.
template <bool FIRST>
__device__ __forceinline__ bool pair_at(const PairSrc& a, int64_t t, int64_t n, int& key, int& val) {
  const int64_t tc = t < n ? t : n - 1;
  if constexpr (FIRST) {
    const bool isl = tc < a.nl;
    const int64_t il = isl ? tc : 0;
    const int64_t ip = isl ? 0 : tc - a.nl;
    const int kn = a.negs[il];
    const int kp = a.pos[ip];
    key = isl ? kn : kp;
    // list entry t belongs to position (t / k) mod s (lists are [round][position][k])
    const uint32_t q = udiv_rd((uint32_t)il, (uint32_t)a.k, a.rk);
    const uint32_t i = q - (uint32_t)a.s * udiv_rd(q, (uint32_t)a.s, a.rs);
    val = isl ? (int)i : ((int)ip | (int)0x80000000u);
    return (int)(t < n) & (int)(key >= 0) & (int)(key < a.C);   // no short-circuit: no branch between loads
  } else {
    key = a.kin[tc];
    val = a.vin[tc];
    return t < n;
  }
}

// Each pass is one stable counting sort on a digit of at most 8 bits, over tiles
// of RS_TILE records (one 256-thread workgroup each):
//   k_pair_hist     per tile, the count of every digit -> counts[digit][tile];
//   (an exclusive scan of counts in (digit, tile) order: every (digit, tile) gets
//    its first output slot);
//   k_pair_scatter  per tile: the records are ranked in input order (each wave
//                   takes a quarter of the tile, 64 consecutive records at a time;
//                   lanes with equal digits find each other with one ballot per
//                   digit bit and advance the wave's running digit counts; the four
//                   waves' counts are then combined in order), placed in LDS in
//                   digit order, and written out from there so that consecutive
//                   lanes write consecutive slots.
constexpr int RS_THREADS = 256;
constexpr int RS_GROUPS_PER_WAVE = 16;
constexpr int RS_GROUPS = 4 * RS_GROUPS_PER_WAVE;   // groups of 64 records per tile
constexpr int RS_TILE = RS_GROUPS * WAVE;           // 4096 records
constexpr int RS_BINS = 256;

template <bool FIRST>
__global__ __launch_bounds__(RS_THREADS) void k_pair_hist(PairSrc a, int64_t n_max, int shift, int nbits, int ntiles,
                                                          uint32_t* __restrict__ counts) {
  __shared__ uint32_t hist[RS_BINS];
  const int nbins = 1 << nbits;
  const uint32_t mask = (uint32_t)nbins - 1u;
  hist[threadIdx.x] = 0u;
  __syncthreads();
  const int64_t n = FIRST ? n_max : (int64_t)*a.nin;
  const int64_t t0 = (int64_t)blockIdx.x * RS_TILE;
  int dig[RS_TILE / RS_THREADS];
  if (n > 0) {
#pragma unroll
    for (int u = 0; u < RS_TILE / RS_THREADS; ++u) {
      const int64_t t = t0 + u * RS_THREADS + threadIdx.x;
      int key, val;
      const bool ok = pair_at<FIRST>(a, t, n, key, val);
      dig[u] = ok ? (int)(((uint32_t)key >> shift) & mask) : -1;
    }
  } else {
#pragma unroll
    for (int u = 0; u < RS_TILE / RS_THREADS; ++u) dig[u] = -1;
  }
#pragma unroll
  for (int u = 0; u < RS_TILE / RS_THREADS; ++u)
    if (dig[u] >= 0) atomicAdd(&hist[dig[u]], 1u);
  __syncthreads();
  if ((int)threadIdx.x < nbins) counts[(int64_t)threadIdx.x * ntiles + blockIdx.x] = hist[threadIdx.x];
  if (blockIdx.x == 0 && threadIdx.x == 0) counts[(int64_t)nbins * ntiles] = 0u;   // becomes the total
}

template <bool FIRST>
__global__ __launch_bounds__(RS_THREADS) void k_pair_scatter(PairSrc a, int64_t n_max, int shift, int nbits,
                                                             int ntiles, const uint32_t* __restrict__ offs,
                                                             int32_t* __restrict__ kout, int32_t* __restrict__ vout,
                                                             uint32_t* __restrict__ ntot) {
  __shared__ uint32_t wcnt[4][RS_BINS];   // per wave: running count of each digit, then its prefix over waves
  __shared__ uint32_t dstart[RS_BINS];    // first local slot of each digit
  __shared__ uint32_t gbase[RS_BINS];     // first global slot of each digit (this tile)
  __shared__ uint32_t wsum[4];
  __shared__ int32_t skey[RS_TILE];
  __shared__ int32_t sval[RS_TILE];
  const int nbins = 1 << nbits;
  const uint32_t mask = (uint32_t)nbins - 1u;
  const int tid = threadIdx.x, w = tid >> 6, l = lane_id();
  if (blockIdx.x == 0 && tid == 0) *ntot = offs[(int64_t)nbins * ntiles];
#pragma unroll
  for (int q = 0; q < 4; ++q) wcnt[q][tid] = 0u;
  gbase[tid] = tid < nbins ? offs[(int64_t)tid * ntiles + blockIdx.x] : 0u;
  const int64_t n = FIRST ? n_max : (int64_t)*a.nin;
  const int64_t t0 = (int64_t)blockIdx.x * RS_TILE;
  // wave w ranks records 1024 w .. 1024 w + 1023 of the tile, 64 at a time in input
  // order, against its own running digit counts
  int rkey[RS_GROUPS_PER_WAVE], rval[RS_GROUPS_PER_WAVE], rinfo[RS_GROUPS_PER_WAVE];   // info: digit | rank << 8, -1 invalid
  bool rok[RS_GROUPS_PER_WAVE];
#pragma unroll
  for (int it = 0; it < RS_GROUPS_PER_WAVE; ++it) rkey[it] = rval[it] = 0;
  // all the wave's records first (every load in flight), then the ranks
#pragma unroll
  for (int it = 0; it < RS_GROUPS_PER_WAVE; ++it) {
    const int64_t t = t0 + (int64_t)(w * RS_GROUPS_PER_WAVE + it) * WAVE + l;
    const bool okr = pair_at<FIRST>(a, t, n > 0 ? n : 1, rkey[it], rval[it]);
    rok[it] = (n > 0) & okr;   // no short-circuit: no branch between the records' loads
  }
  __syncthreads();   // counters cleared
  uint32_t* ctr = wcnt[w];
#pragma unroll
  for (int it = 0; it < RS_GROUPS_PER_WAVE; ++it) {
    const bool valid = rok[it];
    const int dg = valid ? (int)(((uint32_t)rkey[it] >> shift) & mask) : 0;
    uint64_t same = ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (dg >> bit) & 1;
      const uint64_t bm = ballot(on);
      same &= on ? bm : ~bm;
    }
    const int rank = popc(same & lanemask_lt());
    uint32_t base = 0;
    if (valid) base = ctr[dg];
    wave_sync();
    if (valid && rank == 0) ctr[dg] = base + (uint32_t)popc(same);
    wave_sync();
    rinfo[it] = valid ? (dg | (int)((base + (uint32_t)rank) << 8)) : -1;
  }
  __syncthreads();
  // per digit: prefix over the waves and the tile total; then an exclusive scan of
  // the totals over the digits
  uint32_t tot = 0;
  if (tid < nbins) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t c = wcnt[q][tid];
      wcnt[q][tid] = tot;
      tot += c;
    }
  }
  {
    uint32_t x = tot;
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
      const uint32_t y = __shfl_up(x, o);
      if (l >= o) x += y;
    }
    if (l == WAVE - 1) wsum[w] = x;
    __syncthreads();
    uint32_t pre = 0;
    for (int q = 0; q < w; ++q) pre += wsum[q];
    dstart[tid] = pre + x - tot;
  }
  __syncthreads();
  const uint32_t nvalid = wsum[0] + wsum[1] + wsum[2] + wsum[3];
#pragma unroll
  for (int it = 0; it < RS_GROUPS_PER_WAVE; ++it) {
    if (rinfo[it] < 0) continue;
    const int dg = rinfo[it] & 0xFF;
    const uint32_t local = dstart[dg] + wcnt[w][dg] + ((uint32_t)rinfo[it] >> 8);
    skey[local] = rkey[it];
    sval[local] = rval[it];
  }
  __syncthreads();
  for (uint32_t q = tid; q < nvalid; q += RS_THREADS) {
    const int key = skey[q];
    const int dg = (int)(((uint32_t)key >> shift) & mask);
    const uint32_t slot = gbase[dg] + (q - dstart[dg]);
    kout[slot] = key;
    vout[slot] = sval[q];
  }
}

// ------------------------------------------------------------------ dY from the sorted pairs
constexpr int DY_SUB = 256;   // sorted pairs per lane group

// Per sub-piece: flags (1 = its first item started in an earlier sub-piece, 2 = that
// item also continues into the next one, 4 = its last item starts here and
// continues), the items of the head and tail partial rows, and the rows.
struct DyArea {
  float* partial;    // [nsub][2][D]
  int32_t* flags;    // [nsub]
  int32_t* items;    // [nsub][2]
  int64_t nsub;
};

// One lane group (LPR lanes, 16 bytes of a row each) per sub-piece of DY_SUB sorted
// pairs.  For each pair (j, i): l = x_i . y_j (float32, the same lane split and
// order as k_dx_lists), g = gbar_i exp(l - lse_i), or the position's positive
// coefficient for a positive record, summed as g x_i per item in pair order.  An item
// wholly inside the sub-piece is written to dY here; an item continuing from the
// previous or into the next sub-piece leaves a partial row for k_dy_combine.  The
// items with no pair between two consecutive keys get zero rows from the sub-piece
// holding the earlier key (sub-piece 0 also clears the items before the first key).
template <class E, int D>
__global__ __launch_bounds__(256) void k_dy_pieces(BwdArgs p, const int32_t* __restrict__ K,
                                                   const int32_t* __restrict__ V, const uint32_t* __restrict__ ntot,
                                                   DyArea area) {
  constexpr int EPL = 16 / (int)sizeof(E);
  constexpr int LPR = D / EPL;
  constexpr int RPI = WAVE / LPR;
  constexpr int UNR = 4;
  const E* __restrict__ X = reinterpret_cast<const E*>(p.X);
  const E* __restrict__ Y = reinterpret_cast<const E*>(p.Y);
  const int l = lane_id();
  const int q = l / LPR, sub = l % LPR;
  const int64_t piece = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPI + q;
  const int64_t n = (int64_t)*ntot;
  const int64_t C = p.C;
  const int64_t t0 = piece * DY_SUB;
  if (piece >= area.nsub || (t0 >= n && piece != 0)) return;   // whole groups leave together
  const int64_t t1 = min(n, t0 + DY_SUB);
  float zero[EPL];
#pragma unroll
  for (int t = 0; t < EPL; ++t) zero[t] = 0.0f;
  void* dY = p.dY;
  const bool b16 = p.grad_bf16 != 0;
  if (n == 0) {   // no pair at all: piece 0 clears every row
    for (int64_t j = 0; j < C; ++j) store_grad<EPL>(dY, j * D + sub * EPL, zero, b16);
    if (sub == 0) area.flags[0] = 0;
    return;
  }
  const int prev_key = t0 > 0 ? K[t0 - 1] : -1;
  const int next_key = t1 < n ? K[t1] : (int)C;   // C: no later key
  const float4* __restrict__ PC = reinterpret_cast<const float4*>(p.pcoef);
  int cur = -1;
  int64_t run_start = t0;
  int flags = 0, head_item = -1, tail_item = -1;
  float acc[EPL];
#pragma unroll
  for (int t = 0; t < EPL; ++t) acc[t] = 0.0f;

  // rows of items [a, b) cleared
  auto clear_rows = [&](int64_t a, int64_t b) {
    for (int64_t j = a; j < b; ++j) store_grad<EPL>(dY, j * D + sub * EPL, zero, b16);
  };
  // the run of item cur over [run_start, t_end) is complete
  auto flush = [&](int64_t t_end) {
    const bool head = run_start == t0 && cur == prev_key;
    const bool tail = t_end == t1 && t1 < n && cur == next_key;
    if (!head && !tail) {
      store_grad<EPL>(dY, (int64_t)cur * D + sub * EPL, acc, b16);
    } else if (head) {
      store_row<EPL>(area.partial + (piece * 2 + 0) * D + sub * EPL, acc);
      head_item = cur;
      flags |= tail ? 3 : 1;
    } else {
      store_row<EPL>(area.partial + (piece * 2 + 1) * D + sub * EPL, acc);
      tail_item = cur;
      flags |= 4;
    }
  };
  // keys and values of the batch at tb (key -1 past the sub-piece; addresses clamped)
  auto load_kv = [&](int64_t tb, int (&kk)[UNR], int (&vv)[UNR]) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t t = tb + u;
      const int64_t tc = t < t1 ? t : t1 - 1;
      kk[u] = K[tc];
      vv[u] = V[tc];
      if (t >= t1) kk[u] = -1;
    }
  };

  // Pipelined: the rows and coefficients of batch b are requested before the keys
  // and values of batch b + 1, which then arrive while batch b is summed.  An item
  // row is fetched only for a record whose key differs from the one before it.
  int kn[UNR], vn[UNR];
  load_kv(t0, kn, vn);
  int ykey = -1;
  u32x4 ycur = u32x4{0u, 0u, 0u, 0u};
  for (int64_t tb = t0; tb < t1; tb += UNR) {
    int key[UNR], val[UNR];
    u32x4 xr[UNR], yr[UNR];
    float4 pc[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      key[u] = kn[u];
      val[u] = vn[u];
      const int64_t i = key[u] >= 0 ? (int64_t)(val[u] & 0x7FFFFFFF) : 0;
      xr[u] = *reinterpret_cast<const u32x4*>(X + i * D + sub * EPL);
      pc[u] = PC[i];
      const int kprev = u == 0 ? ykey : key[u - 1];
      yr[u] = u32x4{0u, 0u, 0u, 0u};
      if (key[u] >= 0 && key[u] != kprev) yr[u] = *reinterpret_cast<const u32x4*>(Y + (int64_t)key[u] * D + sub * EPL);
    }
    load_kv(tb + UNR, kn, vn);
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (key[u] < 0) break;
      if (key[u] != cur) {
        if (cur >= 0) {
          flush(tb + u);
          clear_rows(cur + 1, key[u]);
        } else if (piece == 0) {
          clear_rows(0, key[u]);
        }
        cur = key[u];
        run_start = tb + u;
#pragma unroll
        for (int t = 0; t < EPL; ++t) acc[t] = 0.0f;
      }
      if (key[u] != ykey) {
        ycur = yr[u];
        ykey = key[u];
      }
      float x[EPL], y[EPL];
      cvt16f(xr[u], x);
      cvt16f(ycur, y);
      float dot = 0.0f;
#pragma unroll
      for (int t = 0; t < EPL; ++t) dot = fmaf(x[t], y[t], dot);
#pragma unroll
      for (int o = 1; o < LPR; o <<= 1) dot += __shfl_xor(dot, o);
      const float g = val[u] < 0 ? pc[u].z : __expf(dot - pc[u].x) * pc[u].y;
#pragma unroll
      for (int t = 0; t < EPL; ++t) acc[t] = fmaf(g, x[t], acc[t]);
    }
  }
  flush(t1);
  if (cur != next_key) clear_rows(cur + 1, next_key);
  if (sub == 0) {
    area.flags[piece] = flags;
    area.items[piece * 2 + 0] = head_item;
    area.items[piece * 2 + 1] = tail_item;
  }
}

// Items spanning sub-pieces: the sub-piece where such an item starts adds the head
// rows of the following sub-pieces, in order, to its tail row and writes dY.
template <int D>
__global__ __launch_bounds__(256) void k_dy_combine(void* __restrict__ dY, int b16, const uint32_t* __restrict__ ntot,
                                                    DyArea area) {
  constexpr int EPL = 4;
  constexpr int LPR = D / EPL;
  constexpr int RPI = WAVE / LPR > 0 ? WAVE / LPR : 1;
  const int l = lane_id();
  const int q = l / LPR, sub = l % LPR;
  if (q >= RPI) return;
  const int64_t piece = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPI + q;
  const int64_t n = (int64_t)*ntot;
  const int64_t nact = (n + DY_SUB - 1) / DY_SUB;
  if (piece >= nact || !(area.flags[piece] & 4)) return;
  float acc[EPL];
  load16f(area.partial + (piece * 2 + 1) * D + sub * EPL, acc);
  for (int64_t qq = piece + 1; qq < nact; ++qq) {
    float h[EPL];
    load16f(area.partial + (qq * 2 + 0) * D + sub * EPL, h);
#pragma unroll
    for (int t = 0; t < EPL; ++t) acc[t] += h[t];
    if (!(area.flags[qq] & 2)) break;
  }
  store_grad<EPL>(dY, (int64_t)area.items[piece * 2 + 1] * D + sub * EPL, acc, b16 != 0);
}

// ------------------------------------------------------------------ launchers
PairSortGeom pair_sort_geom(int64_t E, int64_t C) {
  PairSortGeom g{};
  g.E = E;
  int kb = 1;
  while (((int64_t)1 << kb) < C) ++kb;
  g.npass = (kb + 7) / 8;
  int shift = 0;
  for (int pss = 0; pss < g.npass; ++pss) {
    const int left = g.npass - pss;
    const int b = (kb - shift + left - 1) / left;
    g.shift[pss] = shift;
    g.bits[pss] = b;
    shift += b;
  }
  g.seg_len = RS_TILE;
  g.nseg = (E + RS_TILE - 1) / RS_TILE;
  g.count_words = (int64_t)RS_BINS * g.nseg + 1;
  const int64_t nb = (g.count_words + 4095) / 4096;
  g.scratch_bytes = (size_t)(g.count_words + nb + 64 + 8) * 4;
  return g;
}

template <bool FIRST>
static hipError_t pair_pass(const PairSrc& a, const PairSortGeom& g, int pss, uint32_t* counts, uint32_t* bsum,
                            int32_t* kout, int32_t* vout, uint32_t* ntot, hipStream_t st) {
  const int nbits = g.bits[pss], nbins = 1 << nbits;
  hipLaunchKernelGGL(k_pair_hist<FIRST>, dim3((unsigned)g.nseg), dim3(RS_THREADS), 0, st, a, g.E, g.shift[pss],
                     nbits, (int)g.nseg, counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_exclusive_scan(counts, (int64_t)nbins * g.nseg + 1, bsum, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_pair_scatter<FIRST>, dim3((unsigned)g.nseg), dim3(RS_THREADS), 0, st, a, g.E, g.shift[pss],
                     nbits, (int)g.nseg, counts, kout, vout, ntot);
  return hipGetLastError();
}

hipError_t launch_pair_sort(const PairSortGeom& g, const int32_t* negs, int64_t nl, int k, int64_t s,
                            const int32_t* pos, int64_t C, void* scratch, int32_t* kA, int32_t* vA, int32_t* kB,
                            int32_t* vB, const int32_t** kout, const int32_t** vout, const uint32_t** nout,
                            hipStream_t st) {
  uint32_t* base = static_cast<uint32_t*>(scratch);
  uint32_t* ntot = base;              // [8] record counts after each pass
  uint32_t* counts = base + 8;
  uint32_t* bsum = counts + g.count_words;
  PairSrc a{};
  a.negs = negs;
  a.pos = pos;
  a.nl = nl;
  a.s = s;
  a.C = C;
  a.k = k > 0 ? k : 1;
  a.rk = 1.0 / (double)a.k;
  a.rs = 1.0 / (double)(s > 0 ? s : 1);
  int32_t* kbuf[2] = {kA, kB};
  int32_t* vbuf[2] = {vA, vB};
  for (int pss = 0; pss < g.npass; ++pss) {
    int32_t* ko = kbuf[pss & 1];
    int32_t* vo = vbuf[pss & 1];
    hipError_t e;
    if (pss == 0) {
      e = pair_pass<true>(a, g, pss, counts, bsum, ko, vo, ntot + pss, st);
    } else {
      a.kin = kbuf[(pss - 1) & 1];
      a.vin = vbuf[(pss - 1) & 1];
      a.nin = ntot + pss - 1;
      e = pair_pass<false>(a, g, pss, counts, bsum, ko, vo, ntot + pss, st);
    }
    if (e != hipSuccess) return e;
  }
  *kout = kbuf[(g.npass - 1) & 1];
  *vout = vbuf[(g.npass - 1) & 1];
  *nout = ntot + g.npass - 1;
  return hipSuccess;
}

static int64_t dy_nsub(int64_t E) { return (E + DY_SUB - 1) / DY_SUB > 0 ? (E + DY_SUB - 1) / DY_SUB : 1; }

size_t dy_area_bytes(int64_t E, int d) {
  const int64_t nsub = dy_nsub(E);
  return (size_t)nsub * 2 * d * 4 + (size_t)nsub * 3 * 4 + 256;
}

static DyArea dy_area(void* base, int64_t E, int d) {
  DyArea a;
  a.nsub = dy_nsub(E);
  a.partial = static_cast<float*>(base);
  a.flags = reinterpret_cast<int32_t*>(a.partial + a.nsub * 2 * d);
  a.items = a.flags + a.nsub;
  return a;
}

template <class E, int D>
static hipError_t launch_dy_t(const BwdArgs& a, const int32_t* K, const int32_t* V, const uint32_t* ntot, int64_t En,
                              void* area, hipStream_t st) {
  constexpr int RPI = WAVE / (D / (16 / (int)sizeof(E)));
  const DyArea ar = dy_area(area, En, D);
  const int64_t groups_per_block = 4 * RPI;
  hipLaunchKernelGGL((k_dy_pieces<E, D>), dim3((unsigned)((ar.nsub + groups_per_block - 1) / groups_per_block)),
                     dim3(256), 0, st, a, K, V, ntot, ar);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int CRPI = WAVE / (D / 4) > 0 ? WAVE / (D / 4) : 1;
  hipLaunchKernelGGL((k_dy_combine<D>), dim3((unsigned)((ar.nsub + 4 * CRPI - 1) / (4 * CRPI))), dim3(256), 0, st,
                     a.dY, a.grad_bf16, ntot, ar);
  return hipGetLastError();
}

hipError_t launch_dy(bool bf16v, int d, const BwdArgs& a, const int32_t* K, const int32_t* V, const uint32_t* ntot,
                     int64_t E, void* area, hipStream_t st) {
#define RECE_DY(EE, DD) \
  if (d == DD) return launch_dy_t<EE, DD>(a, K, V, ntot, E, area, st);
  if (bf16v) {
    RECE_DY(bf16, 32) RECE_DY(bf16, 64) RECE_DY(bf16, 128) RECE_DY(bf16, 256)
  } else {
    RECE_DY(float, 32) RECE_DY(float, 64) RECE_DY(float, 128) RECE_DY(float, 256)
  }
#undef RECE_DY
  return hipErrorInvalidValue;
}

hipError_t launch_pos_coef(const BwdArgs& a, float* out, hipStream_t st) {
  if (a.s == 0) return hipSuccess;
  hipLaunchKernelGGL(k_pos_coef, dim3((unsigned)((a.s + 255) / 256)), dim3(256), 0, st, a,
                     reinterpret_cast<float4*>(out));
  return hipGetLastError();
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

hipError_t launch_union_ids(const int32_t* negs, int64_t s, int k, int rounds, int32_t* dst, hipStream_t st) {
  if (s == 0 || k == 0) return hipSuccess;
  hipLaunchKernelGGL(k_union_ids, dim3((unsigned)((s + 3) / 4)), dim3(256), 0, st, negs, s, k, rounds, dst);
  return hipGetLastError();
}

}  // namespace rece
