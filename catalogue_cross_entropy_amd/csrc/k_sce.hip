// Bucket (SCE) variant kernels.  The SCE page ("Scalable Cross-Entropy Loss for
// Sequential Recommendations with Large Item Catalogs", abstract) scores each
// position against a subset of the catalogue found by maximum inner product
// search; in the bucket variant, each of n_b projection vectors (buckets) takes
// the b_x positions and the b_y items with the largest scores and the positions
// keep their k largest logits over the union of their buckets.
//
// Pipeline (the chunk kernel is shared with RECE: a bucket is a "chunk" whose
// window is its own item list):
//   k_project_scores  scores of every row against every bucket, float32 matrix
//                     cores, stored one column per bucket (plus row norms);
//   k_col_select      per bucket column, the b largest scores, decided exactly
//                     (histogram -> boundary bin -> float64 recomputation of
//                     the entries within 2*beta of the boundary);
//   k_group_bounds    groups of a sorted key list (slots of each position,
//                     slots of each item);
//   k_sce_merge       per position, the exact top-k of the union of its bucket
//                     lists (duplicates removed), its threshold and sums, and
//                     its kept list, which the backward pass reads as RECE's.
#include <algorithm>

#include "rece_device.h"
#include "rece_internal.h"
#include "rece_kth.h"

namespace rece {

// ------------------------------------------------------------ projection scores
// Block: 4 waves x 32 rows.  Bucket vectors stream through LDS in tiles of TB.
template <class E, int D>
__global__ __launch_bounds__(256) void k_project_scores(const E* __restrict__ V, int64_t n,
                                                        const E* __restrict__ Bt, int n_b, float* __restrict__ PT,
                                                        float* __restrict__ norms,
                                                        uint32_t* __restrict__ norm_max_bits) {
  constexpr int P = Pitch<E, D>::value;
  constexpr int TB = D * (int)sizeof(E) > 512 ? 32 : 64;   // bucket rows per LDS tile
  constexpr int CPR = D * (int)sizeof(E) / 16;             // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) E tile[TB * P];
  const int w = threadIdx.x >> 6, l = lane_id(), g = l >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * 128 + w * 32;
  Frag<E, D> a[2];
  float ss[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int64_t r = row0 + 16 * f + (l & 15);
    const E* rp = r < n ? V + r * D : nullptr;
    a[f].load_global(rp);
    // squared norm of row (l & 15) of fragment f: this lane's coordinates, then the 4 lanes of the row
    float acc = 0.0f;
    if (rp) {
      if constexpr (sizeof(E) == 2) {
        for (int ks = 0; ks < D / 32; ++ks)
          for (int t = 0; t < 8; ++t) {
            const float x = to_f32(rp[32 * ks + 8 * g + t]);
            acc = fmaf(x, x, acc);
          }
      } else {
        for (int ks = 0; ks < D / 4; ++ks) {
          const float x = to_f32(rp[4 * ks + g]);
          acc = fmaf(x, x, acc);
        }
      }
    }
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    ss[f] = acc;
  }
  float nmx = 0.0f;   // largest norm of the wave's rows (rows past n count 0)
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int64_t r = row0 + 16 * f + (l & 15);
    // float32 sum of squares: relative error below d * 2^-24 < 2^-12; round the norm up
    const float nrm = r < n ? sqrtf(ss[f]) * (1.0f + 0.0005f) : 0.0f;
    if (norms && l < 16 && r < n) norms[r] = nrm;
    nmx = fmaxf(nmx, nrm);
  }
  if (norm_max_bits) {   // at most one atomic per wave
    nmx = wave_max(nmx);
    if (l == 0) raise_max_bits(norm_max_bits, nmx);
  }

  for (int b0 = 0; b0 < n_b; b0 += TB) {
    __syncthreads();
    for (int e = threadIdx.x; e < TB * CPR; e += 256) {
      const int rr = e / CPR, ch = e % CPR;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (b0 + rr < n_b) v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(Bt + (int64_t)(b0 + rr) * D) + ch * 16);
      *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(tile + rr * P) + ch * 16) = v;
    }
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < TB / 16; ++cb) {
      const int bb = b0 + cb * 16;
      if (bb >= n_b) break;
      Frag<E, D> bf;
      bf.load_lds(tile + (cb * 16 + (l & 15)) * P);
      const int bcol = bb + (l & 15);
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const f32x4 c = mma_block(a[f], bf, f32x4{0.f, 0.f, 0.f, 0.f});
        if (bcol < n_b) {
          // element v: row 4*(l/16)+v, bucket l%16: four consecutive rows of one column
          float* dst = PT + (int64_t)bcol * n;
          const int64_t r = row0 + 16 * f + 4 * g;
          if (r + 4 <= n && ((uintptr_t)(dst + r) & 15) == 0) {
            *reinterpret_cast<f32x4*>(dst + r) = c;
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (r + v < n) dst[r + v] = c[v];
          }
        }
      }
    }
  }
}

template <class E, int D>
static hipError_t launch_ps(const void* V, int64_t n, const void* Bt, int n_b, float* PT, float* norms,
                            uint32_t* nmax, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_project_scores<E, D>), dim3((unsigned)((n + 127) / 128)), dim3(256), 0, st,
                     static_cast<const E*>(V), n, static_cast<const E*>(Bt), n_b, PT, norms, nmax);
  return hipGetLastError();
}

hipError_t launch_project_scores(bool is_bf16, int d, const void* V, int64_t n, const void* Bt, int n_b, float* PT,
                                 float* norms, uint32_t* norm_max_bits, hipStream_t st) {
#define RECE_PS(E, DD) \
  if (d == DD) return launch_ps<E, DD>(V, n, Bt, n_b, PT, norms, norm_max_bits, st);
  if (is_bf16) {
    RECE_PS(bf16, 32) RECE_PS(bf16, 64) RECE_PS(bf16, 128) RECE_PS(bf16, 256)
  } else {
    RECE_PS(float, 32) RECE_PS(float, 64) RECE_PS(float, 128) RECE_PS(float, 256)
  }
#undef RECE_PS
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------ column top-m
constexpr int CS_BINS = 4096;
constexpr int CS_NEAR = 2048;               // entries within the boundary band
constexpr int CS_SLACK = 256;               // room for band entries outside the boundary bin
constexpr float CS_XTOP = 4095.9998f;       // largest histogram coordinate below 4096
constexpr int CS_THREADS = 1024;

// One workgroup per bucket column.  Selection order: (float64 score desc, index asc).
template <class E, int D>
__global__ __launch_bounds__(CS_THREADS) void k_col_select(ColSelectArgs a) {
  __shared__ uint32_t hist[CS_BINS];
  __shared__ int32_t near_idx[CS_NEAR];
  __shared__ float near_val[CS_NEAR];
  __shared__ double near_e[CS_NEAR];
  __shared__ uint32_t wtot[2][CS_THREADS / 64];
  __shared__ int32_t bcast[4];
  const int b = blockIdx.x;
  const int64_t N = a.N;
  const int m = a.m;
  const float* __restrict__ col = a.PT + (int64_t)b * N;
  int32_t* out = a.out + (int64_t)b * m;
  const int tid = threadIdx.x, l = lane_id(), w = tid >> 6;
  constexpr int NW = CS_THREADS / 64;
  if ((int64_t)m >= N) {   // the bucket takes every entry
    for (int64_t t = tid; t < N; t += CS_THREADS) out[t] = (int32_t)t;
    return;
  }
  const E* V = static_cast<const E*>(a.V);
  const E* brow = static_cast<const E*>(a.Bt) + (int64_t)b * D;
  const float vmax = __uint_as_float(a.vmax_bits[0]), bn = a.bnorm_max[0];
  const float beta = a.beta_coef * vmax * bn;   // bounds |float32 score - float64 score|
  const float bnd = f_up((double)vmax * (double)bn * (1.0 + 1e-5) + 2.0 * (double)beta) + 1e-30f;
  const float lo0 = -bnd, sc0 = (float)CS_BINS / (2.0f * bnd);

  float xa = 0.0f, mul = 1.0f, tlo = 0.0f, thi = 0.0f;
  int kk = m;
  for (int pass = 0;; ++pass) {
    for (int i = tid; i < CS_BINS; i += CS_THREADS) hist[i] = 0u;
    __syncthreads();
    // eight loads in flight per thread before their bins are counted
    constexpr int CS_BATCH = 8;
    for (int64_t t0 = tid; t0 < N; t0 += (int64_t)CS_BATCH * CS_THREADS) {
      float v[CS_BATCH];
#pragma unroll
      for (int q = 0; q < CS_BATCH; ++q) {
        const int64_t t = t0 + (int64_t)q * CS_THREADS;
        v[q] = t < N ? col[t] : 0.0f;
      }
#pragma unroll
      for (int q = 0; q < CS_BATCH; ++q) {
        const int64_t t = t0 + (int64_t)q * CS_THREADS;
        const float x = fminf(fmaxf((v[q] - lo0) * sc0, 0.0f), CS_XTOP);
        const float y = (x - xa) * mul;
        if (t < N && y >= 0.0f && y < (float)CS_BINS) atomicAdd(&hist[(int)y], 1u);
      }
    }
    __syncthreads();
    // thread tid owns bins 4*tid .. 4*tid+3; suffix sums from the top bin down
    uint32_t h[4], own = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      h[q] = hist[4 * tid + q];
      own += h[q];
    }
    uint32_t suf = own;   // inclusive suffix within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_down(suf, o);
      if (l + o < 64) suf += y;
    }
    if (l == 0) wtot[0][w] = suf;
    __syncthreads();
    uint32_t later = 0;
    for (int q = w + 1; q < NW; ++q) later += wtot[0][q];
    uint32_t acc = suf - own + later;   // entries in bins above this thread's
#pragma unroll
    for (int q = 3; q >= 0; --q) {
      if (acc < (uint32_t)kk && acc + h[q] >= (uint32_t)kk) {
        bcast[0] = 4 * tid + q;
        bcast[1] = (int)acc;
        bcast[2] = (int)h[q];
      }
      acc += h[q];
    }
    __syncthreads();
    const int bstar = bcast[0], above = bcast[1], cnt = bcast[2];
    __syncthreads();   // bcast and wtot are rewritten by the next pass
    const float nxa = xa + (float)bstar / mul;   // exact: at most 24 significant bits
    const double vlo = (double)lo0 + (double)nxa / (double)sc0;
    const double vhi = (double)lo0 + ((double)nxa + 1.0 / (double)mul) / (double)sc0;
    const double pad = (fabs(vlo) + fabs(vhi) + fabs((double)lo0)) * 1e-6 + 1e-30;
    tlo = f_down(vlo - 2.0 * (double)beta - pad);
    thi = f_up(vhi + 2.0 * (double)beta + pad);
    // one nested level reaches the float spacing of the coordinate; finer gains nothing
    if (cnt > CS_NEAR - CS_SLACK && pass < 1 && vhi - vlo > 4.0 * (double)beta) {
      xa = nxa;
      mul *= (float)CS_BINS;
      kk -= above;
      continue;
    }
    break;
  }

  // collect pass, in index order: sure members straight to the output, band entries to LDS
  int base_s = 0, base_n = 0;
  constexpr int CS_CBATCH = 4;   // blocks of CS_THREADS entries whose loads are in flight together
  float vb[CS_CBATCH];
  for (int64_t t0 = 0; t0 < N; t0 += CS_THREADS) {
    const int qb = (int)((t0 / CS_THREADS) % CS_CBATCH);
    if (qb == 0)
#pragma unroll
      for (int q = 0; q < CS_CBATCH; ++q) {
        const int64_t tq = t0 + (int64_t)q * CS_THREADS + tid;
        vb[q] = tq < N ? col[tq] : NEG_INF;
      }
    const int64_t t = t0 + tid;
    float v = vb[0];
#pragma unroll
    for (int q = 1; q < CS_CBATCH; ++q)
      if (qb == q) v = vb[q];
    const bool sure = t < N && v > thi;
    const bool band = t < N && v >= tlo && v <= thi;
    const uint64_t ms = ballot(sure), mn = ballot(band);
    if (l == 0) {
      wtot[0][w] = (uint32_t)popc(ms);
      wtot[1][w] = (uint32_t)popc(mn);
    }
    __syncthreads();
    int off_s = base_s, off_n = base_n, tot_s = 0, tot_n = 0;
    for (int q = 0; q < NW; ++q) {
      const int cs = (int)wtot[0][q], cn = (int)wtot[1][q];
      if (q < w) {
        off_s += cs;
        off_n += cn;
      }
      tot_s += cs;
      tot_n += cn;
    }
    if (sure) {
      const int dst = off_s + popc(ms & lanemask_lt());
      if (dst < m) out[dst] = (int32_t)t;
    }
    if (band) {
      const int dst = off_n + popc(mn & lanemask_lt());
      if (dst < CS_NEAR) {
        near_idx[dst] = (int32_t)t;
        near_val[dst] = v;
      }
    }
    base_s += tot_s;
    base_n += tot_n;
    __syncthreads();
  }
  const int n_sure = base_s, n_band = base_n < CS_NEAR ? base_n : CS_NEAR;
  const int need = m - n_sure;
  if (n_sure > m || base_n > CS_NEAR || need > n_band) {
    if (tid == 0) {
      atomicAdd(a.counters + CNT_OVERFLOW, 1u);
      atomicOr(a.counters + CNT_ERROR, (uint32_t)ERRBIT_OVERFLOW);
    }
    return;
  }
  // float64 scores of the band, then rank by (score desc, index asc)
  for (int e = tid; e < n_band; e += CS_THREADS) near_e[e] = exact_dot<E, D>(V + (int64_t)near_idx[e] * D, brow);
  if (tid == 0 && n_band > 0) atomicAdd(a.counters + CNT_LOGIT_EXACT, (uint32_t)n_band);
  __syncthreads();
  uint32_t* chosen = hist;   // reuse
  for (int e = tid; e < n_band; e += CS_THREADS) {
    const double me = near_e[e];
    const int mi = near_idx[e];
    int rank = 0;
    for (int u = 0; u < n_band; ++u) {
      const double eu = near_e[u];
      rank += (eu > me) || (eu == me && near_idx[u] < mi);
    }
    chosen[e] = rank < need ? 1u : 0u;
  }
  __syncthreads();
  if (w == 0) {   // chosen band entries after the sure ones, in index order
    int off = n_sure;
    for (int base = 0; base < n_band; base += 64) {
      const int e = base + l;
      const bool c = e < n_band && chosen[e] != 0u;
      const uint64_t mk = ballot(c);
      if (c) out[off + popc(mk & lanemask_lt())] = near_idx[e];
      off += popc(mk);
    }
  }
}

template <class E, int D>
static hipError_t launch_cs(const ColSelectArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((k_col_select<E, D>), dim3((unsigned)a.n_b), dim3(CS_THREADS), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_col_select(bool is_bf16, int d, const ColSelectArgs& a, hipStream_t st) {
#define RECE_CS(E, DD) \
  if (d == DD) return launch_cs<E, DD>(a, st);
  if (is_bf16) {
    RECE_CS(bf16, 32) RECE_CS(bf16, 64) RECE_CS(bf16, 128) RECE_CS(bf16, 256)
  } else {
    RECE_CS(float, 32) RECE_CS(float, 64) RECE_CS(float, 128) RECE_CS(float, 256)
  }
#undef RECE_CS
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------ small helpers
// start[key], end[key]: the range of sorted positions q whose element keys[sorted[q]] is key.
__global__ __launch_bounds__(256) void k_group_bounds(const int32_t* __restrict__ keys,
                                                      const int32_t* __restrict__ sorted, int64_t n,
                                                      int32_t* __restrict__ start, int32_t* __restrict__ end) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= n) return;
  const int key = keys[sorted[q]];
  if (q == 0 || keys[sorted[q - 1]] != key) start[key] = (int32_t)q;
  if (q == n - 1 || keys[sorted[q + 1]] != key) end[key] = (int32_t)(q + 1);
}

hipError_t launch_group_bounds(const int32_t* keys, const int32_t* sorted, int64_t n, int32_t* start, int32_t* end,
                               hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_group_bounds, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, keys, sorted, n, start,
                     end);
  return hipGetLastError();
}

// ------------------------------------------------------------ merge per position
// Per wave: the merge list (up to 2k entries, as topk_wave_bytes), then a hash set of
// the ids in the list (open addressing, at most a quarter full).
__host__ __device__ constexpr int merge_hash_size(int k) {
  int h = 256;
  while (h < 4 * k) h *= 2;
  return h;
}
__host__ __device__ constexpr size_t merge_list_bytes(int k) { return (topk_wave_bytes(2 * k) + 15) / 16 * 16; }
__host__ __device__ constexpr size_t merge_wave_bytes(int k) {
  return merge_list_bytes(k) + (size_t)merge_hash_size(k) * 4;
}
constexpr uint32_t HASH_EMPTY = 0xFFFFFFFFu;

// Insert item id j (>= 0) into the wave's hash set; true if it was not there.
__device__ __forceinline__ bool hash_insert(uint32_t* tab, int hmask, int j) {
  int h = (int)(((uint32_t)j * 2654435761u) >> 8) & hmask;
  while (true) {
    const uint32_t old = atomicCAS(tab + h, HASH_EMPTY, (uint32_t)j);
    if (old == HASH_EMPTY) return true;
    if (old == (uint32_t)j) return false;
    h = (h + 1) & hmask;
  }
}
size_t merge_lds_bytes(int k) { return 4 * ((merge_wave_bytes(k) + 15) / 16 * 16); }

template <class E, int D>
__device__ __forceinline__ void sce_merge_row(const MergeArgs& a, char* smem, int w, int64_t i, uint32_t& nexact) {
  const int l = lane_id();
  const int k = a.k;
  char* base = smem + (size_t)w * ((merge_wave_bytes(k) + 15) / 16 * 16);
  const MergeLds L = carve_topk(base, 2 * k);
  uint32_t* tab = reinterpret_cast<uint32_t*>(base + merge_list_bytes(k));   // the ids in L
  const int hmask = merge_hash_size(k) - 1;
  for (int t = l; t <= hmask; t += WAVE) tab[t] = HASH_EMPTY;
  wave_sync();
  const E* X = static_cast<const E*>(a.X);
  const E* Y = static_cast<const E*>(a.Y);
  const E* xrow = X + i * D;
  const float beta = a.beta_coef * a.xnorm[i] * __uint_as_float(a.ymax_bits[0]);

  const int g0 = a.pstart[i], g1 = a.pend[i];
  int cnt = 0;
  bool reduced = false, truncated = false;
  double te = -__builtin_huge_val();
  int tid = -1;
  int trunc_slot = -1;
  for (int q = g0; q < g1; ++q) {
    const int slot = a.sorted[q];
    if (a.slot_tid[slot] != -1) {   // this bucket had more than k candidates
      if (!truncated) trunc_slot = slot;
      truncated = true;
    }
    for (int e0 = 0; e0 < k; e0 += WAVE) {
      const int e = e0 + l;
      const int j = e < k ? a.slot_negs[(int64_t)slot * k + e] : -1;
      const bool keep = j >= 0 && hash_insert(tab, hmask, j);   // ids already in L are dropped
      const uint64_t mk = ballot(keep);
      if (keep) {
        const int dst = cnt + popc(mk & lanemask_lt());
        L.ids[dst] = j;
        L.vals[dst] = a.slot_negl[(int64_t)slot * k + e];
      }
      cnt += popc(mk);
      if (!ballot(j >= 0)) break;   // lists are -1 padded at the end
    }
    wave_sync();
    if (cnt > k) {
      reduce_to_k<E, D>(L, cnt, k, beta, xrow, Y, te, tid, nexact, a.counters);
      cnt = k;
      reduced = true;
      // the set again holds exactly the ids left in L
      for (int t = l; t <= hmask; t += WAVE) tab[t] = HASH_EMPTY;
      wave_sync();
      for (int t = l; t < cnt; t += WAVE) hash_insert(tab, hmask, L.ids[t]);
      wave_sync();
    }
  }
  if (!reduced && truncated) {   // the union is one bucket's list: its threshold stands
    te = a.slot_te[trunc_slot];
    tid = a.slot_tid[trunc_slot];
  }
  const bool none = g1 <= g0 || k == 0;
  const bool all = !none && !reduced && !truncated;

  float mx = NEG_INF;
  for (int t = l; t < cnt; t += WAVE) mx = fmaxf(mx, L.vals[t]);
  mx = wave_max(mx);
  float se = 0.0f;
  for (int t = l; t < cnt; t += WAVE) se += __expf(L.vals[t] - mx);
  se = wave_sumf(se);
  if (a.negs)
    for (int t = l; t < k; t += WAVE) a.negs[i * k + t] = t < cnt ? L.ids[t] : -1;
  if (l == 0) {
    const double b2 = (double)beta * (1.0 + 1e-6);
    if (none) {
      a.thr_e[i] = __builtin_huge_val();
      a.thr_id[i] = -2;
      a.thr_lo[i] = a.thr_hi[i] = __builtin_huge_valf();
    } else if (all) {
      a.thr_e[i] = -__builtin_huge_val();
      a.thr_id[i] = -1;
      a.thr_lo[i] = a.thr_hi[i] = NEG_INF;
    } else {
      a.thr_e[i] = te;
      a.thr_id[i] = tid;
      a.thr_lo[i] = f_down(te - b2);
      a.thr_hi[i] = f_up(te + b2);
    }
    a.mshift[i] = cnt > 0 ? mx : 0.0f;
    a.ssum[i] = cnt > 0 ? se : 0.0f;
    a.nmem[i] = cnt;
  }
}

// A fixed grid: each wave takes positions w0, w0 + waves, ... (no block barrier in
// this kernel); the float64 count is flushed once per wave (one shared address).
template <class E, int D>
__global__ __launch_bounds__(256) void k_sce_merge(MergeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int w = threadIdx.x >> 6;
  const int64_t waves = (int64_t)gridDim.x * 4;
  uint32_t nexact = 0;
  for (int64_t i = (int64_t)blockIdx.x * 4 + w; i < a.s; i += waves) sce_merge_row<E, D>(a, smem, w, i, nexact);
  flush_count(a.counters + CNT_LOGIT_EXACT, nexact);
}

template <class E, int D>
static hipError_t launch_mg(const MergeArgs& a, hipStream_t st) {
  const size_t lds = merge_lds_bytes(a.k);
  auto kern = k_sce_merge<E, D>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  int64_t fit = 0;
  e = resident_blocks(reinterpret_cast<const void*>(kern), 256, lds, &fit);
  if (e != hipSuccess) return e;
  const int64_t want = (a.s + 3) / 4;
  hipLaunchKernelGGL(kern, dim3((unsigned)std::max<int64_t>(1, std::min(want, fit))), dim3(256), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_sce_merge(bool is_bf16, int d, const MergeArgs& a, hipStream_t st) {
#define RECE_MG(E, DD) \
  if (d == DD) return launch_mg<E, DD>(a, st);
  if (is_bf16) {
    RECE_MG(bf16, 32) RECE_MG(bf16, 64) RECE_MG(bf16, 128) RECE_MG(bf16, 256)
  } else {
    RECE_MG(float, 32) RECE_MG(float, 64) RECE_MG(float, 128) RECE_MG(float, 256)
  }
#undef RECE_MG
  return hipErrorInvalidValue;
}

}  // namespace rece
