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

// ------------------------------------------------------------ listed column selection
// The b largest scores of every bucket column without storing the score matrix:
// the scores are recomputed by matrix cores in each pass over the rows.
//   CP_MINMAX  row norms, largest norm, smallest and largest score of each column;
//   CP_HIST    per row block, a 32-bin histogram of each undecided column at the
//              current level (bins of the column's [smallest, largest] range at
//              level 1, of the previous level's listing bins after that);
//   k_col_thresh  per column, the boundary bin and the listing bin below the
//              lowest float32 score a member can have (boundary minus 2 beta), or,
//              when the listed entries would not fit the list, the next level;
//   CP_LIST    every entry at or above the listing bin, with its float32 score,
//              into the column's list (each row block its own stretch of it);
//   k_col_select  (listed) the exact b largest of the list.
// Every pass computes a score with the same instructions, so a score falls into
// the same bin in each of them and the per-block counts of the histogram pass are
// the per-block list lengths of the listing pass.
constexpr float COL_XTOP = 31.999998f;     // largest float below 32
constexpr int CP_WAVES = 8;
constexpr int CP_CG = 512;                 // columns per workgroup at most
constexpr int CP_HSTRIDE = COL_BINS + 1;   // words per column histogram (odd stride)

// Inverse of fkey.
__device__ __forceinline__ float fkey_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// Histogram coordinate at a level: the same float operations in every pass and in
// the threshold kernel.
__device__ __forceinline__ float col_x(float v, float sc, float nlsc) {
  return __builtin_amdgcn_fmed3f(fmaf(v, sc, nlsc), 0.0f, COL_XTOP);
}
__device__ __forceinline__ float col_y(float v, float sc, float nlsc, float mul, float nxm) {
  return fmaf(col_x(v, sc, nlsc), mul, nxm);
}
// Smallest float32 v with col_y(v) >= yt (col_y does not decrease with v), found by
// bisection over the order keys of -inf .. +inf; +inf when no finite score gets
// there.  The passes then test v >= that value instead of computing y.
__device__ float col_vmin(const ColState& s, float yt) {
  uint32_t lo = fkey(NEG_INF), hi = fkey(__builtin_huge_valf());
  auto ok = [&](uint32_t k) { return col_y(fkey_inv(k), s.sc, s.nlsc, s.mul, s.nxm) >= yt; };
  if (ok(lo)) return NEG_INF;
  if (!ok(hi)) return __builtin_huge_valf();
  while (hi - lo > 1u) {   // ok(hi), !ok(lo)
    const uint32_t mid = lo + (hi - lo) / 2u;
    if (ok(mid)) hi = mid;
    else lo = mid;
  }
  return fkey_inv(hi);
}

// Squared norm of this lane's part of a fragment row, one k-slice at a time.
__device__ __forceinline__ float slice_sq(bf16x8 a, float acc) {
  const u32x4 w = __builtin_bit_cast(u32x4, a);
#pragma unroll
  for (int q = 0; q < 4; ++q) acc = bf16_pair_sq_acc(w[q], acc);
  return acc;
}
__device__ __forceinline__ float slice_sq(float a, float acc) { return fmaf(a, a, acc); }

// Bucket vectors of a wave: CBW column blocks of 16, held in registers (at most
// 128 registers of fragments).
template <class E, int D> struct ColPassShape {
  static constexpr int FV = D * (int)sizeof(E) / 16;   // registers of one fragment
  static constexpr int CBW = FV >= 64 ? 1 : (128 / FV >= 4 ? 4 : 128 / FV);
  static constexpr int CG = CP_WAVES * CBW * 16;       // columns of a workgroup
  static constexpr int RT = D * (int)sizeof(E) > 512 ? 32 : 64;   // rows per LDS tile
};

// One workgroup: a row block against CG bucket columns; wave w owns columns
// w*CBW*16 .. +CBW*16 (bucket vectors in registers) and the workgroup's rows
// stream through LDS in tiles of RT, double buffered.
template <class E, int D, int MODE>
__global__ __launch_bounds__(CP_WAVES * 64) void k_col_pass(ColPassArgs a) {
  using S = ColPassShape<E, D>;
  constexpr int P = Pitch<E, D>::value;
  constexpr int CBW = S::CBW, CG = S::CG, RT = S::RT;
  constexpr int CPR = D * (int)sizeof(E) / 16;   // 16-byte chunks per row
  constexpr int TCH = RT * CPR;                  // chunks per tile
  constexpr int NT = CP_WAVES * 64;
  constexpr int LPT = (TCH + NT - 1) / NT;       // chunks per thread
  __shared__ __attribute__((aligned(16))) E tile[2][RT * P];
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  if (MODE == CP_HIST && a.level > 1 && a.active[a.level] == 0u) return;   // nothing undecided
  const int g = blockIdx.x % a.n_g, r = blockIdx.x / a.n_g;
  const int c0 = g * CG;
  const int ncol = min(CG, a.nb_pad - c0);
  const int tid = threadIdx.x, w = tid >> 6, l = lane_id(), grp = l >> 4;
  // per-column state in LDS (CP_HIST, CP_LIST)
  float* s_nl = reinterpret_cast<float*>(dyn);   // nlsc
  float* s_sc = s_nl + CG;
  float* s_nx = s_sc + CG;                        // nxm
  float* s_mul = s_nx + CG;
  float* s_fl = s_mul + CG;   // CP_HIST: smallest score counted; CP_LIST: smallest score listed (+inf: none)
  int32_t* s_off = reinterpret_cast<int32_t*>(s_fl + CG);
  int32_t* s_pos = s_off + CG;
  uint32_t* h = reinterpret_cast<uint32_t*>(s_pos + CG);   // CP_HIST: [CG][CP_HSTRIDE]
  if (MODE != CP_MINMAX) {
    // every column of the group's width (a wave's last blocks may lie past ncol):
    // columns past n_b are neither counted nor listed
    for (int i = tid; i < CG; i += NT) {
      const int c = c0 + i;
      ColState cs{};
      cs.level = -1;
      if (i < ncol && c < a.n_b) cs = a.cs[c];
      s_nl[i] = cs.nlsc;
      s_sc[i] = cs.sc;
      s_nx[i] = cs.nxm;
      s_mul[i] = cs.mul;
      if (MODE == CP_HIST) {
        const bool on = i < ncol && c < a.n_b && cs.level == a.level;
        s_fl[i] = on ? cs.vgate : __builtin_huge_valf();
      } else {
        const bool on = i < ncol && c < a.n_b && cs.level == 0 && cs.nlist > 0;
        s_fl[i] = on ? cs.vlist : __builtin_huge_valf();
        s_off[i] = on ? a.offs[(int64_t)c * a.n_rb + r] : 0;
        s_pos[i] = 0;
      }
    }
    if (MODE == CP_HIST)
      for (int i = tid; i < ncol * CP_HSTRIDE; i += NT) h[i] = 0u;
  }

  const E* __restrict__ V = static_cast<const E*>(a.V);
  const E* __restrict__ Bt = static_cast<const E*>(a.Bt);
  const int64_t N = a.N;
  const int64_t row0 = (int64_t)r * a.rows_pb;
  const int ntile = (int)(a.rows_pb / RT);
  // this wave's bucket vectors: column blocks 0 .. nbw-1 of its CBW lie inside the group
  const int wc0 = w * CBW * 16;   // first local column of the wave
  const int nbw = min(CBW, max(0, (ncol - wc0) / 16));   // ncol is a multiple of 16
  const bool wave_on = nbw > 0;
  Frag<E, D> bf[CBW];
#pragma unroll
  for (int cb = 0; cb < CBW; ++cb) {
    const int bc = c0 + wc0 + cb * 16 + (l & 15);
    bf[cb].load_global(bc < a.n_b ? Bt + (int64_t)bc * D : nullptr);
  }
  float mx[CBW], mn[CBW];
#pragma unroll
  for (int cb = 0; cb < CBW; ++cb) {
    mx[cb] = NEG_INF;
    mn[cb] = __builtin_huge_valf();
  }
  float nmax = 0.0f;
  // column blocks with a counted (CP_HIST) or listed (CP_LIST) column
  bool cb_on[CBW];
#pragma unroll
  for (int cb = 0; cb < CBW; ++cb) cb_on[cb] = true;
  u32x4 pre[LPT];
  // tile t of the row block into registers (zeros past N)
#define CP_LOAD_TILE(t)                                                                         \
  _Pragma("unroll") for (int q = 0; q < LPT; ++q) {                                             \
    const int e = tid + q * NT;                                                                 \
    const int64_t row = row0 + (int64_t)(t) * RT + e / CPR;                                     \
    pre[q] = u32x4{0u, 0u, 0u, 0u};                                                             \
    if (e < TCH && row < N)                                                                     \
      pre[q] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(V + row * D) + (e % CPR) * 16); \
  }
#define CP_STORE_TILE(buf)                                                                      \
  _Pragma("unroll") for (int q = 0; q < LPT; ++q) {                                             \
    const int e = tid + q * NT;                                                                 \
    if (e < TCH) *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(tile[buf] + (e / CPR) * P) + (e % CPR) * 16) = pre[q]; \
  }
  CP_LOAD_TILE(0)
  CP_STORE_TILE(0)
  __syncthreads();
  if (MODE != CP_MINMAX) {
#pragma unroll
    for (int cb = 0; cb < CBW; ++cb)
      cb_on[cb] = cb < nbw && ballot(s_fl[wc0 + cb * 16 + (l & 15)] < __builtin_huge_valf()) != 0;
  }

  for (int it = 0; it < ntile; ++it) {
    if (it + 1 < ntile) {
      CP_LOAD_TILE(it + 1)
    }
    const E* tb = tile[it & 1];
    const int64_t trow = row0 + (int64_t)it * RT;
    const bool tile_full = trow + RT <= N;
#pragma unroll
    for (int rf = 0; rf < RT / 16; ++rf) {
      const E* arow = tb + (rf * 16 + (l & 15)) * P;
      const bool norm_wave = MODE == CP_MINMAX && g == 0 && w == rf;   // row norms, one wave per fragment
      f32x4 sv[CBW];
#pragma unroll
      for (int cb = 0; cb < CBW; ++cb) sv[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
      Frag<E, D> af;
      af.load_lds(arow);
      float nacc = 0.0f;
      if (norm_wave)
#pragma unroll
        for (int ks = 0; ks < Frag<E, D>::KS; ++ks) nacc = slice_sq(af.v[ks], nacc);
#pragma unroll
      for (int cb = 0; cb < CBW; ++cb)
        if (cb < nbw && cb_on[cb]) sv[cb] = mma_block(af, bf[cb], sv[cb]);
      if (norm_wave) {
        float acc = nacc;
        acc += __shfl_xor(acc, 16);
        acc += __shfl_xor(acc, 32);
        const int64_t row = trow + rf * 16 + (l & 15);
        // float32 sum of squares: relative error below d * 2^-24 < 2^-12; round the norm up
        const float nrm = row < N ? sqrtf(acc) * (1.0f + 0.0005f) : 0.0f;
        if (a.norms && grp == 0 && row < N) a.norms[row] = nrm;
        nmax = fmaxf(nmax, nrm);
      }
      if (!wave_on) continue;
      // element v of block cb: row trow + 16 rf + 4 grp + v, local column wc0 + 16 cb + (l & 15)
      const int64_t rg = trow + rf * 16 + 4 * grp;
      const int nv = (int)min<int64_t>(4, max<int64_t>(0, N - rg));   // valid rows of this lane
#pragma unroll
      for (int cb = 0; cb < CBW; ++cb) {
        if (cb >= nbw || !cb_on[cb]) continue;
        const int col = wc0 + cb * 16 + (l & 15);
        if (MODE == CP_MINMAX) {
          if (tile_full) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              mx[cb] = fmaxf(mx[cb], sv[cb][v]);
              mn[cb] = fminf(mn[cb], sv[cb][v]);
            }
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (v < nv) {
                mx[cb] = fmaxf(mx[cb], sv[cb][v]);
                mn[cb] = fminf(mn[cb], sv[cb][v]);
              }
          }
        } else if (MODE == CP_HIST && a.level == 1) {
          // every score counted: x is the level-1 coordinate
          const float sc = s_sc[col], nl = s_nl[col];
          uint32_t* hc = h + col * CP_HSTRIDE;
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (tile_full || v < nv) atomicAdd(&hc[(int)col_x(sv[cb][v], sc, nl)], 1u);
        } else if (MODE == CP_HIST) {
          const float gate = s_fl[col];
          uint32_t qm = 0u;   // bit v: at or above the gate
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (sv[cb][v] >= gate && v < nv) qm |= 1u << v;
          if (qm) {
            const float sc = s_sc[col], nl = s_nl[col], mul = s_mul[col], nx = s_nx[col];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float y = col_y(sv[cb][v], sc, nl, mul, nx);
              if ((qm & (1u << v)) && y < (float)COL_BINS) atomicAdd(&h[col * CP_HSTRIDE + (int)y], 1u);
            }
          }
        } else {
          const float gate = s_fl[col];
          uint32_t qm = 0u;   // bit v: listed
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (sv[cb][v] >= gate && (tile_full || v < nv)) qm |= 1u << v;
          if (qm) {
            int slot = s_off[col] + atomicAdd(&s_pos[col], __builtin_popcount(qm));
            const int64_t base = (int64_t)(c0 + col) * a.capl;
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (qm & (1u << v)) {
                if (slot >= 0 && slot < a.capl) {
                  a.lidx[base + slot] = (int32_t)(rg + v);
                  a.lval[base + slot] = sv[cb][v];
                }
                ++slot;
              }
          }
        }
      }
    }
    if (it + 1 < ntile) CP_STORE_TILE((it + 1) & 1)
    __syncthreads();
  }
#undef CP_LOAD_TILE
#undef CP_STORE_TILE
  if (MODE == CP_MINMAX) {
    if (g == 0 && a.norm_max_bits) {
      nmax = wave_max(nmax);
      if (l == 0) raise_max_bits(a.norm_max_bits, nmax);
    }
#pragma unroll
    for (int cb = 0; cb < CBW; ++cb) {
      float x = mx[cb], y = mn[cb];
      x = fmaxf(x, __shfl_xor(x, 16));
      x = fmaxf(x, __shfl_xor(x, 32));
      y = fminf(y, __shfl_xor(y, 16));
      y = fminf(y, __shfl_xor(y, 32));
      const int c = c0 + wc0 + cb * 16 + (l & 15);
      if (cb < nbw && grp == 0 && c < a.n_b && x >= y) {
        atomicMax(a.key_max + c, fkey(x));
        atomicMax(a.key_min + c, ~fkey(y));
      }
    }
  } else if (MODE == CP_HIST) {
    for (int i = tid; i < ncol * COL_BINS; i += NT) {
      const int col = i / COL_BINS, bin = i % COL_BINS;
      if (s_fl[col] < __builtin_huge_valf())
        a.hist[((int64_t)r * a.nb_pad + c0 + col) * COL_BINS + bin] = h[col * CP_HSTRIDE + bin];
    }
  }
}

template <class E, int D>
static int col_group_width() {
  return ColPassShape<E, D>::CG;
}
static int col_group_width(bool is_bf16, int d) {
#define RECE_CW(E, DD) \
  if (d == DD) return col_group_width<E, DD>();
  if (is_bf16) {
    RECE_CW(bf16, 32) RECE_CW(bf16, 64) RECE_CW(bf16, 128) RECE_CW(bf16, 256)
  } else {
    RECE_CW(float, 32) RECE_CW(float, 64) RECE_CW(float, 128) RECE_CW(float, 256)
  }
#undef RECE_CW
  return CP_CG;
}

void col_pass_shape(bool is_bf16, int d, int64_t n, int nb_pad, int64_t* rows_pb, int* n_rb, int* cg, int* n_g) {
  constexpr int64_t STEP = 64;
  *cg = col_group_width(is_bf16, d);
  *n_g = (nb_pad + *cg - 1) / *cg;
  // about one workgroup per compute unit over all groups, at most 32768 rows per
  // block (16-bit histogram counts)
  const int64_t want = std::max<int64_t>(1, 256 / *n_g);
  int64_t rpb = (n + want - 1) / want;
  rpb = std::min<int64_t>(std::max<int64_t>(rpb, 1), 32768);
  rpb = (rpb + STEP - 1) / STEP * STEP;
  *rows_pb = rpb;
  *n_rb = (int)((n + rpb - 1) / rpb);
}

template <class E, int D>
static hipError_t launch_cp(int mode, const ColPassArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)a.n_rb * a.n_g)), block(CP_WAVES * 64);
  constexpr size_t CG = ColPassShape<E, D>::CG;
  if (a.cg != (int)CG) return hipErrorInvalidValue;
  if (mode == CP_MINMAX) {
    hipLaunchKernelGGL((k_col_pass<E, D, CP_MINMAX>), grid, block, 0, st, a);
  } else if (mode == CP_HIST) {
    hipLaunchKernelGGL((k_col_pass<E, D, CP_HIST>), grid, block, 7 * CG * 4 + CG * CP_HSTRIDE * 4, st, a);
  } else {
    hipLaunchKernelGGL((k_col_pass<E, D, CP_LIST>), grid, block, 7 * CG * 4, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_col_pass(bool is_bf16, int d, int mode, const ColPassArgs& a, hipStream_t st) {
  if (a.N <= 0) return hipSuccess;
#define RECE_CP(E, DD) \
  if (d == DD) return launch_cp<E, DD>(mode, a, st);
  if (is_bf16) {
    RECE_CP(bf16, 32) RECE_CP(bf16, 64) RECE_CP(bf16, 128) RECE_CP(bf16, 256)
  } else {
    RECE_CP(float, 32) RECE_CP(float, 64) RECE_CP(float, 128) RECE_CP(float, 256)
  }
#undef RECE_CP
  return hipErrorInvalidValue;
}

// Level-1 state of every column from its smallest and largest score.
__global__ void k_col_init(ColState* __restrict__ cs, const uint32_t* __restrict__ key_max,
                           const uint32_t* __restrict__ key_min, uint32_t* __restrict__ active, int n_b) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c < COL_LEVELS + 1) active[c] = 0u;
  if (c >= n_b) return;
  const float hi = fkey_inv(key_max[c]), lo = fkey_inv(~key_min[c]);
  float sc = hi > lo ? (float)COL_BINS / (hi - lo) : 0.0f;
  if (!(sc < __builtin_huge_valf())) sc = 0.0f;   // range below the float range's resolution: one bin
  ColState s{};
  s.lo = lo;
  s.sc = sc;
  s.nlsc = -(lo * sc);
  s.xa = 0.0f;
  s.mul = 1.0f;
  s.nxm = -0.0f;
  s.tlo = NEG_INF;
  s.level = 1;
  s.bl = COL_NONE;
  s.nlist = 0;
  s.above = 0;
  s.vgate = NEG_INF;
  s.vlist = __builtin_huge_valf();
  cs[c] = s;
}

hipError_t launch_col_init(ColState* cs, const uint32_t* key_max, const uint32_t* key_min, uint32_t* active, int n_b,
                           hipStream_t st) {
  const int n = std::max(n_b, COL_LEVELS + 1);
  hipLaunchKernelGGL(k_col_init, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, cs, key_max, key_min, active,
                     n_b);
  return hipGetLastError();
}

// One workgroup per column waiting for this level: boundary bin, listing bin, and
// either the list layout (per row block offsets) or the next level.
__global__ __launch_bounds__(256) void k_col_thresh(ColThreshArgs a) {
  __shared__ uint32_t part[8][COL_BINS];
  __shared__ uint32_t H[COL_BINS];
  __shared__ int sh[4];
  __shared__ int32_t wsum[4];
  const int c = blockIdx.x;
  if (c >= a.n_b) return;
  if (a.level > 1 && a.active[a.level] == 0u) return;
  ColState s = a.cs[c];
  if (s.level != a.level) return;
  const int tid = threadIdx.x, l = lane_id(), w = tid >> 6;
  {
    const int bin = tid % COL_BINS, sl = tid / COL_BINS;
    uint32_t acc = 0;
    for (int r = sl; r < a.n_rb; r += 8) acc += a.hist[((int64_t)r * a.nb_pad + c) * COL_BINS + bin];
    part[sl][bin] = acc;
  }
  __syncthreads();
  if (tid < COL_BINS) {
    uint32_t t = 0;
    for (int q = 0; q < 8; ++q) t += part[q][tid];
    H[tid] = t;
  }
  __syncthreads();
  if (tid == 0) {
    int64_t cum = s.above;
    int bstar = -1;
    for (int b = COL_BINS - 1; b >= 0; --b) {
      cum += H[b];
      if (cum >= a.m) {
        bstar = b;
        break;
      }
    }
    int bl = COL_NONE;
    float tlo = s.tlo;
    if (bstar >= 0 && s.sc > 0.0f) {
      // a member's float64 score is at least the boundary bin's lower end less beta
      // (at least m scores reach that end); its float32 score is within beta of it.
      // Value of coordinate x: (x - nlsc) / sc, up to the float32 rounding of x
      // (relative 2^-24), which the pad covers.
      const float vmax = __uint_as_float(a.vmax_bits[0]), bn = a.bnorm_max[0];
      const double beta = (double)(a.beta_coef * vmax * bn);
      const double xlo = (double)s.xa + (double)bstar / (double)s.mul;
      const double xhi = (double)s.xa + (double)(bstar + 1) / (double)s.mul;
      const double vlo = (xlo - (double)s.nlsc) / (double)s.sc;
      const double vhi = (xhi - (double)s.nlsc) / (double)s.sc;
      const double pad = (fabs(vlo) + fabs(vhi) + fabs((double)s.lo)) * 1e-6 + 1e-30;
      tlo = fmaxf(f_down(vlo - 2.0 * beta - pad), s.tlo);
      const float y = col_y(tlo, s.sc, s.nlsc, s.mul, s.nxm);
      bl = y > 0.0f ? (int)y : 0;
      bl = min(bl, bstar);
    } else if (bstar >= 0) {
      bl = 0;   // one bin holds every score
    }
    int64_t nl = s.above;
    if (bl != COL_NONE)
      for (int b = bl; b < COL_BINS; ++b) nl += H[b];
    int refine = 0, hi_bin = COL_BINS;
    if (bl != COL_NONE && nl > a.capl && a.level < COL_LEVELS && s.sc > 0.0f) {
      int span = 1;   // the listing bins up to the boundary bin, cut in 32 again
      while (span < bstar - bl + 1) span <<= 1;
      refine = 1;
      hi_bin = bl + span;
    }
    if (refine) {
      int64_t ab = s.above;
      for (int b = hi_bin; b < COL_BINS; ++b) ab += H[b];
      s.above = (int)ab;
      s.xa = s.xa + (float)bl / s.mul;
      s.mul = s.mul * ((float)COL_BINS / (float)(hi_bin - bl));
      s.nxm = -(s.xa * s.mul);   // exact: xa has few significant bits, mul is a power of two
      s.tlo = tlo;
      s.vgate = col_vmin(s, 0.0f);
      s.level = a.level + 1;
      a.active[a.level + 1] = 1u;
      atomicAdd(a.counters + CNT_COL_REFINE, 1u);
    } else {
      s.level = 0;
      s.tlo = tlo;
      if (bl == COL_NONE || nl > a.capl) {   // fewer than m counted, or the list does not fit
        atomicOr(a.counters + CNT_ERROR, (uint32_t)ERRBIT_OVERFLOW);
        atomicAdd(a.counters + CNT_OVERFLOW, 1u);
        s.bl = COL_NONE;
        s.nlist = -1;
        bl = COL_NONE;
      } else {
        s.bl = bl;
        s.nlist = (int)nl;
        s.vlist = col_vmin(s, (float)bl);
      }
    }
    a.cs[c] = s;
    sh[0] = bl;
    sh[1] = refine;
    sh[2] = hi_bin;
  }
  __syncthreads();
  const int bl = sh[0], refine = sh[1], hi_bin = sh[2];
  int32_t* ab = a.above_r + (int64_t)c * a.n_rb;
  if (refine) {
    // entries above the next level's range, per row block
    for (int r = tid; r < a.n_rb; r += 256) {
      const uint32_t* hr = a.hist + ((int64_t)r * a.nb_pad + c) * COL_BINS;
      int32_t n = a.level > 1 ? ab[r] : 0;
      for (int b = hi_bin; b < COL_BINS; ++b) n += (int32_t)hr[b];
      ab[r] = n;
    }
    return;
  }
  if (bl == COL_NONE) return;
  // list offsets: per row block, the entries at or above the listing bin
  int32_t* off = a.offs + (int64_t)c * a.n_rb;
  int32_t carry = 0;
  for (int r0 = 0; r0 < a.n_rb; r0 += 256) {
    const int r = r0 + tid;
    int32_t n = 0;
    if (r < a.n_rb) {
      const uint32_t* hr = a.hist + ((int64_t)r * a.nb_pad + c) * COL_BINS;
      n = a.level > 1 ? ab[r] : 0;
      for (int b = bl; b < COL_BINS; ++b) n += (int32_t)hr[b];
    }
    int32_t x = n;   // inclusive scan in the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t y = __shfl_up(x, o);
      if (l >= o) x += y;
    }
    if (l == 63) wsum[w] = x;
    __syncthreads();
    int32_t before = carry;
    for (int q = 0; q < w; ++q) before += wsum[q];
    if (r < a.n_rb) off[r] = before + x - n;
    int32_t tot = 0;
    for (int q = 0; q < 4; ++q) tot += wsum[q];
    carry += tot;
    __syncthreads();
  }
}

hipError_t launch_col_thresh(const ColThreshArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_col_thresh, dim3((unsigned)a.n_b), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ column top-m
constexpr int CS_BINS = 4096;
constexpr int CS_NEAR = 2048;               // entries within the boundary band
constexpr int CS_SLACK = 256;               // room for band entries outside the boundary bin
constexpr float CS_XTOP = 4095.9998f;       // largest histogram coordinate below 4096
constexpr int CS_THREADS = 1024;

// One workgroup per bucket column.  Selection order: (float64 score desc, index asc).
// Dense: the column's N scores.  Listed: the column's list (a superset of the b
// largest, in no particular order); the chosen rows are then sorted by index.
template <class E, int D, bool LISTED>
__global__ __launch_bounds__(CS_THREADS) void k_col_select(ColSelectArgs a) {
  __shared__ uint32_t hist[CS_BINS];
  __shared__ int32_t near_idx[CS_NEAR];
  __shared__ float near_val[CS_NEAR];
  __shared__ double near_e[CS_NEAR];
  __shared__ uint32_t wtot[2][CS_THREADS / 64];
  __shared__ int32_t bcast[4];
  __shared__ int32_t chosen_rows[LISTED ? COL_LIST_MAX_M : 1];
  const int b = blockIdx.x;
  const int m = a.m;
  int32_t* out = a.out + (int64_t)b * m;
  const int tid = threadIdx.x, l = lane_id(), w = tid >> 6;
  constexpr int NW = CS_THREADS / 64;
  if ((int64_t)m >= a.N) {   // the bucket takes every entry
    for (int64_t t = tid; t < a.N; t += CS_THREADS) out[t] = (int32_t)t;
    return;
  }
  int64_t N = a.N;
  const float* __restrict__ col;
  const int32_t* __restrict__ rows = nullptr;
  // on an error (reported through the counters) the bucket takes rows 0..m-1, so
  // that the kernels after this one still read valid rows
  auto fail_fill = [&]() {
    for (int t = tid; t < m; t += CS_THREADS) out[t] = t;
  };
  if constexpr (LISTED) {
    const int nl = a.cs[b].nlist;
    if (nl < 0) {   // did not fit its list: reported by the threshold kernel
      fail_fill();
      return;
    }
    N = nl;
    col = a.lval + (int64_t)b * a.capl;
    rows = a.lidx + (int64_t)b * a.capl;
  } else {
    col = a.PT + (int64_t)b * N;
  }
  // row of entry t
  auto row_of = [&](int64_t t) -> int32_t {
    if constexpr (LISTED) return rows[t];
    else return (int32_t)t;
  };
  // the chosen rows: straight to the output (dense), or to LDS for the sort (listed)
  auto put = [&](int slot, int32_t row) {
    if constexpr (LISTED) chosen_rows[slot] = row;
    else out[slot] = row;
  };
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

  // collect pass, in entry order: sure members to the output, band entries to LDS
  int base_s = 0, base_n = 0;
  int bad_row = 0;   // listed: a row outside [0, N) (a list inconsistent with its counts)
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
    const int32_t rw = t < N ? row_of(t) : 0;
    const bool ok = t < N && (!LISTED || (rw >= 0 && (int64_t)rw < a.N));
    bad_row |= (t < N && !ok) ? 1 : 0;
    const bool sure = ok && v > thi;
    const bool band = ok && v >= tlo && v <= thi;
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
      if (dst < m) put(dst, rw);
    }
    if (band) {
      const int dst = off_n + popc(mn & lanemask_lt());
      if (dst < CS_NEAR) {
        near_idx[dst] = rw;
        near_val[dst] = v;
      }
    }
    base_s += tot_s;
    base_n += tot_n;
    __syncthreads();
  }
  const int n_sure = base_s, n_band = base_n < CS_NEAR ? base_n : CS_NEAR;
  const int need = m - n_sure;
  const int any_bad = LISTED ? __syncthreads_or(bad_row) : 0;
  if (n_sure > m || base_n > CS_NEAR || need > n_band || any_bad) {
    if (tid == 0) {
      atomicAdd(a.counters + CNT_OVERFLOW, 1u);
      atomicOr(a.counters + CNT_ERROR, (uint32_t)ERRBIT_OVERFLOW);
    }
    fail_fill();
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
      if (c) put(off + popc(mk & lanemask_lt()), near_idx[e]);
      off += popc(mk);
    }
  }
  if constexpr (LISTED) {
    // bitonic sort of the m chosen rows (padded to a power of two), then out
    int p2 = 1;
    while (p2 < m) p2 <<= 1;
    __syncthreads();
    for (int e = m + tid; e < p2; e += CS_THREADS) chosen_rows[e] = 0x7fffffff;
    __syncthreads();
    for (int kb = 2; kb <= p2; kb <<= 1)
      for (int jb = kb >> 1; jb > 0; jb >>= 1) {
        for (int e = tid; e < p2; e += CS_THREADS) {
          const int f = e ^ jb;
          if (f > e) {
            const int32_t x = chosen_rows[e], y = chosen_rows[f];
            if ((x > y) == ((e & kb) == 0)) {
              chosen_rows[e] = y;
              chosen_rows[f] = x;
            }
          }
        }
        __syncthreads();
      }
    for (int e = tid; e < m; e += CS_THREADS) out[e] = chosen_rows[e];
  }
}

template <class E, int D>
static hipError_t launch_cs(const ColSelectArgs& a, hipStream_t st) {
  if (a.lidx) {
    if (a.m > COL_LIST_MAX_M && (int64_t)a.m < a.N) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_col_select<E, D, true>), dim3((unsigned)a.n_b), dim3(CS_THREADS), 0, st, a);
  } else {
    hipLaunchKernelGGL((k_col_select<E, D, false>), dim3((unsigned)a.n_b), dim3(CS_THREADS), 0, st, a);
  }
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
