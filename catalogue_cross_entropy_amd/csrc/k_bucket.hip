// Bucketing: the argmax over n_b random vectors of the signed scalar product
// b.v, for every position and every item (RECE page, Section 3, Algorithm 1,
// the two argmax lines; "index of the nearest vector from B in terms of dot
// product").  Ties go to the lowest index.
//
// The scores are computed on the matrix cores in float32 (bf16 or f32 inputs)
// and never stored.  The decision is the argmax of the float64 coordinate-order
// sums: a row whose float32 top-2 gap exceeds twice the error bound is decided
// by the float32 argmax; the others (rare) are appended to a list, and a second
// kernel decides them in float64 from the few vectors within twice the bound of
// the row's float32 maximum, so the slow rows neither stall the matrix-core
// kernel nor sit on its critical path.  (Small inputs decide their undecided
// rows inside the matrix-core kernel, all vectors in float64.)
#include <algorithm>
#include <type_traits>
#include <utility>

#include "rece_device.h"
#include "rece_internal.h"
#include "rece_stream.h"

namespace rece {

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), unrolled at compile time.
template <class F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

__global__ void k_fill_u32(uint32_t* p, uint32_t v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, v, n);
  return hipGetLastError();
}

// Zero three small regions in one launch (block y = region).
__global__ void k_zero3(uint32_t* a, int na, uint32_t* b, int nb, uint32_t* c, int nc) {
  uint32_t* p = blockIdx.y == 0 ? a : (blockIdx.y == 1 ? b : c);
  const int n = blockIdx.y == 0 ? na : (blockIdx.y == 1 ? nb : nc);
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

hipError_t launch_zero3(uint32_t* a, int na, uint32_t* b, int nb, uint32_t* c, int nc, hipStream_t st) {
  hipLaunchKernelGGL(k_zero3, dim3(1, 3), dim3(256), 0, st, a, na, b, nb, c, nc);
  return hipGetLastError();
}

// Bt[rho][b][t] = B[rho][t][b]; bnorm_max[rho] = max_b ||b_b||_2 (rounded up).
// bnorm_max must be zero on entry.
template <class E>
__global__ void k_prep_b(const E* __restrict__ B, int d, int n_b, E* __restrict__ Bt,
                         uint32_t* __restrict__ bnorm_max_bits) {
  const int rho = blockIdx.y;
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= n_b) return;
  const E* src = B + (int64_t)rho * d * n_b;
  E* dst = Bt + ((int64_t)rho * n_b + b) * d;
  double ss = 0.0;
  for (int t0 = 0; t0 < d; t0 += 8) {   // d is a multiple of 8: eight loads in flight
    E v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[(int64_t)(t0 + u) * n_b + b];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      dst[t0 + u] = v[u];
      const double f = (double)to_f32(v[u]);
      ss = fma(f, f, ss);
    }
  }
  const float nrm = f_up(sqrt(ss) * (1.0 + 1e-12));
  atomicMax(bnorm_max_bits + rho, __float_as_uint(nrm));
}

hipError_t launch_prep_b(bool is_bf16, int d, const void* B, int rounds, int n_b, void* Bt, float* bnorm_max,
                         int zero_words, hipStream_t st) {
  // bnorm_max[0 .. rounds) and the zero_words following it are cleared (zero_words < 0:
  // the caller has cleared them)
  hipError_t e = zero_words < 0 ? hipSuccess
                                : launch_fill_u32(reinterpret_cast<uint32_t*>(bnorm_max), 0u, rounds + zero_words, st);
  if (e != hipSuccess) return e;
  dim3 grid((n_b + 255) / 256, rounds);
  if (is_bf16)
    hipLaunchKernelGGL(k_prep_b<bf16>, grid, dim3(256), 0, st, (const bf16*)B, d, n_b, (bf16*)Bt,
                       reinterpret_cast<uint32_t*>(bnorm_max));
  else
    hipLaunchKernelGGL(k_prep_b<float>, grid, dim3(256), 0, st, (const float*)B, d, n_b, (float*)Bt,
                       reinterpret_cast<uint32_t*>(bnorm_max));
  return hipGetLastError();
}

// Median of three integers (one v_med3_i32).
__device__ __forceinline__ int med3_i(int a, int b, int c) { return max(min(a, b), min(max(a, b), c)); }
// Maximum of three integers as one v_max3_i32 (the compiler splits max(max(a, b), c)
// into two instructions when it shares max(b, c) with a neighbouring med3).
__device__ __forceinline__ int max3_i(int a, int b, int c) {
  int r;
  asm("v_max3_i32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Wave-collective float64 argmax of x . b over the n_b vectors (lowest index
// among ties): every lane scores n_b / 64 of them in coordinate order.
template <class E, int D>
__device__ __forceinline__ int argmax_exact_wave(const E* __restrict__ x, const E* __restrict__ Bt, int n_b) {
  const int l = lane_id();
  double be = -__builtin_huge_val();
  int bi = 0x7fffffff;
#pragma unroll 1
  for (int b = l; b < n_b; b += WAVE) {
    const double e = exact_dot<E, D, 4>(x, Bt + (int64_t)b * D);
    if (e > be) {
      be = e;
      bi = b;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const double oe = __shfl_xor(be, o);
    const int ob = __shfl_xor(bi, o);
    if (oe > be || (oe == be && ob < bi)) {
      be = oe;
      bi = ob;
    }
  }
  return bi;
}

// One workgroup = 4 waves x 16*RF rows; each wave keeps the matrix-core
// fragments of its rows in registers.  The random vectors stream through a
// ring of three LDS tiles fed by asynchronous copies two tiles ahead, every
// tile used by all the workgroup's rows (RF > 1 for large inputs: fewer loads
// of the vectors per row).  Each lane keeps the running best and second-best
// scores of its share branch-free, as integer keys (max3 / med3 / max); equal
// scores leave best = second, which sends the row to the float64 decision
// (lowest index among exact ties).  256-byte rows: three workgroups per CU,
// with no spills (a spill reload inside the tile loop would wait for every
// copy in flight).
template <class E, int D, int RF>
__global__ __launch_bounds__(256, (D * sizeof(E) == 256) ? 3 : 1) void k_project_argmax(
    const E* __restrict__ V, int64_t n, const E* __restrict__ Bt, int n_b,
    const float* __restrict__ bnorm_max, float beta_coef, int32_t* __restrict__ ids,
    float* __restrict__ norms, uint32_t* __restrict__ norm_max_bits, int32_t* __restrict__ und,
    uint32_t* __restrict__ und_n, uint32_t* __restrict__ counters) {
  using G = TileGeom<E, D>;
  constexpr int NW = 4;
  // bf16: a ring of two tiles, copies one tile ahead (16 KB at 256-byte vectors; the
  // random vectors stay in the L2, so one tile of lead hides their copies, and the
  // smaller footprint leaves LDS to a kernel running beside this one); float32: three
  constexpr int RING = sizeof(E) == 2 ? 2 : 3;
  __shared__ __attribute__((aligned(1024))) char ring[RING * G::ROW_BYTES];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = lane_id();
  const int g = l >> 4;
  const int nt = (n_b + G::TI - 1) / G::TI;

  // the first two tiles of vectors are on their way while the rows load; every
  // tile takes the same number of copies from this wave
  dma_rows<E, D, NW>(ring, Bt, 0, n_b, w);
  if (RING == 3 && nt > 1) dma_rows<E, D, NW>(ring + G::ROW_BYTES, Bt, G::TI, n_b, w);

  Frag<E, D> a[RF];
#pragma unroll
  for (int f = 0; f < RF; ++f) {
    const int64_t rA = ((int64_t)blockIdx.x * NW + w) * 16 * RF + 16 * f + (l & 15);
    const E* rp = rA < n ? V + rA * D : nullptr;
    a[f].load_global(rp);
    a[f].settle();
  }

  // Running top-2 per output element as integer keys: the score's float32 bits with
  // the low `ib` bits replaced by the vector index.  Non-negative floats order like
  // their bits, so among non-negative scores the keys order as the truncated scores
  // (ties broken by index); negative scores order below every non-negative one.
  const int ib = n_b > 1 ? 32 - __builtin_clz((unsigned)(n_b - 1)) : 0;
  const int imask = (1 << ib) - 1;
  // bf16: the products are taken vectors x rows, so a lane's four scores of a block
  // belong to one row (l & 15) and four vectors (4g + v); the running top-2 is one
  // pair of keys per fragment (t1, t2), updated two keys at a time:
  //   top-2 of {t1 >= t2, kA, kB} = (max3(t1, kA, kB), max(t2, med3(t1, kA, kB))).
  // Per score: one and-or and, per two scores, one med3, one max3 and half of a
  // max3.  float32: vectors as columns (one vector, four rows per lane) and a pair
  // of keys per output element (best1, best2): one and-or, one max, one med3 per
  // score.
  int t1[RF], t2[RF];
  int best1[RF][4], best2[RF][4];
#pragma unroll
  for (int f = 0; f < RF; ++f) {
    t1[f] = INT32_MIN;
    t2[f] = INT32_MIN;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      best1[f][v] = INT32_MIN;
      best2[f][v] = INT32_MIN;
    }
  }

  if constexpr (sizeof(E) == 2) {
    // bf16: every fragment read is this lane's slot-0 address for its k-step plus
    // an immediate offset (the ring slot where it is known at compile time, and the
    // 16-vector block); only a last tile that passes n_b pads its scores.
    constexpr int KS = Frag<E, D>::KS;
    constexpr int NCB = G::TI / 16;
    const int q = l >> 4, n0 = l & 15;
    uint32_t fa0[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) fa0[ks] = lds_addr(ring + n0 * G::RB + (((4 * ks + q) ^ (n0 & G::SWM)) * 16));
    // this wave's copies of a tile: a uniform tile address plus this lane's 32-bit
    // offset inside the tile (tiles that pass n_b take dma_rows, which clamps)
    constexpr int NQ = G::ROW_DMA / NW;
    static_assert(G::ROW_DMA % NW == 0, "whole copies per wave");
    constexpr int LRB = ilog2(G::RB);
    uint32_t goff[NQ];   // byte offset of this lane's 16 bytes of copy qq inside a tile
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
      const int byte = (w + qq * NW) * 1024 + 16 * l;
      goff[qq] = (uint32_t)(byte ^ (((byte >> LRB) & G::SWM) << 4));
    }
    const int nfull_t = n_b / G::TI;   // tiles with no row past n_b
    // score: the NCB blocks of 16 vectors of tile t, fragment reads at offset OFF
    // from the addresses fa.  A tile: wait for its copies, meet the other waves,
    // issue the copies of tile t + 2, then score.  tile_fixed: the ring slot is
    // known at compile time (immediate offsets from the slot-0 addresses) and tile
    // t + 2 is full.  tile: the general form (runtime slot, clamped copies near the
    // end of the vectors, padded scores in a last partial tile).
    auto score = [&](auto pad_c, auto off_c, const uint32_t* fa, int t) {
      constexpr bool PAD = decltype(pad_c)::value;
      constexpr int OFF = decltype(off_c)::value;
      const int tb = t * G::TI + 4 * g;   // vector of element v of the tile's first block: tb + v
      static_for<NCB>([&](auto cb_c) {
        constexpr int cb = decltype(cb_c)::value;
        Frag<E, D> bf;
        u32x4 raw[KS];
        LdsReadOff128<KS, OFF + cb * 16 * G::RB>::run(fa, raw);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bf.v[ks] = __builtin_bit_cast(bf16x8, raw[ks]);
        const int i0 = tb + cb * 16;
        f32x4 c0{0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (PAD) {
#pragma unroll
          for (int v = 0; v < 4; ++v) c0[v] = i0 + v < n_b ? 0.0f : NEG_INF;
        }
        // the RF product chains k-step outer (independent chains back to back), then
        // the updates
        f32x4 acc[RF];
#pragma unroll
        for (int f = 0; f < RF; ++f) acc[f] = c0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int f = 0; f < RF; ++f)
            acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf.v[ks], a[f].v[ks], acc[f], 0, 0, 0);
#pragma unroll
        for (int f = 0; f < RF; ++f) {
          int key[4];   // acc[f][v]: vector 4g + v, row l & 15
#pragma unroll
          for (int v = 0; v < 4; ++v) key[v] = (__float_as_int(acc[f][v]) & ~imask) | (i0 + v);
#pragma unroll
          for (int h = 0; h < 4; h += 2) {
            const int m = med3_i(t1[f], key[h], key[h + 1]);
            t1[f] = max3_i(t1[f], key[h], key[h + 1]);
            t2[f] = max(t2[f], m);
          }
        }
      });
    };
    auto tile_fixed = [&](auto slot_c, int t) {   // t % 2 == SLOT and t + 1 < nfull_t
      constexpr int SLOT = decltype(slot_c)::value;
      wait_vmcnt_c<0>();   // tile t's copies (the only ones outstanding) landed
      raw_barrier();       // ... for every wave, and every wave is done with slot (t + 1) % 2
      const char* src = reinterpret_cast<const char*>(Bt) + (int64_t)(t + 1) * G::ROW_BYTES;
      char* dst = ring + ((SLOT + 1) % 2) * G::ROW_BYTES;
#pragma unroll
      for (int qq = 0; qq < NQ; ++qq) dma_copy16(src + goff[qq], dst + (w + qq * NW) * 1024);
      score(std::false_type{}, std::integral_constant<int, SLOT * G::ROW_BYTES>{}, fa0, t);
    };
    auto tile = [&](auto pad_c, int t) {
      wait_vmcnt_c<0>();
      raw_barrier();   // every wave's copies of tile t landed; slot (t + 1) % 2 is free
      const int slot = t % 2;
      if (t + 1 < nfull_t) {
        char* dst = ring + (size_t)((t + 1) % 2) * G::ROW_BYTES;
        const char* src = reinterpret_cast<const char*>(Bt) + (int64_t)(t + 1) * G::ROW_BYTES;
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq) dma_copy16(src + goff[qq], dst + (w + qq * NW) * 1024);
      } else if (t + 1 < nt) {
        dma_rows<E, D, NW>(ring + (size_t)((t + 1) % 2) * G::ROW_BYTES, Bt, (int64_t)(t + 1) * G::TI, n_b, w);
      }
      uint32_t fa[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) fa[ks] = fa0[ks] + (uint32_t)(slot * G::ROW_BYTES);
      score(pad_c, std::integral_constant<int, 0>{}, fa, t);
    };
    // tiles [0, tmain) in pairs of ring slots, the rest in the general form
    const int tmain = nfull_t >= 1 ? (nfull_t - 1) / 2 * 2 : 0;
    int t0 = 0;
    for (; t0 < tmain; t0 += 2) {
      tile_fixed(std::integral_constant<int, 0>{}, t0);
      tile_fixed(std::integral_constant<int, 1>{}, t0 + 1);
    }
    const int nfull = n_b % G::TI != 0 ? nt - 1 : nt;   // tiles without padding
    for (int t = t0; t < nfull; ++t) tile(std::false_type{}, t);
    if (nfull < nt) tile(std::true_type{}, nfull);
  } else {
  for (int t = 0; t < nt; ++t) {
      // tile t's copies are complete once only tile t+1's remain outstanding
      if (t + 1 < nt)
        wait_vmcnt_c<G::ROW_DMA / NW>();   // the fewest copies any wave issues per tile
      else
        wait_vmcnt_c<0>();
      raw_barrier();   // every wave's copies of tile t landed; slot (t+2) % 3 is free
      if (t + 2 < nt)
        dma_rows<E, D, NW>(ring + (size_t)((t + 2) % 3) * G::ROW_BYTES, Bt, (int64_t)(t + 2) * G::TI, n_b, w);
      const char* rows = ring + (size_t)(t % 3) * G::ROW_BYTES;
      const int b0 = t * G::TI;
      // vectors past n_b (last tile only) score -inf
      const int nvalid = n_b - b0;
  #pragma unroll
      for (int cb = 0; cb < G::TI / 16; ++cb) {
        Frag<E, D> bf;
        TileFrag<E, D>::load(bf, rows, cb * 16 + (l & 15));
        // the vector index as one register (one and-or per score below)
        const int bcol = settled(b0 + cb * 16 + (l & 15));
        const float pad = cb * 16 + (l & 15) < nvalid ? 0.0f : NEG_INF;
  #pragma unroll
        for (int f = 0; f < RF; ++f) {
          const f32x4 acc = mma_block(a[f], bf, f32x4{pad, pad, pad, pad});
  #pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int key = (__float_as_int(acc[v]) & ~imask) | bcol;
            best2[f][v] = med3_i(best1[f][v], best2[f][v], key);
            best1[f][v] = max(best1[f][v], key);
          }
        }
      }
    }
  
  }
  // Row norms from the fragments, after the scan (no registers held across it):
  // each lane sums the squares of its part of row (l & 15), then the row's 4 lanes add.
  float my_norm[RF];
#pragma unroll
  for (int f = 0; f < RF; ++f) {
    float ss = 0.0f;
#pragma unroll
    for (int ks = 0; ks < Frag<E, D>::KS; ++ks) {
      if constexpr (sizeof(E) == 2) {
        // pairs of squares per instruction (exact products, float32 sums)
        const u32x4 w4 = __builtin_bit_cast(u32x4, a[f].v[ks]);
#pragma unroll
        for (int t = 0; t < 4; ++t) ss = bf16_pair_sq_acc(w4[t], ss);
      } else {
        ss = fmaf(a[f].v[ks], a[f].v[ks], ss);
      }
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    // float32 sum of squares has relative error below d * 2^-24 < 2^-12 for d <= 512.
    my_norm[f] = sqrtf(ss) * (1.0f + 0.0005f);
  }
  const float bmax = bnorm_max[0];
  // Decision of one row from its top-2 keys: the winner's float32 score is at least
  // s1; every other one is below s2 plus the truncation (at most s2 * 2^(ib - 23)),
  // or negative when the second key is; |float32 score - float64 score| <= beta
  // (matrix-core accumulation bound + float64 rounding).
  auto decided_row = [&](int k1, int k2, float nrm) {
    const double beta = (double)beta_coef * (double)nrm * (double)bmax;
    const double s1 = (double)__int_as_float(k1 & ~imask), s2 = (double)__int_as_float(k2 & ~imask);
    const double other = k2 < 0 ? 0.0 : s2 + s2 * ldexp(1.0, ib - 22);
    return k1 >= 0 && s1 - other > 2.0 * beta;
  };
#pragma unroll
  for (int f = 0; f < RF; ++f) {
    const int64_t row0 = ((int64_t)blockIdx.x * NW + w) * 16 * RF + 16 * f;
    // need_all: the fragment's undecided rows, bit b standing for row row0 + rowof(b)
    uint64_t need_all = 0;
    int shift_g = 0;   // rowof(b) = 4 (b >> 4) + (b & 15) (float32), b (bf16)
    if constexpr (sizeof(E) == 2) {
      // Merge the top-2 keys of the four lanes (l & 15) + 16 g that hold the row.
#pragma unroll
      for (int o = 16; o < 64; o <<= 1) {
        const int o1 = __shfl_xor(t1[f], o);
        const int o2 = __shfl_xor(t2[f], o);
        t2[f] = max(min(t1[f], o1), max(t2[f], o2));
        t1[f] = max(t1[f], o1);
      }
      const int64_t row = row0 + (l & 15);
      const bool decided = decided_row(t1[f], t2[f], my_norm[f]);
      if (decided && g == 0 && row < n) ids[row] = t1[f] & imask;
      need_all = ballot(!decided && row < n) & 0xFFFFull;   // bit r: row row0 + r
    } else {
      // Merge the top-2 keys of the 16 lanes that hold each row.
#pragma unroll
      for (int v = 0; v < 4; ++v) {
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const int ob1 = __shfl_xor(best1[f][v], o);
          const int ob2 = __shfl_xor(best2[f][v], o);
          best2[f][v] = max(min(best1[f][v], ob1), max(best2[f][v], ob2));
          best1[f][v] = max(best1[f][v], ob1);
        }
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 4 * g + v;                       // row of this output element within the fragment
        const float nrm = __shfl(my_norm[f], r);       // lane r holds row r's norm
        const int64_t row = row0 + r;
        const bool decided = decided_row(best1[f][v], best2[f][v], nrm);
        if (decided && (l & 15) == 0 && row < n) ids[row] = best1[f][v] & imask;
        const uint64_t und = ballot(!decided && row < n);
        need_all |= (und & 0x0001000100010001ull) << v;    // bit 16*g + v
      }
      shift_g = 1;
    }
    auto row_of = [&](int bit) -> int64_t {
      return row0 + (shift_g ? 4 * (bit >> 4) + (bit & 15) : bit);
    };
    // undecided rows: decided here by the whole wave (small inputs), or listed for
    // the float64 kernel (one atomic per wave)
    if (need_all && !und) {
      uint32_t nfb = 0;
      while (need_all) {
        const int bit = __builtin_ctzll(need_all);
        need_all &= need_all - 1;
        const int64_t row = row_of(bit);
        int bi = argmax_exact_wave<E, D>(V + row * D, Bt, n_b);
        if (bi >= n_b) bi = 0;   // only reachable with NaN scores
        if (l == 0) ids[row] = bi;
        ++nfb;
      }
      if (l == 0) atomicAdd(counters + CNT_ARGMAX_EXACT, nfb);
    }
    if (need_all) {
      uint32_t base = 0;
      if (l == 0) base = atomicAdd(und_n, (uint32_t)__popcll(need_all));
      base = __builtin_amdgcn_readfirstlane(base);
      for (int e = 0; need_all; ++e) {
        const int bit = __builtin_ctzll(need_all);
        need_all &= need_all - 1;
        if (l == 0) und[base + e] = (int32_t)row_of(bit);
      }
    }
    const int64_t rA = row0 + (l & 15);
    if (norms && l < 16 && rA < n) norms[rA] = my_norm[f];
  }
  if (norm_max_bits) {
    // the largest norm of the wave's rows (rows past n count 0), at most one atomic
    float mx = 0.0f;
#pragma unroll
    for (int f = 0; f < RF; ++f) mx = fmaxf(mx, my_norm[f]);
    mx = wave_max(mx);
    if (l == 0) raise_max_bits(norm_max_bits, mx);
  }
}

// Float64 decision of the listed rows.  A workgroup takes 64 listed rows at a
// time (16 per wave); the vectors stream once through an LDS ring shared by the
// four waves, and each score is computed on the matrix cores as in the main
// kernel (vectors x rows: lane l holds row l % 16 and vectors 4 (l / 16) + v of
// every 16-block).  Per lane the four largest keys of its share of the vectors
// are kept (score bits, vector index in the low bits).  The float64 argmax is
// among the vectors whose float32 score is at least m - 2 beta (m the row's
// float32 maximum): its float32 score is at least its float64 score less beta,
// which is at least the float64 score of the float32 winner, at least m - beta.
// When m - 2 beta > 0 those vectors score above zero, where keys order like
// scores, so each lane's band members are among its four keys unless its fourth
// key is itself inside the band; those (and rows with m - 2 beta <= 0) are redone
// by the wave over every vector in float64.  Band members are scored in float64;
// exact ties go to the lowest index, as in the oracle.
template <class E, int D>
__global__ __launch_bounds__(256) void k_argmax_near(const E* __restrict__ V, const E* __restrict__ Bt, int n_b,
                                                     const float* __restrict__ bnorm_max, float beta_coef,
                                                     const int32_t* __restrict__ und,
                                                     const uint32_t* __restrict__ und_n, int32_t* __restrict__ ids,
                                                     uint32_t* __restrict__ counters) {
  using G = TileGeom<E, D>;
  constexpr int NW = 4;
  constexpr int NCB = G::TI / 16;
  __shared__ __attribute__((aligned(1024))) char ring[3 * G::ROW_BYTES];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = lane_id(), r = l & 15, g = l >> 4;
  const int64_t nund = *und_n;
  const int nt = (n_b + G::TI - 1) / G::TI;
  const int ib = n_b > 1 ? 32 - __builtin_clz((unsigned)(n_b - 1)) : 0;
  const int imask = (1 << ib) - 1;
  const double tau = ldexp(1.0, ib - 23);   // relative truncation of a key's score
  const float bmax = bnorm_max[0];
  uint32_t done = 0;
  for (int64_t g0 = (int64_t)blockIdx.x * 64; g0 < nund; g0 += (int64_t)gridDim.x * 64) {
    const int64_t slot = g0 + 16 * w + r;
    const bool rv = slot < nund;
    const int64_t row = rv ? und[slot] : 0;
    Frag<E, D> afr;
    afr.load_global(rv ? V + row * D : nullptr);
    afr.settle();
    // the row's norm from its fragment (spread over the row's four lanes), as in
    // the matrix-core kernel
    float ss = 0.0f;
#pragma unroll
    for (int ks = 0; ks < Frag<E, D>::KS; ++ks) {
      if constexpr (sizeof(E) == 2) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float x = to_f32(afr.v[ks][t]);
          ss = fmaf(x, x, ss);
        }
      } else {
        ss = fmaf(afr.v[ks], afr.v[ks], ss);
      }
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const double beta = (double)beta_coef * (double)(sqrtf(ss) * (1.0f + 0.0005f)) * (double)bmax;

    int k1 = INT32_MIN, k2 = INT32_MIN, k3 = INT32_MIN, k4 = INT32_MIN;
    __syncthreads();   // the previous group's reads of the ring are done
    dma_rows<E, D, NW>(ring, Bt, 0, n_b, w);
    if (nt > 1) dma_rows<E, D, NW>(ring + G::ROW_BYTES, Bt, G::TI, n_b, w);
    for (int t = 0; t < nt; ++t) {
      if (t + 1 < nt)
        wait_vmcnt_c<G::ROW_DMA / NW>();
      else
        wait_vmcnt_c<0>();
      raw_barrier();
      if (t + 2 < nt)
        dma_rows<E, D, NW>(ring + (size_t)((t + 2) % 3) * G::ROW_BYTES, Bt, (int64_t)(t + 2) * G::TI, n_b, w);
      const char* rows = ring + (size_t)(t % 3) * G::ROW_BYTES;
      const bool pad = (t + 1) * G::TI > n_b;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        Frag<E, D> bf;
        TileFrag<E, D>::load(bf, rows, cb * 16 + r);
        const int b0 = t * G::TI + cb * 16 + 4 * g;   // vector of element v: b0 + v
        f32x4 c0{0.0f, 0.0f, 0.0f, 0.0f};
        if (pad) {
#pragma unroll
          for (int v = 0; v < 4; ++v) c0[v] = b0 + v < n_b ? 0.0f : NEG_INF;
        }
        const f32x4 acc = mma_block(bf, afr, c0);   // [vector 4g+v][row r]
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int key = (__float_as_int(acc[v]) & ~imask) | (b0 + v);
          k4 = med3_i(k3, k4, key);
          k3 = med3_i(k2, k3, key);
          k2 = med3_i(k1, k2, key);
          k1 = max(k1, key);
        }
      }
    }
    // the band [m - 2 beta, m] of the row, from its largest key
    int km = max(k1, __shfl_xor(k1, 16));
    km = max(km, __shfl_xor(km, 32));
    const double sm = (double)__int_as_float(km & ~imask);   // m is at least this
    const double thr = sm - 2.0 * beta;
    auto in_band = [&](int kq) {
      const double sq = (double)__int_as_float(kq & ~imask);
      return kq >= 0 && sq + fabs(sq) * tau >= thr;   // the key's score is at most sq + |sq| tau
    };
    bool redo = !(km >= 0 && thr > 0.0) || in_band(k4);
    redo = redo || __shfl_xor(redo, 16);
    redo = redo || __shfl_xor(redo, 32);
    double be = -__builtin_huge_val();
    int bi = 0x7fffffff;
    if (rv && !redo) {
      const int kk[3] = {k1, k2, k3};   // the fourth key is outside the band here
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        if (!in_band(kk[q])) continue;
        const int b = kk[q] & imask;
        const double e = exact_dot<E, D, 4>(V + row * D, Bt + (int64_t)b * D);
        if (e > be || (e == be && b < bi)) {
          be = e;
          bi = b;
        }
      }
    }
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const double oe = __shfl_xor(be, o);
      const int ob = __shfl_xor(bi, o);
      if (oe > be || (oe == be && ob < bi)) {
        be = oe;
        bi = ob;
      }
    }
    if (rv && !redo && g == 0) ids[row] = bi < n_b ? bi : 0;
    // rows the four keys cannot settle: every vector in float64, one row at a time
    uint64_t rm = ballot(rv && redo && g == 0);
    while (rm) {
      const int rr = __builtin_ctzll(rm);
      rm &= rm - 1;
      const int64_t rrow = lane_val((int)row, rr);
      int bx = argmax_exact_wave<E, D>(V + rrow * D, Bt, n_b);
      if (bx >= n_b) bx = 0;   // only reachable with NaN scores
      if (l == 0) ids[rrow] = bx;
    }
    done += (uint32_t)popc(ballot(rv && g == 0));
  }
  if (l == 0 && done) atomicAdd(counters + CNT_ARGMAX_EXACT, done);
}

template <class E, int D>
static hipError_t launch_pa(const void* V, int64_t n, const void* Bt, int n_b, const float* bmax, float beta,
                            int32_t* ids, float* norms, uint32_t* nmax, int32_t* und, uint32_t* und_n,
                            uint32_t* counters, hipStream_t st) {
  // several row fragments per wave (as many as registers allow at two waves per
  // SIMD) once the input still gives every CU several workgroups
  constexpr int RF = D * (int)sizeof(E) >= 512 ? 2 : 4;
  if (n >= (int64_t)64 * RF * 2048) {
    const unsigned blocks = (unsigned)((n + 64 * RF - 1) / (64 * RF));
    hipLaunchKernelGGL((k_project_argmax<E, D, RF>), dim3(blocks), dim3(256), 0, st, (const E*)V, n, (const E*)Bt,
                       n_b, bmax, beta, ids, norms, nmax, und, und_n, counters);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the listed rows, 16 per wave: about one row in 2048 expected, a few times
    // that many waves
    const int64_t eb = std::min<int64_t>(1024, std::max<int64_t>(16, n / 16384));
    hipLaunchKernelGGL((k_argmax_near<E, D>), dim3((unsigned)eb), dim3(256), 0, st, (const E*)V, (const E*)Bt, n_b,
                       bmax, beta, und, und_n, ids, counters);
  } else {   // small input: undecided rows are decided inside the kernel
    const unsigned blocks = (unsigned)((n + 63) / 64);
    hipLaunchKernelGGL((k_project_argmax<E, D, 1>), dim3(blocks), dim3(256), 0, st, (const E*)V, n, (const E*)Bt,
                       n_b, bmax, beta, ids, norms, nmax, (int32_t*)nullptr, (uint32_t*)nullptr, counters);
  }
  return hipGetLastError();
}

hipError_t launch_project_argmax(bool is_bf16, int d, const void* V, int64_t n, const void* Bt, int n_b,
                                 const float* bnorm_max, float beta_coef, int32_t* ids, float* norms,
                                 uint32_t* norm_max_bits, int32_t* und, uint32_t* und_n, uint32_t* counters,
                                 hipStream_t st) {
  if (n <= 0) return hipSuccess;
#define RECE_PA(E, DD)                                                                                       \
  if (d == DD)                                                                                               \
    return launch_pa<E, DD>(V, n, Bt, n_b, bnorm_max, beta_coef, ids, norms, norm_max_bits, und, und_n, counters, \
                            st);
  if (is_bf16) {
    RECE_PA(bf16, 32) RECE_PA(bf16, 64) RECE_PA(bf16, 128) RECE_PA(bf16, 256)
  } else {
    RECE_PA(float, 32) RECE_PA(float, 64) RECE_PA(float, 128) RECE_PA(float, 256)
  }
#undef RECE_PA
  return hipErrorInvalidValue;
}

}  // namespace rece
