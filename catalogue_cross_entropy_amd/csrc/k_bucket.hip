// Bucketing: the argmax over n_b random vectors of the signed scalar product
// b.v, for every position and every item (RECE page, Section 3, Algorithm 1,
// the two argmax lines; "index of the nearest vector from B in terms of dot
// product").  Ties go to the lowest index.
//
// The scores are computed on the matrix cores in float32 (bf16 or f32 inputs)
// and never stored.  The decision is the argmax of the float64 coordinate-order
// sums: a row whose float32 top-2 gap exceeds twice the error bound is decided
// by the float32 argmax; otherwise the wave recomputes all n_b scores of that
// row in float64 (rare).
#include "rece_device.h"
#include "rece_internal.h"

namespace rece {

__global__ void k_fill_u32(uint32_t* p, uint32_t v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, v, n);
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
  for (int t = 0; t < d; ++t) {
    const E v = src[(int64_t)t * n_b + b];
    dst[t] = v;
    const double f = (double)to_f32(v);
    ss = fma(f, f, ss);
  }
  const float nrm = f_up(sqrt(ss) * (1.0 + 1e-12));
  atomicMax(bnorm_max_bits + rho, __float_as_uint(nrm));
}

hipError_t launch_prep_b(bool is_bf16, int d, const void* B, int rounds, int n_b, void* Bt, float* bnorm_max,
                         hipStream_t st) {
  hipError_t e = launch_fill_u32(reinterpret_cast<uint32_t*>(bnorm_max), 0u, rounds, st);
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

// One workgroup = 4 waves x 16 rows.  The random vectors stream through LDS in
// tiles of 64; each wave keeps its rows' fragments in registers.
template <class E, int D>
__global__ __launch_bounds__(256) void k_project_argmax(
    const E* __restrict__ V, int64_t n, const E* __restrict__ Bt, int n_b,
    const float* __restrict__ bnorm_max, float beta_coef, int32_t* __restrict__ ids,
    float* __restrict__ norms, uint32_t* __restrict__ norm_max_bits, uint32_t* __restrict__ counters) {
  constexpr int P = Pitch<E, D>::value;
  __shared__ __attribute__((aligned(16))) E tile[64 * P];
  const int w = threadIdx.x >> 6;
  const int l = lane_id();
  const int g = l >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * 64 + w * 16;
  const int64_t rA = row0 + (l & 15);

  Frag<E, D> a;
  a.load_global(rA < n ? V + rA * D : nullptr);

  // Squared norm of row (l & 15): each lane sums its fragment, then the 4 lanes of the row.
  float ss = 0.0f;
  {
    const E* rp = rA < n ? V + rA * D : nullptr;
    if (rp) {
      const int q = g;
      if constexpr (sizeof(E) == 2) {
        for (int ks = 0; ks < D / 32; ++ks)
          for (int t = 0; t < 8; ++t) {
            const float f = to_f32(rp[32 * ks + 8 * q + t]);
            ss = fmaf(f, f, ss);
          }
      } else {
        for (int ks = 0; ks < D / 4; ++ks) {
          const float f = to_f32(rp[4 * ks + q]);
          ss = fmaf(f, f, ss);
        }
      }
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
  }
  // float32 sum of squares has relative error below d * 2^-24 < 2^-12 for d <= 512.
  const float my_norm = sqrtf(ss) * (1.0f + 0.0005f);

  float best1[4], best2[4];
  int idx1[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    best1[v] = NEG_INF;
    best2[v] = NEG_INF;
    idx1[v] = 0;
  }

  for (int b0 = 0; b0 < n_b; b0 += 64) {
    __syncthreads();
    // stage 64 random vectors (rows of Bt) in LDS, 16 bytes per thread per step
    constexpr int PIECES = D * (int)sizeof(E) / 16;   // 16-byte pieces per vector
    for (int pc = threadIdx.x; pc < 64 * PIECES; pc += 256) {
      const int nb = pc / PIECES, part = pc % PIECES;
      constexpr int EPP = 16 / (int)sizeof(E);
      u32x4 val = {0u, 0u, 0u, 0u};
      if (b0 + nb < n_b) val = *reinterpret_cast<const u32x4*>(Bt + (int64_t)(b0 + nb) * D + part * EPP);
      *reinterpret_cast<u32x4*>(tile + nb * P + part * EPP) = val;
    }
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      if (b0 + cb * 16 >= n_b) break;
      Frag<E, D> bf;
      bf.load_lds(tile + (cb * 16 + (l & 15)) * P);
      const f32x4 acc = mma_block(a, bf, f32x4{0.f, 0.f, 0.f, 0.f});
      const int bcol = b0 + cb * 16 + (l & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float sc = bcol < n_b ? acc[v] : NEG_INF;
        if (sc > best1[v]) {
          best2[v] = best1[v];
          best1[v] = sc;
          idx1[v] = bcol;
        } else if (sc > best2[v]) {
          best2[v] = sc;
        }
      }
    }
  }

  // Merge the top-2 summaries of the 16 lanes that hold each row.
#pragma unroll
  for (int v = 0; v < 4; ++v) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const float ob1 = __shfl_xor(best1[v], o);
      const float ob2 = __shfl_xor(best2[v], o);
      const int oi = __shfl_xor(idx1[v], o);
      const float lo1 = fminf(best1[v], ob1);
      const bool take = ob1 > best1[v] || (ob1 == best1[v] && oi < idx1[v]);
      best2[v] = fmaxf(lo1, fmaxf(best2[v], ob2));
      if (take) {
        best1[v] = ob1;
        idx1[v] = oi;
      }
    }
  }

  const float bmax = bnorm_max[0];
  uint64_t need_all = 0;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r = 4 * g + v;                       // row of this output element within the wave
    const float nrm = __shfl(my_norm, r);          // lane r holds row r's norm
    const int64_t row = row0 + r;
    // |float32 score - float64 score| <= beta (matrix-core accumulation bound + float64 rounding)
    const double beta = (double)beta_coef * (double)nrm * (double)bmax;
    const bool decided = (double)best1[v] - (double)best2[v] > 2.0 * beta;
    if (decided && (l & 15) == 0 && row < n) ids[row] = idx1[v];
    const uint64_t und = ballot(!decided && row < n);
    need_all |= (und & 0x0001000100010001ull) << v;    // bit 16*g + v
  }
  // Float64 fallback: the whole wave recomputes every score of an undecided row.
  while (need_all) {
    const int bit = __builtin_ctzll(need_all);
    need_all &= need_all - 1;
    const int r = 4 * (bit >> 4) + (bit & 15);
    const int64_t row = row0 + r;
    const E* x = V + row * D;
    double be = -__builtin_huge_val();
    int bi = 0x7fffffff;
    for (int b = l; b < n_b; b += WAVE) {
      const double e = exact_dot<E, D>(x, Bt + (int64_t)b * D);
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
    if (bi >= n_b) bi = 0;   // only reachable with NaN scores
    if (l == 0) {
      ids[row] = bi;
      atomicAdd(counters + CNT_ARGMAX_EXACT, 1u);
    }
  }

  if (l < 16 && rA < n) {
    if (norms) norms[rA] = my_norm;
    if (norm_max_bits) atomicMax(norm_max_bits, __float_as_uint(my_norm));
  }
}

template <class E, int D>
static hipError_t launch_pa(const void* V, int64_t n, const void* Bt, int n_b, const float* bmax, float beta,
                            int32_t* ids, float* norms, uint32_t* nmax, uint32_t* counters, hipStream_t st) {
  const unsigned blocks = (unsigned)((n + 63) / 64);
  hipLaunchKernelGGL((k_project_argmax<E, D>), dim3(blocks), dim3(256), 0, st, (const E*)V, n, (const E*)Bt,
                     n_b, bmax, beta, ids, norms, nmax, counters);
  return hipGetLastError();
}

hipError_t launch_project_argmax(bool is_bf16, int d, const void* V, int64_t n, const void* Bt, int n_b,
                                 const float* bnorm_max, float beta_coef, int32_t* ids, float* norms,
                                 uint32_t* norm_max_bits, uint32_t* counters, hipStream_t st) {
  if (n <= 0) return hipSuccess;
#define RECE_PA(E, DD) \
  if (d == DD) return launch_pa<E, DD>(V, n, Bt, n_b, bnorm_max, beta_coef, ids, norms, norm_max_bits, counters, st);
  if (is_bf16) {
    RECE_PA(bf16, 32) RECE_PA(bf16, 64) RECE_PA(bf16, 128) RECE_PA(bf16, 256)
  } else {
    RECE_PA(float, 32) RECE_PA(float, 64) RECE_PA(float, 128) RECE_PA(float, 256)
  }
#undef RECE_PA
  return hipErrorInvalidValue;
}

}  // namespace rece
