// Exact full cross-entropy over the whole catalogue, forward and backward (RECE
// page, Section 3: Eq. 3, the loss over every item, and Eq. 4, its gradient
// softmax minus one-hot), the dense baseline that the reduced losses approximate.
// Every logit is computed on the matrix cores and consumed on chip; no [s, C]
// array exists anywhere.
//
// One kernel template, three passes, each an "owner x streamed" sweep: a wave
// keeps the matrix-core fragments of 16 owner vectors in registers and the other
// side streams through LDS in tiles (two tiles in flight), its logit block
// computed transposed (streamed x owners), so lane l holds owner l % 16 and
// streamed 4*(l/16) + v of every 16-block.
//   FCE_LSE (owners = positions, streamed = items): online log-sum-exp of each
//     position's logits, the positive's logit, the loss.
//   FCE_DX  (owners = positions, streamed = items): G = g_i (softmax - one-hot)
//     recomputed per block and multiplied into the streamed rows: dX_i.
//   FCE_DY  (owners = items, streamed = positions): the same G transposed times
//     the position rows: dY_j.  The streamed positions' log-sum-exp, upstream
//     gradient and positive id ride with each tile.
// G enters the gradient product in the layout the logit block leaves it in (the
// A operand, k = streamed vectors); the streamed rows enter transposed through
// the LDS transpose read.  bf16: G split into bf16 hi + lo (about 16 significant
// bits) for the product; f32: the float32 matrix cores.
#include <algorithm>
#include <cmath>

#include "rece_device.h"
#include "rece_internal.h"
#include "rece_stream.h"

namespace rece {

enum FceMode { FCE_LSE = 0, FCE_DX = 1, FCE_DY = 2 };
constexpr int FCE_RING = 3;
constexpr float FCE_LOG2E = 1.4426950408889634f;

// Slot: the tile's rows, then (FCE_DY) 64 positive ids, 64 log-sum-exp and 64
// upstream gradients of the tile's positions.
template <class E, int D>
__host__ __device__ constexpr size_t fce_slot_bytes() {
  return (size_t)TileGeom<E, D>::ROW_BYTES + 3 * 256;
}

typedef __attribute__((address_space(3))) short4v lds_short4;

// Four 16-bit values of coordinate 16*nb + (l % 16) for rows r0 .. r0 + 3 of a
// swizzled bf16 tile, r0 = base + 4*(l/16): one LDS transpose read.  Within each
// 16-lane group, source lane j names 4 coordinates of one row (row r0 + j/4,
// coordinates 16*nb + 4*(j%4) .. +3); the read hands lane i coordinate i of the
// group's 4 rows.
template <int D>
__device__ __forceinline__ short4v tile_tr4(const char* rows, int base, int nb) {
  using G = TileGeom<bf16, D>;
  const int l = lane_id(), j = l & 15;
  const int row = base + 4 * (l >> 4) + (j >> 2);
  const int dim0 = 16 * nb + 4 * (j & 3);
  const int ch = (dim0 >> 3) ^ (row & G::SWM);
  const char* addr = rows + row * G::RB + ch * 16 + ((dim0 >> 2) & 1) * 8;
  short4v v;
  asm volatile("ds_read_b64_tr_b16 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(addr)) : "memory");
  return v;
}

// acc[nb] += G[16 owners][TI streamed] . tile[TI streamed][D] where lane l holds
// G[owner l % 16][streamed 16*cb + 4*(l/16) + v] in gv[cb][v].  bf16: k = 32
// streamed rows per step, in the order (4 of block 2ks, 4 of block 2ks + 1) on
// both operands; f32: k = 4 rows per step.  Output: lane l holds owner
// 4*(l/16) + v, coordinate 16*nb + l % 16 in acc[nb][v].
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
        const uint32_t h0 = bf16_bits_rne(g0), h1 = bf16_bits_rne(g1);
        const uint32_t l0 = bf16_bits_rne(g0 - __uint_as_float(h0 << 16)), l1 = bf16_bits_rne(g1 - __uint_as_float(h1 << 16));
        ph[e / 2] = h0 | (h1 << 16);
        pl[e / 2] = l0 | (l1 << 16);
      }
      const bf16x8 ahi = __builtin_bit_cast(bf16x8, u32x4{ph[0], ph[1], ph[2], ph[3]});
      const bf16x8 alo = __builtin_bit_cast(bf16x8, u32x4{pl[0], pl[1], pl[2], pl[3]});
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) {
        const short4v b0 = tile_tr4<D>(rows, 32 * ks, nb);
        const short4v b1 = tile_tr4<D>(rows, 32 * ks + 16, nb);
        const short4v b8[2] = {b0, b1};
        const bf16x8 b = __builtin_bit_cast(bf16x8, b8);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b, acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, b, acc[nb], 0, 0, 0);
      }
    }
  } else {
    constexpr int NB = D / 16;
    const int g = l >> 4;
#pragma unroll
    for (int cb = 0; cb < G::TI / 16; ++cb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        // coordinate 16*nb + l % 16 of row n of the tile, one per output block
        const int n = 16 * cb + 4 * g + v;
        uint32_t ad[NB];
        float tv[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int t = 16 * u + (l & 15);
          const int c = (t >> 2) ^ (n & G::SWM);
          ad[u] = lds_addr(rows + n * G::RB + c * 16 + 4 * (t & 3));
        }
        LdsReadB32<NB>::run(ad, tv);
#pragma unroll
        for (int u = 0; u < NB; ++u) acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(gv[cb][v], tv[u], acc[u], 0, 0, 0);
      }
  }
}

struct FceArgs {
  const void* own;       // owner vectors: X (LSE, DX) or Y (DY), [n_own][d]
  const void* str;       // streamed vectors: Y (LSE, DX) or X (DY), [n_str][d]
  int64_t n_own, n_str;
  const int32_t* pos;    // [s] positive item of every position
  float* lg;             // [2][s]: log-sum-exp, then upstream gradient g_i of each position
  float* loss_pp;        // [s] (LSE, may be null)
  double* partial;       // [blocks * waves] loss sums (LSE)
  float* out;            // dX (DX) or dY (DY), [n_own][d] float32
};

// The streamed tile t (rows, then for FCE_DY the positions' id, lse, gradient).
template <class E, int D, int NW, int MODE>
__device__ __forceinline__ void fce_issue(char* ring, const FceArgs& a, int64_t t, int w) {
  using G = TileGeom<E, D>;
  const int64_t q0 = t * G::TI;
  char* slot = ring + (size_t)(t % FCE_RING) * fce_slot_bytes<E, D>();
  dma_rows<E, D, NW>(slot, reinterpret_cast<const E*>(a.str), q0, a.n_str, w);
  if constexpr (MODE == FCE_DY) {
    // three 64-int copies, by waves ROW_DMA, ROW_DMA + 1, ROW_DMA + 2 (mod NW)
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      if ((G::ROW_DMA + m) % NW != w) continue;
      const int32_t* src = m == 0 ? a.pos : reinterpret_cast<const int32_t*>(a.lg) + (int64_t)(m - 1) * a.n_str;
      dma_ints(reinterpret_cast<int32_t*>(slot + G::ROW_BYTES) + 64 * m, src, q0, a.n_str);
    }
  }
}

template <class E, int D, int NW, int MODE>
__global__ __launch_bounds__(64 * NW, 2) void k_fce(FceArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  using G = TileGeom<E, D>;
  constexpr int TI = G::TI;
  constexpr int NCB = TI / 16;
  // copies of one tile issued by the wave with the fewest
  constexpr int NCOPY = G::ROW_DMA + (MODE == FCE_DY ? 3 : 0);
  constexpr int MINC = NCOPY / NW;
  char* ring = smem;
  const int w = threadIdx.x >> 6, l = lane_id(), g = l >> 4, r = l & 15;
  const int64_t o0 = ((int64_t)blockIdx.x * NW + w) * 16;
  const int64_t oA = o0 + r;
  const bool ov = oA < a.n_own;
  const int64_t ntiles = (a.n_str + TI - 1) / TI;

  Frag<E, D> afr;
  afr.load_global(ov ? reinterpret_cast<const E*>(a.own) + oA * D : nullptr);
  afr.settle();
  // owner constants (positions: lse, gradient, positive; items: the item id)
  const int pos_r = settled(MODE != FCE_DY && ov ? a.pos[oA] : -1);
  const float lseL = settled(MODE == FCE_DX && ov ? a.lg[oA] * FCE_LOG2E : 0.0f);
  const float gb_r = settled(MODE == FCE_DX && ov ? a.lg[a.n_own + oA] : 0.0f);

  float m = NEG_INF, z = 0.0f, lp = 0.0f;   // FCE_LSE: running max, sum of exp(x - m), positive logit
  f32x4 acc[D / 16];
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t t0 = 0; t0 < FCE_RING - 1 && t0 < ntiles; ++t0) fce_issue<E, D, NW, MODE>(ring, a, t0, w);
  for (int64_t t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles)
      wait_vmcnt_c<MINC>();
    else
      wait_vmcnt_c<0>();
    raw_barrier();   // every wave's copies of tile t landed; slot (t - 1) % RING is free
    if (t + FCE_RING - 1 < ntiles) fce_issue<E, D, NW, MODE>(ring, a, t + FCE_RING - 1, w);
    const char* slot = ring + (size_t)(t % FCE_RING) * fce_slot_bytes<E, D>();
    const int64_t q0 = t * TI;
    const int nlim = (int)std::min<int64_t>(TI, a.n_str - q0);

    float gv[NCB][4];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      Frag<E, D> bf;
      TileFrag<E, D>::load(bf, slot, cb * 16 + r);
      const f32x4 lg = mma_block(bf, afr, f32x4{0.f, 0.f, 0.f, 0.f});   // [streamed 4g+v][owner r]
      if constexpr (MODE == FCE_LSE) {
        float x[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int n = cb * 16 + 4 * g + v;
          x[v] = n < nlim ? lg[v] : NEG_INF;
          if (q0 + n == pos_r) lp = lg[v];
        }
        const float mn = fmaxf(m, fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        if (mn != NEG_INF) {
          float s4 = 0.0f;
#pragma unroll
          for (int v = 0; v < 4; ++v) s4 += exp2f((x[v] - mn) * FCE_LOG2E);
          z = z * exp2f((m - mn) * FCE_LOG2E) + s4;
          m = mn;
        }
      } else if constexpr (MODE == FCE_DX) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int n = cb * 16 + 4 * g + v;
          const float p = exp2f(fmaf(lg[v], FCE_LOG2E, -lseL));
          gv[cb][v] = n < nlim && ov ? gb_r * (p - (q0 + n == pos_r ? 1.0f : 0.0f)) : 0.0f;
        }
      } else {
        const int32_t* tpos = reinterpret_cast<const int32_t*>(slot + G::ROW_BYTES);
        const float* tlse = reinterpret_cast<const float*>(slot + G::ROW_BYTES + 256);
        const float* tgb = reinterpret_cast<const float*>(slot + G::ROW_BYTES + 512);
        u32x4 ip, il, ig;
        const uint32_t ai[3] = {lds_addr(tpos + cb * 16 + 4 * g), lds_addr(tlse + cb * 16 + 4 * g),
                                lds_addr(tgb + cb * 16 + 4 * g)};
        LdsRead128<1>::run(&ai[0], &ip);
        LdsRead128<1>::run(&ai[1], &il);
        LdsRead128<1>::run(&ai[2], &ig);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int n = cb * 16 + 4 * g + v;
          const float p = exp2f(fmaf(lg[v], FCE_LOG2E, -__uint_as_float(il[v]) * FCE_LOG2E));
          gv[cb][v] = n < nlim && ov ? __uint_as_float(ig[v]) * (p - ((int64_t)(int)ip[v] == oA ? 1.0f : 0.0f)) : 0.0f;
        }
      }
    }
    if constexpr (MODE != FCE_LSE) accumulate_rows<E, D>(acc, gv, slot);
  }

  if constexpr (MODE == FCE_LSE) {
    // combine the row's four lanes
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float om = __shfl_xor(m, o), oz = __shfl_xor(z, o), ol = __shfl_xor(lp, o);
      const float mn = fmaxf(m, om);
      z = (mn == NEG_INF) ? 0.0f : z * exp2f((m - mn) * FCE_LOG2E) + oz * exp2f((om - mn) * FCE_LOG2E);
      m = mn;
      lp += ol;   // one lane of the row saw the positive
    }
    const float lse = m + logf(z);
    const float loss = lse - lp;
    if (ov && g == 0) {
      a.lg[oA] = lse;
      if (a.loss_pp) a.loss_pp[oA] = loss;
    }
    double sw = (ov && g == 0) ? (double)loss : 0.0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sw += __shfl_xor(sw, o);
    if (l == 0) a.partial[(int64_t)blockIdx.x * NW + w] = sw;
  } else {
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t ow = o0 + 4 * g + v;
        if (ow < a.n_own) a.out[ow * D + 16 * nb + r] = acc[nb][v];
      }
  }
}

// g_i: the upstream gradient of position i's loss times the mean's 1/s.
__global__ void k_fce_gbar(float* gb, int64_t s, const float* dloss, const float* dloss_pp) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < s) gb[i] = dloss_pp ? dloss_pp[i] : dloss[0] / (float)s;
}

__global__ __launch_bounds__(256) void k_fce_mean(const double* __restrict__ partial, int64_t n, int64_t s,
                                                  float* __restrict__ loss) {
  __shared__ double sh[256];
  double t = 0.0;
  for (int64_t q = threadIdx.x; q < n; q += 256) t += partial[q];
  sh[threadIdx.x] = t;
  __syncthreads();
  for (int off = 128; off >= 1; off >>= 1) {
    if ((int)threadIdx.x < off) sh[threadIdx.x] += sh[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = (float)(sh[0] / (double)s);
}

constexpr int FCE_NW = 4;

template <class E, int D, int MODE>
static hipError_t launch_fce_t(const FceArgs& a, hipStream_t st) {
  const size_t lds = FCE_RING * fce_slot_bytes<E, D>();
  auto kern = k_fce<E, D, FCE_NW, MODE>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  const int64_t blocks = (a.n_own + 16 * FCE_NW - 1) / (16 * FCE_NW);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * FCE_NW), lds, st, a);
  return hipGetLastError();
}

template <class E, int D>
static hipError_t launch_fce_d(int mode, const FceArgs& a, hipStream_t st) {
  if (mode == FCE_LSE) return launch_fce_t<E, D, FCE_LSE>(a, st);
  if (mode == FCE_DX) return launch_fce_t<E, D, FCE_DX>(a, st);
  return launch_fce_t<E, D, FCE_DY>(a, st);
}

static hipError_t launch_fce(bool bf16v, int d, int mode, const FceArgs& a, hipStream_t st) {
#define RECE_F(E, DD) \
  if (d == DD) return launch_fce_d<E, DD>(mode, a, st);
  if (bf16v) {
    RECE_F(bf16, 32) RECE_F(bf16, 64) RECE_F(bf16, 128) RECE_F(bf16, 256)
  } else {
    RECE_F(float, 32) RECE_F(float, 64) RECE_F(float, 128) RECE_F(float, 256)
  }
#undef RECE_F
  return hipErrorInvalidValue;
}

size_t full_ce_workspace_bytes(int64_t s) {
  const int64_t waves = (s + 15) / 16 + FCE_NW;
  return ((size_t)2 * s * 4 + 255) / 256 * 256 + (size_t)waves * 8;
}

hipError_t full_ce_forward(bool bf16v, int d, int64_t s, int64_t C, const void* X, const void* Y, const int32_t* pos,
                           void* ws, float* loss, float* loss_pp, hipStream_t st) {
  FceArgs a{};
  a.own = X;
  a.str = Y;
  a.n_own = s;
  a.n_str = C;
  a.pos = pos;
  a.lg = reinterpret_cast<float*>(ws);
  a.loss_pp = loss_pp;
  a.partial = reinterpret_cast<double*>(static_cast<char*>(ws) + ((size_t)2 * s * 4 + 255) / 256 * 256);
  hipError_t e = launch_fce(bf16v, d, FCE_LSE, a, st);
  if (e != hipSuccess) return e;
  const int64_t nparts = (s + 16 * FCE_NW - 1) / (16 * FCE_NW) * FCE_NW;
  hipLaunchKernelGGL(k_fce_mean, dim3(1), dim3(256), 0, st, a.partial, nparts, s, loss);
  return hipGetLastError();
}

hipError_t full_ce_backward(bool bf16v, int d, int64_t s, int64_t C, const void* X, const void* Y, const int32_t* pos,
                            void* ws, const float* dloss, const float* dloss_pp, float* dX, float* dY, hipStream_t st) {
  float* lg = reinterpret_cast<float*>(ws);
  hipLaunchKernelGGL(k_fce_gbar, dim3((unsigned)((s + 255) / 256)), dim3(256), 0, st, lg + s, s, dloss, dloss_pp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  FceArgs a{};
  a.pos = pos;
  a.lg = lg;
  a.own = X;
  a.str = Y;
  a.n_own = s;
  a.n_str = C;
  a.out = dX;
  e = launch_fce(bf16v, d, FCE_DX, a, st);
  if (e != hipSuccess) return e;
  a.own = Y;
  a.str = X;
  a.n_own = C;
  a.n_str = s;
  a.out = dY;
  return launch_fce(bf16v, d, FCE_DY, a, st);
}

}  // namespace rece
