// Device helpers shared by the librece kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rece {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Storage tag of a bfloat16 input element (raw bits).
struct bf16 {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return __uint_as_float((uint32_t)v.bits << 16); }

constexpr int WAVE = 64;
constexpr float NEG_INF = -__builtin_huge_valf();

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }
__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}
__device__ __forceinline__ int popc(uint64_t m) { return __popcll(m); }

// Orders LDS traffic between lanes of one wave (no hardware barrier needed:
// a wave executes its LDS instructions in order; this stops compiler motion).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
// Raise the device word *bits (a non-negative float's bit pattern, which orders
// like the float) to v.  The atomic is skipped when the stored value already
// covers v: the stored value only grows, so a stale read can cost an extra atomic
// but never loses one.  Thousands of waves raising one word otherwise queue on
// that address (same-address atomics run one at a time).
__device__ __forceinline__ void raise_max_bits(uint32_t* bits, float v) {
  const uint32_t b = __float_as_uint(v);
  if (__hip_atomic_load(bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < b) atomicMax(bits, b);
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  return v;
}
// Hand a value loaded from memory on as a plain register value (the compiler
// waits for the load here, once, instead of at every use inside a later loop,
// where the wait would also cover every asynchronous copy in flight).
template <class T>
__device__ __forceinline__ T settled(T v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// Value of `v` in lane `lane`, which must be the same in every active lane (a
// scalar read of the register, no LDS round trip as with __shfl).
__device__ __forceinline__ int lane_val(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ uint32_t lane_val(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}
__device__ __forceinline__ float lane_val(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ double lane_val(double v, int lane) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive prefix sum over the 64 lanes (lane l gets the sum of lanes 0..l), in
// registers with data-parallel-primitive moves: shifts within each 16-lane row,
// then the last lane of row 0 (and of row 2) added to row 1 (row 3), then lane 31
// added to rows 2 and 3.  Every lane must be active.
__device__ __forceinline__ uint32_t wave_prefix_incl(uint32_t v) {
  int p = (int)v;
  p += __builtin_amdgcn_update_dpp(0, p, 0x111, 0xF, 0xF, true);   // row_shr:1
  p += __builtin_amdgcn_update_dpp(0, p, 0x112, 0xF, 0xF, true);   // row_shr:2
  p += __builtin_amdgcn_update_dpp(0, p, 0x114, 0xF, 0xF, true);   // row_shr:4
  p += __builtin_amdgcn_update_dpp(0, p, 0x118, 0xF, 0xF, true);   // row_shr:8
  p += __builtin_amdgcn_update_dpp(0, p, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  p += __builtin_amdgcn_update_dpp(0, p, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return (uint32_t)p;
}

// Sum over the 64 lanes in a fixed order (the prefix pattern above, in float),
// returned in every lane.  Every lane must be active.
template <int CTRL, int ROWS, bool BC>
__device__ __forceinline__ float dpp_movf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, BC));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_movf<0x111, 0xF, true>(v);
  v += dpp_movf<0x112, 0xF, true>(v);
  v += dpp_movf<0x114, 0xF, true>(v);
  v += dpp_movf<0x118, 0xF, true>(v);
  v += dpp_movf<0x142, 0xA, false>(v);
  v += dpp_movf<0x143, 0xC, false>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_sumf(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Order-preserving map float -> uint32 (larger float -> larger key; -0 < +0).
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Float64 scalar product summed in coordinate order t = 0..D-1.  Products of
// float32 / bfloat16 values are exact in float64, so fma(a, b, acc) equals
// acc + a*b rounded once: this is the reference value every selection uses.
// Both rows are read in 16-byte pieces, a batch of pieces in flight at a time;
// only the additions are ordered.  The pointers pass through an empty asm
// statement: in a loop over rows the compiler would otherwise keep a
// loop-invariant row converted to float64 in 2*D registers (or scratch).
template <class E, int D, int MAXB = 8>
__device__ __forceinline__ double exact_dot(const E* __restrict__ a, const E* __restrict__ b) {
  constexpr int EPP = 16 / (int)sizeof(E);     // elements per piece
  constexpr int NP = D / EPP;                  // pieces per row
  constexpr int BATCH = NP < MAXB ? NP : MAXB;   // pieces in flight (registers: 8 per piece)
  asm volatile("" : "+v"(a), "+v"(b));
  const u32x4* pa = reinterpret_cast<const u32x4*>(a);
  const u32x4* pb = reinterpret_cast<const u32x4*>(b);
  double acc = 0.0;
#pragma unroll
  for (int p0 = 0; p0 < NP; p0 += BATCH) {
    u32x4 ra[BATCH], rb[BATCH];
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      ra[q] = pa[p0 + q];
      rb[q] = pb[p0 + q];
    }
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      const E* ea = reinterpret_cast<const E*>(&ra[q]);
      const E* eb = reinterpret_cast<const E*>(&rb[q]);
#pragma unroll
      for (int t = 0; t < EPP; ++t) acc = fma((double)to_f32(ea[t]), (double)to_f32(eb[t]), acc);
    }
  }
  return acc;
}

// The dispatcher deals workgroups to the 8 XCDs (each with its own L2) in turn:
// block b runs on XCD b % 8.  Renumber so that every XCD gets one contiguous run
// of logical blocks; neighbouring blocks (which read the same chunk window) then
// share an L2.  A bijection of [0, nblocks) whatever the real placement.
__device__ __forceinline__ int xcd_block(int b, int nblocks) {
  constexpr int NX = 8;
  const int per = nblocks / NX, rem = nblocks % NX;
  const int x = b % NX;
  return x * per + (x < rem ? x : rem) + b / NX;
}

// acc + lo^2 + hi^2 for the two bf16 values packed in w (one v_dot2 instruction).
__device__ __forceinline__ float bf16_pair_sq_acc(uint32_t w, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 x2 = __builtin_bit_cast(bf16x2, w);
  return __builtin_amdgcn_fdot2_f32_bf16(x2, x2, acc, false);
}

// Outward rounding of a float64 interval end to float32.
// bf16 bit pattern of x, rounded to nearest even.
__device__ __forceinline__ uint32_t bf16_bits_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float f_down(double v) { return __double2float_rd(v); }
__device__ __forceinline__ float f_up(double v) { return __double2float_ru(v); }

// ---------------------------------------------------------------------------
// Matrix-core fragments.  A 16x16 output block C[m][n] = sum_t A[m][t] * B[n][t]
// over D coordinates.  Lane l supplies row m = l % 16 of A and row n = l % 16 of
// B (both "row = vector" layout); the block result lands as
// C[4*(l/16) + v][l % 16] in element v of the lane's f32x4.
//   bf16: v_mfma_f32_16x16x32_bf16, k-step of 32 coordinates, lane holds the 8
//         coordinates 32*ks + 8*(l/16) .. +7 of its row (same map for A and B, so
//         the pairing of coordinates is right whatever the unit's internal order);
//   f32:  v_mfma_f32_16x16x4_f32, k-step of 4, lane holds coordinate 4*ks + l/16.
// ---------------------------------------------------------------------------
template <class E, int D> struct Frag;

template <int D> struct Frag<bf16, D> {
  static constexpr int KS = D / 32;
  bf16x8 v[KS];
  // After a global load: wait for it here, once, and hand the registers on as
  // plain values.  A loop that uses the fragment then carries no pending load,
  // which the compiler would otherwise wait for (with every copy in flight) at
  // each use.
  __device__ __forceinline__ void settle() {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(v[ks]));
  }
  // Load the fragment of one row (row pointer; nullptr -> zeros).
  __device__ __forceinline__ void load_global(const bf16* row) {
    const int q = lane_id() >> 4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (row) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(row + 32 * ks + 8 * q);
        v[ks] = __builtin_bit_cast(bf16x8, raw);
      } else {
        v[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      }
    }
  }
  __device__ __forceinline__ void load_lds(const bf16* row) {
    const int q = lane_id() >> 4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(row + 32 * ks + 8 * q);
      v[ks] = __builtin_bit_cast(bf16x8, raw);
    }
  }
};

template <int D> struct Frag<float, D> {
  static constexpr int KS = D / 4;
  float v[KS];
  __device__ __forceinline__ void settle() {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(v[ks]));
  }
  __device__ __forceinline__ void load_global(const float* row) {
    const int q = lane_id() >> 4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) v[ks] = row ? row[4 * ks + q] : 0.0f;
  }
  __device__ __forceinline__ void load_lds(const float* row) {
    const int q = lane_id() >> 4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) v[ks] = row[4 * ks + q];
  }
};

template <int D>
__device__ __forceinline__ f32x4 mma_block(const Frag<bf16, D>& a, const Frag<bf16, D>& b, f32x4 acc) {
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v[ks], b.v[ks], acc, 0, 0, 0);
  return acc;
}
template <int D>
__device__ __forceinline__ f32x4 mma_block(const Frag<float, D>& a, const Frag<float, D>& b, f32x4 acc) {
#pragma unroll
  for (int ks = 0; ks < D / 4; ++ks)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[ks], b.v[ks], acc, 0, 0, 0);
  return acc;
}

// Row pitch (elements) of an LDS tile holding vectors of D coordinates.
template <class E, int D> struct Pitch;
template <int D> struct Pitch<bf16, D> { static constexpr int value = D + 8; };
template <int D> struct Pitch<float, D> { static constexpr int value = D + 4; };

// Chunk of sorted slot p among N slots cut into n_c chunks: floor(p * n_c / N).
__device__ __forceinline__ int chunk_of(int64_t p, int64_t N, int n_c) {
  return (int)((p * (int64_t)n_c) / N);
}
// First slot of chunk c: ceil(c * N / n_c).
__host__ __device__ __forceinline__ int64_t chunk_start(int64_t c, int64_t N, int n_c) {
  return (c * N + n_c - 1) / n_c;
}

// Add a per-lane tally to a device counter: one atomic per wave.
__device__ __forceinline__ void flush_count(uint32_t* counter, uint32_t v) {
  const int t = wave_sum((int)v);
  if (lane_id() == 0 && t != 0) atomicAdd(counter, (uint32_t)t);
}

}  // namespace rece
