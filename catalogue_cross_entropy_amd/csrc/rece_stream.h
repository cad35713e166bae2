// Asynchronous tile streaming for gfx950: global -> LDS copies with
// global_load_lds_dwordx4 (lane l of a wave writes 16 bytes at the LDS base
// + 16*l), issued two tiles ahead into a ring of three LDS slots.
//
// A tile holds TI consecutive rows (vectors of D coordinates) of a row-major
// array: rows of RB = D * sizeof(E) bytes, unpadded.  To keep the matrix-core
// fragment reads free of bank conflicts, 16-byte chunk c of row n is stored at
// chunk position c ^ (n & SWM); the DMA picks, per lane, the source chunk that
// belongs at its fixed LDS destination.
//
// Waiting: the waves wait for their own copies with s_waitcnt vmcnt(N) (N = the
// copies they issued after the tile they need, loads complete in order), then
// meet at a raw s_barrier.  The workgroup-scope fence of __syncthreads() would
// wait for every copy in flight, which would serialise the pipeline.
#pragma once
#include "rece_device.h"

namespace rece {

typedef __attribute__((address_space(3))) void lds_void;

template <class E, int D> struct TileGeom {
  static constexpr int RB = D * (int)sizeof(E);             // bytes per row
  // rows per tile: 8 KB row blocks where the matrix-core steps allow (bf16 needs 32 rows)
  static constexpr int TI = RB <= 128 ? 64 : (RB <= 512 ? 32 : 16);
  static constexpr int CPR = RB / 16;                        // 16-byte chunks per row
  static constexpr int SWM = (CPR < 8 ? CPR : 8) - 1;        // swizzle mask
  static constexpr int ROW_BYTES = TI * RB;                  // bytes of the row block
  static constexpr int ROW_DMA = ROW_BYTES / 1024;           // wave copies of the row block
  static_assert(ROW_BYTES % 1024 == 0, "tile rows must fill whole 1 KiB wave copies");
};

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// s_waitcnt vmcnt(n) leaving the LDS and export counters alone (GFX9 encoding).
__device__ __forceinline__ void wait_vmcnt(int n) {
#define RECE_VMCNT_CASE(N) \
  case N:                  \
    __builtin_amdgcn_s_waitcnt(((N)&15) | (7 << 4) | (15 << 8) | ((((N) >> 4) & 3) << 14)); \
    break;
  switch (n) {
    RECE_VMCNT_CASE(0) RECE_VMCNT_CASE(1) RECE_VMCNT_CASE(2) RECE_VMCNT_CASE(3)
    RECE_VMCNT_CASE(4) RECE_VMCNT_CASE(5) RECE_VMCNT_CASE(6) RECE_VMCNT_CASE(7)
    RECE_VMCNT_CASE(8) RECE_VMCNT_CASE(9) RECE_VMCNT_CASE(10) RECE_VMCNT_CASE(11)
    RECE_VMCNT_CASE(12) RECE_VMCNT_CASE(13) RECE_VMCNT_CASE(14) RECE_VMCNT_CASE(15)
    RECE_VMCNT_CASE(16) RECE_VMCNT_CASE(17) RECE_VMCNT_CASE(18) RECE_VMCNT_CASE(19)
    RECE_VMCNT_CASE(20) RECE_VMCNT_CASE(21) RECE_VMCNT_CASE(22) RECE_VMCNT_CASE(23)
    default:
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0)
      break;
  }
#undef RECE_VMCNT_CASE
}

// s_waitcnt vmcnt(N) for a compile-time N.
template <int N>
__device__ __forceinline__ void wait_vmcnt_c() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// LDS stores, atomics and transpose reads issued inside the streaming loops.
// The compiler cannot tell that their addresses lie outside the destinations of
// the asynchronous tile copies in flight, and would wait for every copy before
// each of them (draining the prefetch).  As inline assembly they carry no such
// wait: the stores and atomics have no outputs (later LDS reads of the same
// wave are ordered behind them by the in-order LDS queue), and the transpose
// reads wait for their own results inside the same asm block.  The tile data
// they read has arrived: the loops wait for its copies before the barrier.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void lds_add_u32(void* p, uint32_t v) {
  asm volatile("ds_add_u32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_store_u32(void* p, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
typedef short short4v __attribute__((ext_vector_type(4)));
// Two ds_read_b64_tr_b16 (see tile_tr4 for the lane layout), complete on return.
__device__ __forceinline__ void lds_tr16_pair(const void* a0, const void* a1, short4v& r0, short4v& r1) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %2\n\t"
      "ds_read_b64_tr_b16 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1)
      : "v"(lds_addr(a0)), "v"(lds_addr(a1))
      : "memory");
}

// Every wave: finish its LDS reads, then meet the others (no memory fence).
__device__ __forceinline__ void raw_barrier() {
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

__host__ __device__ constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// One wave copy: 16 bytes per lane from g into LDS at lds (lane l at lds + 16 l).
__device__ __forceinline__ void dma_copy16(const char* g, char* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}

// Copy rows [r0, r0 + TI) of `src` (row-major, RB bytes per row) into a swizzled
// LDS row block; rows at or beyond r_end repeat row r_end - 1 (callers mask them).
// Copy u (0 <= u < ROW_DMA) is issued by wave (u % NW); returns this wave's count.
// A full tile needs one address add per copy: the swizzle is a bit flip of the
// byte offset inside the tile.
template <class E, int D, int NW>
__device__ __forceinline__ int dma_rows(char* lds_rows, const E* __restrict__ src, int64_t r0, int64_t r_end,
                                        int wave) {
  using G = TileGeom<E, D>;
  constexpr int LRB = ilog2(G::RB);
  static_assert((1 << LRB) == G::RB, "row bytes must be a power of two");
  const int l = lane_id();
  const bool full = r0 + G::TI <= r_end;
  const char* base = reinterpret_cast<const char*>(src) + r0 * G::RB;
  int issued = 0;
#pragma unroll
  for (int q = 0; q < (G::ROW_DMA + NW - 1) / NW; ++q) {
    const int u = wave + q * NW;
    if (u >= G::ROW_DMA) break;
    const int byte = u * 1024 + 16 * l;
    const int n = byte >> LRB;
    const int off = byte ^ ((n & G::SWM) << 4);   // chunk c of row n stored at c ^ (n & SWM)
    const char* g;
    if (full) {
      g = base + off;
    } else {
      int64_t row = r0 + n;
      if (row >= r_end) row = r_end - 1;
      g = reinterpret_cast<const char*>(src) + row * G::RB + (off & (G::RB - 1));
    }
    __builtin_amdgcn_global_load_lds(g, (lds_void*)(lds_rows + u * 1024), 16, 0, 0);
    ++issued;
  }
  return issued;
}

// Copy 64 int32 values src[i0 .. i0 + 63] (clamped to i_end - 1) into LDS (one wave).
__device__ __forceinline__ void dma_ints(int32_t* lds, const int32_t* __restrict__ src, int64_t i0, int64_t i_end) {
  const int l = lane_id();
  const int32_t* g = src + i0 + l;
  if (i0 + WAVE > i_end) g = src + (i0 + l < i_end ? i0 + l : i_end - 1);
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 4, 0, 0);
}

// Copy records [r0, r0 + NREC) of an array of REC_BYTES-byte records into LDS
// (record n at lds + n * REC_BYTES).  The tile's copies are numbered; these are
// copies first .. first + copies_of - 1, issued by wave (number % nwaves).
// Records at or beyond r_end repeat record r_end - 1.  Returns this wave's count.
template <int REC_BYTES, int NREC>
struct RecCopy {
  static constexpr int CH = REC_BYTES / 16;
  static constexpr int COPIES = (NREC * CH + 63) / 64;
  static constexpr int LDS_BYTES = COPIES * 1024;
  static_assert(REC_BYTES % 16 == 0, "records must be whole 16-byte chunks");
  template <int NW>
  static __device__ __forceinline__ int issue(char* lds, const void* src, int64_t r0, int64_t r_end, int first,
                                              int wave) {
    const int l = lane_id();
    const bool full = r0 + NREC <= r_end;
    const char* base = static_cast<const char*>(src) + r0 * REC_BYTES;
    int issued = 0;
#pragma unroll
    for (int u = 0; u < COPIES; ++u) {
      if ((first + u) % NW != wave) continue;
      const int cidx = u * 64 + l;
      const char* g;
      if (full) {
        g = base + cidx * 16;
      } else {
        int64_t rr = r0 + cidx / CH;
        if (rr >= r_end) rr = r_end - 1;
        g = static_cast<const char*>(src) + rr * REC_BYTES + (cidx % CH) * 16;
      }
      __builtin_amdgcn_global_load_lds(g, (lds_void*)(lds + u * 1024), 16, 0, 0);
      ++issued;
    }
    return issued;
  }
};

// The window of chunk c: chunks c - n_ec .. c + n_ec of N sorted slots cut into
// n_c chunks (RECE page, Algorithm 1, the adjacent-chunk line, with n_ec
// neighbours on each side as in the method paragraph of Section 3).  Cyclic
// (wrap = 1): chunk indices modulo n_c, taken as a set, so 2 n_ec + 1 >= n_c gives
// all N slots.  Clipped (wrap = 0): only chunks inside [0, n_c).  Consecutive
// chunks are consecutive slots, so every window is at most two slot ranges,
// walked in tiles of TI slots: ascending (a cyclic window that passes an end of
// the order is split there), or, with rot > 0 and a window that passes no end,
// rotated: chunks lo + rot .. hi, then lo .. lo + rot - 1.  Plain scalar members
// assigned in branches: other forms (an indexed array, references to members)
// put the struct in scratch memory.
struct Ranges {
  int64_t s0, s1, e0, e1;   // slot ranges [s_q, e_q); the second may be empty
  int c1, c2;               // cumulative tile counts
  __device__ __forceinline__ void init(int c, int n_c, int64_t N, int TI, int n_ec, int wrap, int rot) {
    const int lo = c - n_ec, hi = c + n_ec;   // chunks lo .. hi (before the modulo or the clip)
    s1 = e1 = 0;
    if (wrap && 2 * n_ec + 1 >= n_c) {
      s0 = 0;
      e0 = N;
    } else if (rot > 0 && (!wrap || (lo >= 0 && hi < n_c))) {
      const int a0 = lo + rot < 0 ? 0 : lo + rot, b0 = hi > n_c - 1 ? n_c - 1 : hi;
      const int a1 = lo < 0 ? 0 : lo, b1 = lo + rot - 1 > n_c - 1 ? n_c - 1 : lo + rot - 1;
      s0 = a0 <= b0 ? chunk_start(a0, N, n_c) : 0;
      e0 = a0 <= b0 ? chunk_start(b0 + 1, N, n_c) : 0;
      s1 = a1 <= b1 ? chunk_start(a1, N, n_c) : 0;
      e1 = a1 <= b1 ? chunk_start(b1 + 1, N, n_c) : 0;
    } else if (!wrap) {
      s0 = chunk_start(lo < 0 ? 0 : lo, N, n_c);
      e0 = chunk_start(hi + 1 > n_c ? n_c : hi + 1, N, n_c);
    } else if (lo < 0) {
      s0 = chunk_start(lo + n_c, N, n_c);
      e0 = N;
      e1 = chunk_start(hi + 1, N, n_c);
    } else if (hi >= n_c) {
      s0 = chunk_start(lo, N, n_c);
      e0 = N;
      e1 = chunk_start(hi + 1 - n_c, N, n_c);
    } else {
      s0 = chunk_start(lo, N, n_c);
      e0 = chunk_start(hi + 1, N, n_c);
    }
    c1 = (int)((e0 - s0 + TI - 1) / TI);
    c2 = c1 + (int)((e1 - s1 + TI - 1) / TI);
  }
  __device__ __forceinline__ int ntiles() const { return c2; }
};

// Rotation of chunk c's window for a walking order: 0 ascending; 1 the chunk's own
// items first; 2 by chunk index modulo 2 n_ec + 1, so that at any time the
// workgroups of neighbouring chunks read the same item chunk (one HBM read serves
// the 2 n_ec + 1 windows that contain it, through the L2).
__host__ __device__ __forceinline__ int window_rotation(int order, int c, int n_ec) {
  const int m = 2 * n_ec + 1;
  if (order == 1) return n_ec;
  if (order == 2) return (int)((((int64_t)n_ec - c) % m + m) % m);
  return 0;
}

// Slot range [q0, q1_end) of tile t (tile rows are q0 .. q0 + TI - 1, clipped at q1_end).
__device__ __forceinline__ int64_t range_tile_start(Ranges r, int t, int TI) {
  return t < r.c1 ? r.s0 + (int64_t)t * TI : r.s1 + (int64_t)(t - r.c1) * TI;
}
__device__ __forceinline__ int64_t range_tile_end(Ranges r, int t) { return t < r.c1 ? r.e0 : r.e1; }

// Issue the copies of window tile t (rows from `rows_src`, then 64 ids from
// `ids_src`, then `nmaps` chunk maps of C ints from `maps_src`) into ring slot t % RING.
template <class E, int D, int NW, int RING = 3>
__device__ __forceinline__ void issue_window_tile(char* ring, size_t slot_bytes, Ranges r, int t,
                                                  const E* rows_src, const int32_t* ids_src,
                                                  const int32_t* maps_src, int64_t map_len, int nmaps, int wave) {
  using G = TileGeom<E, D>;
  const int64_t q0 = range_tile_start(r, t, G::TI), q1 = range_tile_end(r, t);
  char* slot = ring + (size_t)(t % RING) * slot_bytes;
  dma_rows<E, D, NW>(slot, rows_src, q0, q1, wave);
  const int ncopies = G::ROW_DMA + 1 + nmaps;
  for (int u = G::ROW_DMA + ((wave - G::ROW_DMA % NW + NW) % NW); u < ncopies; u += NW) {
    const int m = u - G::ROW_DMA;
    int32_t* dst = reinterpret_cast<int32_t*>(slot + G::ROW_BYTES) + 64 * m;
    if (m == 0)
      dma_ints(dst, ids_src, q0, q1);
    else
      dma_ints(dst, maps_src + (int64_t)(m - 1) * map_len, q0, q1);
  }
}

// Reads of tile data from LDS as inline assembly, waiting for their own results
// inside the block.  As plain loads the compiler cannot tell that they miss the
// destinations of the asynchronous copies in flight and waits for every copy
// before each of them, which would drain the prefetch ring at every tile.
template <int N> struct LdsRead128;
template <> struct LdsRead128<1> {
  static __device__ __forceinline__ void run(const uint32_t* a, u32x4* r) {
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r[0]) : "v"(a[0]) : "memory");
  }
};
template <> struct LdsRead128<2> {
  static __device__ __forceinline__ void run(const uint32_t* a, u32x4* r) {
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]) : "v"(a[0]), "v"(a[1]) : "memory");
  }
};
template <> struct LdsRead128<4> {
  static __device__ __forceinline__ void run(const uint32_t* a, u32x4* r) {
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
  }
};
template <> struct LdsRead128<8> {
  static __device__ __forceinline__ void run(const uint32_t* a, u32x4* r) {
    asm volatile(
        "ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\tds_read_b128 %3, %11\n\t"
        "ds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\tds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
        : "memory");
  }
};
// KS 16-byte reads from LDS at a[ks] + OFF (an immediate), one wait.
template <int KS, int OFF> struct LdsReadOff128;
template <int OFF> struct LdsReadOff128<1, OFF> {
  static __device__ __forceinline__ void run(const uint32_t* a, u32x4* r) {
    asm volatile("ds_read_b128 %0, %1 offset:%2\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r[0]) : "v"(a[0]), "i"(OFF) : "memory");
  }
};
template <int OFF> struct LdsReadOff128<2, OFF> {
  static __device__ __forceinline__ void run(const uint32_t* a, u32x4* r) {
    asm volatile("ds_read_b128 %0, %2 offset:%4\n\tds_read_b128 %1, %3 offset:%4\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]) : "v"(a[0]), "v"(a[1]), "i"(OFF) : "memory");
  }
};
template <int OFF> struct LdsReadOff128<4, OFF> {
  static __device__ __forceinline__ void run(const uint32_t* a, u32x4* r) {
    asm volatile(
        "ds_read_b128 %0, %4 offset:%8\n\tds_read_b128 %1, %5 offset:%8\n\tds_read_b128 %2, %6 offset:%8\n\t"
        "ds_read_b128 %3, %7 offset:%8\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF)
        : "memory");
  }
};
template <int OFF> struct LdsReadOff128<8, OFF> {
  static __device__ __forceinline__ void run(const uint32_t* a, u32x4* r) {
    LdsReadOff128<4, OFF>::run(a, r);
    LdsReadOff128<4, OFF>::run(a + 4, r + 4);
  }
};

// Eight dwords from LDS (addresses a[0..7]), one wait.
__device__ __forceinline__ void lds_read_b32x8(const uint32_t* a, float* r) {
  asm volatile(
      "ds_read_b32 %0, %8\n\tds_read_b32 %1, %9\n\tds_read_b32 %2, %10\n\tds_read_b32 %3, %11\n\t"
      "ds_read_b32 %4, %12\n\tds_read_b32 %5, %13\n\tds_read_b32 %6, %14\n\tds_read_b32 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

// N dwords from LDS (N = 2, 4, 8, 16), waited for inside.
template <int N> struct LdsReadB32;
template <> struct LdsReadB32<8> {
  static __device__ __forceinline__ void run(const uint32_t* a, float* r) { lds_read_b32x8(a, r); }
};
template <> struct LdsReadB32<16> {
  static __device__ __forceinline__ void run(const uint32_t* a, float* r) {
    lds_read_b32x8(a, r);
    lds_read_b32x8(a + 8, r + 8);
  }
};
template <> struct LdsReadB32<4> {
  static __device__ __forceinline__ void run(const uint32_t* a, float* r) {
    asm volatile(
        "ds_read_b32 %0, %4\n\tds_read_b32 %1, %5\n\tds_read_b32 %2, %6\n\tds_read_b32 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
  }
};
template <> struct LdsReadB32<1> {
  static __device__ __forceinline__ void run(const uint32_t* a, float* r) {
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r[0]) : "v"(a[0]) : "memory");
  }
};
template <> struct LdsReadB32<2> {
  static __device__ __forceinline__ void run(const uint32_t* a, float* r) {
    asm volatile("ds_read_b32 %0, %2\n\tds_read_b32 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1])
                 : "v"(a[0]), "v"(a[1])
                 : "memory");
  }
};

// Gather rows into a swizzled LDS row block: row n of the block is row
// ids[n] of `src` (ids in LDS, TileGeom<E, D>::TI of them); the same copy
// numbering and swizzle as dma_rows (copy u by wave u % NW).  Callers mask rows
// past the end of their range (their ids repeat the last one).
template <class E, int D, int NW>
__device__ __forceinline__ void dma_rows_gather(char* lds_rows, const E* __restrict__ src, const int32_t* lds_ids,
                                                int wave) {
  using G = TileGeom<E, D>;
  constexpr int LRB = ilog2(G::RB);
  constexpr int NQ = G::ROW_DMA / NW;   // copies of this wave
  static_assert(G::ROW_DMA % NW == 0 && NQ >= 1, "whole copies per wave");
  const int l = lane_id();
  uint32_t a[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) a[q] = lds_addr(lds_ids + (((wave + q * NW) * 1024 + 16 * l) >> LRB));
  float idf[NQ];
  LdsReadB32<NQ>::run(a, idf);
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int u = wave + q * NW;
    const int byte = u * 1024 + 16 * l;
    const int n = byte >> LRB;
    const int off = byte ^ ((n & G::SWM) << 4);   // chunk c of row n stored at c ^ (n & SWM)
    const char* g = reinterpret_cast<const char*>(src) + (int64_t)__float_as_int(idf[q]) * G::RB + (off & (G::RB - 1));
    __builtin_amdgcn_global_load_lds(g, (lds_void*)(lds_rows + u * 1024), 16, 0, 0);
  }
}

// Matrix-core fragment of tile row n (B operand, "row = vector" layout).
template <class E, int D> struct TileFrag;

template <int D> struct TileFrag<bf16, D> {
  static __device__ __forceinline__ void load(Frag<bf16, D>& f, const char* rows, int n) {
    using G = TileGeom<bf16, D>;
    constexpr int KS = D / 32;
    const int q = lane_id() >> 4;
    uint32_t a[KS];
    u32x4 raw[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = (4 * ks + q) ^ (n & G::SWM);
      a[ks] = lds_addr(rows + n * G::RB + c * 16);
    }
    LdsRead128<KS>::run(a, raw);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) f.v[ks] = __builtin_bit_cast(bf16x8, raw[ks]);
  }
};
template <int D> struct TileFrag<float, D> {
  static __device__ __forceinline__ void load(Frag<float, D>& f, const char* rows, int n) {
    using G = TileGeom<float, D>;
    constexpr int KS = D / 4;
    const int q = lane_id() >> 4;
#pragma unroll
    for (int k0 = 0; k0 < KS; k0 += 8) {
      uint32_t a[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = (k0 + u) ^ (n & G::SWM);
        a[u] = lds_addr(rows + n * G::RB + c * 16 + 4 * q);
      }
      lds_read_b32x8(a, &f.v[k0]);
    }
  }
};

// Element (row n, coordinate t) of a swizzled tile, as float.
template <class E, int D>
__device__ __forceinline__ float tile_elem(const char* rows, int n, int t) {
  using G = TileGeom<E, D>;
  constexpr int EPC = 16 / (int)sizeof(E);   // elements per chunk
  const int c = (t / EPC) ^ (n & G::SWM);
  const E* p = reinterpret_cast<const E*>(rows + n * G::RB + c * 16) + (t % EPC);
  return to_f32(*p);
}

}  // namespace rece
