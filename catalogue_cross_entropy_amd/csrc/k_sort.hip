// Stable counting sort of small integer keys (RECE page, Section 3, Algorithm 1,
// the sorting lines: positions and items reordered by bucket index; read as a
// stable ascending argsort).
//
// Three passes over the keys, no atomics on the output path:
//   1. per segment of keys (256 to SORT_SEG of them), a histogram in LDS -> counts[bin][segment];
//   2. one exclusive scan of counts in (bin, segment) order gives every
//      (bin, segment) its first output slot;
//   3. one wave per segment walks its keys in order, 64 at a time: lanes with
//      equal keys find each other with one ballot per key bit, take ranks from
//      the mask, and the group's running counter in LDS advances by the group
//      size, so equal keys keep their input order.
// When the count matrix is small (at most SMALL_COUNTS entries, at most 256
// bins), step 2 is folded into step 3: every scatter workgroup reads the whole
// matrix (L2-resident) and derives the slots of its own segments, which saves
// the three launches of the scan.
// The same kernels do the LSD passes of a wider radix sort: the key of input
// slot t is (keys[in_perm[t]] >> shift) & (2^nbits - 1).
#include "rece_device.h"
#include "rece_internal.h"

namespace rece {

constexpr int SCAN_BLOCK = 4096;   // elements per scan block (256 threads x 16)
constexpr int64_t SMALL_COUNTS = 65536;   // count matrices scanned inside the scatter kernel
constexpr int SMALL_BINS = 256;

__device__ __forceinline__ int key_at(const int32_t* __restrict__ keys, const int32_t* __restrict__ in_perm,
                                      int64_t t, int shift, uint32_t mask) {
  const int64_t e = in_perm ? in_perm[t] : t;
  return (int)(((uint32_t)keys[e] >> shift) & mask);
}

__global__ __launch_bounds__(256) void k_seg_hist(const int32_t* __restrict__ keys,
                                                  const int32_t* __restrict__ in_perm, int64_t n, int shift,
                                                  int nbits, int seg_len, int nseg, uint32_t* __restrict__ counts) {
  extern __shared__ uint32_t hist[];
  const int nbins = 1 << nbits;
  const uint32_t mask = (uint32_t)nbins - 1u;
  for (int b = threadIdx.x; b < nbins; b += 256) hist[b] = 0u;
  __syncthreads();
  const int64_t seg = blockIdx.x;
  const int64_t t0 = seg * seg_len;
  const int64_t t1 = min(n, t0 + seg_len);
  for (int64_t t = t0 + threadIdx.x; t < t1; t += 256) atomicAdd(&hist[key_at(keys, in_perm, t, shift, mask)], 1u);
  __syncthreads();
  for (int b = threadIdx.x; b < nbins; b += 256) counts[(int64_t)b * nseg + seg] = hist[b];
}

// --- exclusive scan of a uint32 array (in place) ----------------------------

__device__ __forceinline__ uint32_t block_exclusive_scan_256(uint32_t v, uint32_t* sh, uint32_t* total) {
  // inclusive wave scan
  const int l = lane_id(), w = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (l >= o) x += y;
  }
  if (l == 63) sh[w] = x;
  __syncthreads();
  uint32_t wpre = 0, tot = 0;
  for (int i = 0; i < 4; ++i) {
    if (i < w) wpre += sh[i];
    tot += sh[i];
  }
  __syncthreads();
  *total = tot;
  return wpre + x - v;
}

__global__ __launch_bounds__(256) void k_scan_reduce(const uint32_t* __restrict__ a, int64_t n,
                                                     uint32_t* __restrict__ bsum) {
  __shared__ uint32_t sh[4];
  const int64_t base = (int64_t)blockIdx.x * SCAN_BLOCK + threadIdx.x * 16;
  uint32_t s = 0;
  for (int i = 0; i < 16; ++i)
    if (base + i < n) s += a[base + i];
  uint32_t tot;
  block_exclusive_scan_256(s, sh, &tot);
  if (threadIdx.x == 0) bsum[blockIdx.x] = tot;
}

__global__ __launch_bounds__(256) void k_scan_top(uint32_t* __restrict__ bsum, int64_t nb) {
  __shared__ uint32_t sh[4];
  uint32_t carry = 0;
  for (int64_t b0 = 0; b0 < nb; b0 += 256) {
    const int64_t i = b0 + threadIdx.x;
    const uint32_t v = i < nb ? bsum[i] : 0u;
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan_256(v, sh, &tot);
    if (i < nb) bsum[i] = carry + ex;
    carry += tot;
  }
}

__global__ __launch_bounds__(256) void k_scan_apply(uint32_t* __restrict__ a, int64_t n,
                                                    const uint32_t* __restrict__ bsum) {
  __shared__ uint32_t sh[4];
  const int64_t base = (int64_t)blockIdx.x * SCAN_BLOCK + threadIdx.x * 16;
  uint32_t v[16];
  uint32_t s = 0;
  for (int i = 0; i < 16; ++i) {
    v[i] = base + i < n ? a[base + i] : 0u;
    s += v[i];
  }
  uint32_t tot;
  uint32_t run = block_exclusive_scan_256(s, sh, &tot) + bsum[blockIdx.x];
  for (int i = 0; i < 16; ++i) {
    if (base + i < n) a[base + i] = run;
    run += v[i];
  }
}

static hipError_t exclusive_scan(uint32_t* a, int64_t n, uint32_t* bsum, hipStream_t st) {
  const int64_t nb = (n + SCAN_BLOCK - 1) / SCAN_BLOCK;
  hipLaunchKernelGGL(k_scan_reduce, dim3((unsigned)nb), dim3(256), 0, st, a, n, bsum);
  hipLaunchKernelGGL(k_scan_top, dim3(1), dim3(256), 0, st, bsum, nb);
  hipLaunchKernelGGL(k_scan_apply, dim3((unsigned)nb), dim3(256), 0, st, a, n, bsum);
  return hipGetLastError();
}

hipError_t launch_exclusive_scan(uint32_t* a, int64_t n, uint32_t* bsum, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  return exclusive_scan(a, n, bsum, st);
}

// --- stable scatter: one wave per segment -------------------------------------

__global__ __launch_bounds__(256) void k_seg_scatter(const int32_t* __restrict__ keys,
                                                     const int32_t* __restrict__ in_perm, int64_t n, int shift,
                                                     int nbits, int seg_len, int nseg, const uint32_t* __restrict__ offs,
                                                     int32_t* __restrict__ perm_out, int32_t* __restrict__ inv_out) {
  extern __shared__ uint32_t ctr_all[];
  const int nbins = 1 << nbits;
  const uint32_t mask = (uint32_t)nbins - 1u;
  const int w = threadIdx.x >> 6, l = lane_id();
  const int64_t seg = (int64_t)blockIdx.x * 4 + w;
  if (seg >= nseg) return;   // whole wave leaves; no block barrier below
  uint32_t* ctr = ctr_all + (int64_t)w * nbins;
  for (int b = l; b < nbins; b += WAVE) ctr[b] = offs[(int64_t)b * nseg + seg];
  wave_sync();
  const int64_t t0 = seg * seg_len;
  const int64_t t1 = min(n, t0 + seg_len);
  for (int64_t tb = t0; tb < t1; tb += WAVE) {
    const int64_t t = tb + l;
    const bool valid = t < t1;
    int key = 0;
    int64_t e = 0;
    if (valid) {
      e = in_perm ? in_perm[t] : t;
      key = (int)(((uint32_t)keys[e] >> shift) & mask);
    }
    // lanes holding the same key: one ballot per key bit
    uint64_t same = ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (key >> bit) & 1;
      const uint64_t bm = ballot(on);
      same &= on ? bm : ~bm;
    }
    const int rank = popc(same & lanemask_lt());
    const int cnt = popc(same);
    uint32_t base = 0;
    if (valid) base = ctr[key];
    wave_sync();
    if (valid && rank == 0) ctr[key] = base + (uint32_t)cnt;
    wave_sync();
    if (valid) {
      const uint32_t slot = base + (uint32_t)rank;
      perm_out[slot] = (int32_t)e;
      if (inv_out) inv_out[e] = (int32_t)slot;
    }
  }
}

// Scatter with the scan folded in (small count matrices): the workgroup's four
// segments get their first slots from the raw counts.  Thread b < nbins sums
// bin b over all segments (its total) and over the segments before each of the
// four; an exclusive scan of the totals over bins gives the bin bases.
__global__ __launch_bounds__(256) void k_seg_scatter_small(const int32_t* __restrict__ keys,
                                                           const int32_t* __restrict__ in_perm, int64_t n,
                                                           int shift, int nbits, int seg_len, int nseg,
                                                           const uint32_t* __restrict__ counts,
                                                           int32_t* __restrict__ perm_out,
                                                           int32_t* __restrict__ inv_out) {
  __shared__ uint32_t ctr_all[4 * SMALL_BINS];
  __shared__ uint32_t sh[4];
  __shared__ uint32_t red[5 * 256];   // per (part, bin): total, then the four prefixes
  const int nbins = 1 << nbits;
  const uint32_t mask = (uint32_t)nbins - 1u;
  const int w = threadIdx.x >> 6, l = lane_id();
  const int64_t seg0 = (int64_t)blockIdx.x * 4;
  {
    // thread t sums bin t % nbins over its share of the segments (256 / nbins shares)
    const int parts = 256 >> nbits;
    const int b = threadIdx.x & (nbins - 1), part = threadIdx.x >> nbits;
    const int per = (nseg + parts - 1) / parts;
    const int q0 = part * per, q1 = min(nseg, q0 + per);
    uint32_t pre[4] = {0u, 0u, 0u, 0u};
    uint32_t tot = 0;
    const uint32_t* row = counts + (int64_t)b * nseg;
    int q = q0;
    for (; q + 4 <= q1; q += 4) {
      const uint32_t c0 = row[q], c1 = row[q + 1], c2 = row[q + 2], c3 = row[q + 3];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t sg = seg0 + u;
        pre[u] += (q < sg ? c0 : 0u) + (q + 1 < sg ? c1 : 0u) + (q + 2 < sg ? c2 : 0u) + (q + 3 < sg ? c3 : 0u);
      }
      tot += c0 + c1 + c2 + c3;
    }
    for (; q < q1; ++q) {
      const uint32_t c = row[q];
#pragma unroll
      for (int u = 0; u < 4; ++u) pre[u] += q < seg0 + u ? c : 0u;
      tot += c;
    }
    red[threadIdx.x] = tot;
#pragma unroll
    for (int u = 0; u < 4; ++u) red[(1 + u) * 256 + threadIdx.x] = pre[u];
    __syncthreads();
    // shares combined in order (exact integer sums), then the bin bases
    uint32_t btot = 0, bpre[4] = {0u, 0u, 0u, 0u};
    if (threadIdx.x < nbins)
      for (int pt = 0; pt < parts; ++pt) {
        const int t = pt * nbins + threadIdx.x;
        btot += red[t];
#pragma unroll
        for (int u = 0; u < 4; ++u) bpre[u] += red[(1 + u) * 256 + t];
      }
    uint32_t total;
    const uint32_t base = block_exclusive_scan_256(threadIdx.x < nbins ? btot : 0u, sh, &total);
    if (threadIdx.x < nbins)
#pragma unroll
      for (int u = 0; u < 4; ++u) ctr_all[u * SMALL_BINS + threadIdx.x] = base + bpre[u];
  }
  __syncthreads();
  const int64_t seg = seg0 + w;
  if (seg >= nseg) return;   // whole wave leaves; no block barrier below
  uint32_t* ctr = ctr_all + w * SMALL_BINS;
  const int64_t t0 = seg * seg_len;
  const int64_t t1 = min(n, t0 + seg_len);
  for (int64_t tb = t0; tb < t1; tb += WAVE) {
    const int64_t t = tb + l;
    const bool valid = t < t1;
    int key = 0;
    int64_t e = 0;
    if (valid) {
      e = in_perm ? in_perm[t] : t;
      key = (int)(((uint32_t)keys[e] >> shift) & mask);
    }
    uint64_t same = ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (key >> bit) & 1;
      const uint64_t bm = ballot(on);
      same &= on ? bm : ~bm;
    }
    const int rank = popc(same & lanemask_lt());
    const int cnt = popc(same);
    uint32_t base = 0;
    if (valid) base = ctr[key];
    wave_sync();
    if (valid && rank == 0) ctr[key] = base + (uint32_t)cnt;
    wave_sync();
    if (valid) {
      const uint32_t slot = base + (uint32_t)rank;
      perm_out[slot] = (int32_t)e;
      if (inv_out) inv_out[e] = (int32_t)slot;
    }
  }
}

// Keys per segment: about 256 segments for small inputs (enough waves for the
// scatter), at most SORT_SEG keys each for large ones (bounded histogram matrix).
static int64_t seg_len_for(int64_t n) {
  int64_t L = ((n / 256) + 63) / 64 * 64;
  return L < 256 ? 256 : (L > SORT_SEG ? SORT_SEG : L);
}
static int64_t num_segments(int64_t n) {
  const int64_t L = seg_len_for(n);
  return (n + L - 1) / L;
}

// Digit width of an LSD pass over n keys: 8 bits when the count matrix then
// stays small enough for the folded scan, else 12.
int sort_digit_bits(int64_t n) { return num_segments(n) * SMALL_BINS <= SMALL_COUNTS ? 8 : 12; }

size_t sort_scratch_bytes(int64_t n, int nbins) {
  const int64_t cnt = num_segments(n) * (int64_t)nbins;
  const int64_t nb = (cnt + SCAN_BLOCK - 1) / SCAN_BLOCK;
  return (size_t)(cnt + nb + 64) * sizeof(uint32_t);
}

hipError_t launch_counting_sort(const int32_t* keys, const int32_t* in_perm, int64_t n, int shift, int nbits,
                                void* scratch, int32_t* perm_out, int32_t* inv_out, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int nbins = 1 << nbits;
  const int64_t nseg = num_segments(n);
  uint32_t* counts = reinterpret_cast<uint32_t*>(scratch);
  uint32_t* bsum = counts + nseg * nbins;
  const int seg_len = (int)seg_len_for(n);
  hipLaunchKernelGGL(k_seg_hist, dim3((unsigned)nseg), dim3(256), nbins * sizeof(uint32_t), st, keys, in_perm, n,
                     shift, nbits, seg_len, (int)nseg, counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nbins <= SMALL_BINS && nseg * nbins <= SMALL_COUNTS) {
    hipLaunchKernelGGL(k_seg_scatter_small, dim3((unsigned)((nseg + 3) / 4)), dim3(256), 0, st, keys, in_perm, n,
                       shift, nbits, seg_len, (int)nseg, counts, perm_out, inv_out);
    return hipGetLastError();
  }
  e = exclusive_scan(counts, nseg * nbins, bsum, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_seg_scatter, dim3((unsigned)((nseg + 3) / 4)), dim3(256), 4 * nbins * sizeof(uint32_t), st,
                     keys, in_perm, n, shift, nbits, seg_len, (int)nseg, counts, perm_out, inv_out);
  return hipGetLastError();
}

}  // namespace rece
