// Internal interface between the librece host code and its kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/rece.h"
#include "rece_device.h"

namespace rece {

// Device counters (uint32), kept in the saved buffer.
enum Counter {
  CNT_ERROR = 0,          // bit flags, ERRBIT_*
  CNT_ARGMAX_EXACT = 1,   // rows whose bucket was decided in float64
  CNT_TOPK_EXACT = 2,     // rows whose k-th element needed more than one float64 value
  CNT_LOGIT_EXACT = 3,    // logits recomputed in float64 (selection and dedup tests)
  CNT_OVERFLOW = 4,       // selection buffers that could not be compacted
  CNT_SEL_REDO = 5,       // rows whose candidate list went to the exact pass (ties by the hundred)
  CNT_LISTED = 6,         // candidate entries appended to the selection lists
  CNT_COL_REFINE = 7,     // bucket columns whose selection took a finer histogram level
  NUM_COUNTERS = 8
};
enum ErrBit : uint32_t { ERRBIT_BAD_ID = 1u, ERRBIT_OVERFLOW = 2u };

constexpr int MAX_ROUNDS = 8;
constexpr int SORT_SEG = 4096;      // keys per counting-sort segment (one wave each)
constexpr int ALIST = 64;           // near-tie list capacity at the k-th boundary

struct SelectArgs {
  const void* X;
  const void* Y;
  const int32_t* pos;
  const int32_t* perm_x;      // round rho
  const int32_t* perm_y;      // round rho
  int64_t s, C;
  int n_c, k, cap, rho, rounds;   // cap: entries of a row's candidate list
  int selall;                 // 1: every window has at most k candidates (lists never compacted)
  int tiles_per_chunk;
  float beta_coef;            // error-bound coefficient of a float32 logit
  const float* xnorm;         // [s]
  const float* ynorm_max;     // [1]
  double* thr_e;              // [rounds][s]
  int32_t* thr_id;            // [rounds][s]
  float* thr_lo;              // [rounds][s]
  float* thr_hi;              // [rounds][s]
  float* mshift;              // [rounds][s]
  float* ssum;                // [rounds][s]
  int32_t* nmem;              // [rounds][s]
  int32_t* negs;              // [rounds][s][k] kept ids (bit 31: kept in an earlier round; -1 pad) or nullptr
  float* negl;                // [s][k] float32 logits of this round's negs (row = position or slot), or nullptr
  int slot_out;               // 1: outputs indexed by sorted slot, not by position id
  int n_ec;                   // window: chunks c - n_ec .. c + n_ec
  int wrap;                   // 1: chunk indices modulo n_c (cyclic); 0: clipped to [0, n_c)
  int win_order;              // walking order of the window's chunks (window_rotation)
  int prepass;                // 1: a histogram pass over the window sets the first threshold
  int2* clist;                // [rows][cap] candidate lists (item id, float32 logit bits)
  int32_t* clist_n;           // [rows] entries in each list; bit 31: compacted or raised, bit 30: redo
  float* clist_lo;            // [rows] each row's final threshold (no kept entry lies below it)
  double* cdbl;               // [blocks * waves][cap] float64 scratch of each chunk-kernel wave
  uint32_t* counters;
};

struct CeArgs {
  const void* X;
  const void* Y;
  const int32_t* pos;
  int64_t s, C;
  int rounds;
  const float* mshift;
  const float* ssum;
  const int32_t* nmem;
  float* lse;
  float* lpos;
  float* loss_pp;             // nullable
  float* partial;             // [num blocks][2] float64: loss sum, positions counted
  float* wmean;               // [1] out: the mean's weight of a position (1 / positions counted)
  uint32_t* counters;
  int validate;
  int ignore;                 // pos < 0 marks padding (no loss, not counted)
};

// Round dedup (rounds >= 1): the pairs of round rho's kept list that an earlier
// round also kept are marked (bit 31 of the id) and left out of the round's sum.
struct DedupArgs {
  int32_t* negs;              // [rounds][s][k] kept ids (-1 pad); earlier rounds read, round rho marked
  const float* negl;          // [s][k] float32 logits of round rho's kept list
  const float* mshift;        // [rounds][s]
  float* ssum;                // [rounds][s] overwritten for round rho: sum over its new pairs
  int32_t* nmem;              // [rounds][s] overwritten for round rho: its new pairs
  int64_t s;
  int k, rho;
  int hash_bits;              // log2 of the LDS hash slots per wave; 0: linear scan of the earlier lists
};

// Backward pass (both variants): everything is read from the kept lists.
struct BwdArgs {
  const void* X;
  const void* Y;
  const int32_t* pos;
  int64_t s, C;
  int rounds, k;
  const int32_t* negs;        // [rounds][s][k] kept ids (-1 pad; bit 31: kept in an earlier round)
  const float* lse;           // [s]
  const float* lpos;          // [s]
  const float* dloss;         // [1]
  const float* dloss_pp;      // [s] or nullptr
  const float* pcoef;         // [s][4]: lse, upstream gradient, positive coefficient, 0 (launch_pos_coef)
  const float* wmean;         // [1] the mean's weight of a position (forward pass)
  int ignore;                 // pos < 0 marks padding: upstream gradient 0
  int grad_bf16;              // dX, dY written as bf16
  void* dX;                   // [s][d] float32 (or bf16)
  void* dY;                   // [C][d] float32 (or bf16)
};

// Stable LSD counting sort of the (item, position) records of the backward pass:
// npass digit passes over keys below C, segments of seg_len records.
struct PairSortGeom {
  int64_t E;                  // records: rounds * s * k list entries + s positives
  int npass;
  int shift[4], bits[4];
  int64_t seg_len, nseg;
  int64_t count_words;        // count matrix of the widest pass, plus its total
  size_t scratch_bytes;       // counters, count matrix, scan block sums
};

// Launchers (defined in the .hip files).  All enqueue on `st`.
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t st);
// a[0..na), b[0..nb), c[0..nc) = 0 in one launch (each region at most a few thousand words).
hipError_t launch_zero3(uint32_t* a, int na, uint32_t* b, int nb, uint32_t* c, int nc, hipStream_t st);
// bnorm_max[0 .. rounds) and the zero_words 32-bit words after it are cleared first
// (zero_words < 0: already cleared by the caller).
hipError_t launch_prep_b(bool is_bf16, int d, const void* B, int rounds, int n_b, void* Bt, float* bnorm_max,
                         int zero_words, hipStream_t st);
// und: room for n row ids; und_n: a zero counter (rows whose float32 decision is
// not certain are listed there and decided in float64 by a second kernel).
hipError_t launch_project_argmax(bool is_bf16, int d, const void* V, int64_t n, const void* Bt, int n_b,
                                 const float* bnorm_max, float beta_coef, int32_t* ids, float* norms,
                                 uint32_t* norm_max_bits, int32_t* und, uint32_t* und_n, uint32_t* counters,
                                 hipStream_t st);
size_t sort_scratch_bytes(int64_t n, int nbins);
int sort_digit_bits(int64_t n);
hipError_t launch_counting_sort(const int32_t* keys, const int32_t* in_perm, int64_t n, int shift, int nbits,
                                void* scratch, int32_t* perm_out, int32_t* inv_out, hipStream_t st);
hipError_t launch_select(bool is_bf16, int d, int waves, const SelectArgs& a, hipStream_t st);
// Workgroups of `kernel` (threads, dynamic LDS bytes) resident on the current device at once.
hipError_t resident_blocks(const void* kernel, int threads, size_t lds, int64_t* out);
// Exact full cross-entropy (k_fullce.hip): workspace = [2][s] float32 (log-sum-exp,
// upstream gradient) + per-wave float64 loss sums.
size_t full_ce_workspace_bytes(int64_t s);
hipError_t full_ce_forward(bool bf16v, int d, int64_t s, int64_t C, const void* X, const void* Y, const int32_t* pos,
                           void* ws, float* loss, float* loss_pp, hipStream_t st);
hipError_t full_ce_backward(bool bf16v, int d, int64_t s, int64_t C, const void* X, const void* Y, const int32_t* pos,
                            void* ws, const float* dloss, const float* dloss_pp, float* dX, float* dY, hipStream_t st);
size_t select_lds_bytes(bool is_bf16, int d, int waves, int cap_lds);
int select_list_cap(int k, int d, bool bf16);   // entries of a row's candidate list
int select_finish_waves(int cap_lds);            // 0: a list of cap_lds entries does not fit in LDS
int ce_blocks(int64_t s);
hipError_t launch_ce(bool is_bf16, int d, const CeArgs& a, float* loss, hipStream_t st);
// log2 of the per-wave hash slots k_round_dedup uses for rounds earlier lists of k
// ids (0: too many for LDS, the kernel scans the lists instead).
int dedup_hash_bits(int rounds, int k);
hipError_t launch_round_dedup(const DedupArgs& a, hipStream_t st);
// out[s][4] = {lse, upstream gradient, positive coefficient, 0} per position (read by dX and dY).
hipError_t launch_pos_coef(const BwdArgs& a, float* out, hipStream_t st);
// dX of every position from the kept lists of all rounds plus the positive term
// (writes all s rows of dX).
hipError_t launch_dx_lists(bool is_bf16, int d, const BwdArgs& a, hipStream_t st);
// dst[0..n) = src[0..n) with bit 31 cleared, -1 kept (exported kept lists).
hipError_t launch_strip_mark(const int32_t* src, int64_t n, int32_t* dst, hipStream_t st);
// dst[s][rounds * k]: per position the ids no earlier round kept, in (round, list) order, -1 padded.
hipError_t launch_union_ids(const int32_t* negs, int64_t s, int k, int rounds, int32_t* dst, hipStream_t st);
// Exclusive scan of a[0..n) in place; bsum holds ceil(n / 4096) + 64 words.
hipError_t launch_exclusive_scan(uint32_t* a, int64_t n, uint32_t* bsum, hipStream_t st);
PairSortGeom pair_sort_geom(int64_t E, int64_t C);
// Records of the lists (nl = rounds * s * k entries) and the s positives sorted by item
// (stable); *kout / *vout point at the sorted keys / values (kA/vA or kB/vB) and *nout
// at the device count of records (entries < 0 or >= C are dropped).  scratch holds
// geom.scratch_bytes.
hipError_t launch_pair_sort(const PairSortGeom& g, const int32_t* negs, int64_t nl, int k, int64_t s,
                            const int32_t* pos, int64_t C, void* scratch, int32_t* kA, int32_t* vA, int32_t* kB,
                            int32_t* vB, const int32_t** kout, const int32_t** vout, const uint32_t** nout,
                            hipStream_t st);
// Work area of launch_dy for at most E sorted records.
size_t dy_area_bytes(int64_t E, int d);
// Every row of dY from the sorted records (K, V, *ntot of them); E bounds *ntot.
hipError_t launch_dy(bool is_bf16, int d, const BwdArgs& a, const int32_t* K, const int32_t* V, const uint32_t* ntot,
                     int64_t E, void* area, hipStream_t st);
// Bucket (SCE) variant.
// Per bucket column of a listed selection (k_col_pass / k_col_thresh): the
// histogram coordinate of a float32 score v is x = med3(v * sc + nlsc, 0, 32 -)
// (one fma) and, at the current level, y = x * mul + nxm (exactly (x - xa) * mul);
// bins are floor(y) in [0, 32).
struct ColState {
  float lo, sc, nlsc;   // smallest score of the column, 32 / (largest - smallest), -lo * sc
  float xa, mul, nxm;   // level origin (x units), scale, -xa * mul
  float tlo;            // listing threshold of the last decided level (value space)
  float vgate;          // smallest float32 score with y >= 0 at the current level
  float vlist;          // smallest float32 score with y >= bl (listed entries: score >= vlist)
  int level;            // level whose histogram is taken next; 0 once decided
  int bl;               // listing bin (COL_NONE: none)
  int nlist;            // entries listed, -1 when they exceed the list capacity
  int above;            // entries above the current level's range (y >= 32)
  int pad[3];
};
constexpr int COL_BINS = 32;      // bins of a histogram level
constexpr int COL_LEVELS = 3;     // levels at most
constexpr int COL_NONE = 1 << 30;
constexpr int COL_LIST_MAX_M = 4096;   // listed selections take at most this many entries per bucket
struct ColPassArgs {
  const void* V;              // [N][d] rows
  int64_t N;
  const void* Bt;             // [n_b][d] projection vectors
  int n_b, nb_pad;            // buckets, padded to 16
  int cg, n_g;                // columns per workgroup group, groups
  int64_t rows_pb;            // rows per row block (a multiple of 64)
  int n_rb;                   // row blocks
  int level;                  // histogram level of a CP_HIST pass
  float* norms;               // [N] row norms (nullptr: not stored)
  uint32_t* norm_max_bits;    // [1] largest row norm
  uint32_t* key_max;          // [nb_pad] order keys of the column maxima
  uint32_t* key_min;          // [nb_pad] complemented order keys of the column minima
  const ColState* cs;         // [n_b]
  uint32_t* hist;             // [n_rb][nb_pad][COL_BINS]
  const int32_t* offs;        // [nb_pad][n_rb] first list slot of each row block
  int32_t* lidx;              // [nb_pad][capl] listed rows
  float* lval;                // [nb_pad][capl] their float32 scores
  int64_t capl;
  const uint32_t* active;     // [COL_LEVELS + 1]: a column waits for level l
};
struct ColThreshArgs {
  ColState* cs;
  const uint32_t* hist;
  int32_t* above_r;           // [nb_pad][n_rb] entries above the level's range, per row block
  int32_t* offs;              // [nb_pad][n_rb]
  uint32_t* active;
  int n_b, nb_pad, n_rb, level, m;
  int64_t N, capl;
  float beta_coef;
  const uint32_t* vmax_bits;
  const float* bnorm_max;
  uint32_t* counters;
};
enum ColPassMode { CP_MINMAX = 0, CP_HIST = 1, CP_LIST = 2 };
// Row blocks of a listed selection over n rows (rows per block, a multiple of 64,
// and their count) and column groups (width, count).
void col_pass_shape(bool is_bf16, int d, int64_t n, int nb_pad, int64_t* rows_pb, int* n_rb, int* cg, int* n_g);
hipError_t launch_col_pass(bool is_bf16, int d, int mode, const ColPassArgs& a, hipStream_t st);
hipError_t launch_col_init(ColState* cs, const uint32_t* key_max, const uint32_t* key_min, uint32_t* active, int n_b,
                           hipStream_t st);
hipError_t launch_col_thresh(const ColThreshArgs& a, hipStream_t st);
struct ColSelectArgs {
  const float* PT;            // [n_b][N] projection scores, one column per bucket (dense selection)
  const int32_t* lidx;        // listed selection: [n_b][capl] rows and
  const float* lval;          //   their scores, nlist of ColState each
  const ColState* cs;
  int64_t capl;
  const void* V;              // [N][d] rows (float64 recomputation)
  const void* Bt;             // [n_b][d] projection vectors
  int64_t N;
  int m;                      // entries taken per bucket
  int n_b;
  float beta_coef;
  const uint32_t* vmax_bits;  // [1] max row norm (float bits)
  const float* bnorm_max;     // [1] max projection-vector norm
  int32_t* out;               // [n_b][m]
  uint32_t* counters;
};
hipError_t launch_project_scores(bool is_bf16, int d, const void* V, int64_t n, const void* Bt, int n_b, float* PT,
                                 float* norms, uint32_t* norm_max_bits, hipStream_t st);
// Dense selection (PT set) or listed selection (lidx set; output in index order).
hipError_t launch_col_select(bool is_bf16, int d, const ColSelectArgs& a, hipStream_t st);
hipError_t launch_group_bounds(const int32_t* keys, const int32_t* sorted, int64_t n, int32_t* start, int32_t* end,
                               hipStream_t st);
struct MergeArgs {
  const void* Y;
  const void* X;
  int64_t s;
  int k;
  float beta_coef;
  const float* xnorm;         // [s]
  const uint32_t* ymax_bits;  // [1]
  const int32_t* sorted;      // [slots] slots grouped by position
  const int32_t* pstart;      // [s]
  const int32_t* pend;        // [s]
  const int32_t* slot_negs;   // [slots][k] per-slot kept ids, -1 padded
  const float* slot_negl;     // [slots][k] their float32 logits
  const int32_t* slot_tid;    // [slots] per-slot threshold id (-1: every candidate kept)
  const double* slot_te;      // [slots] per-slot threshold logit (float64)
  double* thr_e;              // [s]
  int32_t* thr_id;
  float* thr_lo;
  float* thr_hi;
  float* mshift;
  float* ssum;
  int32_t* nmem;
  int32_t* negs;              // [s][k] or nullptr
  uint32_t* counters;
};
size_t merge_lds_bytes(int k);

// Host side (rece_host.cpp), for entry points defined in other files.
size_t plan_forward_scratch_bytes(rece_plan_t plan);      // scratch the forward pass alone uses
// rece_forward with every launch on `stream` (no second stream, no events created).
rece_status forward_single_stream(rece_plan_t plan, void* stream, const void* X, const void* Y, const int32_t* pos,
                                  const void* B, void* scratch, void* saved, float* loss, float* loss_pp);
rece_status set_last_error(rece_status st, const char* msg);   // sets rece_last_error(); returns st
hipError_t launch_sce_merge(bool is_bf16, int d, const MergeArgs& a, hipStream_t st);

}  // namespace rece
