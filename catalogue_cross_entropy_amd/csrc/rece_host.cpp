// librece host side: plan validation, workspace layout and the launch sequence.
// Every entry point is a C function returning rece_status; nothing here
// allocates device memory or waits for the GPU (except rece_check).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "rece_internal.h"

using namespace rece;

namespace {

thread_local std::string g_last_error;

rece_status fail(rece_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

rece_status hip_fail(hipError_t e, const char* where) {
  return fail(RECE_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int bits_for(int64_t n) {   // smallest b with 2^b >= n
  int b = 0;
  while (((int64_t)1 << b) < n) ++b;
  return b;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Layout {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  }
};

constexpr int32_t MAX_N_EC = 1 << 20;

}  // namespace

#define RECE_HIP(call, where)                 \
  do {                                         \
    hipError_t e_ = (call);                    \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

struct Profiler {
  bool on = false;
  uint32_t mask = 0;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<std::pair<int, std::pair<hipEvent_t, hipEvent_t>>> rec;
  hipEvent_t get() {
    if (used == pool.size()) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[used++];
  }
};

// A second stream of the plan (default priority) for launches with no data
// dependence on the main chain, forked from and joined back into the caller's
// stream with events; created on the device current at first use.
struct SideStream {
  std::mutex mu;   // one forward or backward enqueues on the side stream at a time
  hipStream_t s = nullptr;
  hipEvent_t join = nullptr;
  std::vector<hipEvent_t> fork;
};

struct rece_plan_s {
  rece_config cfg;
  mutable Profiler prof;
  mutable SideStream side;
  bool bf16;
  int esize;
  int nbits_b;
  int cap;            // entries of a row's candidate list in the chunk kernels
  int selall;         // every window has at most k candidates
  int prepass;        // windows of a few k: the chunk kernel's histogram pass sets the first threshold
  int waves_sel;
  int win_order;   // walking order of a window's chunks (window_rotation)
  int items_ahead;    // forward stream arrangement: item chains ahead of the chunk kernels
  int tpc_sel;
  int64_t wmax;       // largest window (items)
  float beta_coef;
  int dedup_bits;     // LDS hash size of the round dedup (log2 slots per wave, 0 = list scan)
  PairSortGeom pg;    // backward: sort of the (item, position) records
  int64_t npairs;     // rounds * s * k list entries + s positives
  // saved (forward -> backward)
  size_t o_cnt, o_bx, o_by, o_px, o_py, o_te, o_tid, o_tlo, o_thi, o_msh, o_ssum, o_nmem, o_xnorm, o_ymax, o_lse,
      o_lpos, o_wmean, o_negs, saved_bytes;
  // forward scratch
  size_t o_bt, o_bnorm, o_und, o_undy, o_sorty, o_sort, o_part, o_negl, o_cl0, o_cl1, o_cn0, o_cn1, o_cd0,
      o_cd1, o_clo0, o_clo1;
  // backward scratch (the backward reuses the forward's scratch from offset 0)
  size_t o_pk0, o_pv0, o_pk1, o_pv1, o_psc, o_dya, o_pcoef;
  size_t scratch_bytes;
  size_t scratch_fwd_bytes;   // what the forward pass alone uses of scratch
  // bucket variant: slots = (bucket, position) and (bucket, item) pairs
  int64_t sx, sy;     // n_b * b_x, n_b * b_y
  size_t o_R, o_Q, o_xmax;                                                                  // saved
  size_t o_ssort, o_sinv, o_pstart, o_pend, o_ste, o_stid, o_stlo, o_sthi, o_smsh, o_sssum, o_snmem,
      o_snegs, o_snegl, o_stmp;                                                             // scratch
  // the b_x positions (csx) and b_y items (csy) of every bucket
  struct ColSel {
    int mode;           // COLSEL_ALL, COLSEL_LISTED or COLSEL_DENSE
    int64_t N;
    int m;
    int64_t rows_pb, capl;
    int n_rb, cg, n_g, nb_pad;
    size_t o_cs, o_keys, o_act, o_hist, o_above, o_offs, o_lidx, o_lval, o_pt;   // scratch
  } csx, csy;
};
// A bucket takes every row; the b largest through histogram passes and a list
// (b <= COL_LIST_MAX_M); through the stored score matrix (larger b).
enum { COLSEL_ALL = 0, COLSEL_LISTED = 1, COLSEL_DENSE = 2 };

namespace {
// Brackets the launches of one phase with events when profiling is on.
struct PhaseScope {
  Profiler& pr;
  hipStream_t st;
  int phase;
  hipEvent_t a = nullptr, b = nullptr;
  PhaseScope(Profiler& p, int ph, hipStream_t s) : pr(p), st(s), phase(ph) {
    if (!pr.on || !((pr.mask >> ph) & 1u)) return;
    a = pr.get();
    b = pr.get();
    if (a && b) hipEventRecord(a, st);
  }
  ~PhaseScope() {
    if (!a || !b) return;
    hipEventRecord(b, st);
    pr.rec.push_back({phase, {a, b}});
  }
};
}  // namespace

#define RECE_PHASE(phase, call, where)                 \
  do {                                                 \
    PhaseScope ps_(p.prof, (phase), st);               \
    RECE_HIP(call, where);                             \
  } while (0)

static rece_status validate_config(const rece_config* c) {
  if (!c) return fail(RECE_ERR_INVALID_ARGUMENT, "config is NULL");
  if (c->variant != RECE_VARIANT_RECE && c->variant != RECE_VARIANT_SCE)
    return fail(RECE_ERR_INVALID_ARGUMENT, "unknown variant");
  if (c->s < 1) return fail(RECE_ERR_INVALID_ARGUMENT, "s must be >= 1");
  if (c->C < 2) return fail(RECE_ERR_INVALID_ARGUMENT, "C must be >= 2");
  if (c->s > ((int64_t)1 << 31) - 1 || c->C > ((int64_t)1 << 31) - 1)
    return fail(RECE_ERR_UNSUPPORTED, "s and C must fit in int32");
  if (c->d != 32 && c->d != 64 && c->d != 128 && c->d != 256)
    return fail(RECE_ERR_UNSUPPORTED, "d must be one of 32, 64, 128, 256");
  if (c->n_b < 1 || c->n_b > 4096) return fail(RECE_ERR_INVALID_ARGUMENT, "n_b must be in 1..4096");
  if (c->variant == RECE_VARIANT_RECE) {
    if (c->n_c < 1 || c->n_c > c->s || c->n_c > c->C)
      return fail(RECE_ERR_INVALID_ARGUMENT, "n_c must be in 1..min(s, C)");
    if (c->n_ec < 0 || c->n_ec > MAX_N_EC) return fail(RECE_ERR_INVALID_ARGUMENT, "n_ec must be in 0..2^20");
    if (c->window_wrap != 0 && c->window_wrap != 1)
      return fail(RECE_ERR_INVALID_ARGUMENT, "window_wrap must be 0 (clipped) or 1 (cyclic)");
  }
  if (c->variant == RECE_VARIANT_SCE) {
    if (c->rounds != 1) return fail(RECE_ERR_INVALID_ARGUMENT, "the bucket variant takes rounds = 1");
    if (c->b_x < 1 || c->b_x > c->s) return fail(RECE_ERR_INVALID_ARGUMENT, "b_x must be in 1..s");
    if (c->b_y < 1 || c->b_y > c->C) return fail(RECE_ERR_INVALID_ARGUMENT, "b_y must be in 1..C");
    if ((int64_t)c->n_b * c->b_x > ((int64_t)1 << 31) - 1 || (int64_t)c->n_b * c->b_y > ((int64_t)1 << 31) - 1)
      return fail(RECE_ERR_UNSUPPORTED, "n_b * b_x and n_b * b_y must fit in int32");
    if (c->k > 1024) return fail(RECE_ERR_UNSUPPORTED, "the bucket variant keeps at most k = 1024");
  }
  if (c->k < 0 || c->k > c->C - 1) return fail(RECE_ERR_INVALID_ARGUMENT, "k must be in 0..C-1");
  if (c->rounds < 1 || c->rounds > MAX_ROUNDS) return fail(RECE_ERR_INVALID_ARGUMENT, "rounds must be in 1..8");
  if (c->dtype != RECE_F32 && c->dtype != RECE_BF16) return fail(RECE_ERR_INVALID_ARGUMENT, "unknown dtype");
  if (c->flags & ~(RECE_FLAG_VALIDATE_IDS | RECE_FLAG_KEEP_STAGES | RECE_FLAG_IGNORE_NEGATIVE_POS |
                   RECE_FLAG_BF16_GRADS))
    return fail(RECE_ERR_INVALID_ARGUMENT, "unknown flag bits");
  if ((int64_t)c->rounds * c->s * std::max(c->k, 1) + c->s > ((int64_t)1 << 31) - 1)
    return fail(RECE_ERR_UNSUPPORTED, "rounds * s * k + s must fit in int32 (the backward's pair records)");
  return RECE_OK;
}

// Backward scratch of either variant: the sort of the (item, position) records
// and the dY work area.  Laid out from offset 0: the backward reads nothing of
// the forward's scratch.
static size_t plan_backward_scratch(rece_plan_s* p) {
  const rece_config& c = p->cfg;
  p->npairs = (int64_t)c.rounds * c.s * c.k + c.s;
  p->pg = pair_sort_geom(p->npairs, c.C);
  Layout sc;
  p->o_pk0 = sc.take((size_t)p->npairs * 4);
  p->o_pv0 = sc.take((size_t)p->npairs * 4);
  p->o_pk1 = sc.take((size_t)p->npairs * 4);
  p->o_pv1 = sc.take((size_t)p->npairs * 4);
  p->o_psc = sc.take(p->pg.scratch_bytes);
  p->o_dya = sc.take(dy_area_bytes(p->npairs, c.d));
  p->o_pcoef = sc.take((size_t)c.s * 16);
  return sc.off;
}

// Workspace of the bucket variant.
static void plan_sce_layout(rece_plan_s* p) {
  const rece_config& c = p->cfg;
  const int64_t s = c.s, C = c.C;
  const int d = c.d, k = std::max(c.k, 1), n_b = c.n_b;
  p->sx = (int64_t)n_b * c.b_x;
  p->sy = (int64_t)n_b * c.b_y;
  const int64_t sx = p->sx, sy = p->sy;
  Layout sv;
  p->o_cnt = sv.take(NUM_COUNTERS * 4);
  p->o_R = sv.take((size_t)sx * 4);
  p->o_Q = sv.take((size_t)sy * 4);
  p->o_te = sv.take((size_t)s * 8);
  p->o_tid = sv.take((size_t)s * 4);
  p->o_tlo = sv.take((size_t)s * 4);
  p->o_thi = sv.take((size_t)s * 4);
  p->o_msh = sv.take((size_t)s * 4);
  p->o_ssum = sv.take((size_t)s * 4);
  p->o_nmem = sv.take((size_t)s * 4);
  p->o_xnorm = sv.take((size_t)s * 4);
  p->o_xmax = sv.take(4);
  p->o_ymax = sv.take(4);
  p->o_lse = sv.take((size_t)s * 4);
  p->o_lpos = sv.take((size_t)s * 4);
  p->o_wmean = sv.take(16);
  p->o_negs = sv.take((size_t)s * k * 4);   // the final kept lists: the backward reads them
  p->saved_bytes = sv.off;

  Layout sc;
  p->o_bt = sc.take((size_t)n_b * d * p->esize);
  p->o_bnorm = sc.take(4);
  const size_t sort_b = std::max({sort_scratch_bytes(sx, 1 << std::min(12, bits_for(s))),
                                  sort_scratch_bytes(sy, 1 << std::min(12, bits_for(C)))});
  p->o_sort = sc.take(sort_b);
  p->o_part = sc.take((size_t)ce_blocks(s) * 16);
  p->o_ssort = sc.take((size_t)sx * 4);
  p->o_sinv = sc.take((size_t)sx * 4);
  p->o_pstart = sc.take((size_t)s * 4);
  p->o_pend = sc.take((size_t)s * 4);
  auto colsel = [&](rece_plan_s::ColSel& q, int64_t N, int m) {
    q = rece_plan_s::ColSel{};
    q.N = N;
    q.m = m;
    q.nb_pad = (n_b + 15) / 16 * 16;
    q.mode = (int64_t)m >= N ? COLSEL_ALL : (m <= COL_LIST_MAX_M ? COLSEL_LISTED : COLSEL_DENSE);
    col_pass_shape(p->bf16, d, N, q.nb_pad, &q.rows_pb, &q.n_rb, &q.cg, &q.n_g);
    // the list of a column: the m members, the rest of the boundary bin and the bin
    // below it (the column's score range cut in 32 bins); a finer level is taken
    // when that is more than the capacity
    q.capl = std::min<int64_t>(N, 3 * (int64_t)m + 16384);
    if (q.mode == COLSEL_DENSE) {
      q.o_pt = sc.take((size_t)n_b * N * 4);
    } else {
      q.o_keys = sc.take((size_t)q.nb_pad * 8);
    }
    if (q.mode == COLSEL_LISTED) {
      q.o_cs = sc.take((size_t)q.nb_pad * sizeof(ColState));
      q.o_act = sc.take((COL_LEVELS + 1) * 4);
      q.o_hist = sc.take((size_t)q.n_rb * q.nb_pad * COL_BINS * 4);
      q.o_above = sc.take((size_t)q.nb_pad * q.n_rb * 4);
      q.o_offs = sc.take((size_t)q.nb_pad * q.n_rb * 4);
      q.o_lidx = sc.take((size_t)q.nb_pad * q.capl * 4);
      q.o_lval = sc.take((size_t)q.nb_pad * q.capl * 4);
    }
  };
  colsel(p->csx, s, c.b_x);
  colsel(p->csy, C, c.b_y);
  p->o_ste = sc.take((size_t)sx * 8);
  p->o_stid = sc.take((size_t)sx * 4);
  p->o_stlo = sc.take((size_t)sx * 4);
  p->o_sthi = sc.take((size_t)sx * 4);
  p->o_smsh = sc.take((size_t)sx * 4);
  p->o_sssum = sc.take((size_t)sx * 4);
  p->o_snmem = sc.take((size_t)sx * 4);
  p->o_snegs = sc.take((size_t)sx * k * 4);
  p->o_snegl = sc.take((size_t)sx * k * 4);
  p->o_stmp = sc.take((size_t)sx * 4);
  p->o_cl0 = sc.take((size_t)sx * p->cap * 8);
  p->o_cn0 = sc.take((size_t)sx * 4);
  p->o_clo0 = sc.take((size_t)sx * 4);
  p->o_cd0 = sc.take((size_t)n_b * p->tpc_sel * p->waves_sel * p->cap * 8);
  p->scratch_fwd_bytes = sc.off;
  p->scratch_bytes = std::max(sc.off, plan_backward_scratch(p));
}

// Stable grouping of n elements by an integer key below `nkeys`: LSD passes of up
// to 12 bits; out = element indices in (key, index) order, inv = its inverse.
static rece_status group_by_key(const rece_plan_s& p, const int32_t* keys, int64_t n, int64_t nkeys, char* sort_scratch,
                                int32_t* tmp, int32_t* out, int32_t* inv, hipStream_t st) {
  const int total_bits = std::max(1, bits_for(nkeys));
  const int db = sort_digit_bits(n);
  const int npass = (total_bits + db - 1) / db;
  const int32_t* in = nullptr;
  for (int pass = 0, shift = 0; pass < npass; ++pass, shift += db) {
    const int nb = std::min(db, total_bits - shift);
    int32_t* dst = ((npass - 1 - pass) % 2 == 0) ? out : tmp;   // the last pass lands in out
    RECE_PHASE(RECE_PHASE_SORT,
               launch_counting_sort(keys, in, n, shift, nb, sort_scratch, dst, pass == npass - 1 ? inv : nullptr, st),
               "group by key");
    in = dst;
  }
  return RECE_OK;
}

// The m rows of largest projection score in every bucket column (SCE page, the
// bucket procedure), with the rows' norms and their largest norm.
static rece_status sce_col_select(const rece_plan_s& p, const rece_plan_s::ColSel& q, const void* V, const void* Bt,
                                  const float* bnorm, float* norms, uint32_t* vmax, int32_t* out, uint32_t* counters,
                                  char* sc, hipStream_t st) {
  const rece_config& c = p.cfg;
  const int d = c.d, n_b = c.n_b;
  ColSelectArgs ca{};
  ca.V = V;
  ca.Bt = Bt;
  ca.N = q.N;
  ca.m = q.m;
  ca.n_b = n_b;
  ca.beta_coef = p.beta_coef;
  ca.vmax_bits = vmax;
  ca.bnorm_max = bnorm;
  ca.out = out;
  ca.counters = counters;
  if (q.mode == COLSEL_DENSE) {
    float* pt = reinterpret_cast<float*>(sc + q.o_pt);
    RECE_PHASE(RECE_PHASE_PROJECT, launch_project_scores(p.bf16, d, V, q.N, Bt, n_b, pt, norms, vmax, st),
               "projection scores");
    ca.PT = pt;
    RECE_PHASE(RECE_PHASE_SORT, launch_col_select(p.bf16, d, ca, st), "bucket columns");
    return RECE_OK;
  }
  uint32_t* keys = reinterpret_cast<uint32_t*>(sc + q.o_keys);
  ColPassArgs pa{};
  pa.V = V;
  pa.N = q.N;
  pa.Bt = Bt;
  pa.n_b = n_b;
  pa.nb_pad = q.nb_pad;
  pa.cg = q.cg;
  pa.n_g = q.n_g;
  pa.rows_pb = q.rows_pb;
  pa.n_rb = q.n_rb;
  pa.norms = norms;
  pa.norm_max_bits = vmax;
  pa.key_max = keys;
  pa.key_min = keys + q.nb_pad;
  RECE_PHASE(RECE_PHASE_OTHER, launch_fill_u32(keys, 0u, 2 * q.nb_pad, st), "clear column ranges");
  RECE_PHASE(RECE_PHASE_PROJECT, launch_col_pass(p.bf16, d, CP_MINMAX, pa, st), "row norms and column ranges");
  if (q.mode == COLSEL_LISTED) {
    ColState* cs = reinterpret_cast<ColState*>(sc + q.o_cs);
    uint32_t* act = reinterpret_cast<uint32_t*>(sc + q.o_act);
    pa.cs = cs;
    pa.hist = reinterpret_cast<uint32_t*>(sc + q.o_hist);
    pa.offs = reinterpret_cast<int32_t*>(sc + q.o_offs);
    pa.lidx = reinterpret_cast<int32_t*>(sc + q.o_lidx);
    pa.lval = reinterpret_cast<float*>(sc + q.o_lval);
    pa.capl = q.capl;
    pa.active = act;
    ColThreshArgs ta{};
    ta.cs = cs;
    ta.hist = pa.hist;
    ta.above_r = reinterpret_cast<int32_t*>(sc + q.o_above);
    ta.offs = reinterpret_cast<int32_t*>(sc + q.o_offs);
    ta.active = act;
    ta.n_b = n_b;
    ta.nb_pad = q.nb_pad;
    ta.n_rb = q.n_rb;
    ta.m = q.m;
    ta.N = q.N;
    ta.capl = q.capl;
    ta.beta_coef = p.beta_coef;
    ta.vmax_bits = vmax;
    ta.bnorm_max = bnorm;
    ta.counters = counters;
    RECE_PHASE(RECE_PHASE_OTHER, launch_col_init(cs, pa.key_max, pa.key_min, act, n_b, st), "column ranges");
    for (int lvl = 1; lvl <= COL_LEVELS; ++lvl) {
      pa.level = lvl;
      ta.level = lvl;
      RECE_PHASE(RECE_PHASE_PROJECT, launch_col_pass(p.bf16, d, CP_HIST, pa, st), "column histograms");
      RECE_PHASE(RECE_PHASE_SORT, launch_col_thresh(ta, st), "column thresholds");
    }
    RECE_PHASE(RECE_PHASE_PROJECT, launch_col_pass(p.bf16, d, CP_LIST, pa, st), "column lists");
    ca.lidx = pa.lidx;
    ca.lval = pa.lval;
    ca.cs = cs;
    ca.capl = q.capl;
  }
  RECE_PHASE(RECE_PHASE_SORT, launch_col_select(p.bf16, d, ca, st), "bucket columns");
  return RECE_OK;
}

// Forward pass of the bucket variant (SCE page, abstract; the bucket procedure
// is described with the kernels).
static rece_status ensure_side(const rece_plan_s& p, int nfork);
static rece_status sce_forward(const rece_plan_s& p, hipStream_t st, const void* X, const void* Y,
                               const int32_t* pos, const void* B, char* sc, char* sv, float* loss, float* loss_pp,
                               bool single) {
  const rece_config& c = p.cfg;
  const int64_t s = c.s, C = c.C;
  const int d = c.d, k = c.k, n_b = c.n_b;
  uint32_t* counters = reinterpret_cast<uint32_t*>(sv + p.o_cnt);
  uint32_t* xmax = reinterpret_cast<uint32_t*>(sv + p.o_xmax);
  uint32_t* ymax = reinterpret_cast<uint32_t*>(sv + p.o_ymax);
  float* xnorm = reinterpret_cast<float*>(sv + p.o_xnorm);
  float* bnorm = reinterpret_cast<float*>(sc + p.o_bnorm);
  void* Bt = sc + p.o_bt;
  int32_t* R = reinterpret_cast<int32_t*>(sv + p.o_R);
  int32_t* Q = reinterpret_cast<int32_t*>(sv + p.o_Q);

  RECE_PHASE(RECE_PHASE_OTHER, launch_fill_u32(counters, 0u, NUM_COUNTERS, st), "clear counters");
  RECE_PHASE(RECE_PHASE_OTHER, launch_fill_u32(xmax, 0u, 1, st), "clear norm max");
  RECE_PHASE(RECE_PHASE_OTHER, launch_fill_u32(ymax, 0u, 1, st), "clear norm max");
  RECE_PHASE(RECE_PHASE_OTHER, launch_prep_b(p.bf16, d, B, 1, n_b, Bt, bnorm, 0, st), "prepare projection vectors");
  // the b_x positions and b_y items of every bucket (row norms on the way): the
  // positions on the side stream (unless single), alongside the items
  {
    std::unique_lock<std::mutex> side_lock(p.side.mu, std::defer_lock);
    hipStream_t side = st;
    if (!single) {
      side_lock.lock();
      const rece_status ss = ensure_side(p, 2);
      if (ss != RECE_OK) return ss;
      side = p.side.s;
      RECE_HIP(hipEventRecord(p.side.fork[0], st), "fork");
      RECE_HIP(hipStreamWaitEvent(side, p.side.fork[0], 0), "fork");
    }
    const rece_status ex = sce_col_select(p, p.csx, X, Bt, bnorm, xnorm, xmax, R, counters, sc, side);
    if (ex != RECE_OK) return ex;
    const rece_status ey = sce_col_select(p, p.csy, Y, Bt, bnorm, nullptr, ymax, Q, counters, sc, st);
    if (ey != RECE_OK) return ey;
    if (!single) {
      RECE_HIP(hipEventRecord(p.side.fork[1], side), "join");
      RECE_HIP(hipStreamWaitEvent(st, p.side.fork[1], 0), "join");
    }
  }

  // per (bucket, position) slot, the top-k of the bucket's items (the chunk kernel,
  // one chunk per bucket, window = the chunk's own items)
  SelectArgs a{};
  a.X = X;
  a.Y = Y;
  a.rounds = 1;
  a.pos = pos;
  a.perm_x = R;
  a.perm_y = Q;
  a.s = p.sx;
  a.C = p.sy;
  a.n_c = n_b;
  a.k = k;
  a.rho = 0;
  a.tiles_per_chunk = p.tpc_sel;
  a.beta_coef = p.beta_coef;
  a.xnorm = xnorm;
  a.ynorm_max = reinterpret_cast<const float*>(ymax);
  a.thr_e = reinterpret_cast<double*>(sc + p.o_ste);
  a.thr_id = reinterpret_cast<int32_t*>(sc + p.o_stid);
  a.thr_lo = reinterpret_cast<float*>(sc + p.o_stlo);
  a.thr_hi = reinterpret_cast<float*>(sc + p.o_sthi);
  a.mshift = reinterpret_cast<float*>(sc + p.o_smsh);
  a.ssum = reinterpret_cast<float*>(sc + p.o_sssum);
  a.nmem = reinterpret_cast<int32_t*>(sc + p.o_snmem);
  a.negs = reinterpret_cast<int32_t*>(sc + p.o_snegs);
  a.negl = reinterpret_cast<float*>(sc + p.o_snegl);
  a.slot_out = 1;
  a.n_ec = 0;
  a.prepass = p.prepass;
  a.wrap = 0;
  a.cap = p.cap;
  a.selall = p.selall;
  a.clist = reinterpret_cast<int2*>(sc + p.o_cl0);
  a.clist_n = reinterpret_cast<int32_t*>(sc + p.o_cn0);
  a.clist_lo = reinterpret_cast<float*>(sc + p.o_clo0);
  a.cdbl = reinterpret_cast<double*>(sc + p.o_cd0);
  a.counters = counters;
  RECE_PHASE(RECE_PHASE_SELECT, launch_select(p.bf16, d, p.waves_sel, a, st), "bucket logits and top-k");

  // slots grouped by position (bucket order inside a group), then the merge
  int32_t* ssort = reinterpret_cast<int32_t*>(sc + p.o_ssort);
  int32_t* sinv = reinterpret_cast<int32_t*>(sc + p.o_sinv);
  int32_t* pstart = reinterpret_cast<int32_t*>(sc + p.o_pstart);
  int32_t* pend = reinterpret_cast<int32_t*>(sc + p.o_pend);
  const rece_status gs =
      group_by_key(p, R, p.sx, s, sc + p.o_sort, reinterpret_cast<int32_t*>(sc + p.o_stmp), ssort, sinv, st);
  if (gs != RECE_OK) return gs;
  RECE_PHASE(RECE_PHASE_OTHER, launch_fill_u32(reinterpret_cast<uint32_t*>(pstart), 0u, s, st), "clear groups");
  RECE_PHASE(RECE_PHASE_OTHER, launch_fill_u32(reinterpret_cast<uint32_t*>(pend), 0u, s, st), "clear groups");
  RECE_PHASE(RECE_PHASE_OTHER, launch_group_bounds(R, ssort, p.sx, pstart, pend, st), "position groups");
  MergeArgs m{};
  m.X = X;
  m.Y = Y;
  m.s = s;
  m.k = k;
  m.beta_coef = p.beta_coef;
  m.xnorm = xnorm;
  m.ymax_bits = ymax;
  m.sorted = ssort;
  m.pstart = pstart;
  m.pend = pend;
  m.slot_negs = a.negs;
  m.slot_negl = a.negl;
  m.slot_tid = a.thr_id;
  m.slot_te = a.thr_e;
  m.thr_e = reinterpret_cast<double*>(sv + p.o_te);
  m.thr_id = reinterpret_cast<int32_t*>(sv + p.o_tid);
  m.thr_lo = reinterpret_cast<float*>(sv + p.o_tlo);
  m.thr_hi = reinterpret_cast<float*>(sv + p.o_thi);
  m.mshift = reinterpret_cast<float*>(sv + p.o_msh);
  m.ssum = reinterpret_cast<float*>(sv + p.o_ssum);
  m.nmem = reinterpret_cast<int32_t*>(sv + p.o_nmem);
  m.negs = reinterpret_cast<int32_t*>(sv + p.o_negs);
  m.counters = counters;
  RECE_PHASE(RECE_PHASE_SELECT, launch_sce_merge(p.bf16, d, m, st), "merge bucket lists");

  CeArgs ce{};
  ce.X = X;
  ce.Y = Y;
  ce.pos = pos;
  ce.s = s;
  ce.C = C;
  ce.rounds = 1;
  ce.mshift = m.mshift;
  ce.ssum = m.ssum;
  ce.nmem = m.nmem;
  ce.lse = reinterpret_cast<float*>(sv + p.o_lse);
  ce.lpos = reinterpret_cast<float*>(sv + p.o_lpos);
  ce.loss_pp = loss_pp;
  ce.partial = reinterpret_cast<float*>(sc + p.o_part);
  ce.counters = counters;
  ce.validate = (c.flags & RECE_FLAG_VALIDATE_IDS) ? 1 : 0;
  ce.ignore = (c.flags & RECE_FLAG_IGNORE_NEGATIVE_POS) ? 1 : 0;
  ce.wmean = reinterpret_cast<float*>(sv + p.o_wmean);
  RECE_PHASE(RECE_PHASE_LOSS, launch_ce(p.bf16, d, ce, loss, st), "loss");
  return RECE_OK;
}

extern "C" {

rece_status rece_plan(const rece_config* cfg, rece_plan_t* out) {
  if (!out) return fail(RECE_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  const rece_status vs = validate_config(cfg);
  if (vs != RECE_OK) return vs;
  rece_plan_s* p = new (std::nothrow) rece_plan_s();
  if (!p) return fail(RECE_ERR_INTERNAL, "host allocation failed");
  p->cfg = *cfg;
  rece_config& c = p->cfg;
  const int64_t s = c.s, C = c.C;
  const bool sce = c.variant == RECE_VARIANT_SCE;
  if (sce) {   // a bucket is a chunk whose window is its own item list
    c.n_ec = 0;
    c.window_wrap = 0;
  }
  const int d = c.d, r = c.rounds, k = c.k, n_c = sce ? c.n_b : c.n_c;
  p->bf16 = c.dtype == RECE_BF16;
  p->esize = p->bf16 ? 2 : 4;
  p->nbits_b = bits_for(c.n_b);
  const int64_t rows_chunk = sce ? c.b_x : (s + n_c - 1) / n_c;
  // the largest window (items)
  if (sce) {
    p->wmax = c.b_y;
  } else {
    const int64_t items_chunk = (C + n_c - 1) / n_c;
    const int64_t span = 2 * (int64_t)c.n_ec + 1;
    p->wmax = (c.window_wrap && span >= n_c) ? C : std::min<int64_t>(C, span * items_chunk);
  }
  // every candidate is kept when k reaches the largest window (a window of the whole
  // catalogue has C - 1 candidates, the positive being excluded); the candidate lists
  // then hold whole windows and are never compacted
  p->selall = sce ? (k >= c.b_y) : (p->wmax >= C ? (k >= C - 1) : (k >= p->wmax));
  // Windows of up to 24 k: a first pass over the window (histogram only) lists a few
  // k entries per row instead of about k (1 + ln(W / k)) with a threshold that
  // starts at -inf; with larger windows the extra pass costs more than it saves.
  p->prepass = !p->selall && k > 0 && p->wmax <= 24 * (int64_t)k;
  p->cap = p->selall ? (int)std::max<int64_t>(p->wmax, 1) : select_list_cap(k, d, p->bf16);
  if (p->selall && p->wmax >= ((int64_t)1 << 30)) {   // list lengths share a word with two flag bits
    delete p;
    return fail(RECE_ERR_UNSUPPORTED, "k covers a window of 2^30 or more items");
  }
  const int cap_lds = p->selall ? 0 : p->cap;
  if (!p->selall && select_finish_waves(cap_lds) == 0) {
    delete p;
    return fail(RECE_ERR_UNSUPPORTED, "k too large for a selection list held in LDS (k must cover the window, "
                                      "or stay below about 9000)");
  }
  // waves per chunk-kernel workgroup: 16 positions each, no more than a chunk has
  p->waves_sel = rows_chunk <= 16 ? 1 : (rows_chunk <= 32 ? 2 : 4);
  // Window walking order: with item chunks of a megabyte or more, by chunk index
  // modulo 2 n_ec + 1 (the workgroups of neighbouring chunks read each item chunk
  // at the same time, one HBM read for the windows that share it through the L2);
  // smaller chunks are L2-resident anyway and start with their own chunk, whose
  // logits raise the thresholds soonest.
  {
    const int64_t chunk_bytes = (sce ? c.b_y : (C + n_c - 1) / n_c) * (int64_t)d * p->esize;
    p->win_order = sce ? 0 : (chunk_bytes >= ((int64_t)1 << 20) ? 2 : 1);
  }
  // The item chains go ahead of the chunk kernels when the bucketing of the items
  // (C n_b products per round) outweighs the chunk logits (s times the window) four
  // times over: the chunk kernels then wait the least with one round's chain hidden
  // behind the previous round's chunk kernel.  Below that the chunk kernels of
  // different rounds are better run side by side.
  p->items_ahead = !sce && (int64_t)C * c.n_b >= 4 * (int64_t)s * p->wmax;
  while (p->waves_sel > 1 && select_lds_bytes(p->bf16, d, p->waves_sel, cap_lds) > 160 * 1024) p->waves_sel /= 2;
  if (select_lds_bytes(p->bf16, d, p->waves_sel, cap_lds) > 160 * 1024) {
    delete p;
    return fail(RECE_ERR_UNSUPPORTED, "k too large for the chunk kernel's LDS");
  }
  p->tpc_sel = (int)((rows_chunk + 16 * p->waves_sel - 1) / (16 * p->waves_sel));
  // |float32 matrix-core dot - float64 coordinate-order dot| <= beta_coef * ||x|| * ||y||:
  // d products and d additions, each with relative error at most 2^-23 (round or
  // chop), doubled for safety; the float64 side adds d * 2^-53.
  p->beta_coef = (float)(4.0 * (d + 2) * std::ldexp(1.0, -24) * (1.0 + 1e-6) + d * std::ldexp(1.0, -52));
  if (sce) {
    plan_sce_layout(p);
    *out = p;
    return RECE_OK;
  }

  Layout sv;
  p->o_cnt = sv.take(NUM_COUNTERS * 4);
  p->o_bx = sv.take((size_t)r * s * 4);
  p->o_by = sv.take((size_t)r * C * 4);
  p->o_px = sv.take((size_t)r * s * 4);
  p->o_py = sv.take((size_t)r * C * 4);
  p->o_te = sv.take((size_t)r * s * 8);
  p->o_tid = sv.take((size_t)r * s * 4);
  p->o_tlo = sv.take((size_t)r * s * 4);
  p->o_thi = sv.take((size_t)r * s * 4);
  p->o_msh = sv.take((size_t)r * s * 4);
  p->o_ssum = sv.take((size_t)r * s * 4);
  p->o_nmem = sv.take((size_t)r * s * 4);
  p->o_xnorm = sv.take((size_t)s * 4);
  p->o_ymax = sv.take(4);
  p->o_lse = sv.take((size_t)s * 4);
  p->o_lpos = sv.take((size_t)s * 4);
  p->o_wmean = sv.take(16);
  p->o_negs = sv.take((size_t)r * s * std::max(k, 1) * 4);   // kept lists: the backward reads them
  p->saved_bytes = sv.off;

  Layout sc;
  p->o_bt = sc.take((size_t)r * c.n_b * d * p->esize);
  p->o_bnorm = sc.take((size_t)r * 4 + (size_t)2 * r * 4);   // norms, then one list counter per bucketing launch
  p->o_und = sc.take((size_t)s * 4);    // undecided bucketing rows: positions,
  p->o_undy = sc.take((size_t)std::max(s, C) * 4);   // chains on the side stream (items, later positions)
  p->o_sorty = sc.take(std::max(sort_scratch_bytes(C, 1 << p->nbits_b), sort_scratch_bytes(s, 1 << p->nbits_b)));
  p->o_sort = sc.take(std::max(sort_scratch_bytes(s, 1 << p->nbits_b), sort_scratch_bytes(C, 1 << p->nbits_b)));
  p->o_part = sc.take((size_t)ce_blocks(s) * 16);
  // float32 logits of the kept lists of rounds >= 1 (the round dedup sums the new pairs)
  p->o_negl = sc.take((size_t)(r - 1) * s * k * 4);
  // candidate lists of the chunk kernels: round 0 (caller's stream), rounds >= 1 (side stream, in turn)
  p->o_cl0 = sc.take((size_t)s * p->cap * 8);
  p->o_cn0 = sc.take((size_t)s * 4);
  p->o_cl1 = r > 1 ? sc.take((size_t)s * p->cap * 8) : p->o_cl0;
  p->o_cn1 = r > 1 ? sc.take((size_t)s * 4) : p->o_cn0;
  p->o_clo0 = sc.take((size_t)s * 4);
  p->o_clo1 = r > 1 ? sc.take((size_t)s * 4) : p->o_clo0;
  const size_t cd = (size_t)c.n_c * p->tpc_sel * p->waves_sel * p->cap * 8;   // per chunk-kernel wave
  p->o_cd0 = sc.take(cd);
  p->o_cd1 = r > 1 ? sc.take(cd) : p->o_cd0;
  p->dedup_bits = dedup_hash_bits(r, k);
  p->scratch_fwd_bytes = sc.off;
  p->scratch_bytes = std::max(sc.off, plan_backward_scratch(p));
  *out = p;
  return RECE_OK;
}

rece_status rece_plan_destroy(rece_plan_t plan) {
  if (plan) {
    for (hipEvent_t e : plan->prof.pool) hipEventDestroy(e);
    for (hipEvent_t e : plan->side.fork) hipEventDestroy(e);
    if (plan->side.join) hipEventDestroy(plan->side.join);
    if (plan->side.s) hipStreamDestroy(plan->side.s);
  }
  delete plan;
  return RECE_OK;
}

// The plan's side stream and nfork fork events (created once).
static rece_status ensure_side(const rece_plan_s& p, int nfork) {
  SideStream& sd = p.side;
  if (!sd.s) RECE_HIP(hipStreamCreateWithFlags(&sd.s, hipStreamNonBlocking), "create side stream");
  if (!sd.join) RECE_HIP(hipEventCreateWithFlags(&sd.join, hipEventDisableTiming), "create event");
  while ((int)sd.fork.size() < nfork) {
    hipEvent_t e = nullptr;
    RECE_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming), "create event");
    sd.fork.push_back(e);
  }
  return RECE_OK;
}

rece_status rece_profile_enable(rece_plan_t plan, int mask) {
  if (!plan) return fail(RECE_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (mask) {
    plan->prof.rec.clear();
    plan->prof.used = 0;
  }
  plan->prof.on = mask != 0;
  plan->prof.mask = (uint32_t)mask;
  return RECE_OK;
}

rece_status rece_profile_read(rece_plan_t plan, int phase, double* total_ms, int64_t* launches) {
  if (!plan || !total_ms || !launches) return fail(RECE_ERR_INVALID_ARGUMENT, "NULL argument");
  if (phase < 0 || phase >= RECE_NUM_PHASES) return fail(RECE_ERR_INVALID_ARGUMENT, "unknown phase");
  double tot = 0.0;
  int64_t n = 0;
  for (auto& r : plan->prof.rec) {
    if (r.first != phase) continue;
    RECE_HIP(hipEventSynchronize(r.second.second), "profile: wait for event");
    float ms = 0.0f;
    RECE_HIP(hipEventElapsedTime(&ms, r.second.first, r.second.second), "profile: elapsed time");
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return RECE_OK;
}

rece_status rece_auto_size(int64_t s, int64_t C, int32_t n_ec, double alpha_bc, int32_t rounds, int32_t* n_b,
                           int32_t* n_c, double* model_elems, double* full_ratio) {
  if (s < 1 || C < 1 || n_ec < 0 || !(alpha_bc > 0.0) || rounds < 1)
    return fail(RECE_ERR_INVALID_ARGUMENT, "need s, C, rounds >= 1, n_ec >= 0 and alpha_bc > 0");
  const double mn = (double)std::min(C, s), mx = (double)std::max(C, s);
  const double span = 1.0 + 2.0 * (double)n_ec;
  const double nb = std::sqrt(4.0 * alpha_bc * span * mn);
  const int32_t nbi = (int32_t)std::max(1.0, std::min(std::floor(nb + 0.5), 2147483647.0));
  if (n_b) *n_b = nbi;
  if (n_c) *n_c = (int32_t)std::max(1.0, std::min(std::floor(nbi / alpha_bc + 0.5), 2147483647.0));
  const double root = std::sqrt(alpha_bc * span * mn);
  if (model_elems) *model_elems = 2.0 * rounds * root * mx;
  if (full_ratio) *full_ratio = std::sqrt(mn) / (2.0 * rounds * std::sqrt(alpha_bc * span));
  return RECE_OK;
}

static rece_status check_full_ce(int64_t s, int64_t C, int32_t d, int32_t dtype, const void* X, const void* Y,
                                 const int32_t* pos, const void* ws, size_t ws_bytes) {
  if (s < 1 || C < 1) return fail(RECE_ERR_INVALID_ARGUMENT, "s and C must be >= 1");
  if (s > ((int64_t)1 << 31) - 1 || C > ((int64_t)1 << 31) - 1)
    return fail(RECE_ERR_UNSUPPORTED, "s and C must fit in int32");
  if (d != 32 && d != 64 && d != 128 && d != 256) return fail(RECE_ERR_UNSUPPORTED, "d must be one of 32, 64, 128, 256");
  if (dtype != RECE_F32 && dtype != RECE_BF16) return fail(RECE_ERR_UNSUPPORTED, "dtype must be RECE_F32 or RECE_BF16");
  if (!X || !Y || !pos || !ws) return fail(RECE_ERR_INVALID_ARGUMENT, "NULL input or workspace pointer");
  if ((reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(Y) | reinterpret_cast<uintptr_t>(ws)) % 16)
    return fail(RECE_ERR_INVALID_ARGUMENT, "X, Y and workspace must be 16-byte aligned");
  if (ws_bytes < rece::full_ce_workspace_bytes(s))
    return fail(RECE_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than rece_full_ce_workspace_bytes(s)");
  return RECE_OK;
}

rece_status rece_full_ce_workspace_bytes(int64_t s, size_t* bytes) {
  if (s < 1 || !bytes) return fail(RECE_ERR_INVALID_ARGUMENT, "s must be >= 1 and bytes non-NULL");
  *bytes = rece::full_ce_workspace_bytes(s);
  return RECE_OK;
}

rece_status rece_full_ce_forward(void* stream, int64_t s, int64_t C, int32_t d, int32_t dtype, const void* X,
                                 const void* Y, const int32_t* pos, void* workspace, size_t workspace_bytes,
                                 float* loss, float* loss_pp) {
  const rece_status v = check_full_ce(s, C, d, dtype, X, Y, pos, workspace, workspace_bytes);
  if (v != RECE_OK) return v;
  if (!loss) return fail(RECE_ERR_INVALID_ARGUMENT, "loss is NULL");
  RECE_HIP(rece::full_ce_forward(dtype == RECE_BF16, d, s, C, X, Y, pos, workspace, loss, loss_pp,
                                 static_cast<hipStream_t>(stream)),
           "full cross-entropy forward");
  return RECE_OK;
}

rece_status rece_full_ce_backward(void* stream, int64_t s, int64_t C, int32_t d, int32_t dtype, const void* X,
                                  const void* Y, const int32_t* pos, void* workspace, size_t workspace_bytes,
                                  const float* dloss, const float* dloss_pp, float* dX, float* dY) {
  const rece_status v = check_full_ce(s, C, d, dtype, X, Y, pos, workspace, workspace_bytes);
  if (v != RECE_OK) return v;
  if (!dloss && !dloss_pp) return fail(RECE_ERR_INVALID_ARGUMENT, "dloss and dloss_pp are both NULL");
  if (!dX || !dY) return fail(RECE_ERR_INVALID_ARGUMENT, "dX or dY is NULL");
  RECE_HIP(rece::full_ce_backward(dtype == RECE_BF16, d, s, C, X, Y, pos, workspace, dloss, dloss_pp, dX, dY,
                                  static_cast<hipStream_t>(stream)),
           "full cross-entropy backward");
  return RECE_OK;
}

rece_status rece_workspace_bytes(rece_plan_t plan, size_t* scratch_bytes, size_t* saved_bytes) {
  if (!plan) return fail(RECE_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (scratch_bytes) *scratch_bytes = plan->scratch_bytes;
  if (saved_bytes) *saved_bytes = plan->saved_bytes;
  return RECE_OK;
}

// The forward pass.  single: everything on `st` (no side stream, no events), for
// callers that may create no HIP object.
static rece_status forward_impl(const rece_plan_s& p, hipStream_t st, const void* X, const void* Y,
                                const int32_t* pos, const void* B, char* sc, char* sv, float* loss, float* loss_pp,
                                bool single) {
  const rece_config& c = p.cfg;
  const int64_t s = c.s, C = c.C;
  const int d = c.d;
  uint32_t* counters = reinterpret_cast<uint32_t*>(sv + p.o_cnt);
  float* ymax = reinterpret_cast<float*>(sv + p.o_ymax);
  float* xnorm = reinterpret_cast<float*>(sv + p.o_xnorm);
  float* bnorm = reinterpret_cast<float*>(sc + p.o_bnorm);
  void* Bt = sc + p.o_bt;

  if (c.variant == RECE_VARIANT_SCE) return sce_forward(p, st, X, Y, pos, B, sc, sv, loss, loss_pp, single);
  std::unique_lock<std::mutex> side_lock(p.side.mu, std::defer_lock);
  if (!single) side_lock.lock();
  uint32_t* und_n = reinterpret_cast<uint32_t*>(bnorm + c.rounds);   // cleared with the norms
  int32_t* und = reinterpret_cast<int32_t*>(sc + p.o_und);
  RECE_PHASE(RECE_PHASE_OTHER,
             launch_zero3(counters, NUM_COUNTERS, reinterpret_cast<uint32_t*>(ymax), 1,
                          reinterpret_cast<uint32_t*>(bnorm), 3 * c.rounds, st),
             "clear counters and maxima");
  RECE_PHASE(RECE_PHASE_OTHER, launch_prep_b(p.bf16, d, B, c.rounds, c.n_b, Bt, bnorm, -1, st),
             "prepare random vectors");

  // Two streams.  With a catalogue much larger than the rounds' windows
  // (items_ahead), the item chain of every round (bucketing and sort of the C
  // items, then the largest part of the forward pass) runs on the side stream
  // ahead of the chunk kernels, which run in turn on the caller's stream after the
  // position chains: the chain of round rho + 1 runs while the chunk kernel of
  // round rho does.  Otherwise the side stream takes the item chains, the position
  // chains of rounds >= 1 and the chunk kernels of rounds >= 1, while round 0's
  // position chain and chunk kernel run on the caller's stream (the chunk kernels
  // of different rounds then run at the same time).  Events: fork[rounds] starts
  // the side stream, fork[rho] marks the end of round rho's item chain,
  // fork[rounds + 1] the position norms (second arrangement), fork[rounds + 2]
  // the end of the side stream.
  hipStream_t side = st;
  if (!single) {
    const rece_status ss = ensure_side(p, c.rounds + 3);
    if (ss != RECE_OK) return ss;
    side = p.side.s;
  }
  // event record / wait between the two streams (nothing when single)
  auto record = [&](int e, hipStream_t on) { return single ? hipSuccess : hipEventRecord(p.side.fork[e], on); };
  auto wait = [&](hipStream_t on, int e) { return single ? hipSuccess : hipStreamWaitEvent(on, p.side.fork[e], 0); };
  int32_t* undy = reinterpret_cast<int32_t*>(sc + p.o_undy);
  RECE_HIP(record(c.rounds, st), "fork");
  RECE_HIP(wait(side, c.rounds), "fork");

  auto select_args = [&](int rho) {
    SelectArgs a{};
    a.X = X;
    a.Y = Y;
    a.rounds = c.rounds;
    a.pos = pos;
    a.perm_x = reinterpret_cast<int32_t*>(sv + p.o_px) + (int64_t)rho * s;
    a.perm_y = reinterpret_cast<int32_t*>(sv + p.o_py) + (int64_t)rho * C;
    a.s = s;
    a.C = C;
    a.n_c = c.n_c;
    a.k = c.k;
    a.rho = rho;
    a.tiles_per_chunk = p.tpc_sel;
    a.beta_coef = p.beta_coef;
    a.xnorm = xnorm;
    a.ynorm_max = ymax;
    a.thr_e = reinterpret_cast<double*>(sv + p.o_te);
    a.thr_id = reinterpret_cast<int32_t*>(sv + p.o_tid);
    a.thr_lo = reinterpret_cast<float*>(sv + p.o_tlo);
    a.thr_hi = reinterpret_cast<float*>(sv + p.o_thi);
    a.mshift = reinterpret_cast<float*>(sv + p.o_msh);
    a.ssum = reinterpret_cast<float*>(sv + p.o_ssum);
    a.nmem = reinterpret_cast<int32_t*>(sv + p.o_nmem);
    a.negs = reinterpret_cast<int32_t*>(sv + p.o_negs);
    a.slot_out = 0;
    a.n_ec = c.n_ec;
    a.wrap = c.window_wrap;
    a.win_order = p.win_order;
    a.prepass = p.prepass;
    a.cap = p.cap;
    a.selall = p.selall;
    a.clist = reinterpret_cast<int2*>(sc + (rho == 0 ? p.o_cl0 : p.o_cl1));
    a.clist_n = reinterpret_cast<int32_t*>(sc + (rho == 0 ? p.o_cn0 : p.o_cn1));
    a.clist_lo = reinterpret_cast<float*>(sc + (rho == 0 ? p.o_clo0 : p.o_clo1));
    a.cdbl = reinterpret_cast<double*>(sc + (rho == 0 ? p.o_cd0 : p.o_cd1));
    a.counters = counters;
    a.negl = rho > 0 ? reinterpret_cast<float*>(sc + p.o_negl) + (int64_t)(rho - 1) * s * c.k : nullptr;
    return a;
  };

  if (p.items_ahead) {
    // position chains of every round (the caller's stream; round 0's bucketing also
    // writes the position norms every chunk kernel reads)
    for (int rho = 0; rho < c.rounds; ++rho) {
      int32_t* bx = reinterpret_cast<int32_t*>(sv + p.o_bx) + (int64_t)rho * s;
      int32_t* px = reinterpret_cast<int32_t*>(sv + p.o_px) + (int64_t)rho * s;
      const void* Btr = static_cast<const char*>(Bt) + (size_t)rho * c.n_b * d * p.esize;
      RECE_PHASE(RECE_PHASE_PROJECT, launch_project_argmax(p.bf16, d, X, s, Btr, c.n_b, bnorm + rho, p.beta_coef, bx,
                                     rho == 0 ? xnorm : nullptr, nullptr, und, und_n + 2 * rho, counters, st),
                 "bucket positions");
      RECE_PHASE(RECE_PHASE_SORT, launch_counting_sort(bx, nullptr, s, 0, p.nbits_b, sc + p.o_sort, px, nullptr, st),
                 "sort positions");
    }
    // item chain of round rho on the side stream; round 0's also takes the largest
    // item norm
    auto item_chain = [&](int rho) -> rece_status {
      hipStream_t st = side;
      int32_t* by = reinterpret_cast<int32_t*>(sv + p.o_by) + (int64_t)rho * C;
      int32_t* py = reinterpret_cast<int32_t*>(sv + p.o_py) + (int64_t)rho * C;
      const void* Btr = static_cast<const char*>(Bt) + (size_t)rho * c.n_b * d * p.esize;
      RECE_PHASE(RECE_PHASE_PROJECT, launch_project_argmax(p.bf16, d, Y, C, Btr, c.n_b, bnorm + rho, p.beta_coef, by, nullptr,
                                     rho == 0 ? reinterpret_cast<uint32_t*>(ymax) : nullptr, undy, und_n + 2 * rho + 1,
                                     counters, st),
                 "bucket items");
      RECE_PHASE(RECE_PHASE_SORT, launch_counting_sort(by, nullptr, C, 0, p.nbits_b, sc + p.o_sorty, py, nullptr, st),
                 "sort items");
      RECE_HIP(record(rho, side), "item chain done");
      return RECE_OK;
    };
    {
      const rece_status e0 = item_chain(0);
      if (e0 != RECE_OK) return e0;
    }
    for (int rho = 0; rho < c.rounds; ++rho) {
      // enqueued in this order, a single stream also runs every chain before its use
      if (rho + 1 < c.rounds) {
        const rece_status e1 = item_chain(rho + 1);
        if (e1 != RECE_OK) return e1;
      }
      RECE_HIP(wait(st, rho), "join the item chain");
      const SelectArgs a = select_args(rho);
      RECE_PHASE(RECE_PHASE_SELECT, launch_select(p.bf16, d, p.waves_sel, a, st), "chunk logits and top-k");
    }
    RECE_HIP(record(c.rounds + 2, side), "side stream done");
    RECE_HIP(wait(st, c.rounds + 2), "join the side stream");
  } else {
    {   // round 0's position chain, alongside the first item chain
      int32_t* bx = reinterpret_cast<int32_t*>(sv + p.o_bx);
      int32_t* px = reinterpret_cast<int32_t*>(sv + p.o_px);
      RECE_PHASE(RECE_PHASE_PROJECT, launch_project_argmax(p.bf16, d, X, s, Bt, c.n_b, bnorm, p.beta_coef, bx,
                                     xnorm, nullptr, und, und_n, counters, st),
                 "bucket positions");
      RECE_HIP(record(c.rounds + 1, st), "position norms");
      RECE_PHASE(RECE_PHASE_SORT, launch_counting_sort(bx, nullptr, s, 0, p.nbits_b, sc + p.o_sort, px, nullptr, st),
                 "sort positions");
    }

    for (int rho = 0; rho < c.rounds; ++rho) {
      hipStream_t st = side;
      int32_t* by = reinterpret_cast<int32_t*>(sv + p.o_by) + (int64_t)rho * C;
      int32_t* py = reinterpret_cast<int32_t*>(sv + p.o_py) + (int64_t)rho * C;
      const void* Btr = static_cast<const char*>(Bt) + (size_t)rho * c.n_b * d * p.esize;
      RECE_PHASE(RECE_PHASE_PROJECT, launch_project_argmax(p.bf16, d, Y, C, Btr, c.n_b, bnorm + rho, p.beta_coef, by, nullptr,
                                     rho == 0 ? reinterpret_cast<uint32_t*>(ymax) : nullptr, undy, und_n + 2 * rho + 1,
                                     counters, st),
               "bucket items");
      RECE_PHASE(RECE_PHASE_SORT, launch_counting_sort(by, nullptr, C, 0, p.nbits_b, sc + p.o_sorty, py, nullptr, st),
                 "sort items");
      if (rho == 0) {
        RECE_HIP(record(0, side), "item chain done");
        continue;
      }
      int32_t* bx = reinterpret_cast<int32_t*>(sv + p.o_bx) + (int64_t)rho * s;
      int32_t* px = reinterpret_cast<int32_t*>(sv + p.o_px) + (int64_t)rho * s;
      RECE_PHASE(RECE_PHASE_PROJECT, launch_project_argmax(p.bf16, d, X, s, Btr, c.n_b, bnorm + rho, p.beta_coef,
                                     bx, nullptr, nullptr, undy, und_n + 2 * rho, counters, st),
                 "bucket positions");
      RECE_PHASE(RECE_PHASE_SORT, launch_counting_sort(bx, nullptr, s, 0, p.nbits_b, sc + p.o_sorty, px, nullptr, st),
                 "sort positions");
      if (rho == 1) RECE_HIP(wait(side, c.rounds + 1), "position norms");
      const SelectArgs a = select_args(rho);
      RECE_PHASE(RECE_PHASE_SELECT, launch_select(p.bf16, d, p.waves_sel, a, st), "chunk logits and top-k");
    }
    RECE_HIP(record(c.rounds + 2, side), "side stream done");

    RECE_HIP(wait(st, 0), "join the first item chain");
    {
      const SelectArgs a = select_args(0);
      RECE_PHASE(RECE_PHASE_SELECT, launch_select(p.bf16, d, p.waves_sel, a, st), "chunk logits and top-k");
    }
    RECE_HIP(wait(st, c.rounds + 2), "join the side stream");
  }
  for (int rho = 1; rho < c.rounds && c.k > 0; ++rho) {
    DedupArgs dd{};
    dd.negs = reinterpret_cast<int32_t*>(sv + p.o_negs);
    dd.negl = reinterpret_cast<const float*>(sc + p.o_negl) + (int64_t)(rho - 1) * s * c.k;
    dd.mshift = reinterpret_cast<const float*>(sv + p.o_msh);
    dd.ssum = reinterpret_cast<float*>(sv + p.o_ssum);
    dd.nmem = reinterpret_cast<int32_t*>(sv + p.o_nmem);
    dd.s = s;
    dd.k = c.k;
    dd.rho = rho;
    // a table sized for this round's earlier ids (rho k): smaller tables for the
    // early rounds, so more workgroups share a CU (the table size bounds occupancy)
    dd.hash_bits = p.dedup_bits ? dedup_hash_bits(rho + 1, c.k) : 0;
    RECE_PHASE(RECE_PHASE_LOSS, launch_round_dedup(dd, st), "round dedup");
  }

  CeArgs ce{};
  ce.X = X;
  ce.Y = Y;
  ce.pos = pos;
  ce.s = s;
  ce.C = C;
  ce.rounds = c.rounds;
  ce.mshift = reinterpret_cast<const float*>(sv + p.o_msh);
  ce.ssum = reinterpret_cast<const float*>(sv + p.o_ssum);
  ce.nmem = reinterpret_cast<const int32_t*>(sv + p.o_nmem);
  ce.lse = reinterpret_cast<float*>(sv + p.o_lse);
  ce.lpos = reinterpret_cast<float*>(sv + p.o_lpos);
  ce.loss_pp = loss_pp;
  ce.partial = reinterpret_cast<float*>(sc + p.o_part);
  ce.counters = counters;
  ce.validate = (c.flags & RECE_FLAG_VALIDATE_IDS) ? 1 : 0;
  ce.ignore = (c.flags & RECE_FLAG_IGNORE_NEGATIVE_POS) ? 1 : 0;
  ce.wmean = reinterpret_cast<float*>(sv + p.o_wmean);
  RECE_PHASE(RECE_PHASE_LOSS, launch_ce(p.bf16, d, ce, loss, st), "loss");
  return RECE_OK;
}

static rece_status check_forward_args(rece_plan_t plan, const void* X, const void* Y, const int32_t* pos,
                                      const void* B, const void* scratch, const void* saved, const float* loss) {
  if (!plan) return fail(RECE_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!X || !Y || !pos || !B || !scratch || !saved || !loss)
    return fail(RECE_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (!aligned16(X) || !aligned16(Y) || !aligned16(B) || !aligned16(scratch) || !aligned16(saved))
    return fail(RECE_ERR_INVALID_ARGUMENT, "X, Y, B, scratch and saved must be 16-byte aligned");
  return RECE_OK;
}

rece_status rece_forward(rece_plan_t plan, void* stream, const void* X, const void* Y, const int32_t* pos,
                         const void* B, void* scratch, void* saved, float* loss, float* loss_pp) {
  const rece_status cs = check_forward_args(plan, X, Y, pos, B, scratch, saved, loss);
  if (cs != RECE_OK) return cs;
  return forward_impl(*plan, reinterpret_cast<hipStream_t>(stream), X, Y, pos, B, static_cast<char*>(scratch),
                      static_cast<char*>(saved), loss, loss_pp, false);
}

}  // extern "C"

namespace rece {
size_t plan_forward_scratch_bytes(rece_plan_t plan) { return plan->scratch_fwd_bytes; }

rece_status forward_single_stream(rece_plan_t plan, void* stream, const void* X, const void* Y, const int32_t* pos,
                                  const void* B, void* scratch, void* saved, float* loss, float* loss_pp) {
  const rece_status cs = check_forward_args(plan, X, Y, pos, B, scratch, saved, loss);
  if (cs != RECE_OK) return cs;
  return forward_impl(*plan, reinterpret_cast<hipStream_t>(stream), X, Y, pos, B, static_cast<char*>(scratch),
                      static_cast<char*>(saved), loss, loss_pp, true);
}

rece_status set_last_error(rece_status st, const char* msg) { return fail(st, msg); }
}  // namespace rece

extern "C" {

rece_status rece_backward(rece_plan_t plan, void* stream, const void* X, const void* Y, const int32_t* pos,
                          const float* dloss, const float* dloss_pp, void* scratch, const void* saved, void* dX,
                          void* dY) {
  if (!plan) return fail(RECE_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!X || !Y || !pos || !scratch || !saved || !dX || !dY || (!dloss && !dloss_pp))
    return fail(RECE_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (!aligned16(X) || !aligned16(Y) || !aligned16(scratch) || !aligned16(saved) || !aligned16(dX) ||
      !aligned16(dY))
    return fail(RECE_ERR_INVALID_ARGUMENT, "X, Y, dX, dY, scratch and saved must be 16-byte aligned");
  const rece_plan_s& p = *plan;
  const rece_config& c = p.cfg;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const char* sv = static_cast<const char*>(saved);
  char* sc = static_cast<char*>(scratch);
  const int rounds = c.variant == RECE_VARIANT_SCE ? 1 : c.rounds;
  std::lock_guard<std::mutex> side_lock(p.side.mu);

  BwdArgs b{};
  b.X = X;
  b.Y = Y;
  b.pos = pos;
  b.s = c.s;
  b.C = c.C;
  b.rounds = rounds;
  b.k = c.k;
  b.negs = reinterpret_cast<const int32_t*>(sv + p.o_negs);
  b.lse = reinterpret_cast<const float*>(sv + p.o_lse);
  b.lpos = reinterpret_cast<const float*>(sv + p.o_lpos);
  b.dloss = dloss;
  b.dloss_pp = dloss_pp;
  b.wmean = reinterpret_cast<const float*>(sv + p.o_wmean);
  b.ignore = (c.flags & RECE_FLAG_IGNORE_NEGATIVE_POS) ? 1 : 0;
  b.grad_bf16 = (c.flags & RECE_FLAG_BF16_GRADS) ? 1 : 0;
  b.dX = dX;
  b.dY = dY;
  b.pcoef = reinterpret_cast<const float*>(sc + p.o_pcoef);
  RECE_PHASE(RECE_PHASE_OTHER, launch_pos_coef(b, reinterpret_cast<float*>(sc + p.o_pcoef), st),
             "per-position coefficients");
  // dY (the sort of the pairs by item, then the per-item sums) runs on the side
  // stream and dX on the caller's stream; the caller's stream then waits.  With
  // three or more sort passes (large catalogues) dX waits for the sort and runs
  // beside the per-item sums only: the sort's passes are short and latency-bound,
  // and the row gathers of dX slow them down (ten million items: 20.55 -> 20.25 ms
  // per step).  Two-pass sorts run beside dX (equal within noise at SASRec scale).
  const bool dx_after_sort = p.pg.npass >= 3;
  const rece_status ss = ensure_side(p, 2);
  if (ss != RECE_OK) return ss;
  hipStream_t side = p.side.s;
  RECE_HIP(hipEventRecord(p.side.fork[0], st), "fork");
  RECE_HIP(hipStreamWaitEvent(side, p.side.fork[0], 0), "fork");
  {
    hipStream_t st = side;
    const int32_t *K = nullptr, *V = nullptr;
    const uint32_t* ntot = nullptr;
    RECE_PHASE(RECE_PHASE_BWD_SORT,
               launch_pair_sort(p.pg, b.negs, (int64_t)rounds * c.s * c.k, c.k, c.s, pos, c.C, sc + p.o_psc,
                                reinterpret_cast<int32_t*>(sc + p.o_pk0), reinterpret_cast<int32_t*>(sc + p.o_pv0),
                                reinterpret_cast<int32_t*>(sc + p.o_pk1), reinterpret_cast<int32_t*>(sc + p.o_pv1), &K,
                                &V, &ntot, st),
               "sort pairs by item");
    if (dx_after_sort) RECE_HIP(hipEventRecord(p.side.fork[1], st), "sorted");
    RECE_PHASE(RECE_PHASE_BWD_DY, launch_dy(p.bf16, c.d, b, K, V, ntot, p.npairs, sc + p.o_dya, st), "dY");
  }
  if (dx_after_sort) RECE_HIP(hipStreamWaitEvent(st, p.side.fork[1], 0), "sorted");
  RECE_PHASE(RECE_PHASE_BWD_DX, launch_dx_lists(p.bf16, c.d, b, st), "dX");
  RECE_HIP(hipEventRecord(p.side.join, side), "join");
  RECE_HIP(hipStreamWaitEvent(st, p.side.join, 0), "join");
  return RECE_OK;
}

rece_status rece_export_bytes(rece_plan_t plan, int stage, size_t* bytes) {
  if (!plan || !bytes) return fail(RECE_ERR_INVALID_ARGUMENT, "NULL argument");
  const rece_config& c = plan->cfg;
  const bool sce = c.variant == RECE_VARIANT_SCE;
  const int rounds = sce ? 1 : c.rounds;
  switch (stage) {
    case RECE_STAGE_BUCKET_X:
    case RECE_STAGE_PERM_X:
      *bytes = sce ? 0 : (size_t)c.s * 4;
      break;
    case RECE_STAGE_THRESH_ID:
    case RECE_STAGE_LSE:
      *bytes = (size_t)c.s * 4;
      break;
    case RECE_STAGE_BUCKET_Y:
    case RECE_STAGE_PERM_Y:
      *bytes = sce ? 0 : (size_t)c.C * 4;
      break;
    case RECE_STAGE_SCE_ROWS:
      *bytes = sce ? (size_t)plan->sx * 4 : 0;
      break;
    case RECE_STAGE_SCE_ITEMS:
      *bytes = sce ? (size_t)plan->sy * 4 : 0;
      break;
    case RECE_STAGE_THRESH_LOGIT:
      *bytes = (size_t)c.s * 8;
      break;
    case RECE_STAGE_NEG_IDS:
      *bytes = (size_t)c.s * std::max(c.k, 1) * 4;
      break;
    case RECE_STAGE_UNION_IDS:
      *bytes = (size_t)c.s * rounds * std::max(c.k, 1) * 4;
      break;
    case RECE_STAGE_COUNTERS:
      *bytes = NUM_COUNTERS * 4;
      break;
    default:
      return fail(RECE_ERR_INVALID_ARGUMENT, "unknown stage");
  }
  return RECE_OK;
}

rece_status rece_export(rece_plan_t plan, void* stream, const void* saved, int stage, int round, void* dst) {
  if (!plan || !saved || !dst) return fail(RECE_ERR_INVALID_ARGUMENT, "NULL argument");
  const rece_plan_s& p = *plan;
  const rece_config& c = p.cfg;
  if (round < 0 || round >= c.rounds) return fail(RECE_ERR_INVALID_ARGUMENT, "round out of range");
  size_t bytes = 0;
  const rece_status bs = rece_export_bytes(plan, stage, &bytes);
  if (bs != RECE_OK) return bs;
  if (bytes == 0) return fail(RECE_ERR_INVALID_ARGUMENT, "stage not kept by this plan's variant");
  const char* sv = static_cast<const char*>(saved);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t s = c.s, C = c.C;
  const int kk = std::max(c.k, 1);
  size_t off = 0;
  switch (stage) {
    case RECE_STAGE_BUCKET_X: off = p.o_bx + (size_t)round * s * 4; break;
    case RECE_STAGE_BUCKET_Y: off = p.o_by + (size_t)round * C * 4; break;
    case RECE_STAGE_PERM_X: off = p.o_px + (size_t)round * s * 4; break;
    case RECE_STAGE_PERM_Y: off = p.o_py + (size_t)round * C * 4; break;
    case RECE_STAGE_THRESH_ID: off = p.o_tid + (size_t)round * s * 4; break;
    case RECE_STAGE_THRESH_LOGIT: off = p.o_te + (size_t)round * s * 8; break;
    case RECE_STAGE_NEG_IDS: off = p.o_negs + (size_t)round * s * kk * 4; break;
    case RECE_STAGE_UNION_IDS: off = p.o_negs; break;
    case RECE_STAGE_LSE: off = p.o_lse; break;
    case RECE_STAGE_COUNTERS: off = p.o_cnt; break;
    case RECE_STAGE_SCE_ROWS: off = p.o_R; break;
    case RECE_STAGE_SCE_ITEMS: off = p.o_Q; break;
    default: return fail(RECE_ERR_INVALID_ARGUMENT, "unknown stage");
  }
  if (stage == RECE_STAGE_NEG_IDS) {   // ids without the earlier-round mark
    if (c.k == 0) {
      RECE_HIP(launch_fill_u32(static_cast<uint32_t*>(dst), 0xFFFFFFFFu, (int64_t)(bytes / 4), st), "export");
      return RECE_OK;
    }
    RECE_HIP(launch_strip_mark(reinterpret_cast<const int32_t*>(sv + off), (int64_t)(bytes / 4),
                               static_cast<int32_t*>(dst), st),
             "export");
    return RECE_OK;
  }
  if (stage == RECE_STAGE_UNION_IDS) {
    const int rounds = c.variant == RECE_VARIANT_SCE ? 1 : c.rounds;
    if (c.k == 0) {
      RECE_HIP(launch_fill_u32(static_cast<uint32_t*>(dst), 0xFFFFFFFFu, (int64_t)(bytes / 4), st), "export");
      return RECE_OK;
    }
    RECE_HIP(launch_union_ids(reinterpret_cast<const int32_t*>(sv + off), s, c.k, rounds, static_cast<int32_t*>(dst),
                              st),
             "export");
    return RECE_OK;
  }
  RECE_HIP(hipMemcpyAsync(dst, sv + off, bytes, hipMemcpyDeviceToDevice, st), "export");
  return RECE_OK;
}

rece_status rece_check(rece_plan_t plan, void* stream, const void* saved) {
  if (!plan || !saved) return fail(RECE_ERR_INVALID_ARGUMENT, "NULL argument");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  RECE_HIP(hipStreamSynchronize(st), "stream synchronize");
  uint32_t cnt[NUM_COUNTERS];
  RECE_HIP(hipMemcpy(cnt, static_cast<const char*>(saved) + plan->o_cnt, sizeof(cnt), hipMemcpyDeviceToHost),
           "read counters");
  if (cnt[CNT_ERROR] & ERRBIT_BAD_ID) return fail(RECE_ERR_DEVICE_CHECK, "positive id out of range [0, C)");
  if (cnt[CNT_ERROR] & ERRBIT_OVERFLOW)
    return fail(RECE_ERR_DEVICE_CHECK, "candidate list overflow (too many near-equal logits at the k-th place)");
  return RECE_OK;
}

const char* rece_status_string(rece_status status) {
  switch (status) {
    case RECE_OK: return "ok";
    case RECE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case RECE_ERR_UNSUPPORTED: return "unsupported";
    case RECE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case RECE_ERR_HIP: return "HIP runtime error";
    case RECE_ERR_DEVICE_CHECK: return "device check failed";
    case RECE_ERR_INTERNAL: return "internal error";
  }
  return "unknown status";
}

const char* rece_last_error(void) { return g_last_error.c_str(); }

const char* rece_version(void) { return "librece 0.2 (gfx950)"; }

}  // extern "C"
