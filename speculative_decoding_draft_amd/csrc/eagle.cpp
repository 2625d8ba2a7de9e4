// Host side of the C interface in include/eagle.h: configuration checks,
// the weight table, carving of the caller's buffers, and the sequence of
// kernel launches for prefill, the draft passes and the verify pass.
#include "eagle.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <deque>
#include <string>
#include <vector>

#include "kernels.h"

namespace {

constexpr int KV_PAGE = 64;
constexpr uint64_t ALIGN = 256;

enum { ST_EMPTY = 0, ST_READY = 1, ST_DRAFTED = 2, ST_FAILED = 3 };

uint64_t align_up(uint64_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// ------------------------------------------------------------ derived shape
struct Derived {
  int H, nq, nkv, d, F, V, NL, dt, esz;
  int qkv_rows, kin_draft, fc_in;
  int k_b, k_e, D, budget, dynamic;
  int Mv, n_nodes_max, tree_rows_max;
  int B;           // sequences served together (eagle_config.batch)
  int chunk, Mmax, lane_rows;
  int t_slots, d_slots, t_pages, d_pages, max_pos, max_chunks;
  int rows_per_pass[EAGLE_MAX_DEPTH + 1];   // rows of draft pass p (p >= 2)
  // static plan
  int s_depth[EAGLE_MAX_STATIC], s_prow[EAGLE_MAX_STATIC];
  int s_nexp[EAGLE_MAX_DEPTH + 1];
  int s_exp[EAGLE_MAX_DEPTH + 1][TREE_MAXEXP];
};

bool fail(std::string* why, const char* fmt, ...) {
  if (why) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    *why = buf;
  }
  return false;
}

bool derive(const eagle_config* c, Derived* z, std::string* why) {
  if (!c) return fail(why, "config is NULL");
  std::memset(z, 0, sizeof(*z));
  if (c->dtype != EAGLE_F32 && c->dtype != EAGLE_BF16) return fail(why, "dtype must be EAGLE_F32 or EAGLE_BF16");
  if (c->head != EAGLE_HEAD_E1 && c->head != EAGLE_HEAD_E3) return fail(why, "head must be E1 or E3");
  if (c->n_layers < 1) return fail(why, "n_layers must be >= 1");
  if (c->hidden < 64 || c->hidden % 64 || c->hidden > 16384)
    return fail(why, "hidden must be a multiple of 64 in [64, 16384]");
  if (c->n_heads < 1 || c->hidden % c->n_heads) return fail(why, "n_heads must divide hidden");
  if (c->n_kv_heads < 1 || c->n_heads % c->n_kv_heads) return fail(why, "n_kv_heads must divide n_heads");
  const int d = c->hidden / c->n_heads;
  if (d % 2) return fail(why, "head_dim must be even");
  if (c->dtype == EAGLE_BF16 && d != 128) return fail(why, "bf16 path needs head_dim 128");
  if (c->dtype == EAGLE_F32 && d > 256) return fail(why, "fp32 path needs head_dim <= 256");
  if (1024 % d) return fail(why, "head_dim must divide 1024");
  const int kq = c->dtype == EAGLE_BF16 ? 32 : 16;
  if (c->ffn < kq || c->ffn % kq) return fail(why, "ffn must be a positive multiple of %d", kq);
  if (c->vocab < 2) return fail(why, "vocab must be >= 2");
  if (!(c->rope_base > 0.f) || !(c->rms_eps > 0.f)) return fail(why, "rope_base and rms_eps must be > 0");
  if (c->max_ctx < 2) return fail(why, "max_ctx must be >= 2");
  if (c->prefill_chunk < 0 || c->prefill_chunk > 1024) return fail(why, "prefill_chunk must be in [0, 1024]");
  if (!(c->temperature >= 0.f) || !(c->temperature <= 1e4f))
    return fail(why, "temperature must be in [0, 1e4] (0 = greedy)");
  if (c->temperature > 0.f && !sample_vocab_ok(c->vocab))
    return fail(why, "sampling supports vocab <= 131072");
  if (c->head == EAGLE_HEAD_E3)
    for (int i = 0; i < 3; ++i)
      if (c->feat_layers[i] < 0 || c->feat_layers[i] >= c->n_layers)
        return fail(why, "feat_layers[%d] out of range", i);
  if (c->topk < 1 || c->topk > EAGLE_MAX_TOPK) return fail(why, "topk must be in [1, %d]", EAGLE_MAX_TOPK);
  if (c->topk > c->vocab) return fail(why, "topk must be <= vocab");
  if (c->depth < 1 || c->depth > EAGLE_MAX_DEPTH) return fail(why, "depth must be in [1, %d]", EAGLE_MAX_DEPTH);
  static_assert(EAGLE_MAX_BATCH <= MAX_LANES, "a launch serves at most MAX_LANES sequences");
  if (c->batch < 0 || c->batch > EAGLE_MAX_BATCH) return fail(why, "batch must be in [0, %d] (0 = 1)", EAGLE_MAX_BATCH);
  z->B = c->batch > 0 ? c->batch : 1;

  z->H = c->hidden; z->nq = c->n_heads; z->nkv = c->n_kv_heads; z->d = d; z->F = c->ffn;
  z->V = c->vocab; z->NL = c->n_layers; z->dt = c->dtype; z->esz = c->dtype == EAGLE_BF16 ? 2 : 4;
  z->qkv_rows = (z->nq + 2 * z->nkv) * d;
  z->kin_draft = c->head == EAGLE_HEAD_E3 ? 2 * z->H : z->H;
  z->fc_in = c->head == EAGLE_HEAD_E3 ? 3 * z->H : 2 * z->H;
  z->k_b = c->topk; z->D = c->depth;
  z->dynamic = c->tree == EAGLE_TREE_DYNAMIC;
  if (c->tree == EAGLE_TREE_DYNAMIC) {
    z->k_e = c->expand > 0 ? c->expand : c->topk;
    if (z->k_e > TREE_MAXEXP) return fail(why, "expand must be <= %d", TREE_MAXEXP);
    if (c->budget < 0 || c->budget > EAGLE_MAX_VERIFY - 1)
      return fail(why, "budget must be in [0, %d]", EAGLE_MAX_VERIFY - 1);
    z->budget = c->budget;
    long nodes = z->k_b;
    int tree_rows = 0, width = z->k_b;
    for (int p = 2; p <= z->D; ++p) {
      const int rows = std::min(z->k_e, width);
      z->rows_per_pass[p] = rows;
      tree_rows += rows;
      nodes += (long)rows * z->k_b;
      width = rows * z->k_b;
    }
    if (nodes > EAGLE_MAX_NODES) return fail(why, "tree generates %ld nodes (> %d)", nodes, EAGLE_MAX_NODES);
    if (tree_rows > TREE_MAXROWS) return fail(why, "tree uses %d draft rows (> %d)", tree_rows, TREE_MAXROWS);
    z->n_nodes_max = (int)nodes;
    z->tree_rows_max = tree_rows;
    z->Mv = 1 + std::min<long>(z->budget, nodes);
    if (z->budget == 0) z->tree_rows_max = 0;
  } else if (c->tree == EAGLE_TREE_STATIC) {
    const int n = c->n_static;
    if (n < 1 || n > EAGLE_MAX_STATIC) return fail(why, "n_static must be in [1, %d]", EAGLE_MAX_STATIC);
    int maxd = 0;
    for (int j = 0; j < n; ++j) {
      const int p = c->static_parent[j], r = c->static_rank[j];
      if (p < -1 || p >= j) return fail(why, "static_parent[%d] must be -1 or an earlier node", j);
      if (r < 0 || r >= c->topk) return fail(why, "static_rank[%d] must be in [0, topk)", j);
      for (int i = 0; i < j; ++i)
        if (c->static_parent[i] == p && c->static_rank[i] == r) return fail(why, "static node %d duplicates node %d", j, i);
      z->s_depth[j] = p < 0 ? 1 : z->s_depth[p] + 1;
      if (j > 0 && z->s_depth[j] < z->s_depth[j - 1]) return fail(why, "static tree must be in breadth-first order");
      maxd = std::max(maxd, z->s_depth[j]);
    }
    if (maxd != z->D) return fail(why, "depth must equal the static tree's depth (%d)", maxd);
    int tree_rows = 0;
    for (int dd = 1; dd < z->D; ++dd) {
      int cnt = 0;
      for (int j = 0; j < n; ++j) {
        if (z->s_depth[j] != dd) continue;
        bool has = false;
        for (int i = j + 1; i < n; ++i) has |= c->static_parent[i] == j;
        if (has) {
          if (cnt >= TREE_MAXEXP) return fail(why, "static tree expands more than %d nodes per level", TREE_MAXEXP);
          z->s_exp[dd][cnt++] = j;
        }
      }
      z->s_nexp[dd] = cnt;
      z->rows_per_pass[dd + 1] = cnt;
      tree_rows += cnt;
    }
    for (int j = 0; j < n; ++j) {
      const int p = c->static_parent[j];
      z->s_prow[j] = 0;
      if (p >= 0)
        for (int i = 0; i < z->s_nexp[z->s_depth[p]]; ++i)
          if (z->s_exp[z->s_depth[p]][i] == p) z->s_prow[j] = i;
    }
    z->k_e = TREE_MAXEXP;
    z->budget = n;
    z->n_nodes_max = n;
    z->tree_rows_max = tree_rows;
    z->Mv = 1 + n;
  } else {
    return fail(why, "tree must be EAGLE_TREE_DYNAMIC or EAGLE_TREE_STATIC");
  }
  z->chunk = c->prefill_chunk > 0 ? c->prefill_chunk : 512;
  int pass_rows = 1;
  for (int p = 2; p <= z->D; ++p) pass_rows = std::max(pass_rows, z->rows_per_pass[p]);
  // one pass serves every sequence: B times the rows of one
  z->Mmax = std::max({z->chunk, z->B * z->Mv, z->B * (z->D + 1), z->B * pass_rows});
  z->lane_rows = std::max(z->chunk, z->D + 1);   // rows of a prefill chunk or a catch-up
  z->t_slots = c->max_ctx + z->Mv + 1;
  z->d_slots = c->max_ctx + 2 + z->tree_rows_max + z->D + 1;
  z->t_pages = (z->t_slots + KV_PAGE - 1) / KV_PAGE;
  z->d_pages = (z->d_slots + KV_PAGE - 1) / KV_PAGE;
  z->max_pos = std::max(z->t_slots, z->d_slots) + z->D + 2;
  const int ck = attn_chunk_keys();
  z->max_chunks = (std::max(z->t_pages, z->d_pages) * KV_PAGE + ck - 1) / ck + 1;
  if (z->max_chunks > attn_max_chunks()) return fail(why, "max_ctx too large for the attention combine (%d key chunks max)", attn_max_chunks());
  return true;
}

// ------------------------------------------------------------ weight table
std::vector<eagle_tensor> tensor_table(const eagle_config* c, const Derived& z) {
  std::vector<eagle_tensor> t;
  uint64_t off = 0;
  auto add = [&](int kind, int group, int layer, int dtype, int64_t rows, int64_t cols) {
    eagle_tensor e;
    e.kind = kind; e.group = group; e.layer = layer; e.dtype = dtype;
    e.rows = rows; e.cols = cols;
    e.offset = off;
    off = align_up(off + (uint64_t)rows * cols * (dtype == EAGLE_BF16 ? 2 : 4));
    t.push_back(e);
  };
  const int dt = c->dtype;
  add(EAGLE_T_EMBED, EAGLE_G_GLOBAL, 0, dt, z.V, z.H);
  add(EAGLE_T_LM_HEAD, EAGLE_G_GLOBAL, 0, dt, z.V, z.H);
  add(EAGLE_T_FINAL_NORM, EAGLE_G_GLOBAL, 0, EAGLE_F32, 1, z.H);
  auto layer = [&](int group, int l, int kin) {
    add(EAGLE_T_ATTN_NORM, group, l, EAGLE_F32, 1, kin);
    add(EAGLE_T_WQ, group, l, dt, (int64_t)z.nq * z.d, kin);
    add(EAGLE_T_WK, group, l, dt, (int64_t)z.nkv * z.d, kin);
    add(EAGLE_T_WV, group, l, dt, (int64_t)z.nkv * z.d, kin);
    add(EAGLE_T_WO, group, l, dt, z.H, (int64_t)z.nq * z.d);
    add(EAGLE_T_FFN_NORM, group, l, EAGLE_F32, 1, z.H);
    add(EAGLE_T_WGATE, group, l, dt, z.F, z.H);
    add(EAGLE_T_WUP, group, l, dt, z.F, z.H);
    add(EAGLE_T_WDOWN, group, l, dt, z.H, z.F);
  };
  for (int l = 0; l < z.NL; ++l) layer(EAGLE_G_TARGET, l, z.H);
  add(EAGLE_T_FC, EAGLE_G_GLOBAL, 0, dt, z.H, z.fc_in);
  layer(EAGLE_G_DRAFT, 0, z.kin_draft);
  return t;
}

uint64_t table_bytes(const std::vector<eagle_tensor>& t) {
  const eagle_tensor& e = t.back();
  return align_up(e.offset + (uint64_t)e.rows * e.cols * (e.dtype == EAGLE_BF16 ? 2 : 4));
}

// ------------------------------------------------------------ scratch plan
struct Carve {
  uint64_t off = 0;
  char* base = nullptr;
  template <typename T>
  T* take(uint64_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off = align_up(off + count * sizeof(T));
    return p;
  }
};

uint64_t gemm_ws_floats(const Derived& z) {
  // split-K partial planes: max over the projections and row counts of
  // splits * M * output width
  struct S { int rows, K; };
  const S shapes[] = {{z.qkv_rows, z.H}, {z.H, z.nq * z.d}, {z.H, z.F},
                      {z.qkv_rows, z.kin_draft}, {z.H, z.fc_in}};
  uint64_t mx = 0;
  for (const S& s : shapes)
    for (int M = 1; M <= z.Mmax; ++M) {
      GemmPlan p = gemm_plan(M, s.rows, s.K, z.dt, EPI_PART);
      mx = std::max(mx, gemm_part_floats(p, s.rows, M));
    }
  // SwiGLU over many rows: the gate|up partial planes (2F wide)
  for (int M = 1; M <= z.Mmax; ++M)
    if (swiglu_by_planes(z.dt, M)) {
      GemmPlan p = gemm_plan(M, 2 * z.F, z.H, z.dt, EPI_PART);
      mx = std::max(mx, gemm_part_floats(p, 2 * z.F, M));
    }
  return mx;
}

// One sequence of a batch: its host state and its device state (tree,
// acceptance result, committed tokens, per-row descriptors). The device
// arrays of every sequence share one layout, lane_bytes apart (see
// carve_lane), so one launch can serve all sequences.
struct Lane {
  TreeDev t;
  int32_t *acc, *new_tok, *cu_src, *seq;
  int32_t *rpos, *rslot, *rprehi;
  uint64_t* rmask;
  float* dout;   // draft outputs: row 0 = the root row, then each pass's rows
  // acceptance result in pinned, coherent host memory: [0] tag, [1] L,
  // [2 ..] committed tokens; written by the acceptance kernel through hres_dev
  int32_t* hres = nullptr;
  int32_t* hres_dev = nullptr;
  uint32_t step = 0;   // sampling draw step: 0 = the prefill's token, i = the i-th verify
  int state = ST_EMPTY;
  int ctx_len = 0;
  std::vector<int32_t> committed;
};
constexpr int HRES_INTS = 64;   // pinned result ints per sequence (one 256-byte line)
static_assert(HRES_INTS >= 2 + EAGLE_MAX_DEPTH + 2, "result block too small");

}  // namespace

// ------------------------------------------------------------ context
struct eagle_ctx {
  eagle_config cfg;
  Derived z;
  hipStream_t st = nullptr;
  int device = 0;
  char *W = nullptr, *KV = nullptr, *S = nullptr;
  struct LW {
    const float *attn_norm, *ffn_norm;
    const void *wqkv, *wo, *wgu, *wdown;
  };
  std::vector<LW> tl;
  LW dl;
  const void *embed, *lm, *fc;
  const float* final_norm;
  KVView tkv0, dkv;
  int64_t t_layer_elems = 0;
  // scratch
  float *cos_t, *sin_t;
  int32_t *tpt, *dpt;
  float *h, *tfeat, *gbuf, *hcat, *dout, *opart, *mlpart, *gpart, *hpart, *logits, *margin, *logp;
  int64_t dout_stride = 0;   // floats between two sequences' draft outputs
  float* rss;                // per-slice sums of squares of the sliced RMSNorm
  const float* xrs = nullptr;   // rss when xop holds RMSNorm numerators, else null
  float* ebuf;
  double* zpart;
  void *xop, *qop, *aop, *fop, *lmh, *lmh2;   // activation operands (two planes for bf16)
  int64_t xlo = 0, qlo = 0, alo = 0, flo = 0, lmhlo = 0, lmh2lo = 0;  // lo-plane offsets (elements)
  int32_t *g, *ids, *iota;
  TreeParams tp;
  std::vector<Lane> lanes;   // one per sequence (config batch)
  int64_t lane_bytes = 0;    // distance between two sequences' device state
  int32_t* hres = nullptr;   // pinned block of every sequence's result
  int32_t verify_tag = 0;
  bool debug = false;
  int last_target_rows = 0, last_verify_rows = 0;
  std::string err;
  // profiling (eagle_profile_enable)
  uint32_t prof = 0;   // class mask
  int prof_every = 1;  // bracket one launch in prof_every of each class
  int64_t prof_seen[EAGLE_PROF_CLASSES] = {};
  struct ProfRec { int cls; double bytes; hipEvent_t a, b; };
  std::deque<ProfRec> recs;            // recorded, not yet read back (oldest first)
  std::vector<hipEvent_t> free_ev;     // events ready for reuse
  std::vector<hipEvent_t> all_ev;      // every event created; destroyed with the context
  eagle_profile ptot{};                // totals of the records already read back
  ~eagle_ctx() {
    if (hres) (void)hipHostFree(hres);
  }
};

namespace {

#define TAKE(field, T, count)                      \
  do {                                             \
    T* p_ = cv.take<T>((uint64_t)(count));         \
    if (x) x->field = p_;                          \
  } while (0)

#define LTAKE(field, T, count)                     \
  do {                                             \
    T* p_ = cv.take<T>((uint64_t)(count));         \
    if (l) l->field = p_;                          \
  } while (0)

// The device state of one sequence, carved from `base` (NULL: sizing only).
// Every sequence's block has this layout, so sequence b's copy of an array
// sits b * lane_bytes after sequence 0's.
uint64_t carve_lane(const Derived& z, char* base, Lane* l) {
  Carve cv;
  cv.base = base;
  LTAKE(acc, int32_t, 2 + EAGLE_MAX_DEPTH + 2);
  LTAKE(new_tok, int32_t, EAGLE_MAX_DEPTH + 2);
  LTAKE(cu_src, int32_t, EAGLE_MAX_DEPTH + 2);
  LTAKE(seq, int32_t, (uint64_t)z.t_slots + z.D + 4);
  LTAKE(rpos, int32_t, z.lane_rows);
  LTAKE(rslot, int32_t, z.lane_rows);
  LTAKE(rprehi, int32_t, z.lane_rows);
  LTAKE(rmask, uint64_t, 2 * (uint64_t)z.lane_rows);
  LTAKE(t.tok, int32_t, TREE_MAXN);
  LTAKE(t.parent, int32_t, TREE_MAXN);
  LTAKE(t.depth, int32_t, TREE_MAXN);
  LTAKE(t.srcrow, int32_t, TREE_MAXN);
  LTAKE(t.rank, int32_t, TREE_MAXN);
  LTAKE(t.row_of_node, int32_t, TREE_MAXN);
  LTAKE(t.logv, float, TREE_MAXN);
  LTAKE(t.logp, float, TREE_MAXN);
  LTAKE(t.counts, int32_t, 8);
  LTAKE(t.exp_nodes, int32_t, TREE_MAXEXP);
  LTAKE(t.row_tok, int32_t, TREE_MAXEXP);
  LTAKE(t.row_src, int32_t, TREE_MAXEXP);
  LTAKE(t.row_pos, int32_t, TREE_MAXEXP);
  LTAKE(t.row_slot, int32_t, TREE_MAXEXP);
  LTAKE(t.row_prehi, int32_t, TREE_MAXEXP);
  LTAKE(t.row_mask, uint64_t, 2 * TREE_MAXEXP);
  LTAKE(t.tmask, uint64_t, 2 * TREE_MAXROWS);
  LTAKE(t.v_tok, int32_t, TREE_MAXROWS);
  LTAKE(t.v_parent, int32_t, TREE_MAXROWS);
  LTAKE(t.v_depth, int32_t, TREE_MAXROWS);
  LTAKE(t.v_node, int32_t, TREE_MAXROWS);
  LTAKE(t.v_pos, int32_t, TREE_MAXROWS);
  LTAKE(t.v_slot, int32_t, TREE_MAXROWS);
  LTAKE(t.v_prehi, int32_t, TREE_MAXROWS);
  LTAKE(t.v_logv, float, TREE_MAXROWS);
  LTAKE(t.v_mask, uint64_t, 2 * TREE_MAXROWS);
  LTAKE(t.s_parent, int32_t, EAGLE_MAX_STATIC);
  LTAKE(t.s_rank, int32_t, EAGLE_MAX_STATIC);
  LTAKE(t.s_depth, int32_t, EAGLE_MAX_STATIC);
  LTAKE(t.s_prow, int32_t, EAGLE_MAX_STATIC);
  LTAKE(t.s_exp, int32_t, (EAGLE_MAX_DEPTH + 1) * TREE_MAXEXP);
  LTAKE(t.s_nexp, int32_t, EAGLE_MAX_DEPTH + 1);
  return cv.off;
}
#undef LTAKE

uint64_t plan_scratch(const Derived& z, eagle_ctx* x) {
  Carve cv;
  cv.base = x ? x->S : nullptr;
  const int M = z.Mmax;
  const uint64_t B = z.B;
  const uint64_t kmax = std::max({z.H, z.fc_in, z.kin_draft, z.F, z.nq * z.d});
  const uint64_t es = z.esz;
  TAKE(cos_t, float, (uint64_t)z.max_pos * z.d / 2);
  TAKE(sin_t, float, (uint64_t)z.max_pos * z.d / 2);
  TAKE(tpt, int32_t, z.t_pages);
  TAKE(dpt, int32_t, z.d_pages);
  TAKE(h, float, (uint64_t)M * z.H);
  TAKE(tfeat, float, (uint64_t)M * z.H);
  TAKE(gbuf, float, (uint64_t)M * z.H);
  TAKE(hcat, float, (uint64_t)M * z.H);
  TAKE(dout, float, B * (1 + z.tree_rows_max) * z.H);
  TAKE(opart, float, (uint64_t)z.max_chunks * M * z.nq * z.d);
  TAKE(mlpart, float, (uint64_t)z.max_chunks * M * z.nq * 2);
  TAKE(gpart, float, gemm_ws_floats(z));
  TAKE(rss, float, (uint64_t)M * RS_SLICES);
  // LM-head partials: the largest need over every row count a call can take
  // (calls above 80 rows run in 64-row passes)
  uint64_t hp = 0;
  for (int m = 1; m <= (int)B * std::max(z.Mv, TREE_MAXEXP); ++m)
    hp = std::max(hp, lmhead_part_floats(m, z.V, z.k_b));
  TAKE(hpart, float, hp);
  TAKE(logits, float, B * z.Mv * z.V);
  TAKE(ebuf, float, B * z.Mv * z.V);                              // sampling: exp((l - max) / T)
  TAKE(zpart, double, sample_zpart_doubles((int)B * z.Mv, z.V));  // sampling: block sums of e
  TAKE(margin, float, B * z.Mv);
  TAKE(logp, float, B * TREE_MAXEXP * EAGLE_MAX_TOPK);
  TAKE(xop, char, 2 * (uint64_t)M * kmax * es);
  TAKE(qop, char, 2 * (uint64_t)M * z.nq * z.d * es);
  TAKE(aop, char, 2 * (uint64_t)M * z.nq * z.d * es);
  TAKE(fop, char, 2 * (uint64_t)M * z.F * es);
  TAKE(lmh, char, 2 * (uint64_t)M * 3 * z.H * es);
  TAKE(lmh2, char, 2 * B * (z.D + 1) * 3 * z.H * es);
  if (x) {
    x->xlo = (int64_t)M * kmax;
    x->qlo = x->alo = (int64_t)M * z.nq * z.d;
    x->flo = (int64_t)M * z.F;
    x->lmhlo = (int64_t)M * 3 * z.H;
    x->lmh2lo = (int64_t)B * (z.D + 1) * 3 * z.H;
    x->dout_stride = (int64_t)(1 + z.tree_rows_max) * z.H;
  }
  TAKE(g, int32_t, B * z.Mv);
  TAKE(ids, int32_t, B * TREE_MAXEXP * EAGLE_MAX_TOPK);
  TAKE(iota, int32_t, M);
  // per-sequence state
  const uint64_t lb = carve_lane(z, nullptr, nullptr);
  char* l0 = cv.take<char>(B * lb);
  if (x) {
    x->lane_bytes = (int64_t)lb;
    x->lanes.assign(B, Lane());
    for (uint64_t b = 0; b < B; ++b) carve_lane(z, l0 + b * lb, &x->lanes[b]);
    for (uint64_t b = 0; b < B; ++b) x->lanes[b].dout = x->dout + b * x->dout_stride;
  }
  // eagle_load stages weight blocks of 16 rows through scratch when it
  // packs bf16 matrices: keep room for at least one block of the widest.
  return std::max<uint64_t>(cv.off, 16 * kmax * es);
}
#undef TAKE

// Target cache [layer][sequence][page], then draft cache [sequence][page].
uint64_t kv_bytes_of(const Derived& z) {
  const uint64_t page_elems = (uint64_t)kv_planes(z.dt) * z.nkv * KV_PAGE * z.d;
  return align_up((uint64_t)z.NL * z.B * z.t_pages * page_elems * z.esz) +
         align_up((uint64_t)z.B * z.d_pages * page_elems * z.esz);
}

eagle_status set_err(eagle_ctx* c, eagle_status s, const char* fmt, ...) {
  if (c) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    c->err = buf;
    if (s == EAGLE_E_HIP || s == EAGLE_E_DEVICE)
      for (Lane& l : c->lanes) l.state = ST_FAILED;
  }
  return s;
}

#define HCHK(expr)                                                                      \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess)                                                               \
      return set_err(c, EAGLE_E_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));    \
  } while (0)

#define SCHK(expr)                       \
  do {                                   \
    eagle_status s_ = (expr);            \
    if (s_ != EAGLE_OK) return s_;       \
  } while (0)

// Moves finished records into the totals and their events back to the free
// list; with wait, first waits for every recorded event.
void prof_settle(eagle_ctx* c, bool wait) {
  while (!c->recs.empty()) {
    const eagle_ctx::ProfRec r = c->recs.front();
    if (wait) {
      if (hipEventSynchronize(r.b) != hipSuccess) break;
    } else if (hipEventQuery(r.b) != hipSuccess) {
      break;
    }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      c->ptot.launches[r.cls]++;
      c->ptot.ms[r.cls] += ms;
      c->ptot.bytes[r.cls] += r.bytes;
    }
    c->free_ev.push_back(r.a);
    c->free_ev.push_back(r.b);
    c->recs.pop_front();
  }
}

// An event for a profile record: reused once its record has been read back,
// so the number of events stays near the number of launches in flight.
hipEvent_t take_event(eagle_ctx* c) {
  if (c->free_ev.empty()) prof_settle(c, false);
  if (c->free_ev.empty()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    c->all_ev.push_back(e);
    return e;
  }
  hipEvent_t e = c->free_ev.back();
  c->free_ev.pop_back();
  return e;
}

// Whether this launch of class cls is bracketed (class enabled, and the
// launch falls on the sampling stride).
bool prof_pick(eagle_ctx* c, int cls) {
  if (!((c->prof >> cls) & 1u)) return false;
  return c->prof_seen[cls]++ % c->prof_every == 0;
}

// Brackets the launches of its scope with events when profiling is on.
struct Prof {
  eagle_ctx* c;
  int cls;
  double bytes;
  hipEvent_t a = nullptr;
  Prof(eagle_ctx* c_, int cls_, double bytes_) : c(c_), cls(cls_), bytes(bytes_) {
    if (prof_pick(c, cls) && (a = take_event(c))) (void)hipEventRecord(a, c->st);
  }
  ~Prof() {
    if (!a) return;
    hipEvent_t b = take_event(c);
    if (!b) return;
    (void)hipEventRecord(b, c->st);
    c->recs.push_back({cls, bytes, a, b});
  }
};

#define PROFILED(cls, bytes, expr)        \
  do {                                    \
    Prof p_(c, (cls), (double)(bytes));   \
    HCHK(expr);                           \
  } while (0)

// Events for a class that is one kernel dispatch: they are handed to the
// launch (tm_), which attaches them to the dispatch packet, so no extra
// packets enter the stream and the interval is the kernel's own.
const KTiming* prof_kernel(eagle_ctx* c, int cls, double bytes, KTiming* t) {
  if (!prof_pick(c, cls)) return nullptr;
  t->start = take_event(c);
  t->stop = take_event(c);
  if (!t->start || !t->stop) return nullptr;
  c->recs.push_back({cls, bytes, t->start, t->stop});
  return t;
}

#define PROFILED_KERNEL(cls, bytes, expr)                                   \
  do {                                                                      \
    KTiming t_;                                                             \
    const KTiming* tm_ = prof_kernel(c, (cls), (double)(bytes), &t_);       \
    HCHK(expr);                                                             \
  } while (0)

// Algorithmic bytes: each weight byte once, activation operands (two bf16
// planes or fp32), outputs (read and written for residual updates).
double opnd_bytes(const Derived&) { return 4.0; }   // fp32 or bf16 hi + lo
double gemm_bytes(const Derived& z, int M, int rows, int K, int n_out, int epi) {
  const double w = (double)rows * K * z.esz;
  const double x = (double)M * K * opnd_bytes(z);
  const double y = (double)M * n_out * 4.0;
  return w + x + y;
}
double attn_bytes(const Derived& z, int M, const RowVis& v, const Lanes& ln) {
  double keys = 0.0;
  for (int b = 0; b < ln.n; ++b) keys += (double)(v.key_end + ln.off[b] - v.pre_lo);
  return keys * z.nkv * z.d * 2.0 * 4.0 + 2.0 * M * z.nq * z.d * 4.0;   // K,V: fp32 or hi + lo
}

// ------------------------------------------------------------ sequences
// The sequences one pass serves: lanes [first, first + n), `rows` rows each,
// sequence by sequence.
struct Span {
  int first, n, rows;
  int M() const { return n * rows; }
};

// Per-launch description of a span for the kernels that serve several
// sequences: row split, per-row input stride and each sequence's key shift
// relative to the first (their context lengths differ).
Lanes lanes_of(const eagle_ctx* c, Span s) {
  Lanes ln;
  ln.n = s.n;
  ln.rows = s.rows;
  ln.bytes = c->lane_bytes;
  for (int b = 0; b < s.n; ++b)
    ln.off[b] = c->lanes[s.first + b].ctx_len - c->lanes[s.first].ctx_len;
  return ln;
}

// A cache view that starts at sequence `b`.
KVView lane_view(KVView v, int b, int esz) {
  v.base = (char*)v.base + (int64_t)b * v.lane_elems * esz;
  return v;
}

// ------------------------------------------------------------ passes
// Applies the pending split-K partial planes of a projection to the
// residual stream h (or sets h to their sum) and writes the next operand:
// RMSNorm(h) * gain, or h itself when gain is null.
// bf16 rows without an fp32 copy of the result take the sliced form: the
// operand is then gain * h and xrs points at the sums of squares, which the
// projection that reads xop next (q|k|v or gate|up) turns into each row's
// RMSNorm factor (RowScale).
eagle_status resnorm(eagle_ctx* c, float* h, int M, int S, bool set, const float* gain,
                     float* out_f) {
  const Derived& z = c->z;
  if (z.dt == 1 && !out_f && resnorm_slices_fit(z.H)) {
    PROFILED(EAGLE_PROF_ROWS, (double)M * z.H * (12.0 + 4.0 * S),
             launch_resnorm_slices(z.dt, h, z.H, M, c->gpart, S, (int64_t)M * z.H, set ? 1 : 0,
                                   gain, c->xop, c->xlo, c->rss, c->st));
    c->xrs = gain ? c->rss : nullptr;
    return EAGLE_OK;
  }
  PROFILED(EAGLE_PROF_ROWS, (double)M * z.H * (12.0 + 4.0 * S),
           launch_resnorm(z.dt, h, z.H, M, c->gpart, S, (int64_t)M * z.H, set ? 1 : 0, gain,
                          c->cfg.rms_eps, c->xop, c->xlo, out_f, c->st));
  c->xrs = nullptr;
  return EAGLE_OK;
}

// The RowScale of a projection whose operand is xop.
RowScale xop_scale(const eagle_ctx* c) {
  RowScale r;
  r.ss = c->xrs;
  r.H = c->z.H;
  r.eps = c->cfg.rms_eps;
  return r;
}

// One decoder layer over M rows (the rows of every sequence of `ln`). On
// entry xop holds the normed layer input (row width kin), or its RMSNorm
// numerator with xrs set (the q|k|v projection then applies the factor); on
// exit the down-projection partials are pending in gpart (*s_down planes)
// for the caller's resnorm.
eagle_status layer_core(eagle_ctx* c, const eagle_ctx::LW& w, int kin, int M, float* h,
                        const int32_t* pos, const int32_t* slot, KVView kv, RowVis vis,
                        const Lanes& ln, bool target, int* s_down) {
  const Derived& z = c->z;
  const int dt = z.dt;
  const int cls_part = target ? EAGLE_PROF_GEMM : EAGLE_PROF_DRAFT;
  const int cls_glu = target ? EAGLE_PROF_SWIGLU : EAGLE_PROF_DRAFT;
  int S = 1;
  PROFILED_KERNEL(cls_part, gemm_bytes(z, M, z.qkv_rows, kin, z.qkv_rows, EPI_PART),
           launch_gemm(dt, EPI_PART, w.wqkv, c->xop, c->xlo, M, z.qkv_rows, kin, c->gpart,
                       z.qkv_rows, nullptr, 0, &S, c->st, tm_, xop_scale(c)));
  PROFILED(EAGLE_PROF_ROWS, (double)M * z.qkv_rows * 4.0 * (S + 1),
           launch_rope_kv(dt, c->gpart, S, (int64_t)M * z.qkv_rows, M, z.nq, z.nkv, z.d, pos, slot,
                          c->cos_t, c->sin_t, c->qop, c->qlo, kv, c->st, ln));
  PROFILED(EAGLE_PROF_ATTN, attn_bytes(z, M, vis, ln),
           launch_attention(dt, c->qop, c->qlo, kv, vis, M, z.nq, z.d,
                            1.0f / std::sqrt((float)z.d), c->opart, c->mlpart, c->aop, c->alo,
                            c->st, ln));
  PROFILED_KERNEL(cls_part, gemm_bytes(z, M, z.H, z.nq * z.d, z.H, EPI_PART),
           launch_gemm(dt, EPI_PART, w.wo, c->aop, c->alo, M, z.H, z.nq * z.d, c->gpart, z.H,
                       nullptr, 0, &S, c->st, tm_));
  SCHK(resnorm(c, h, M, S, false, w.ffn_norm, nullptr));
  PROFILED_KERNEL(cls_glu, gemm_bytes(z, M, 2 * z.F, z.H, z.F, EPI_SWIGLU),
           launch_gemm(dt, EPI_SWIGLU, w.wgu, c->xop, c->xlo, M, z.F, z.H, c->gpart, 2 * z.F,
                       c->fop, c->flo, nullptr, c->st, tm_, xop_scale(c)));
  PROFILED_KERNEL(cls_part, gemm_bytes(z, M, z.H, z.F, z.H, EPI_PART),
           launch_gemm(dt, EPI_PART, w.wdown, c->fop, c->flo, M, z.H, z.F, c->gpart, z.H, nullptr,
                       0, s_down, c->st, tm_));
  return EAGLE_OK;
}

// Target forward over the rows of span s; leaves f in tfeat and its operand
// in xop. tok, pos, slot and vis's per-row arrays are the first sequence's.
eagle_status target_pass(eagle_ctx* c, Span s, const int32_t* tok, const int32_t* pos,
                         const int32_t* slot, RowVis vis) {
  const Derived& z = c->z;
  const int M = s.M();
  const Lanes ln = lanes_of(c, s);
  PROFILED(EAGLE_PROF_ROWS, (double)M * z.H * 4.0,
           launch_embed(z.dt, c->embed, z.H, tok, M, c->h, c->st, ln));
  SCHK(resnorm(c, c->h, M, 0, false, c->tl[0].attn_norm, nullptr));
  for (int l = 0; l < z.NL; ++l) {
    KVView kv = c->tkv0;
    kv.base = (char*)c->tkv0.base + (int64_t)l * c->t_layer_elems * z.esz;
    kv = lane_view(kv, s.first, z.esz);
    int sd = 1;
    SCHK(layer_core(c, c->tl[l], z.H, M, c->h, pos, slot, kv, vis, ln, true, &sd));
    const bool last = l + 1 == z.NL;
    SCHK(resnorm(c, c->h, M, sd, false, last ? c->final_norm : c->tl[l + 1].attn_norm,
                 last ? c->tfeat : nullptr));
    if (c->cfg.head == EAGLE_HEAD_E3)
      for (int j = 0; j < 3; ++j)
        if (c->cfg.feat_layers[j] == l)
          PROFILED(EAGLE_PROF_ROWS, (double)M * z.H * 8.0,
                   launch_store_feat(z.dt, c->h, z.H, M, (char*)c->lmh + (int64_t)j * z.H * z.esz,
                                     3 * z.H, c->lmhlo, c->st));
  }
  c->last_target_rows = M;
  return EAGLE_OK;
}

// Draft rows of span s -> residual stream hout (M rows); leaves the LM-head
// operand of every row in xop. Row r of sequence b pairs token tok_b[r] with
// the feature row idx_b[r] of feat + b * feat_stride, where tok_b, idx_b are
// sequence b's copies (idx: idx_bytes apart; 0 = one shared index array).
eagle_status draft_pass(eagle_ctx* c, Span s, const int32_t* tok, const float* feat,
                        int64_t feat_stride, const int32_t* idx, int64_t idx_bytes,
                        const int32_t* pos, const int32_t* slot, RowVis vis, float* hout) {
  const Derived& z = c->z;
  const int M = s.M();
  const Lanes ln = lanes_of(c, s);
  if (c->cfg.head == EAGLE_HEAD_E1) {
    int S = 1;
    PROFILED(EAGLE_PROF_ROWS, (double)M * z.H * 12.0,
             launch_draft_input_e1(z.dt, c->embed, tok, feat, idx, M, z.H, c->xop, c->xlo, c->st,
                                   ln, feat_stride, idx_bytes));
    c->xrs = nullptr;   // [E[t]; f] feeds the FC unscaled
    PROFILED_KERNEL(EAGLE_PROF_DRAFT, gemm_bytes(z, M, z.H, 2 * z.H, z.H, EPI_PART),
             launch_gemm(z.dt, EPI_PART, c->fc, c->xop, c->xlo, M, z.H, 2 * z.H, c->gpart, z.H,
                         nullptr, 0, &S, c->st, tm_));
    SCHK(resnorm(c, hout, M, S, true, c->dl.attn_norm, nullptr));
  } else {
    PROFILED(EAGLE_PROF_ROWS, (double)M * z.H * 16.0,
             launch_draft_input_e3(z.dt, c->embed, tok, feat, idx, c->dl.attn_norm, c->cfg.rms_eps,
                                   M, z.H, c->xop, c->xlo, hout, c->st, ln, feat_stride,
                                   idx_bytes));
    c->xrs = nullptr;   // that operand is normalized
  }
  int sd = 1;
  SCHK(layer_core(c, c->dl, z.kin_draft, M, hout, pos, slot, lane_view(c->dkv, s.first, z.esz),
                  vis, ln, false, &sd));
  SCHK(resnorm(c, hout, M, sd, false, nullptr, nullptr));
  return EAGLE_OK;
}

// Draft catch-up of sequence b over M committed pairs at positions
// first..first+M-1; the features are feat[idx[r]] (true target features,
// EAGLE-3: fused). If final, the last row becomes the root row: its top-k
// are the depth-1 nodes.
eagle_status catch_up(eagle_ctx* c, int b, int M, int first, const int32_t* tok, const float* feat,
                      const int32_t* idx, bool final, int ctx_after) {
  const Derived& z = c->z;
  Lane& q = c->lanes[b];
  HCHK(launch_rows_causal(first, M, q.rpos, q.rslot, q.rprehi, q.rmask, c->st));
  RowVis vis{q.rprehi, q.rmask, 1, 0, 0, first + M};
  SCHK(draft_pass(c, Span{b, 1, M}, tok, feat, 0, idx, 0, q.rpos, q.rslot, vis, c->hcat));
  if (!final) return EAGLE_OK;
  HCHK(hipMemcpyAsync(q.dout, c->hcat + (int64_t)(M - 1) * z.H, sizeof(float) * z.H,
                      hipMemcpyDeviceToDevice, c->st));
  const void* xl = (const char*)c->xop + (int64_t)(M - 1) * z.H * z.esz;
  PROFILED(EAGLE_PROF_LMHEAD, (double)z.V * z.H * z.esz + (double)z.H * 4.0,
           launch_lmhead_topk(z.dt, c->lm, xl, c->xlo, 1, z.V, z.H, z.k_b, c->hpart, c->ids,
                              c->logp, c->st));
  PROFILED(EAGLE_PROF_TREE, 0.0, launch_tree_append(q.t, c->tp, c->ids, c->logp, 1, ctx_after, c->st));
  return EAGLE_OK;
}

// The verify's catch-up, for every sequence, before the acceptance lengths
// are known on the host: all depth + 1 rows after each root are drafted
// (rows past the committed ones read the filler the acceptance kernel wrote
// and only touch draft KV slots that the next cycle overwrites before
// reading; every row attends causally, so the committed rows are exactly
// what a catch-up over them alone computes). Sequence b's new root row is
// its row L = acc[0], picked on the device for the LM head, and its tree is
// restarted at position ctx + L + 1. Features: feat + b * feat_stride,
// rows idx_b[r] (idx_bytes apart per sequence).
eagle_status catch_up_fixed(eagle_ctx* c, const float* feat, int64_t feat_stride,
                            const int32_t* idx, int64_t idx_bytes) {
  const Derived& z = c->z;
  const int M1 = z.D + 1, B = z.B;
  const Lane& q0 = c->lanes[0];
  const Lanes ln = lanes_of(c, Span{0, B, M1});
  HCHK(launch_rows_causal(q0.ctx_len + 1, M1, q0.rpos, q0.rslot, q0.rprehi, q0.rmask, c->st, ln));
  RowVis vis{q0.rprehi, q0.rmask, 1, 0, 0, q0.ctx_len + 1 + M1};
  SCHK(draft_pass(c, Span{0, B, M1}, q0.new_tok, feat, feat_stride, idx, idx_bytes, q0.rpos,
                  q0.rslot, vis, c->hcat));
  // each sequence's root row: its draft output to dout row 0 and its LM-head
  // operand to row b of the (now free) q operand buffer
  PROFILED(EAGLE_PROF_ROWS, (double)B * z.H * 16.0,
           launch_gather_roots(z.dt, c->hcat, c->xop, c->xlo, M1, q0.acc, z.H, q0.dout,
                               c->dout_stride, c->qop, c->qlo, ln, c->st));
  PROFILED(EAGLE_PROF_LMHEAD, (double)z.V * z.H * z.esz + (double)B * z.H * 4.0,
           launch_lmhead_topk(z.dt, c->lm, c->qop, c->qlo, B, z.V, z.H, z.k_b, c->hpart, c->ids,
                              c->logp, c->st));
  PROFILED(EAGLE_PROF_TREE, 0.0,
           launch_tree_append(q0.t, c->tp, c->ids, c->logp, 1, q0.ctx_len, c->st, q0.acc, ln,
                              z.k_b));
  return EAGLE_OK;
}

// E3: g = FC([l;m;h]) for M committed rows whose [l;m;h] operands are at src.
eagle_status fuse_rows(eagle_ctx* c, int M, const void* src, int64_t src_lo) {
  const Derived& z = c->z;
  int S = 1;
  PROFILED_KERNEL(EAGLE_PROF_DRAFT, gemm_bytes(z, M, z.H, 3 * z.H, z.H, EPI_PART),
           launch_gemm(z.dt, EPI_PART, c->fc, src, src_lo, M, z.H, 3 * z.H, c->gpart, z.H, nullptr,
                       0, &S, c->st, tm_));
  PROFILED(EAGLE_PROF_ROWS, (double)M * z.H * 4.0 * (S + 1),
           launch_sum_planes(c->gpart, S, (int64_t)M * z.H, M, z.H, c->gbuf, 0, c->st));
  return EAGLE_OK;
}

eagle_status check_ready(eagle_ctx* c) {
  if (!c) return EAGLE_E_INVALID;
  for (const Lane& l : c->lanes)
    if (l.state == ST_FAILED) return set_err(c, EAGLE_E_STATE, "context failed earlier; call eagle_prefill");
  return EAGLE_OK;
}

bool plain_mode(const eagle_ctx* c) { return c->z.dynamic && c->z.budget == 0; }
bool sampling(const eagle_ctx* c) { return c->cfg.temperature > 0.f; }
uint64_t seed_of(const eagle_ctx* c) { return ((uint64_t)c->cfg.seed_hi << 32) | c->cfg.seed_lo; }

}  // namespace

// ============================================================ C interface
extern "C" {

const char* eagle_status_string(eagle_status s) {
  switch (s) {
    case EAGLE_OK: return "ok";
    case EAGLE_E_INVALID: return "invalid argument";
    case EAGLE_E_STATE: return "wrong state";
    case EAGLE_E_CAPACITY: return "capacity exceeded";
    case EAGLE_E_BUFFER: return "buffer missing or too small";
    case EAGLE_E_HIP: return "HIP error";
    case EAGLE_E_DEVICE: return "device check failed";
  }
  return "unknown status";
}

eagle_status eagle_query(const eagle_config* cfg, eagle_sizes* out) {
  Derived z;
  if (!out) return EAGLE_E_INVALID;
  if (!derive(cfg, &z, nullptr)) return EAGLE_E_INVALID;
  std::vector<eagle_tensor> t = tensor_table(cfg, z);
  out->weight_bytes = table_bytes(t);
  out->kv_bytes = kv_bytes_of(z);
  out->scratch_bytes = plan_scratch(z, nullptr);
  out->n_tensors = (int32_t)t.size();
  out->verify_rows = z.Mv;
  out->max_nodes = z.n_nodes_max;
  out->kv_page = KV_PAGE;
  out->ctx_headroom = z.D;
  return EAGLE_OK;
}

eagle_status eagle_tensor_info(const eagle_config* cfg, int32_t index, eagle_tensor* out) {
  Derived z;
  if (!out || !derive(cfg, &z, nullptr)) return EAGLE_E_INVALID;
  std::vector<eagle_tensor> t = tensor_table(cfg, z);
  if (index < 0 || index >= (int32_t)t.size()) return EAGLE_E_INVALID;
  *out = t[index];
  return EAGLE_OK;
}

eagle_status eagle_load(const eagle_config* cfg, const eagle_buffers* bufs, void* hip_stream,
                        eagle_ctx** out) {
  if (!out) return EAGLE_E_INVALID;
  *out = nullptr;
  Derived z;
  std::string why;
  if (!derive(cfg, &z, &why)) return EAGLE_E_INVALID;
  if (!bufs || !bufs->weights || !bufs->kv || !bufs->scratch) return EAGLE_E_BUFFER;
  std::vector<eagle_tensor> tab = tensor_table(cfg, z);
  if (bufs->weight_bytes < table_bytes(tab) || bufs->kv_bytes < kv_bytes_of(z) ||
      bufs->scratch_bytes < plan_scratch(z, nullptr))
    return EAGLE_E_BUFFER;
  eagle_ctx* c = new eagle_ctx();
  c->cfg = *cfg;
  c->z = z;
  c->st = (hipStream_t)hip_stream;
  c->W = (char*)bufs->weights;
  c->KV = (char*)bufs->kv;
  c->S = (char*)bufs->scratch;
  int32_t* hres_dev = nullptr;
  const size_t hres_bytes = sizeof(int32_t) * HRES_INTS * z.B;
  if (hipGetDevice(&c->device) != hipSuccess ||
      hipHostMalloc((void**)&c->hres, hres_bytes, hipHostMallocMapped | hipHostMallocCoherent) !=
          hipSuccess ||
      hipHostGetDevicePointer((void**)&hres_dev, c->hres, 0) != hipSuccess) {
    delete c;
    return EAGLE_E_HIP;
  }
  std::memset(c->hres, 0, hres_bytes);
  // weights
  auto ptr = [&](int kind, int group, int layer) -> const void* {
    for (const eagle_tensor& e : tab)
      if (e.kind == kind && e.group == group && e.layer == layer) return c->W + e.offset;
    return nullptr;
  };
  c->embed = ptr(EAGLE_T_EMBED, EAGLE_G_GLOBAL, 0);
  c->lm = ptr(EAGLE_T_LM_HEAD, EAGLE_G_GLOBAL, 0);
  c->final_norm = (const float*)ptr(EAGLE_T_FINAL_NORM, EAGLE_G_GLOBAL, 0);
  c->fc = ptr(EAGLE_T_FC, EAGLE_G_GLOBAL, 0);
  auto lw = [&](int group, int l) {
    eagle_ctx::LW w;
    w.attn_norm = (const float*)ptr(EAGLE_T_ATTN_NORM, group, l);
    w.ffn_norm = (const float*)ptr(EAGLE_T_FFN_NORM, group, l);
    w.wqkv = ptr(EAGLE_T_WQ, group, l);   // WQ | WK | WV are contiguous
    w.wo = ptr(EAGLE_T_WO, group, l);
    w.wgu = ptr(EAGLE_T_WGATE, group, l); // WGATE | WUP are contiguous
    w.wdown = ptr(EAGLE_T_WDOWN, group, l);
    return w;
  };
  for (int l = 0; l < z.NL; ++l) c->tl.push_back(lw(EAGLE_G_TARGET, l));
  c->dl = lw(EAGLE_G_DRAFT, 0);
  // KV views
  // KV views: each sequence has its own pages (the page tables are shared)
  const int64_t page_elems = (int64_t)kv_planes(z.dt) * z.nkv * KV_PAGE * z.d;
  c->t_layer_elems = (int64_t)z.B * z.t_pages * page_elems;
  plan_scratch(z, c);
  for (int b = 0; b < z.B; ++b) {
    c->lanes[b].hres = c->hres + HRES_INTS * b;
    c->lanes[b].hres_dev = hres_dev + HRES_INTS * b;
  }
  c->tkv0 = KVView{c->KV, c->tpt, page_elems, KV_PAGE, z.nkv, z.d, (int64_t)z.t_pages * page_elems};
  c->dkv = KVView{c->KV + align_up((uint64_t)z.NL * c->t_layer_elems * z.esz), c->dpt, page_elems,
                  KV_PAGE, z.nkv, z.d, (int64_t)z.d_pages * page_elems};
  // bf16 matrices the GEMM and LM-head kernels stream are fragment-packed in
  // place, a batch of 16-row blocks at a time through the (still unused)
  // scratch buffer; the embedding stays row-major (rows are gathered).
  if (z.dt == 1) {
    hipError_t e = hipSuccess;
    for (const eagle_tensor& t : tab) {
      if (t.dtype != EAGLE_BF16 || t.kind == EAGLE_T_EMBED || t.rows < 16) continue;
      const uint64_t blk = 16ull * (uint64_t)t.cols * 2;
      const int64_t nrb = t.rows / 16;
      const int64_t per = (int64_t)(bufs->scratch_bytes / blk);
      if (per < 1 || t.cols % 32) {
        delete c;
        return EAGLE_E_BUFFER;
      }
      for (int64_t b0 = 0; b0 < nrb && e == hipSuccess; b0 += per) {
        const int64_t nb = std::min(per, nrb - b0);
        char* p = c->W + t.offset + (uint64_t)b0 * blk;
        e = hipMemcpyAsync(c->S, p, (size_t)nb * blk, hipMemcpyDeviceToDevice, c->st);
        if (e == hipSuccess) e = launch_pack_frag(c->S, p, nb, (int)t.cols, c->st);
      }
    }
    if (e == hipSuccess) e = hipStreamSynchronize(c->st);
    if (e != hipSuccess) {
      delete c;
      return EAGLE_E_HIP;
    }
  }
  c->tp = TreeParams{z.dynamic, z.k_b, z.k_e, z.D, z.budget, cfg->tree == EAGLE_TREE_STATIC ? cfg->n_static : 0};
  // host-built tables: RoPE, page tables (identity), iota, static plan
  {
    const int half = z.d / 2;
    std::vector<float> cs((size_t)z.max_pos * half), sn((size_t)z.max_pos * half);
    for (int p = 0; p < z.max_pos; ++p)
      for (int i = 0; i < half; ++i) {
        const double theta = std::pow((double)cfg->rope_base, -2.0 * i / z.d);
        const double ang = (double)p * theta;
        cs[(size_t)p * half + i] = (float)std::cos(ang);
        sn[(size_t)p * half + i] = (float)std::sin(ang);
      }
    std::vector<int32_t> tp(z.t_pages), dp(z.d_pages), io(z.Mmax);
    for (int i = 0; i < z.t_pages; ++i) tp[i] = i;
    for (int i = 0; i < z.d_pages; ++i) dp[i] = i;
    for (int i = 0; i < z.Mmax; ++i) io[i] = i;
    std::vector<int32_t> sp(EAGLE_MAX_STATIC, -1), sr(EAGLE_MAX_STATIC, 0), sd(EAGLE_MAX_STATIC, 0),
        sw(EAGLE_MAX_STATIC, 0), se((EAGLE_MAX_DEPTH + 1) * TREE_MAXEXP, -1), sne(EAGLE_MAX_DEPTH + 1, 0);
    if (cfg->tree == EAGLE_TREE_STATIC) {
      for (int j = 0; j < cfg->n_static; ++j) {
        sp[j] = cfg->static_parent[j];
        sr[j] = cfg->static_rank[j];
        sd[j] = z.s_depth[j];
        sw[j] = z.s_prow[j];
      }
      for (int dd = 0; dd <= EAGLE_MAX_DEPTH; ++dd) {
        sne[dd] = z.s_nexp[dd];
        for (int i = 0; i < z.s_nexp[dd]; ++i) se[dd * TREE_MAXEXP + i] = z.s_exp[dd][i];
      }
    }
    hipError_t e = hipSuccess;
    auto up = [&](void* dst, const void* src, size_t n) {
      if (e == hipSuccess) e = hipMemcpy(dst, src, n, hipMemcpyHostToDevice);
    };
    up(c->cos_t, cs.data(), cs.size() * 4);
    up(c->sin_t, sn.data(), sn.size() * 4);
    up(c->tpt, tp.data(), tp.size() * 4);
    up(c->dpt, dp.data(), dp.size() * 4);
    up(c->iota, io.data(), io.size() * 4);
    for (const Lane& q : c->lanes) {
      up(q.t.s_parent, sp.data(), sp.size() * 4);
      up(q.t.s_rank, sr.data(), sr.size() * 4);
      up(q.t.s_depth, sd.data(), sd.size() * 4);
      up(q.t.s_prow, sw.data(), sw.size() * 4);
      up(q.t.s_exp, se.data(), se.size() * 4);
      up(q.t.s_nexp, sne.data(), sne.size() * 4);
    }
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      delete c;
      return EAGLE_E_HIP;
    }
  }
  *out = c;
  return EAGLE_OK;
}

eagle_status eagle_prefill_lane(eagle_ctx* c, int32_t lane, const int32_t* prompt, int32_t n,
                                int32_t* first_token) {
  if (!c) return EAGLE_E_INVALID;
  const Derived& z = c->z;
  if (lane < 0 || lane >= z.B) return set_err(c, EAGLE_E_INVALID, "lane %d is not in [0, batch = %d)", lane, z.B);
  if (!prompt || n < 1) return set_err(c, EAGLE_E_INVALID, "prompt must hold at least one token");
  if (n + 1 > c->cfg.max_ctx) return set_err(c, EAGLE_E_CAPACITY, "prompt of %d tokens exceeds max_ctx", n);
  for (int i = 0; i < n; ++i)
    if (prompt[i] < 0 || prompt[i] >= z.V) return set_err(c, EAGLE_E_INVALID, "prompt[%d] = %d is not in [0, vocab)", i, prompt[i]);
  Lane& q = c->lanes[lane];
  q.state = ST_EMPTY;
  q.committed.clear();
  q.step = 0;
  q.ctx_len = 0;
  HCHK(hipMemcpyAsync(q.seq, prompt, sizeof(int32_t) * n, hipMemcpyHostToDevice, c->st));
  for (int c0 = 0; c0 < n; c0 += z.chunk) {
    const int M = std::min(z.chunk, n - c0);
    const bool last = c0 + M == n;
    HCHK(launch_rows_causal(c0, M, q.rpos, q.rslot, q.rprehi, q.rmask, c->st));
    RowVis vis{q.rprehi, q.rmask, 0, 0, 0, c0 + M};
    SCHK(target_pass(c, Span{lane, 1, M}, q.seq + c0, q.rpos, q.rslot, vis));
    if (last) {
      const void* xl = (const char*)c->xop + (int64_t)(M - 1) * z.H * z.esz;
      const bool smp = sampling(c);
      HCHK(launch_lmhead_argmax(z.dt, c->lm, xl, c->xlo, 1, z.V, z.H, c->hpart, c->g, c->margin,
                                smp ? c->logits : nullptr, c->st));
      if (smp) {
        HCHK(launch_row_exp(c->logits, c->g, 1, z.V, c->cfg.temperature, c->ebuf, c->zpart, c->st));
        HCHK(launch_sample_token(c->ebuf, c->zpart, z.V, seed_of(c), 0, (uint32_t)lane, q.seq + n,
                                 c->st));
      }
      else
        HCHK(hipMemcpyAsync(q.seq + n, c->g, 4, hipMemcpyDeviceToDevice, c->st));
    }
    if (plain_mode(c)) continue;
    const float* feat = c->tfeat;
    if (c->cfg.head == EAGLE_HEAD_E3) {
      SCHK(fuse_rows(c, M, c->lmh, c->lmhlo));
      feat = c->gbuf;
    }
    SCHK(catch_up(c, lane, M, c0 + 1, q.seq + c0 + 1, feat, c->iota, last, n));
  }
  int32_t b = 0;
  HCHK(hipMemcpyAsync(&b, q.seq + n, 4, hipMemcpyDeviceToHost, c->st));
  HCHK(hipStreamSynchronize(c->st));
  q.committed.push_back(b);
  q.ctx_len = n;
  q.state = ST_READY;
  if (first_token) *first_token = b;
  return EAGLE_OK;
}

eagle_status eagle_prefill(eagle_ctx* c, const int32_t* prompt, int32_t n, int32_t* first_token) {
  return eagle_prefill_lane(c, 0, prompt, n, first_token);
}

namespace {
eagle_status copy_tree_out(eagle_ctx* c, int lane, eagle_tree* out) {
  const Lane& q = c->lanes[lane];
  int32_t counts[8];
  HCHK(hipMemcpyAsync(counts, q.t.counts, sizeof(counts), hipMemcpyDeviceToHost, c->st));
  HCHK(hipStreamSynchronize(c->st));
  std::memset(out, 0, sizeof(*out));
  const int nr = counts[3], nn = counts[0];
  out->n_rows = nr;
  out->n_nodes = nn;
  auto d2h = [&](void* dst, const void* src, size_t bytes) {
    return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, c->st);
  };
  HCHK(d2h(out->token, q.t.v_tok, 4 * nr));
  HCHK(d2h(out->parent, q.t.v_parent, 4 * nr));
  HCHK(d2h(out->depth, q.t.v_depth, 4 * nr));
  HCHK(d2h(out->logv, q.t.v_logv, 4 * nr));
  HCHK(d2h(out->node, q.t.v_node, 4 * nr));
  if (nn > 0) {
    HCHK(d2h(out->node_token, q.t.tok, 4 * nn));
    HCHK(d2h(out->node_parent, q.t.parent, 4 * nn));
    HCHK(d2h(out->node_depth, q.t.depth, 4 * nn));
    HCHK(d2h(out->node_logv, q.t.logv, 4 * nn));
    HCHK(d2h(out->node_logp, q.t.logp, 4 * nn));
  }
  HCHK(hipStreamSynchronize(c->st));
  return EAGLE_OK;
}
}  // namespace

eagle_status eagle_draft_tree(eagle_ctx* c, eagle_tree* out) {
  SCHK(check_ready(c));
  for (const Lane& q : c->lanes)
    if (q.state != ST_READY)
      return set_err(c, EAGLE_E_STATE, "eagle_draft_tree needs every sequence READY (call eagle_prefill / eagle_verify)");
  const Derived& z = c->z;
  const int B = z.B;
  const Lane& q0 = c->lanes[0];
  if (plain_mode(c)) {
    HCHK(launch_tree_masks(q0.t, 1, q0.ctx_len, q0.seq + q0.ctx_len, c->st,
                           lanes_of(c, Span{0, B, 1})));
  } else {
    // each pass drafts the same number of rows for every sequence
    const int ctx0 = q0.ctx_len;
    int t0 = 0;
    for (int pass = 2; pass <= z.D; ++pass) {
      const int M = z.rows_per_pass[pass];
      if (M <= 0) break;
      RowVis vis{q0.t.row_prehi, q0.t.row_mask, 1, ctx0 + 1, t0 + M, ctx0 + 1 + t0 + M};
      // one sequence writes its draft outputs in place; several go through
      // hcat and are scattered to each sequence's rows afterwards
      float* hout = B == 1 ? q0.dout + (int64_t)(1 + t0) * z.H : c->hcat;
      SCHK(draft_pass(c, Span{0, B, M}, q0.t.row_tok, q0.dout, c->dout_stride, q0.t.row_src,
                      c->lane_bytes, q0.t.row_pos, q0.t.row_slot, vis, hout));
      if (B > 1)
        HCHK(hipMemcpy2DAsync(q0.dout + (int64_t)(1 + t0) * z.H, sizeof(float) * c->dout_stride,
                              c->hcat, sizeof(float) * M * z.H, sizeof(float) * M * z.H, B,
                              hipMemcpyDeviceToDevice, c->st));
      PROFILED(EAGLE_PROF_LMHEAD, (double)z.V * z.H * z.esz + (double)B * M * z.H * 4.0,
               launch_lmhead_topk(z.dt, c->lm, c->xop, c->xlo, B * M, z.V, z.H, z.k_b, c->hpart,
                                  c->ids, c->logp, c->st));
      PROFILED(EAGLE_PROF_TREE, 0.0,
               launch_tree_append(q0.t, c->tp, c->ids, c->logp, pass, ctx0, c->st, nullptr,
                                  lanes_of(c, Span{0, B, M}), (int64_t)M * z.k_b));
      t0 += M;
    }
    PROFILED(EAGLE_PROF_TREE, 0.0,
             launch_tree_finalize(q0.t, c->tp, ctx0, q0.seq + ctx0, c->st,
                                  lanes_of(c, Span{0, B, 1})));
  }
  for (Lane& q : c->lanes) q.state = ST_DRAFTED;
  if (out) SCHK(copy_tree_out(c, 0, out));
  return EAGLE_OK;
}

eagle_status eagle_read_tree(eagle_ctx* c, int32_t lane, eagle_tree* out) {
  if (!c || !out) return EAGLE_E_INVALID;
  if (lane < 0 || lane >= c->z.B) return set_err(c, EAGLE_E_INVALID, "lane %d is not in [0, batch = %d)", lane, c->z.B);
  if (c->lanes[lane].state != ST_DRAFTED)
    return set_err(c, EAGLE_E_STATE, "eagle_read_tree needs a drafted tree (call eagle_draft_tree)");
  return copy_tree_out(c, lane, out);
}

namespace {
// Spins until sequence `lane`'s acceptance kernel has posted `tag` to its
// pinned result block. Every 4096 polls it asks whether the stream has
// drained: a drained stream without the tag (an earlier kernel failed) or a
// stream error ends the wait with an error instead of spinning forever.
eagle_status wait_result(eagle_ctx* c, int lane, int32_t tag) {
  const int32_t* h = c->lanes[lane].hres;
  for (uint32_t spin = 1;; ++spin) {
    if (__atomic_load_n(h, __ATOMIC_ACQUIRE) == tag) return EAGLE_OK;
    if ((spin & 4095) == 0) {
      const hipError_t qs = hipStreamQuery(c->st);
      if (qs == hipErrorNotReady) continue;
      if (__atomic_load_n(h, __ATOMIC_ACQUIRE) == tag) return EAGLE_OK;
      if (qs != hipSuccess) return set_err(c, EAGLE_E_HIP, "stream failed during verify: %s", hipGetErrorString(qs));
      return set_err(c, EAGLE_E_DEVICE, "acceptance result was not posted");
    }
  }
}

// Verify of every sequence's drafted tree (or, with one sequence, the
// planted tree) in one target pass. Sequence b's committed tokens go to
// out_tokens + b * (EAGLE_MAX_DEPTH + 1) and their count to n_committed[b]
// (either may be NULL).
eagle_status verify_all(eagle_ctx* c, const eagle_tree* planted, int32_t* out_tokens,
                        int32_t* n_committed) {
  SCHK(check_ready(c));
  const Derived& z = c->z;
  const int B = z.B;
  for (const Lane& q : c->lanes)
    if (planted ? (q.state != ST_READY && q.state != ST_DRAFTED) : q.state != ST_DRAFTED)
      return set_err(c, EAGLE_E_STATE, "eagle_verify needs a drafted tree (or a planted tree after prefill)");
  Lane& q0 = c->lanes[0];
  int Mv;
  if (planted) {
    const int n = planted->n_rows;
    if (n < 1 || n > z.Mv) return set_err(c, EAGLE_E_INVALID, "planted tree must have 1..%d rows", z.Mv);
    std::vector<int> depth(n, 0);
    for (int r = 1; r < n; ++r) {
      const int p = planted->parent[r];
      if (p < 0 || p >= r) return set_err(c, EAGLE_E_INVALID, "planted parent[%d] must be in [0, %d)", r, r);
      if (planted->token[r] < 0 || planted->token[r] >= z.V) return set_err(c, EAGLE_E_INVALID, "planted token[%d] out of range", r);
      depth[r] = depth[p] + 1;
      if (depth[r] > z.D) return set_err(c, EAGLE_E_INVALID, "planted tree deeper than depth");
      for (int s = 1; s < r; ++s)
        if (planted->parent[s] == p && planted->token[s] == planted->token[r])
          return set_err(c, EAGLE_E_INVALID, "planted rows %d and %d are siblings with one token", s, r);
    }
    Mv = n;
  } else {
    Mv = z.Mv;
  }
  // the cycle may commit up to depth + 1 tokens after each root
  for (const Lane& q : c->lanes)
    if (q.ctx_len + z.D + 2 > c->cfg.max_ctx)
      return set_err(c, EAGLE_E_CAPACITY, "sequence would exceed max_ctx (%d)", c->cfg.max_ctx);
  if (planted) {
    std::vector<int32_t> par(planted->parent, planted->parent + Mv);
    par[0] = -1;
    HCHK(hipMemcpyAsync(q0.t.v_tok, planted->token, 4 * Mv, hipMemcpyHostToDevice, c->st));
    HCHK(hipMemcpyAsync(q0.t.v_parent, par.data(), 4 * Mv, hipMemcpyHostToDevice, c->st));
    HCHK(launch_tree_masks(q0.t, Mv, q0.ctx_len, q0.seq + q0.ctx_len, c->st));
  }
  const int ctx0 = q0.ctx_len;
  RowVis vis{q0.t.v_prehi, q0.t.v_mask, 0, ctx0, Mv, ctx0 + Mv};
  SCHK(target_pass(c, Span{0, B, Mv}, q0.t.v_tok, q0.t.v_pos, q0.t.v_slot, vis));
  const bool smp = sampling(c);
  PROFILED(EAGLE_PROF_LMHEAD, (double)z.V * z.H * z.esz + (double)B * Mv * z.H * 4.0,
           launch_lmhead_argmax(z.dt, c->lm, c->xop, c->xlo, B * Mv, z.V, z.H, c->hpart, c->g,
                                c->margin, (c->debug || smp) ? c->logits : nullptr, c->st));
  c->last_verify_rows = B * Mv;
  // Each acceptance kernel commits its sequence's tokens into seq on the
  // device and posts (L, tokens) to pinned host memory under a fresh tag. The
  // host waits for that tag only, so the KV compaction queued behind it
  // overlaps the wait and the catch-up launches queue behind it with no
  // stream drain in between.
  const int32_t tag = c->verify_tag = c->verify_tag == INT32_MAX ? 1 : c->verify_tag + 1;
  if (smp) {
    const int64_t nb = (int64_t)sample_zpart_doubles(1, z.V);
    PROFILED(EAGLE_PROF_TREE, 0.0,
             launch_row_exp(c->logits, c->g, B * Mv, z.V, c->cfg.temperature, c->ebuf, c->zpart,
                            c->st));
    for (int b = 0; b < B; ++b) {
      Lane& q = c->lanes[b];
      ++q.step;
      PROFILED(EAGLE_PROF_TREE, 0.0,
               launch_accept_sample(q.t, c->ebuf + (int64_t)b * Mv * z.V, c->zpart + b * Mv * nb,
                                    z.V, seed_of(c), q.step, (uint32_t)b, z.D, q.acc, q.new_tok,
                                    q.cu_src, q.seq + q.ctx_len + 1, q.hres_dev, tag, c->st));
    }
  } else {
    PROFILED(EAGLE_PROF_TREE, 0.0,
             launch_accept(q0.t, c->g, z.D, q0.acc, q0.new_tok, q0.cu_src, q0.seq + ctx0 + 1,
                           q0.hres_dev, tag, c->st, lanes_of(c, Span{0, B, Mv}), Mv, HRES_INTS));
  }
  PROFILED(EAGLE_PROF_KV, 0.0,
           launch_kv_compact(z.dt, c->tkv0, c->t_layer_elems, z.NL, q0.acc, q0.acc + 2, ctx0,
                             c->st, lanes_of(c, Span{0, B, Mv})));
  if (!plain_mode(c)) {
    // the catch-up is queued before the host learns L, so the GPU runs on
    // while the host waits for the acceptance results
    if (c->cfg.head == EAGLE_HEAD_E3) {
      const int64_t w3 = 3 * (int64_t)z.H;
      for (int b = 0; b < B; ++b)
        HCHK(launch_gather_t(z.dt, (const char*)c->lmh + (int64_t)b * Mv * w3 * z.esz, w3,
                             c->lmhlo, c->lanes[b].cu_src, z.D + 1, (int)w3,
                             (char*)c->lmh2 + (int64_t)b * (z.D + 1) * w3 * z.esz, c->lmh2lo,
                             c->st));
      SCHK(fuse_rows(c, B * (z.D + 1), c->lmh2, c->lmh2lo));
      SCHK(catch_up_fixed(c, c->gbuf, (int64_t)(z.D + 1) * z.H, c->iota, 0));
    } else {
      SCHK(catch_up_fixed(c, c->tfeat, (int64_t)Mv * z.H, q0.cu_src, c->lane_bytes));
    }
  }
  for (int b = 0; b < B; ++b) SCHK(wait_result(c, b, tag));
  int Ls[EAGLE_MAX_BATCH];
  for (int b = 0; b < B; ++b) {
    Ls[b] = c->lanes[b].hres[1];
    if (Ls[b] < 0 || Ls[b] > z.D) return set_err(c, EAGLE_E_DEVICE, "acceptance length %d out of range", Ls[b]);
  }
  for (int b = 0; b < B; ++b) {
    Lane& q = c->lanes[b];
    const int L = Ls[b];
    const int32_t* nt = q.hres + 2;
    for (int i = 0; i <= L; ++i) q.committed.push_back(nt[i]);
    q.ctx_len += L + 1;
    q.state = ST_READY;
    if (out_tokens) std::memcpy(out_tokens + b * (EAGLE_MAX_DEPTH + 1), nt, sizeof(int32_t) * (L + 1));
    if (n_committed) n_committed[b] = L + 1;
  }
  return EAGLE_OK;
}
}  // namespace

eagle_status eagle_verify(eagle_ctx* c, const eagle_tree* planted, int32_t* out_tokens,
                          int32_t* n_committed) {
  if (!c) return EAGLE_E_INVALID;
  if (c->z.B != 1) return set_err(c, EAGLE_E_STATE, "eagle_verify serves batch 1; use eagle_verify_batch");
  return verify_all(c, planted, out_tokens, n_committed);
}

eagle_status eagle_verify_batch(eagle_ctx* c, int32_t* out_tokens, int32_t* n_committed) {
  if (!c) return EAGLE_E_INVALID;
  return verify_all(c, nullptr, out_tokens, n_committed);
}

eagle_status eagle_generate(eagle_ctx* c, const int32_t* prompt, int32_t n, int32_t max_new,
                            int32_t* out, int32_t* n_out, eagle_stats* stats) {
  if (!c) return EAGLE_E_INVALID;
  if (c->z.B != 1) return set_err(c, EAGLE_E_STATE, "eagle_generate serves batch 1");
  if (max_new < 1 || !out) return set_err(c, EAGLE_E_INVALID, "max_new must be >= 1 and out non-NULL");
  if (n + max_new + c->z.D > c->cfg.max_ctx)
    return set_err(c, EAGLE_E_CAPACITY, "prompt + max_new + depth exceeds max_ctx");
  SCHK(eagle_prefill(c, prompt, n, nullptr));
  eagle_stats s;
  std::memset(&s, 0, sizeof(s));
  hipEvent_t e0, e1;
  HCHK(hipEventCreate(&e0));
  HCHK(hipEventCreate(&e1));
  HCHK(hipEventRecord(e0, c->st));
  const Lane& q = c->lanes[0];
  while ((int)q.committed.size() < max_new) {
    SCHK(eagle_draft_tree(c, nullptr));
    int32_t cnt = 0;
    SCHK(eagle_verify(c, nullptr, nullptr, &cnt));
    s.cycles++;
    s.accept_hist[std::min(cnt - 1, EAGLE_MAX_DEPTH)]++;
  }
  HCHK(hipEventRecord(e1, c->st));
  HCHK(hipEventSynchronize(e1));
  float ms = 0.f;
  HCHK(hipEventElapsedTime(&ms, e0, e1));
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  s.seconds = ms * 1e-3;
  s.committed = (int64_t)q.committed.size();
  std::memcpy(out, q.committed.data(), sizeof(int32_t) * max_new);
  if (n_out) *n_out = max_new;
  if (stats) *stats = s;
  return EAGLE_OK;
}

eagle_status eagle_committed_lane(eagle_ctx* c, int32_t lane, int32_t* out, int32_t cap, int32_t* n) {
  if (!c || (!out && cap > 0)) return EAGLE_E_INVALID;
  if (lane < 0 || lane >= c->z.B) return set_err(c, EAGLE_E_INVALID, "lane %d is not in [0, batch = %d)", lane, c->z.B);
  const std::vector<int32_t>& v = c->lanes[lane].committed;
  const int k = std::min<int>(cap, (int)v.size());
  if (k > 0) std::memcpy(out, v.data(), sizeof(int32_t) * k);
  if (n) *n = (int32_t)v.size();
  return EAGLE_OK;
}

eagle_status eagle_committed(eagle_ctx* c, int32_t* out, int32_t cap, int32_t* n) {
  return eagle_committed_lane(c, 0, out, cap, n);
}

eagle_status eagle_set_sampling(eagle_ctx* c, float temperature, uint32_t seed_lo,
                                uint32_t seed_hi) {
  if (!c) return EAGLE_E_INVALID;
  if (!(temperature >= 0.f) || !(temperature <= 1e4f))
    return set_err(c, EAGLE_E_INVALID, "temperature must be in [0, 1e4] (0 = greedy)");
  if (temperature > 0.f && !sample_vocab_ok(c->z.V))
    return set_err(c, EAGLE_E_INVALID, "sampling supports vocab <= 131072");
  c->cfg.temperature = temperature;
  c->cfg.seed_lo = seed_lo;
  c->cfg.seed_hi = seed_hi;
  return EAGLE_OK;
}

eagle_status eagle_set_debug(eagle_ctx* c, int32_t on) {
  if (!c) return EAGLE_E_INVALID;
  c->debug = on != 0;
  return EAGLE_OK;
}

eagle_status eagle_debug_read(eagle_ctx* c, int32_t what, void* host_dst, uint64_t bytes,
                              int32_t* rows) {
  if (!c || !host_dst) return EAGLE_E_INVALID;
  const Derived& z = c->z;
  const void* src;
  uint64_t avail;
  int r;
  switch (what) {
    case 0: src = c->tfeat; r = c->last_target_rows; avail = (uint64_t)r * z.H * 4; break;
    case 1: src = c->logits; r = c->last_verify_rows; avail = (c->debug || sampling(c)) ? (uint64_t)r * z.V * 4 : 0; break;
    case 2: src = c->g; r = c->last_verify_rows; avail = (uint64_t)r * 4; break;
    case 3: src = c->margin; r = c->last_verify_rows; avail = (uint64_t)r * 4; break;
    default: return set_err(c, EAGLE_E_INVALID, "unknown debug buffer %d", what);
  }
  if (rows) *rows = r;
  const uint64_t n = std::min(bytes, avail);
  if (n) {
    HCHK(hipMemcpyAsync(host_dst, src, n, hipMemcpyDeviceToHost, c->st));
    HCHK(hipStreamSynchronize(c->st));
  }
  return EAGLE_OK;
}

eagle_status eagle_profile_enable(eagle_ctx* c, uint32_t class_mask, int32_t every) {
  if (!c || every < 1) return EAGLE_E_INVALID;
  prof_settle(c, true);
  c->prof = class_mask;
  c->prof_every = every;
  std::memset(c->prof_seen, 0, sizeof(c->prof_seen));
  std::memset(&c->ptot, 0, sizeof(c->ptot));
  return EAGLE_OK;
}

eagle_status eagle_profile_read(eagle_ctx* c, eagle_profile* out) {
  if (!c || !out) return EAGLE_E_INVALID;
  HCHK(hipStreamSynchronize(c->st));
  prof_settle(c, true);
  *out = c->ptot;
  return EAGLE_OK;
}

void eagle_free(eagle_ctx* c) {
  if (!c) return;
  if (c->st) (void)hipStreamSynchronize(c->st);
  for (hipEvent_t e : c->all_ev) (void)hipEventDestroy(e);
  delete c;
}

const char* eagle_last_error(const eagle_ctx* c) { return c ? c->err.c_str() : "null context"; }

}  // extern "C"
