// Host launchers of the gfx950 kernels (all enqueue on `stream`, no sync).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

enum { EPI_PART = 0, EPI_SWIGLU = 2 };

// ---------------------------------------------------------------- GEMM
// y = x W^T for a skinny x (M rows) and a weight W [N, K] streamed from HBM.
//   EPI_PART  : fp32 partial planes Y[split][M][ldy] (split over K; the
//               consumer sums *splits_out planes in order; plane = M * ldy)
//   EPI_SWIGLU: W = [gate (N rows); up (N rows)], Yt[m, n] = silu(g) * u
//               written as an operand (two bf16 planes, lo at Yt + ytlo)
// dtype 0 = fp32, 1 = bf16 for W. x is an operand (see Opnd in common.h):
// for bf16 two planes, the lo plane xlo elements after the hi plane.
struct GemmPlan { int mt, nb, splits, m_chunks, n_tiles, nw, xg = 1; };
GemmPlan gemm_plan(int M, int N_rows, int K, int dtype, int epi);
uint64_t gemm_part_floats(const GemmPlan& p, int N_rows, int M);
// SwiGLU projections of M rows that run as a split-K gate|up projection plus
// a SiLU pass: they need split * M * 2F floats of partial-plane scratch in Y.
bool swiglu_by_planes(int dtype, int M);
// Optional device timestamps of one kernel dispatch: the events ride on the
// dispatch itself (hipExtLaunchKernel), so they time that kernel alone.
struct KTiming {
  hipEvent_t start, stop;
};

// Optional scale of output rows, for an operand whose rows are the RMSNorm
// numerators gain * h (launch_resnorm_slices): the sums of squares of row m
// sit in ss[RS_SLICES m .. RS_SLICES m + RS_SLICES - 1], and output row m is
// multiplied by 1 / sqrt((their sum) / H + eps), the row's RMSNorm factor.
// By linearity every partial plane, and so their sum, carries the factor.
constexpr int RS_SLICES = 4;
struct RowScale {
  const float* ss = nullptr;   // null: no scaling
  int H = 0;
  float eps = 0.f;
};

hipError_t launch_gemm(int dtype, int epi, const void* W, const void* x, int64_t xlo, int M, int N,
                       int K, float* Y, int64_t ldy, void* Yt, int64_t ytlo, int* splits_out,
                       hipStream_t stream, const KTiming* tm = nullptr, RowScale rs = RowScale());

// Fragment packing of the first 16*n_blocks rows of a bf16 [*, K] matrix
// from row-major `src` to `dst` (non-overlapping; same byte range per block).
// Every bf16 weight the GEMM and LM-head kernels stream is in this form.
hipError_t launch_pack_frag(const void* src, void* dst, int64_t n_blocks, int K, hipStream_t stream);

// ---------------------------------------------------------------- LM head
// Verify: g[m] = argmax_v (x W^T)[m, v] (lowest id on ties), margin[m] =
// top-1 minus top-2; logits stored to `logits` [M, V] when not null.
hipError_t launch_lmhead_argmax(int dtype, const void* W, const void* x, int64_t xlo, int M, int V,
                                int H, float* part, int32_t* g, float* margin, float* logits,
                                hipStream_t stream);
// Draft: per row the k best ids by (logit desc, id asc) and their
// log-probabilities l - max - log(sum exp(l - max)) over the full vocabulary.
hipError_t launch_lmhead_topk(int dtype, const void* W, const void* x, int64_t xlo, int M, int V,
                              int H, int k, float* part, int32_t* ids, float* logp,
                              hipStream_t stream);
uint64_t lmhead_part_floats(int M, int V, int k);

// ---------------------------------------------------------------- paged KV
// One layer of a paged KV cache. Element (slot, plane, kv head h, i) lives at
//   base + page_table[slot / page] * page_elems
//        + ((plane * n_kv + h) * page + slot % page) * d + i
// so each (page, plane, head) is a contiguous [page, d] tile. fp32 caches
// have planes K, V; bf16 caches keep each fp32 value as a hi + lo pair with
// planes K_hi, K_lo, V_hi, V_lo (16 significant bits).
struct KVView {
  void* base;
  const int32_t* page_table;
  int64_t page_elems;   // planes * n_kv * page * d
  int page, n_kv, d;
  int64_t lane_elems = 0;   // sequence b's cache starts b * lane_elems elements after base
};
inline int kv_planes(int dtype) { return dtype == 1 ? 4 : 2; }

// ---------------------------------------------------------------- rows
// Attention visibility of row r: key slots [pre_lo, prehi[r]) plus the
// tree slots tree_base + j whose bit j is set in mask[2r..2r+1].
struct RowVis {
  const int32_t* prehi;
  const uint64_t* mask;
  int pre_lo, tree_base, n_tree, key_end;
};

// Several sequences in one launch. Rows [b * rows, (b + 1) * rows) belong to
// sequence b (b < n). Its per-row inputs (pos, slot, prehi, mask) start
// `bytes` bytes after sequence 0's, its cache at KVView::lane_elems * b, and
// its key positions are shifted by off[b]: sequence b sees the tree slots
// from tree_base + off[b] and keys up to key_end + off[b]. The default is one
// sequence whose rows are all M rows of the launch.
#define MAX_LANES 8
struct Lanes {
  int n = 1, rows = 0;
  int64_t bytes = 0;
  int off[MAX_LANES] = {};
};

// Device side of Lanes: sequence b's key shift (picked with selects, not a
// dynamic index into the kernel arguments) and sequence b's copy of a
// per-sequence array given sequence 0's.
__device__ __forceinline__ int lane_shift(const Lanes& ln, int b) {
  int o = 0;
#pragma unroll
  for (int i = 0; i < MAX_LANES; ++i) o = i == b ? ln.off[i] : o;
  return o;
}
template <typename T>
__device__ __forceinline__ T* lane_at(T* p, int b, int64_t bytes) {
  return (T*)((char*)p + (int64_t)b * bytes);
}

// Sequence-aware forms (ln.n > 1): row r of sequence b = r / ln.rows takes
// its token (and feature index) from sequence b's copy of the array
// (ln.bytes apart) and its feature from feat + b * feat_stride.
hipError_t launch_embed(int dtype, const void* E, int H, const int32_t* tok, int M, float* h,
                        hipStream_t st, const Lanes& ln = Lanes());
// Operand outputs (out_t, q_out, x, dst of store_feat / gather_t) take
// their lo-plane offset `lo` in elements (ignored for fp32).
//
// Residual update + RMSNorm of M rows of width H:
//   h[r] = (set ? 0 : h[r]) + sum_{s < S} part[s][r]   (fixed order; S may be 0)
//   out = gain ? RMSNorm(h[r]) * gain : h[r]   -> operand out_t (and fp32 out_f)
hipError_t launch_resnorm(int dtype, float* h, int H, int M, const float* part, int S,
                          int64_t plane, int set, const float* gain, float eps, void* out_t,
                          int64_t lo, float* out_f, hipStream_t st);
// The same residual update with the RMSNorm spread over RS_SLICES
// workgroups per row (a row's partial planes are more bytes than one CU
// pulls quickly): out = gain * h[r], the RMSNorm numerator, and ss[r] gets
// the per-slice sums of squares of h[r] for the projection that consumes
// out (RowScale). Without a gain out = h[r] and ss is not written. Needs
// H % (64 * RS_SLICES * 4) == 0 and H <= 16384.
bool resnorm_slices_fit(int H);
hipError_t launch_resnorm_slices(int dtype, float* h, int H, int M, const float* part, int S,
                                 int64_t plane, int set, const float* gain, void* out_t, int64_t lo,
                                 float* ss, hipStream_t st);
// dst[r] = (add ? dst[r] : 0) + sum_s part[s][r] for M rows of width W.
hipError_t launch_sum_planes(const float* part, int S, int64_t plane, int M, int W, float* dst,
                             int add, hipStream_t st);
// RoPE on q and k and append of k, v to the cache; qkv = sum of S partial
// planes [M, (nq + 2 nkv) d].
hipError_t launch_rope_kv(int dtype, const float* qkv, int S, int64_t plane, int M, int nq, int nkv,
                          int d, const int32_t* pos, const int32_t* slot, const float* cos_t,
                          const float* sin_t, void* q_out, int64_t qlo, KVView kv, hipStream_t st,
                          const Lanes& ln = Lanes());
uint64_t attn_part_floats(int max_chunks, int M, int nq, int d);
int attn_chunk_keys();
// Most key chunks one attention call may split a row's keys into.
int attn_max_chunks();
hipError_t launch_attention(int dtype, const void* q, int64_t qlo, KVView kv, RowVis vis, int M,
                            int nq, int d, float scale, float* opart, float* mlpart, void* out_t,
                            int64_t olo, hipStream_t st, const Lanes& ln = Lanes());
hipError_t launch_draft_input_e1(int dtype, const void* E, const int32_t* tok, const float* feat,
                                 const int32_t* idx, int M, int H, void* x, int64_t lo,
                                 hipStream_t st, const Lanes& ln = Lanes(),
                                 int64_t feat_stride = 0, int64_t idx_bytes = 0);
hipError_t launch_draft_input_e3(int dtype, const void* E, const int32_t* tok, const float* feat,
                                 const int32_t* idx, const float* gain, float eps, int M, int H,
                                 void* x, int64_t lo, float* h, hipStream_t st,
                                 const Lanes& ln = Lanes(), int64_t feat_stride = 0,
                                 int64_t idx_bytes = 0);
hipError_t launch_gather_f32(const float* src, int64_t ld, const int32_t* idx, int M, int W,
                             float* dst, hipStream_t st);
hipError_t launch_gather_t(int dtype, const void* src, int64_t ld, int64_t src_lo, const int32_t* idx,
                           int M, int W, void* dst, int64_t dst_lo, hipStream_t st);
hipError_t launch_store_feat(int dtype, const float* h, int H, int M, void* dst, int64_t ldd,
                             int64_t lo, hipStream_t st);
// One root row per sequence: row b of dst (dst_f: b * dst_stride floats;
// dst_t: an operand row of width W) = row b * src_rows + r_b of src, where
// r_b = sequence b's acc[0] (acc: sequence 0's copy, ln.bytes apart).
hipError_t launch_gather_roots(int dtype, const float* src_f, const void* src_t, int64_t src_lo,
                               int src_rows, const int32_t* acc, int W, float* dst_f,
                               int64_t dst_stride, void* dst_t, int64_t dst_lo, const Lanes& ln,
                               hipStream_t st);
// Sequence-aware forms: sequence b's rows start at first + ln.off[b] (its
// arrays ln.bytes apart); its cache compaction uses its own cache
// (KVView::lane_elems), L / path copies and context ctx + ln.off[b].
hipError_t launch_rows_causal(int first, int M, int32_t* pos, int32_t* slot, int32_t* prehi,
                              uint64_t* mask, hipStream_t st, const Lanes& ln = Lanes());
hipError_t launch_kv_compact(int dtype, KVView layer0, int64_t layer_elems, int n_layers,
                             const int32_t* L, const int32_t* path, int ctx, hipStream_t st,
                             const Lanes& ln = Lanes());

// ---------------------------------------------------------------- tree
#define TREE_MAXN 1024
#define TREE_MAXROWS 128     // verify rows and tree rows (bit masks of 128)
#define TREE_MAXEXP 16       // rows per draft pass

// Device-side tree state (all arrays in the scratch buffer).
struct TreeDev {
  int32_t *tok, *parent, *depth, *srcrow, *rank, *row_of_node;  // [TREE_MAXN]
  float *logv, *logp;                                                           // [TREE_MAXN]
  int32_t* counts;     // [0] nodes, [1] rows of the next pass, [2] tree rows used, [3] verify rows
  int32_t* exp_nodes;  // [TREE_MAXEXP] nodes expanded by the next pass, in order
  int32_t *row_tok, *row_src, *row_pos, *row_slot, *row_prehi;  // [TREE_MAXEXP]
  uint64_t* row_mask;  // [2 * TREE_MAXEXP]
  uint64_t* tmask;     // [2 * TREE_MAXROWS] visibility mask of each tree row
  int32_t *v_tok, *v_parent, *v_depth, *v_node, *v_pos, *v_slot, *v_prehi;  // [TREE_MAXROWS]
  float* v_logv;
  uint64_t* v_mask;    // [2 * TREE_MAXROWS]
  // static plan (uploaded at load): per static node
  int32_t *s_parent, *s_rank, *s_depth, *s_prow;  // s_prow: row of the parent in its pass
  int32_t *s_exp;      // [EAGLE depth][TREE_MAXEXP] nodes expanded at each depth (-1 padded)
  int32_t* s_nexp;     // [depth] count
};

struct TreeParams {
  int dynamic, k_b, k_e, depth, budget, n_static;
};

// Append the children produced by the last draft pass (pass 1 = the root
// row) and, if pass < depth, choose the nodes the next pass expands and
// write its row descriptors. ids/logp: [rows of the pass, k_b]. The root
// sits at position ctx, or at ctx + ctx_len[0] + 1 when ctx_len (a device
// int, the acceptance length) is given.
// Sequence-aware forms of the tree kernels: one workgroup per sequence b <
// ln.n, whose tree state is t shifted by b * ln.bytes (every TreeDev array)
// and whose context is ctx + ln.off[b]; ids / logp of sequence b start b *
// ids_stride elements in, its root token pointer (and ctx_len, g, acc,
// new_tok, cu_src, seq_out) are sequence 0's shifted by b * ln.bytes (plus
// ln.off[b] elements for pointers into the sequence), g by b * g_stride and
// host by b * host_stride.
hipError_t launch_tree_append(TreeDev t, TreeParams p, const int32_t* ids, const float* logp,
                              int pass, int ctx, hipStream_t st, const int32_t* ctx_len = nullptr,
                              const Lanes& ln = Lanes(), int64_t ids_stride = 0);
// Rerank to the best `budget` nodes, flatten to verify rows (root first,
// then by depth and rerank order), build positions and ancestry masks.
// root_token: device pointer to the last committed token.
hipError_t launch_tree_finalize(TreeDev t, TreeParams p, int ctx, const int32_t* root_token,
                                hipStream_t st, const Lanes& ln = Lanes());
// Masks/positions for verify rows already in v_tok / v_parent (planted tree).
hipError_t launch_tree_masks(TreeDev t, int n_rows, int ctx, const int32_t* root_token,
                             hipStream_t st, const Lanes& ln = Lanes());
// Greedy acceptance walk over the verify rows given the target's choices g.
// acc[0] = L, acc[1] = bonus, acc[2..2+L) = accepted rows; new_tok[0..L]
// = the committed tokens; cu_src[0..L] = feature rows feeding the catch-up.
// The tokens are also written to seq_out[0..L]. host (mapped host memory, or
// NULL) receives host[1] = L and host[2..2+L] = the tokens, then host[0] = tag.
// Rows L+1 .. max_depth of new_tok / cu_src get the bonus token and source
// row 0, so a catch-up over max_depth + 1 rows reads valid inputs.
// Sampling mode (temperature > 0). launch_row_exp: for each of `rows`
// logit rows (logits [rows, V] fp32, g = each row's argmax), e = exp((l -
// max) / T) into ebuf [rows, V] and fp64 sums of e per 1024-token block into
// zpart [rows, sample_zpart_doubles / rows]. launch_accept_sample: the same
// outputs as launch_accept, with the tree's candidates tested by rejection
// sampling against e / Z of each verify row and the last token drawn from
// what is left; draws from Philox4x32-10 keyed by seed, counter (step, depth,
// draw, lane), lane = the sequence's index in a batch (0 alone).
// launch_sample_token draws one token from row 0 (counter (step, 0, 0xFFFF,
// lane)) into out[0]. V must pass sample_vocab_ok.
bool sample_vocab_ok(int V);
uint64_t sample_zpart_doubles(int rows, int V);
hipError_t launch_row_exp(const float* logits, const int32_t* g, int rows, int V, float temperature,
                          float* ebuf, double* zpart, hipStream_t st);
hipError_t launch_accept_sample(TreeDev t, const float* ebuf, const double* zpart, int V,
                                uint64_t seed, uint32_t step, uint32_t lane, int max_depth,
                                int32_t* acc, int32_t* new_tok, int32_t* cu_src, int32_t* seq_out,
                                int32_t* host, int32_t tag, hipStream_t st);
hipError_t launch_sample_token(const float* ebuf, const double* zpart, int V, uint64_t seed,
                               uint32_t step, uint32_t lane, int32_t* out, hipStream_t st);
hipError_t launch_accept(TreeDev t, const int32_t* g, int max_depth, int32_t* acc,
                         int32_t* new_tok, int32_t* cu_src, int32_t* seq_out, int32_t* host,
                         int32_t tag, hipStream_t st, const Lanes& ln = Lanes(),
                         int64_t g_stride = 0, int64_t host_stride = 0);
