/*
 * eagle.h - C interface of one EAGLE / EAGLE-2 draft-and-verify cycle on one
 * AMD Instinct MI355X (gfx950), for one sequence or a small batch of them.
 *
 * What the calls compute (the method, from the source pages):
 *  - "Lesson 13.11 - EAGLE: Feature-Level Drafting for Faster Inference",
 *    section "Speculative decoding in four moves": draft, verify the drafts in
 *    one target pass, accept from the left while the draft equals the
 *    target's greedy choice, correct with the target's token.
 *  - same page, "The big idea: draft at the feature level" and "Resolving the
 *    uncertainty by feeding back the token": the draft row pairs the target
 *    feature f (the vector fed to the LM head) with the next token's
 *    embedding, an FC maps [emb; f] (2H) to H, one decoder layer predicts
 *    the next feature, and the target's frozen LM head gives probabilities.
 *  - "EAGLE-2: Context-Aware Dynamic Draft Trees", sections "Path Value Ranks
 *    Prefixes", "Global Reranking Separates Exploration from Verification",
 *    "The Mask Preserves Tree Semantics in One Target Pass" and the actor
 *    table in "Putting It Together": path value = product of draft
 *    confidences (kept as a sum of logs), expand the top-k newest nodes,
 *    rerank everything to the best m, flatten with an ancestry mask, verify.
 *  - "05 - EAGLE 三代", section 2.3 (draft compute flow: features [B,S,H],
 *    shifted tokens, one draft step per tree level), section 4.3 (EAGLE-3
 *    fusion g = FC([l;m;h]) for verified rows, the draft's own output a for
 *    later steps) and section 3 (the three engine options: branches per
 *    level, tree depth, number of verified draft tokens).
 *
 * Conventions
 *  - One context belongs to one host thread; all device work is ordered on
 *    the stream given to eagle_load. Token ids are int32 in [0, vocab).
 *    Positions are 0-based.
 *  - Batch: a context serves `batch` independent sequences (lanes 0 ..
 *    batch - 1), each with its own prompt, KV cache, tree and committed
 *    stream. Every draft pass and the verify pass run all lanes' rows in one
 *    pass over the weights (the draft and verify row counts are the same for
 *    every lane; the context lengths may differ). A lane computes exactly
 *    what a batch-1 context computes for its sequence, up to the rounding
 *    of split-K sums whose split count depends on the total row count.
 *  - Memory: the library allocates no device memory. The caller allocates
 *    the three device buffers whose sizes eagle_query reports and keeps them
 *    alive until eagle_free. Host pointers are only read during the call.
 *    eagle_load allocates one small pinned host block (freed by eagle_free)
 *    through which eagle_verify receives the acceptance result; eagle_verify
 *    returns once that result is known, with its catch-up work still queued
 *    on the stream.
 *  - Errors: every call returns an eagle_status. Argument, state and
 *    capacity checks run on the host before any device work, so a rejected
 *    call leaves the context unchanged. After EAGLE_E_HIP or EAGLE_E_DEVICE
 *    the context is FAILED: only eagle_prefill (which resets it) and
 *    eagle_free are accepted. eagle_last_error gives a message.
 *  - Greedy (temperature 0, the default): the committed stream equals plain
 *    greedy decoding of the target (ties to the lowest token id). Sampling
 *    (temperature > 0, see eagle_config): it is distributed as plain
 *    sampling from the target.
 */
#ifndef EAGLE_H
#define EAGLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum eagle_status {
  EAGLE_OK = 0,
  EAGLE_E_INVALID = 1,   /* bad argument or configuration */
  EAGLE_E_STATE = 2,     /* call not allowed in the context's current state */
  EAGLE_E_CAPACITY = 3,  /* would exceed max_ctx or a fixed limit below */
  EAGLE_E_BUFFER = 4,    /* a caller buffer is missing or too small */
  EAGLE_E_HIP = 5,       /* a HIP runtime call failed */
  EAGLE_E_DEVICE = 6     /* a device-side check failed */
} eagle_status;

enum { EAGLE_F32 = 0, EAGLE_BF16 = 1 };
enum { EAGLE_HEAD_E1 = 0, EAGLE_HEAD_E3 = 1 };
enum { EAGLE_TREE_DYNAMIC = 0, EAGLE_TREE_STATIC = 1 };

#define EAGLE_MAX_STATIC 64   /* nodes of a static tree */
#define EAGLE_MAX_DEPTH 16    /* draft passes per cycle */
#define EAGLE_MAX_VERIFY 128  /* verify rows = 1 + budget */
#define EAGLE_MAX_NODES 1024  /* generated nodes per cycle */
#define EAGLE_MAX_TOPK 16     /* children per expanded row */
#define EAGLE_MAX_BATCH 8     /* sequences per context */

/* Model and policy. Shapes follow the Llama layout: RMSNorm (gain tensors),
 * rotate-half RoPE, GQA attention, SwiGLU FFN, untied LM head. */
typedef struct eagle_config {
  int32_t n_layers, hidden, n_heads, n_kv_heads, ffn, vocab;
  float rope_base;             /* theta_i = rope_base^(-2i/head_dim) */
  float rms_eps;               /* RMSNorm epsilon */
  int32_t dtype;               /* EAGLE_F32 or EAGLE_BF16 (weights, KV, operands) */
  int32_t head;                /* EAGLE_HEAD_E1 or EAGLE_HEAD_E3 */
  int32_t feat_layers[3];      /* E3: target layers (0-based) fused as [l;m;h] */
  int32_t tree;                /* EAGLE_TREE_DYNAMIC or EAGLE_TREE_STATIC */
  int32_t topk;                /* children kept per expanded row (branching) */
  int32_t expand;              /* dynamic: nodes expanded per level (0 = topk) */
  int32_t depth;               /* draft passes per cycle = deepest node */
  int32_t budget;              /* dynamic: kept nodes m (verify rows = 1 + m);
                                  0 = plain greedy decode, one token per pass */
  int32_t n_static;            /* static: node count (ignored when dynamic) */
  int32_t static_parent[EAGLE_MAX_STATIC]; /* static: parent node, -1 = root;
                                              breadth-first order */
  int32_t static_rank[EAGLE_MAX_STATIC];   /* static: child rank in the
                                              parent's draft top-k */
  int32_t max_ctx;             /* capacity: prompt + generated tokens */
  int32_t prefill_chunk;       /* rows per prefill pass (0 = 512) */
  /* Sampling. temperature 0 = greedy verification (the default). temperature
   * > 0 = sampling from softmax(logits / temperature): the prefill's token is
   * drawn, and verify tests the tree's candidates by rejection sampling, so
   * the committed stream is distributed as plain sampling from the target
   * ("EAGLE: Feature-Level Drafting for Faster Inference", section
   * "Speculative decoding in four moves"; EAGLE-2 page, "How it works").
   * Draws come from Philox4x32-10 keyed by (seed_lo, seed_hi) with counter
   * (step, depth, draw, lane): step 0 is the lane's prefill token, step i
   * its i-th verify after it; draw j tests child j, 0xFFFF draws the
   * residual token; lane is the sequence's index (0 at batch 1). The draft
   * tree is built as in greedy mode. vocab <= 131072 when sampling. */
  float temperature;
  uint32_t seed_lo, seed_hi;
  /* Sequences served together, 1 .. EAGLE_MAX_BATCH (0 = 1). Device buffers
   * grow with it: KV by `batch` caches, scratch by batch times the rows of a
   * pass. */
  int32_t batch;
} eagle_config;

/* Sizes of the caller-owned device buffers, in bytes. */
typedef struct eagle_sizes {
  uint64_t weight_bytes;   /* every weight tensor, at eagle_tensor offsets */
  uint64_t kv_bytes;       /* paged target KV (all layers) + draft KV */
  uint64_t scratch_bytes;  /* activations, partial sums, tree and state */
  int32_t n_tensors;       /* entries of the weight table */
  int32_t verify_rows;     /* 1 + kept nodes */
  int32_t max_nodes;       /* generated nodes per cycle */
  int32_t kv_page;         /* slots per KV page */
  int32_t ctx_headroom;    /* KV slots a generation needs beyond its tokens:
                              max_ctx must be >= prompt + generated +
                              ctx_headroom (the draft depth: the last cycle
                              may commit depth + 1 tokens) */
} eagle_sizes;

/* Weight tensor kinds (one table entry each). */
enum {
  EAGLE_T_EMBED = 0,      /* [vocab, hidden] token embedding (shared) */
  EAGLE_T_LM_HEAD = 1,    /* [vocab, hidden] LM head (shared) */
  EAGLE_T_FINAL_NORM = 2, /* [hidden] fp32 gain */
  EAGLE_T_ATTN_NORM = 3,  /* [hidden] fp32 gain (E3 draft: [2*hidden]) */
  EAGLE_T_WQ = 4,         /* [n_heads*head_dim, in] */
  EAGLE_T_WK = 5,         /* [n_kv_heads*head_dim, in] */
  EAGLE_T_WV = 6,         /* [n_kv_heads*head_dim, in] */
  EAGLE_T_WO = 7,         /* [hidden, n_heads*head_dim] */
  EAGLE_T_FFN_NORM = 8,   /* [hidden] fp32 gain */
  EAGLE_T_WGATE = 9,      /* [ffn, hidden] */
  EAGLE_T_WUP = 10,       /* [ffn, hidden] */
  EAGLE_T_WDOWN = 11,     /* [hidden, ffn] */
  EAGLE_T_FC = 12         /* E1: [hidden, 2*hidden] on [emb; f];
                             E3: [hidden, 3*hidden] on [l; m; h] */
};
enum { EAGLE_G_GLOBAL = 0, EAGLE_G_TARGET = 1, EAGLE_G_DRAFT = 2 };

/* One weight tensor: row-major [rows, cols] at `offset` in the weight
 * buffer. Matrices are stored as in y = x W^T (rows = outputs). Element
 * type is the config dtype, except norm gains, which are always fp32. */
typedef struct eagle_tensor {
  int32_t kind;     /* EAGLE_T_* */
  int32_t group;    /* EAGLE_G_* */
  int32_t layer;    /* target layer index (0 for global and draft) */
  int32_t dtype;    /* EAGLE_F32 or EAGLE_BF16 */
  int64_t rows, cols;
  uint64_t offset;  /* bytes from the start of the weight buffer */
} eagle_tensor;

/* Caller-owned device memory (hipMalloc'd or from a framework allocator). */
typedef struct eagle_buffers {
  void* weights;  uint64_t weight_bytes;
  void* kv;       uint64_t kv_bytes;
  void* scratch;  uint64_t scratch_bytes;
} eagle_buffers;

/* Host view of one drafted tree (eagle_draft_tree) or a caller-planted tree
 * (eagle_verify). Rows are the verify rows: row 0 is the root (the last
 * committed token); every other row's parent row is smaller than itself. */
typedef struct eagle_tree {
  int32_t n_rows;                      /* 1 + kept nodes */
  int32_t token[EAGLE_MAX_VERIFY];
  int32_t parent[EAGLE_MAX_VERIFY];    /* row index, -1 for row 0 */
  int32_t depth[EAGLE_MAX_VERIFY];     /* 0 for row 0 */
  float logv[EAGLE_MAX_VERIFY];        /* log path value (0 for row 0) */
  int32_t node[EAGLE_MAX_VERIFY];      /* generated-node index, -1 for row 0 */
  /* every generated node of the cycle, in generation order (output only) */
  int32_t n_nodes;
  int32_t node_token[EAGLE_MAX_NODES];
  int32_t node_parent[EAGLE_MAX_NODES]; /* node index, -1 = child of the root */
  int32_t node_depth[EAGLE_MAX_NODES];
  float node_logv[EAGLE_MAX_NODES];
  float node_logp[EAGLE_MAX_NODES];     /* the node's own draft log-prob */
} eagle_tree;

typedef struct eagle_stats {
  int64_t cycles;                         /* verify passes */
  int64_t committed;                      /* tokens committed (incl. prefill's) */
  int64_t accept_hist[EAGLE_MAX_DEPTH + 1]; /* cycles by accepted length L */
  double seconds;                         /* device time of the cycle loop */
} eagle_stats;

typedef struct eagle_ctx eagle_ctx;

/* Sizes of the three device buffers for `cfg`; validates `cfg`.
 * The configuration carries the options the pages name for a serving
 * engine: branches per level (topk), draft steps (depth) and verified draft
 * tokens (budget) -- "05 - EAGLE 三代", section 3 (the engine's three
 * options); "Lesson 13.11", section "How EAGLE lives on today" (load the
 * target and a small draft head, set the number of draft steps and the tree
 * size). Pure host call. EAGLE_E_INVALID on a bad config. */
eagle_status eagle_query(const eagle_config* cfg, eagle_sizes* out);

/* Entry `index` (0 <= index < n_tensors) of the weight table of `cfg`.
 * Pure host call. The caller writes each tensor at its offset. */
eagle_status eagle_tensor_info(const eagle_config* cfg, int32_t index, eagle_tensor* out);

/* Loads the target and the draft head ("Lesson 13.11", section "How EAGLE
 * lives on today"; the draft shares the target's embedding and frozen LM
 * head: section "The big idea: draft at the feature level").
 * Creates a context over caller-owned buffers (sizes >= eagle_query's) on
 * HIP stream `hip_stream` (NULL = the default stream). The weights must be
 * in place, in the row-major layout of eagle_tensor, before this call: for
 * EAGLE_BF16 it rewrites every matrix except the embedding, in place, into
 * the fragment-packed form its kernels stream (each full block of 16 rows
 * keeps its byte range; see eagle_op_pack in eagle_ops.h), using the
 * scratch buffer as staging, and synchronises the stream. A weight buffer
 * is therefore loaded by one context once; the caller must not write it
 * afterwards. Binds to the device current at this call. EAGLE_E_BUFFER if
 * a buffer is NULL or too small, EAGLE_E_HIP if packing fails. *out is a
 * host object. */
eagle_status eagle_load(const eagle_config* cfg, const eagle_buffers* bufs, void* hip_stream,
                        eagle_ctx** out);

/* Prefill: the target's pass over the prompt gives the features f and the
 * first token; the draft then runs over the (f_j, t_{j+1}) pairs with the
 * token shifted by one ("Lesson 13.11", section "Resolving the uncertainty
 * by feeding back the token"; "05 - EAGLE 三代", section 2.3).
 * Starts a sequence in lane 0: target prefill over prompt[0..n), the first
 * committed token b = greedy choice after the prompt (sampled when
 * temperature > 0), and the draft's catch-up over the n (feature,
 * next-token) pairs, which leaves the depth-1 candidates ready. Resets any
 * earlier sequence of the lane. The call synchronises the stream and, if
 * first_token is not NULL, writes b. EAGLE_E_CAPACITY if n + 1 > max_ctx. */
eagle_status eagle_prefill(eagle_ctx* ctx, const int32_t* prompt, int32_t n,
                           int32_t* first_token);
/* eagle_prefill for lane `lane` (0 <= lane < batch); the other lanes keep
 * their state, so a finished sequence can be replaced between cycles. */
eagle_status eagle_prefill_lane(eagle_ctx* ctx, int32_t lane, const int32_t* prompt, int32_t n,
                                int32_t* first_token);

/* Draft: grow the tree by path value, expand the best k newest nodes per
 * step, rerank everything generated to the best m and flatten it with an
 * ancestry mask ("EAGLE-2: Context-Aware Dynamic Draft Trees", sections
 * "Path Value Ranks Prefixes, Not Isolated Tokens", "Global Reranking
 * Separates Exploration from Verification", "The Mask Preserves Tree
 * Semantics in One Target Pass"; a static tree when the config says so:
 * "Lesson 13.11", section "EAGLE-2 and dynamic draft trees").
 * Runs the draft passes and the rerank of one cycle for every lane (each
 * lane READY -> DRAFTED). If `out` is not NULL the call synchronises and
 * fills it with lane 0's tree. */
eagle_status eagle_draft_tree(eagle_ctx* ctx, eagle_tree* out);
/* Copies lane `lane`'s drafted tree (state DRAFTED) to `out`. Synchronises. */
eagle_status eagle_read_tree(eagle_ctx* ctx, int32_t lane, eagle_tree* out);

/* Verify: one target pass over the flattened tree, accept from the root
 * while the drafted token equals the target's greedy choice, add the
 * target's own token, and carry the accepted path's KV and features into
 * the next cycle ("Lesson 13.11", section "Speculative decoding in four
 * moves"; "EAGLE-2: Context-Aware Dynamic Draft Trees", section "Putting It
 * Together": verifier, next verified state).
 * Verifies the drafted tree (state DRAFTED), or `planted` when not NULL
 * (state READY or DRAFTED; only n_rows, token and parent are read, rows must
 * be in order with parent[r] < r, siblings with distinct tokens, n_rows <=
 * 1 + budget, depth <= the config depth; token[0] is ignored and taken as
 * the root). Target pass over the rows with the ancestry mask, greedy
 * acceptance, KV compaction of the accepted path, and the draft catch-up.
 * State -> READY. If out_tokens (capacity EAGLE_MAX_DEPTH + 1) or
 * n_committed is not NULL the call synchronises and writes the L + 1
 * tokens committed by this cycle. EAGLE_E_CAPACITY if the context could
 * exceed max_ctx. */
eagle_status eagle_verify(eagle_ctx* ctx, const eagle_tree* planted, int32_t* out_tokens,
                          int32_t* n_committed);
/* Batch form of eagle_verify (any batch; no planted tree): verifies every
 * lane's drafted tree in one target pass and returns once every lane's
 * acceptance result is known. Lane b's L_b + 1 committed tokens go to
 * out_tokens[b * (EAGLE_MAX_DEPTH + 1) ...] (capacity batch *
 * (EAGLE_MAX_DEPTH + 1)) and the count to n_committed[b] (capacity batch);
 * either may be NULL. eagle_verify itself is the batch-1 call
 * (EAGLE_E_STATE when batch > 1), and so is eagle_generate. */
eagle_status eagle_verify_batch(eagle_ctx* ctx, int32_t* out_tokens, int32_t* n_committed);

/* Generate: the draft-verify loop until max_new tokens, whose output equals
 * plain greedy decoding of the target ("Lesson 13.11", sections "Speculative
 * decoding in four moves" and "The big idea"; budget 0 is plain decoding,
 * one token per target pass: the measurement baseline).
 * eagle_prefill, then cycles until at least max_new tokens are committed
 * (the prefill's token is the first); writes exactly max_new tokens to out
 * (capacity max_new) and their count to n_out. stats may be NULL. */
eagle_status eagle_generate(eagle_ctx* ctx, const int32_t* prompt, int32_t n, int32_t max_new,
                            int32_t* out, int32_t* n_out, eagle_stats* stats);

/* Copies the committed tokens of lane 0's sequence (prefill's first) to
 * out (capacity cap); *n gets the total count. Host-side copy. */
eagle_status eagle_committed(eagle_ctx* ctx, int32_t* out, int32_t cap, int32_t* n);
/* eagle_committed for lane `lane`. */
eagle_status eagle_committed_lane(eagle_ctx* ctx, int32_t lane, int32_t* out, int32_t cap,
                                  int32_t* n);

/* Debug read-back of the last target or draft pass, for parity tests:
 * what = 0: target features f [rows, hidden] fp32 of the last target pass;
 * what = 1: target logits [rows, vocab] fp32 of the last verify pass
 *           (recorded after eagle_set_debug(ctx, 1), and always when
 *           sampling); a batch's verify rows are lane by lane;
 * what = 2: greedy choice g [rows] int32 of the last verify pass;
 * what = 3: top-1 minus top-2 logit [rows] fp32 of the last verify pass.
 * Copies min(bytes, available) and writes the row count. Synchronises. */
eagle_status eagle_debug_read(eagle_ctx* ctx, int32_t what, void* host_dst, uint64_t bytes,
                              int32_t* rows);
eagle_status eagle_set_debug(eagle_ctx* ctx, int32_t on);

/* Changes the sampling temperature and seed of a loaded context (the fields
 * of eagle_config of the same names; temperature 0 = greedy). Takes effect
 * at the next call; eagle_prefill restarts the draw steps at 0, a change
 * between cycles keeps the step count. EAGLE_E_INVALID for a temperature
 * outside [0, 1e4] or, when > 0, a vocabulary above 131072. */
eagle_status eagle_set_sampling(eagle_ctx* ctx, float temperature, uint32_t seed_lo,
                                uint32_t seed_hi);

/* Profiling: launches of the enabled classes are bracketed by HIP events on
 * the context's stream; eagle_profile_read synchronises and reports, per
 * class, the bracketed launches, their summed device time and the
 * algorithmic bytes those launches must move (weights read once, activation
 * operands and outputs). eagle_profile_enable takes a bit mask of classes
 * (bit i enables class i; 0 turns profiling off, EAGLE_PROF_ALL enables every
 * class) and a stride `every` >= 1: only one launch in `every` of each class
 * is bracketed, which bounds the cost on a timed run (each bracketed launch
 * adds a few microseconds of stream time). Enabling resets the totals. The
 * single-dispatch projection classes (GEMM, SWIGLU, DRAFT) carry their events
 * on the dispatch itself, so their interval is the kernel's own run time. */
enum {
  EAGLE_PROF_GEMM = 0,      /* target layers: q|k|v, o and down projections (split-K planes) */
  EAGLE_PROF_ATTN = 1,      /* tree-masked attention and its chunk combine */
  EAGLE_PROF_LMHEAD = 2,    /* LM head with argmax or softmax/top-k */
  EAGLE_PROF_ROWS = 3,      /* embedding, norms, RoPE + KV append, gathers */
  EAGLE_PROF_TREE = 4,      /* tree expansion/rerank and acceptance */
  EAGLE_PROF_KV = 5,        /* KV compaction */
  EAGLE_PROF_SWIGLU = 6,    /* target layers: fused gate/up projection and SiLU product */
  EAGLE_PROF_DRAFT = 7,     /* draft head projections: FC, q|k|v, o, gate/up, down */
  EAGLE_PROF_CLASSES = 8
};
#define EAGLE_PROF_ALL 0xffffffffu
typedef struct eagle_profile {
  int64_t launches[EAGLE_PROF_CLASSES];
  double ms[EAGLE_PROF_CLASSES];
  double bytes[EAGLE_PROF_CLASSES];
} eagle_profile;
eagle_status eagle_profile_enable(eagle_ctx* ctx, uint32_t class_mask, int32_t every);
eagle_status eagle_profile_read(eagle_ctx* ctx, eagle_profile* out);

void eagle_free(eagle_ctx* ctx);
const char* eagle_last_error(const eagle_ctx* ctx);
const char* eagle_status_string(eagle_status s);

#ifdef __cplusplus
}
#endif
#endif /* EAGLE_H */
