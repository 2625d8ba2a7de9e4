/*
 * eagle_ops.h - kernel-level entry points of libeagle.so on caller device
 * pointers, for composing other pipelines and for parity testing of the
 * kernels on their own. All calls enqueue on `stream` (NULL = default)
 * and do not synchronise; pointers are device pointers unless stated.
 * Element type `dtype` is EAGLE_F32 or EAGLE_BF16 (raw bf16 bits) of the
 * weights; bf16 weights are passed fragment-packed (eagle_op_pack), fp32
 * weights row-major. Activations are fp32 values: for EAGLE_F32 one fp32 array; for
 * EAGLE_BF16 two bf16 planes of the same shape, back to back, hi = bf16(v)
 * then lo = bf16(v - hi), which the kernels multiply as hi*w + lo*w.
 */
#ifndef EAGLE_OPS_H
#define EAGLE_OPS_H

#include <stdint.h>

#include "eagle.h"

#ifdef __cplusplus
extern "C" {
#endif

enum { EAGLE_EPI_STORE = 0, EAGLE_EPI_ADD = 1, EAGLE_EPI_SWIGLU = 2 };

/* Fragment packing of a bf16 weight W [N, K] (K a multiple of 32), the form
 * every bf16 weight argument below must be in. Row block b (rows 16b ..
 * 16b+15, for b < N/16) keeps its row-major byte range and is stored as K/32
 * fragments of 16 x 32 elements, fragment s at element offset
 * (16 b K + 512 s): lane l = r + 16 g of the fragment (r < 16, g < 4) holds
 * the 8 elements W[16b + r][32s + 8g .. 32s + 8g + 7] at offset 8 l. The
 * last N % 16 rows are copied unchanged (they stay row-major). src and dst
 * are device pointers to non-overlapping N*K-element buffers. The kernels
 * stream one 1 KB fragment per wave load, which the 16x16x32 bf16 MFMA takes
 * as its A operand without reshuffling. EAGLE_E_INVALID on bad sizes or
 * overlapping buffers, EAGLE_E_HIP on a launch failure. */
eagle_status eagle_op_pack(const void* src, void* dst, int32_t N, int32_t K, void* stream);

/* Workspace bytes eagle_op_linear needs for this shape (0 for a bad shape,
 * or when the shape needs none). The workspace holds the split-K partial
 * planes of one call; every byte a call reads there it has written first,
 * so it needs no clearing and carries nothing between calls. */
uint64_t eagle_op_linear_workspace(int32_t dtype, int32_t epilogue, int32_t M, int32_t N, int32_t K);

/* Projection of M activation rows by a weight W, as in a Linear layer
 * (y = x W^T; the decode/verify projections of the target and draft
 * decoder layers, "Lesson 13.11 - EAGLE", section "The big idea").
 *   x: [M, K] activations, row-major. W: [N, K] dtype (EPI_SWIGLU: [2N, K],
 *   the N gate rows then the N up rows).
 *   EPI_STORE : y fp32 [M, N],  y  = x W^T
 *   EPI_ADD   : y fp32 [M, N],  y += x W^T  (residual update)
 *   EPI_SWIGLU: y [M, N] activations, y = silu(x Wg^T) * (x Wu^T)
 * Accumulation is fp32; summation order is fixed, so results repeat
 * bit for bit. Requires K a multiple of 32 (bf16) or 16 (fp32), M >= 1,
 * and for bf16 EPI_SWIGLU N a multiple of 16 (gate and up blocks align).
 * EAGLE_E_INVALID on bad sizes, EAGLE_E_BUFFER if the workspace is too
 * small, EAGLE_E_HIP on a launch failure. */
eagle_status eagle_op_linear(int32_t dtype, int32_t epilogue, const void* x, const void* w, void* y,
                             int32_t M, int32_t N, int32_t K, void* workspace, uint64_t ws_bytes,
                             void* stream);

/* Workspace bytes eagle_op_norm_linear needs for this shape (0 for a bad
 * shape). It holds the normed operand, the per-row sums of squares and the
 * projection's partial planes of one call; every byte a call reads there it
 * has written first. */
uint64_t eagle_op_norm_linear_workspace(int32_t epilogue, int32_t M, int32_t N, int32_t H);

/* The pre-norm step of a decoder layer in the Llama layout the models follow
 * (eagle_config): the residual update, RMSNorm, and the projection that
 * reads the normed rows -- the q|k|v and gate|up inputs of every target and
 * draft layer ("Lesson 13.11 - EAGLE", section "The big idea": the draft
 * head is one such decoder layer). bf16, in the form the layers run it: the
 * norm is spread over four workgroups per row, which write gain * h and
 * each quarter row's sum of squares, and the projection multiplies its
 * output rows by the rows' RMSNorm factors.
 *   h: [M, H] fp32 residual rows, updated in place:
 *      h += part[0] + ... + part[S-1]  (planes of [M, H] fp32, plane s at
 *      part + s*M*H, added in plane order; S may be 0, then part may be NULL)
 *   gain: [H] fp32. w: bf16 packed by eagle_op_pack, [N, H] (EPI_SWIGLU:
 *      [2N, H], the N gate rows then the N up rows).
 *   x = RMSNorm(h) * gain, RMSNorm(h) = h / sqrt(mean(h^2) + eps)
 *   EPI_STORE : y fp32 [M, N] = x w^T
 *   EPI_SWIGLU: y [M, N] bf16 operand (hi plane, then the lo plane M*N
 *               elements later) = silu(x wg^T) * (x wu^T)
 * Accumulation is fp32 in a fixed order, so results repeat bit for bit.
 * Requires M >= 1, N >= 1 (EPI_SWIGLU: a multiple of 16) and H a multiple
 * of 1024, at most 16384. EAGLE_E_INVALID on bad sizes or a NULL pointer,
 * EAGLE_E_BUFFER if the workspace is too small, EAGLE_E_HIP on a launch
 * failure. */
eagle_status eagle_op_norm_linear(int32_t epilogue, float* h, const float* part, int32_t S,
                                  const float* gain, float eps, const void* w, void* y, int32_t M,
                                  int32_t N, int32_t H, void* workspace, uint64_t ws_bytes,
                                  void* stream);

/* Largest workspace eagle_op_linear_noalloc can serve (32 MiB). */
#define EAGLE_OP_NOALLOC_SCRATCH_BYTES (32ull << 20)

/* eagle_op_linear without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, results (bit for bit)
 * and kernels as eagle_op_linear; the partial planes go to a fixed array of
 * EAGLE_OP_NOALLOC_SCRATCH_BYTES that the library holds on each device it
 * runs on until the process ends. The call allocates nothing. It runs on
 * the device current at the call (the stream must belong to it). Every call
 * on one device shares that device's array, so calls that may overlap on a
 * device (different streams, or host threads) race; calls on one stream are
 * ordered and safe. EAGLE_E_CAPACITY, before any launch, if the shape needs
 * more than EAGLE_OP_NOALLOC_SCRATCH_BYTES (eagle_op_linear_workspace gives
 * the need); EAGLE_E_INVALID on bad sizes; EAGLE_E_HIP if the array's
 * address cannot be obtained or a launch fails. */
eagle_status eagle_op_linear_noalloc(int32_t dtype, int32_t epilogue, const void* x, const void* w,
                                     void* y, int32_t M, int32_t N, int32_t K, void* stream);

/* Workspace bytes of eagle_op_lmhead (k = 0 for the greedy variant). */
uint64_t eagle_op_lmhead_workspace(int32_t M, int32_t V, int32_t k);

/* LM head over M feature rows x [M, H] (activations) with W_lm [V, H] ("Lesson 13.11",
 * section "The big idea": the LM head turns a feature into probabilities).
 *   k = 0 (verify): out_ids[m] = argmax_v logits (lowest id on ties),
 *          out_vals[m] = top-1 minus top-2 logit; logits [M, V] fp32 are
 *          also written when `logits` is not NULL.
 *   k >= 1 (draft): out_ids [M, k] = the k best ids by (logit desc, id asc),
 *          out_vals [M, k] = their log-probabilities over the full vocabulary
 *          (EAGLE-2 page, "Calibration Makes Acceptance Estimation Cheap":
 *          the draft confidence is the draft probability).
 * Requires H a multiple of 32 (bf16) or 16 (fp32), 1 <= k <= 16. */
eagle_status eagle_op_lmhead(int32_t dtype, int32_t k, const void* x, const void* w_lm, int32_t M,
                             int32_t V, int32_t H, int32_t* out_ids, float* out_vals, float* logits,
                             void* workspace, uint64_t ws_bytes, void* stream);

/* Keys per page of the paged KV layout eagle_op_attention reads. */
#define EAGLE_OP_KV_PAGE 64

/* Workspace bytes of eagle_op_attention (per-chunk partial outputs and
 * softmax statistics of the split-KV form; 0 for EAGLE_F32). */
uint64_t eagle_op_attention_workspace(int32_t dtype, int32_t M, int32_t n_heads, int32_t head_dim,
                                      int32_t key_end);

/* Tree-masked attention of M query rows over one layer's paged KV cache: the
 * verify pass's attention ("EAGLE-2: Context-Aware Dynamic Draft Trees",
 * section "The Mask Preserves Tree Semantics in One Target Pass": each
 * flattened row sees the context, its ancestors and itself), and the causal
 * attention of prefill rows when there are no tree keys.
 *   q: [M, n_heads * head_dim] query operand after RoPE (bf16: hi plane then
 *      lo plane, see above; fp32: one array).
 *   kv: the cache; key slot s of KV head h, plane p, element i lives at
 *      page_table[s / 64] * (planes * n_kv_heads * 64 * head_dim)
 *        + (p * n_kv_heads + h) * 64 * head_dim + (s % 64) * head_dim + i
 *      with planes K_hi, K_lo, V_hi, V_lo (bf16 raw bits; value = hi + lo) or
 *      K, V (fp32), except that bf16 V planes are transposed within the page:
 *      element i of slot s of V_hi or V_lo lives at
 *        ... + (p * n_kv_heads + h) * 64 * head_dim + i * 64 + s % 64.
 *      page_table: device int32 [key_end / 64 rounded up]. bf16 reads whole
 *      pages: the keys of the first page below pre_lo and of the last page
 *      from key_end on are read and masked, so those slots need no set
 *      contents.
 *   Row r sees key slots [pre_lo, prehi[r]) and the tree slots tree_base + j
 *   (j < n_tree <= 128) whose bit j is set in tree_mask[2r] (j < 64) or
 *   tree_mask[2r + 1] (j >= 64); key_end = one past the last slot any row
 *   sees. prehi [M] int32 and tree_mask [2M] uint64 are device arrays
 *   (tree_mask is read for every row: all zero when n_tree = 0). Query head j reads KV head
 *   j / (n_heads / n_kv_heads) (GQA).
 *   out: [M, n_heads * head_dim] softmax(q k^T * scale) v over the visible
 *      keys, as an operand (bf16: hi and lo planes; fp32: one array).
 * page_table has one entry per 64 slots up to key_end (rounded up), each a
 * page index inside kv: the kernels read whole 64-slot chunks, masked slots
 * included. Requires head_dim = 128 for EAGLE_BF16 (<= 256 for EAGLE_F32),
 * every row with at least one visible key, and key_end - pre_lo <= 131072
 * (2048 chunks of 64 keys). With bf16, no
 * tree keys, M >= 32 and at most 8 query heads per KV head it runs the
 * one-pass (flash) form; otherwise split-KV chunks of 64 keys and a combine.
 * EAGLE_E_INVALID on bad sizes, EAGLE_E_BUFFER if the workspace is too small,
 * EAGLE_E_HIP on a launch failure. */
eagle_status eagle_op_attention(int32_t dtype, const void* q, const void* kv,
                                const int32_t* page_table, int32_t n_kv_heads, int32_t n_heads,
                                int32_t head_dim, int32_t M, int32_t pre_lo, const int32_t* prehi,
                                const uint64_t* tree_mask, int32_t tree_base, int32_t n_tree,
                                int32_t key_end, float scale, void* out, void* workspace,
                                uint64_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* EAGLE_OPS_H */
