// Kernel-level entry points (include/eagle_ops.h).
#include "eagle_ops.h"

#include <hip/hip_runtime.h>

#include <algorithm>

#include "kernels.h"

namespace {

uint64_t align256(uint64_t x) { return (x + 255) / 256 * 256; }

bool linear_ok(int32_t dtype, int32_t epi, int32_t M, int32_t N, int32_t K) {
  if (dtype != EAGLE_F32 && dtype != EAGLE_BF16) return false;
  if (epi < EAGLE_EPI_STORE || epi > EAGLE_EPI_SWIGLU) return false;
  if (dtype == EAGLE_BF16 && epi == EAGLE_EPI_SWIGLU && N % 16) return false;
  const int ks = dtype == EAGLE_BF16 ? 32 : 16;
  return M >= 1 && N >= 1 && K >= ks && K % ks == 0;
}
}  // namespace

extern "C" {

eagle_status eagle_op_pack(const void* src, void* dst, int32_t N, int32_t K, void* stream) {
  if (!src || !dst || N < 1 || K < 32 || K % 32) return EAGLE_E_INVALID;
  const uint64_t bytes = (uint64_t)N * K * 2;
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + bytes && b < a + bytes) return EAGLE_E_INVALID;
  hipStream_t st = (hipStream_t)stream;
  const int64_t nrb = N / 16;
  const uint64_t packed = (uint64_t)nrb * 16 * K * 2;
  hipError_t e = launch_pack_frag(src, dst, nrb, K, st);
  if (e == hipSuccess && packed < bytes)
    e = hipMemcpyAsync((char*)dst + packed, (const char*)src + packed, bytes - packed,
                       hipMemcpyDeviceToDevice, st);
  return e == hipSuccess ? EAGLE_OK : EAGLE_E_HIP;
}

uint64_t eagle_op_linear_workspace(int32_t dtype, int32_t epi, int32_t M, int32_t N, int32_t K) {
  if (!linear_ok(dtype, epi, M, N, K)) return 0;
  if (epi == EAGLE_EPI_SWIGLU) {
    if (!swiglu_by_planes(dtype, M)) return 0;
    GemmPlan p = gemm_plan(M, 2 * N, K, dtype, EPI_PART);
    return align256(gemm_part_floats(p, 2 * N, M) * 4);
  }
  GemmPlan p = gemm_plan(M, N, K, dtype, EPI_PART);
  return align256(gemm_part_floats(p, N, M) * 4);
}

eagle_status eagle_op_linear(int32_t dtype, int32_t epi, const void* x, const void* w, void* y,
                             int32_t M, int32_t N, int32_t K, void* workspace, uint64_t ws_bytes,
                             void* stream) {
  if (!linear_ok(dtype, epi, M, N, K) || !x || !w || !y) return EAGLE_E_INVALID;
  const uint64_t need = eagle_op_linear_workspace(dtype, epi, M, N, K);
  if (need > 0 && (!workspace || ws_bytes < need)) return EAGLE_E_BUFFER;
  const int64_t xlo = (int64_t)M * K;   // bf16: lo plane follows the hi plane
  hipStream_t st = (hipStream_t)stream;
  if (epi == EAGLE_EPI_SWIGLU) {
    hipError_t e = launch_gemm(dtype, EPI_SWIGLU, w, x, xlo, M, N, K, (float*)workspace, 2 * N, y,
                               (int64_t)M * N, nullptr, st);
    return e == hipSuccess ? EAGLE_OK : EAGLE_E_HIP;
  }
  float* part = (float*)workspace;
  int S = 1;
  hipError_t e = launch_gemm(dtype, EPI_PART, w, x, xlo, M, N, K, part, N, nullptr, 0, &S, st);
  if (e == hipSuccess)
    e = launch_sum_planes(part, S, (int64_t)M * N, M, N, (float*)y, epi == EAGLE_EPI_ADD ? 1 : 0, st);
  return e == hipSuccess ? EAGLE_OK : EAGLE_E_HIP;
}

uint64_t eagle_op_norm_linear_workspace(int32_t epi, int32_t M, int32_t N, int32_t H) {
  if (epi != EAGLE_EPI_STORE && epi != EAGLE_EPI_SWIGLU) return 0;
  if (!linear_ok(EAGLE_BF16, epi, M, N, H) || !resnorm_slices_fit(H)) return 0;
  const uint64_t x = align256((uint64_t)M * H * 2 * 2);   // hi and lo planes
  const uint64_t ss = align256((uint64_t)M * RS_SLICES * 4);
  uint64_t planes;
  if (epi == EAGLE_EPI_SWIGLU) {
    planes = swiglu_by_planes(EAGLE_BF16, M)
                 ? gemm_part_floats(gemm_plan(M, 2 * N, H, EAGLE_BF16, EPI_PART), 2 * N, M) * 4
                 : 0;
  } else {
    planes = gemm_part_floats(gemm_plan(M, N, H, EAGLE_BF16, EPI_PART), N, M) * 4;
  }
  return x + ss + align256(planes);
}

eagle_status eagle_op_norm_linear(int32_t epi, float* h, const float* part, int32_t S,
                                  const float* gain, float eps, const void* w, void* y, int32_t M,
                                  int32_t N, int32_t H, void* workspace, uint64_t ws_bytes,
                                  void* stream) {
  const uint64_t need = eagle_op_norm_linear_workspace(epi, M, N, H);
  if (need == 0 || S < 0 || !h || !gain || !w || !y || (S > 0 && !part)) return EAGLE_E_INVALID;
  if (!workspace || ws_bytes < need) return EAGLE_E_BUFFER;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  void* xop = ws;
  float* ss = (float*)(ws + align256((uint64_t)M * H * 2 * 2));
  float* planes = (float*)((char*)ss + align256((uint64_t)M * RS_SLICES * 4));
  const int64_t xlo = (int64_t)M * H;
  hipError_t e = launch_resnorm_slices(EAGLE_BF16, h, H, M, part, S, (int64_t)M * H, 0, gain, xop,
                                       xlo, ss, st);
  RowScale rs;
  rs.ss = ss;
  rs.H = H;
  rs.eps = eps;
  if (e == hipSuccess && epi == EAGLE_EPI_SWIGLU) {
    e = launch_gemm(EAGLE_BF16, EPI_SWIGLU, w, xop, xlo, M, N, H, planes, 2 * N, y, (int64_t)M * N,
                    nullptr, st, nullptr, rs);
  } else if (e == hipSuccess) {
    int SP = 1;
    e = launch_gemm(EAGLE_BF16, EPI_PART, w, xop, xlo, M, N, H, planes, N, nullptr, 0, &SP, st,
                    nullptr, rs);
    if (e == hipSuccess) e = launch_sum_planes(planes, SP, (int64_t)M * N, M, N, (float*)y, 0, st);
  }
  return e == hipSuccess ? EAGLE_OK : EAGLE_E_HIP;
}

uint64_t eagle_op_lmhead_workspace(int32_t M, int32_t V, int32_t k) {
  if (M < 1 || V < 1 || k < 0 || k > EAGLE_MAX_TOPK) return 0;
  return align256(lmhead_part_floats(M, V, k) * 4);
}

eagle_status eagle_op_lmhead(int32_t dtype, int32_t k, const void* x, const void* w_lm, int32_t M,
                             int32_t V, int32_t H, int32_t* out_ids, float* out_vals, float* logits,
                             void* workspace, uint64_t ws_bytes, void* stream) {
  if (dtype != EAGLE_F32 && dtype != EAGLE_BF16) return EAGLE_E_INVALID;
  const int ks = dtype == EAGLE_BF16 ? 32 : 16;
  if (!x || !w_lm || !out_ids || !out_vals || M < 1 || V < 1 || H < ks || H % ks || k < 0 ||
      k > EAGLE_MAX_TOPK || (k > 0 && k > V))
    return EAGLE_E_INVALID;
  if (!workspace || ws_bytes < eagle_op_lmhead_workspace(M, V, k)) return EAGLE_E_BUFFER;
  hipError_t e;
  if (k == 0)
    e = launch_lmhead_argmax(dtype, w_lm, x, (int64_t)M * H, M, V, H, (float*)workspace, out_ids,
                             out_vals, logits, (hipStream_t)stream);
  else
    e = launch_lmhead_topk(dtype, w_lm, x, (int64_t)M * H, M, V, H, k, (float*)workspace, out_ids,
                           out_vals, (hipStream_t)stream);
  return e == hipSuccess ? EAGLE_OK : EAGLE_E_HIP;
}

uint64_t eagle_op_attention_workspace(int32_t dtype, int32_t M, int32_t n_heads, int32_t head_dim,
                                      int32_t key_end) {
  if (dtype != EAGLE_BF16 || M < 1 || n_heads < 1 || head_dim < 1 || key_end < 1) return 0;
  const int64_t chunks = (key_end + attn_chunk_keys() - 1) / attn_chunk_keys();
  return align256(attn_part_floats((int)chunks, M, n_heads, head_dim) * 4);
}

eagle_status eagle_op_attention(int32_t dtype, const void* q, const void* kv,
                                const int32_t* page_table, int32_t n_kv_heads, int32_t n_heads,
                                int32_t head_dim, int32_t M, int32_t pre_lo, const int32_t* prehi,
                                const uint64_t* tree_mask, int32_t tree_base, int32_t n_tree,
                                int32_t key_end, float scale, void* out, void* workspace,
                                uint64_t ws_bytes, void* stream) {
  if (dtype != EAGLE_F32 && dtype != EAGLE_BF16) return EAGLE_E_INVALID;
  if (!q || !kv || !page_table || !prehi || !tree_mask || !out || M < 1 || n_kv_heads < 1 ||
      n_heads < n_kv_heads || n_heads % n_kv_heads || pre_lo < 0 || key_end <= pre_lo ||
      n_tree < 0 || n_tree > 128 ||
      (n_tree > 0 && (tree_base < pre_lo || tree_base + n_tree > key_end)))
    return EAGLE_E_INVALID;
  if (dtype == EAGLE_BF16 ? head_dim != 128 : (head_dim < 1 || head_dim > 256))
    return EAGLE_E_INVALID;
  // bf16 key chunks start on page boundaries at or below pre_lo
  const int ck = attn_chunk_keys();
  const int c0 = dtype == EAGLE_BF16 ? pre_lo / ck * ck : pre_lo;
  const int chunks = (key_end - c0 + ck - 1) / ck;
  if (chunks > attn_max_chunks()) return EAGLE_E_INVALID;
  const uint64_t need = eagle_op_attention_workspace(dtype, M, n_heads, head_dim, key_end);
  if (need > 0 && (!workspace || ws_bytes < need)) return EAGLE_E_BUFFER;
  KVView v;
  v.base = const_cast<void*>(kv);
  v.page_table = page_table;
  v.page = EAGLE_OP_KV_PAGE;
  v.n_kv = n_kv_heads;
  v.d = head_dim;
  v.page_elems = (int64_t)kv_planes(dtype) * n_kv_heads * EAGLE_OP_KV_PAGE * head_dim;
  RowVis vis{prehi, tree_mask, pre_lo, tree_base, n_tree, key_end};
  const int64_t width = (int64_t)n_heads * head_dim;
  float* opart = (float*)workspace;
  const int64_t kc = (key_end + attn_chunk_keys() - 1) / attn_chunk_keys();
  float* mlpart = opart ? opart + kc * M * width : nullptr;
  hipError_t e = launch_attention(dtype, q, (int64_t)M * width, v, vis, M, n_heads, head_dim, scale,
                                  opart, mlpart, out, (int64_t)M * width, (hipStream_t)stream);
  return e == hipSuccess ? EAGLE_OK : EAGLE_E_HIP;
}

}  // extern "C"
