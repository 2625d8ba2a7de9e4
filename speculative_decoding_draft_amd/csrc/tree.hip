// EAGLE-2 tree policy on the device: path values in log space, expansion
// of the best newest nodes, global rerank to a connected top-m, flattening
// with ancestry masks, and the greedy acceptance walk. Each kernel is one
// workgroup; all decisions use fixed total orders on fp32 keys:
//   expansion: (log V desc, generation asc)
//   rerank:    (log V desc, depth asc, generation asc)
//   rows:      (depth asc, rerank order)
#include "eagle.h"
#include "common.h"
#include "kernels.h"

namespace {

// the rerank's LDS arrays hold every node a cycle can generate and every
// verify row a cycle can have
static_assert(EAGLE_MAX_NODES <= TREE_MAXN && EAGLE_MAX_STATIC <= TREE_MAXN, "node arrays");
static_assert(EAGLE_MAX_VERIFY <= TREE_MAXROWS && EAGLE_MAX_STATIC < TREE_MAXROWS, "row arrays");

// Sequence b's tree state: every array of sequence 0's shifted by b * bytes.
__device__ __forceinline__ TreeDev tree_lane(TreeDev t, int b, int64_t bytes) {
  if (b == 0) return t;
  t.tok = lane_at(t.tok, b, bytes);
  t.parent = lane_at(t.parent, b, bytes);
  t.depth = lane_at(t.depth, b, bytes);
  t.srcrow = lane_at(t.srcrow, b, bytes);
  t.rank = lane_at(t.rank, b, bytes);
  t.row_of_node = lane_at(t.row_of_node, b, bytes);
  t.logv = lane_at(t.logv, b, bytes);
  t.logp = lane_at(t.logp, b, bytes);
  t.counts = lane_at(t.counts, b, bytes);
  t.exp_nodes = lane_at(t.exp_nodes, b, bytes);
  t.row_tok = lane_at(t.row_tok, b, bytes);
  t.row_src = lane_at(t.row_src, b, bytes);
  t.row_pos = lane_at(t.row_pos, b, bytes);
  t.row_slot = lane_at(t.row_slot, b, bytes);
  t.row_prehi = lane_at(t.row_prehi, b, bytes);
  t.row_mask = lane_at(t.row_mask, b, bytes);
  t.tmask = lane_at(t.tmask, b, bytes);
  t.v_tok = lane_at(t.v_tok, b, bytes);
  t.v_parent = lane_at(t.v_parent, b, bytes);
  t.v_depth = lane_at(t.v_depth, b, bytes);
  t.v_node = lane_at(t.v_node, b, bytes);
  t.v_pos = lane_at(t.v_pos, b, bytes);
  t.v_slot = lane_at(t.v_slot, b, bytes);
  t.v_prehi = lane_at(t.v_prehi, b, bytes);
  t.v_logv = lane_at(t.v_logv, b, bytes);
  t.v_mask = lane_at(t.v_mask, b, bytes);
  t.s_parent = lane_at(t.s_parent, b, bytes);
  t.s_rank = lane_at(t.s_rank, b, bytes);
  t.s_depth = lane_at(t.s_depth, b, bytes);
  t.s_prow = lane_at(t.s_prow, b, bytes);
  t.s_exp = lane_at(t.s_exp, b, bytes);
  t.s_nexp = lane_at(t.s_nexp, b, bytes);
  return t;
}

__device__ __forceinline__ void set_bit(uint64_t* m, int j) {
  if (j < 64) m[0] |= (1ull << j);
  else m[1] |= (1ull << (j - 64));
}

__global__ __launch_bounds__(256) void tree_append_kernel(TreeDev t, TreeParams p,
                                                          const int32_t* ids, const float* lps,
                                                          int pass, int ctx,
                                                          const int32_t* ctx_len, Lanes ln,
                                                          int64_t ids_stride) {
  __shared__ int s_base, s_nrows, s_nnew, s_nsel, s_tbase;
  __shared__ int sel[TREE_MAXEXP];
  // the new generation (dynamic tree) in LDS: expansion keys, ranked from
  // here, and the token, source row and source-row mask the next pass's rows
  // take, so no row waits on a device re-read
  constexpr int NNEW = TREE_MAXEXP * EAGLE_MAX_TOPK;
  __shared__ uint32_t s_key[NNEW];
  __shared__ int s_tok[NNEW], s_src[NNEW];
  __shared__ uint64_t s_pm[2 * NNEW];
  const int tid = threadIdx.x;
  // this workgroup's sequence
  const int b = blockIdx.x;
  t = tree_lane(t, b, ln.bytes);
  ids += b * ids_stride;
  lps += b * ids_stride;
  ctx += lane_shift(ln, b);
  if (ctx_len) ctx_len = lane_at(ctx_len, b, ln.bytes);
  if (ctx_len) ctx += ctx_len[0] + 1;   // the root sits after the ctx_len[0] + 1 tokens just committed
  if (tid == 0) {
    if (pass == 1) {
      t.counts[0] = 0;
      t.counts[1] = 1;
      t.counts[2] = 0;
      t.counts[3] = 0;
    }
    s_base = t.counts[0];
    s_nrows = t.counts[1];
    s_tbase = t.counts[2];
  }
  __syncthreads();
  const int base = s_base, nrows = s_nrows;
  const int k = p.k_b;

  if (p.dynamic) {
    // children of row i: generation base + i*k + r
    for (int e = tid; e < nrows * k; e += blockDim.x) {
      const int i = e / k, r = e % k;
      const int gen = base + e;
      const int par = (pass == 1) ? -1 : t.exp_nodes[i];
      const float lp = lps[i * k + r];
      const float lv = (par < 0) ? lp : (t.logv[par] + lp);
      const int tok = ids[i * k + r];
      const int src = (par < 0) ? 0 : 1 + t.row_of_node[par];
      uint64_t m0 = 0ull, m1 = 0ull;
      if (src > 0) { m0 = t.tmask[2 * (src - 1)]; m1 = t.tmask[2 * (src - 1) + 1]; }
      t.tok[gen] = tok;
      t.parent[gen] = par;
      t.depth[gen] = pass;
      t.rank[gen] = r;
      t.logp[gen] = lp;
      t.logv[gen] = lv;
      t.srcrow[gen] = src;
      t.row_of_node[gen] = -1;
      s_key[e] = ~float_key(lv);
      s_tok[e] = tok;
      s_src[e] = src;
      s_pm[2 * e] = m0;
      s_pm[2 * e + 1] = m1;
    }
    if (tid == 0) { s_nnew = nrows * k; t.counts[0] = base + nrows * k; }
  } else {
    // static: nodes of depth `pass`, in list order
    for (int j = tid; j < p.n_static; j += blockDim.x) {
      if (t.s_depth[j] != pass) continue;
      const int par = t.s_parent[j];
      const int i = t.s_prow[j];
      const int r = t.s_rank[j];
      const float lp = lps[i * k + r];
      t.tok[j] = ids[i * k + r];
      t.parent[j] = par;
      t.depth[j] = pass;
      t.rank[j] = r;
      t.logp[j] = lp;
      t.logv[j] = (par < 0) ? lp : (t.logv[par] + lp);
      t.srcrow[j] = (par < 0) ? 0 : 1 + t.row_of_node[par];
      t.row_of_node[j] = -1;
    }
    if (tid == 0) {
      int n = 0;
      for (int j = 0; j < p.n_static; ++j) n += (t.s_depth[j] <= pass);
      t.counts[0] = n;
    }
  }
  __syncthreads();
  if (pass >= p.depth) return;

  // choose the nodes the next pass expands
  if (p.dynamic) {
    const int nnew = s_nnew;
    if (tid == 0) s_nsel = min(p.k_e, nnew);
    for (int e = tid; e < nnew; e += blockDim.x) {
      const uint32_t ki = s_key[e];
      int rank = 0;
      for (int f = 0; f < nnew; ++f) {
        const uint32_t kf = s_key[f];
        rank += (kf < ki) || (kf == ki && f < e);
      }
      if (rank < p.k_e) sel[rank] = base + e;
    }
  } else {
    if (tid == 0) s_nsel = t.s_nexp[pass];
    for (int i = tid; i < TREE_MAXEXP; i += blockDim.x)
      if (i < t.s_nexp[pass]) sel[i] = t.s_exp[pass * TREE_MAXEXP + i];
  }
  __syncthreads();
  const int nsel = s_nsel;
  // tree rows are appended in order; masks need the parent row's mask,
  // which belongs to an earlier pass, so rows of this pass are independent
  for (int i = tid; i < nsel; i += blockDim.x) {
    const int e = sel[i];
    const int tr = s_tbase + i;
    int tok, src, dep;
    uint64_t m[2] = {0ull, 0ull};
    if (p.dynamic) {   // a node of the generation written above
      const int le = e - base;
      tok = s_tok[le];
      src = s_src[le];
      dep = pass;
      m[0] = s_pm[2 * le];
      m[1] = s_pm[2 * le + 1];
    } else {
      tok = t.tok[e];
      src = t.srcrow[e];
      dep = t.depth[e];
      if (src > 0) { m[0] = t.tmask[2 * (src - 1)]; m[1] = t.tmask[2 * (src - 1) + 1]; }
    }
    t.exp_nodes[i] = e;
    t.row_of_node[e] = tr;
    t.row_tok[i] = tok;
    t.row_src[i] = src;
    t.row_pos[i] = ctx + dep;
    t.row_slot[i] = ctx + 1 + tr;
    t.row_prehi[i] = ctx + 1;
    set_bit(m, tr);
    t.tmask[2 * tr] = m[0];
    t.tmask[2 * tr + 1] = m[1];
    t.row_mask[2 * i] = m[0];
    t.row_mask[2 * i + 1] = m[1];
  }
  if (tid == 0) {
    t.counts[1] = nsel;
    t.counts[2] = s_tbase + nsel;
  }
}

// masks for verify rows whose parents precede them (level order not needed);
// vpar: the rows' parent rows (LDS in the rerank, the device array otherwise)
__device__ __forceinline__ void build_masks(TreeDev& t, int n, int ctx, const int* vpar) {
  // depth by pointer chasing (n <= 128, depth <= 16)
  for (int r = threadIdx.x; r < n; r += blockDim.x) {
    uint64_t m[2] = {0ull, 0ull};
    int d = 0;
    for (int a = r; a >= 0; a = vpar[a]) {
      set_bit(m, a);
      if (a != 0) ++d;
      if (a == 0) break;
    }
    t.v_mask[2 * r] = m[0];
    t.v_mask[2 * r + 1] = m[1];
    t.v_depth[r] = d;
    t.v_pos[r] = ctx + d;
    t.v_slot[r] = ctx + r;
    t.v_prehi[r] = ctx;
  }
}

__global__ __launch_bounds__(1024) void tree_finalize_kernel(TreeDev t, TreeParams p, int ctx,
                                                             const int32_t* root_token, Lanes ln) {
  __shared__ uint64_t keys[TREE_MAXN];
  __shared__ int kept[TREE_MAXROWS], kdep[TREE_MAXROWS], vpar[TREE_MAXROWS];
  __shared__ int row_of[TREE_MAXN];   // verify row of each kept node, -1 otherwise
  __shared__ int s_n, s_m;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int sh = lane_shift(ln, b);
  t = tree_lane(t, b, ln.bytes);
  ctx += sh;
  root_token = lane_at(root_token, b, ln.bytes) + sh;
  if (tid == 0) {
    s_n = t.counts[0];
    s_m = p.dynamic ? min(p.budget, s_n) : s_n;
  }
  __syncthreads();
  const int n = s_n, m = s_m;
  for (int i = tid; i < n; i += blockDim.x) row_of[i] = -1;
  if (p.dynamic) {
    // bitonic sort, ascending, of the first power of two >= n keys (padding
    // keys ~0 sort last, as they would in any longer sort)
    int np2 = 2;
    while (np2 < n) np2 <<= 1;
    for (int i = tid; i < np2; i += blockDim.x) {
      keys[i] = (i < n) ? (((uint64_t)(~float_key(t.logv[i])) << 32) |
                           ((uint64_t)t.depth[i] << 20) | (uint64_t)i)
                        : ~0ull;
    }
    __syncthreads();
    for (int size = 2; size <= np2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < np2; i += blockDim.x) {
          const int j = i ^ stride;
          if (j > i) {
            const bool up = (i & size) == 0;
            const uint64_t a = keys[i], b = keys[j];
            if ((a > b) == up) { keys[i] = b; keys[j] = a; }
          }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < m; i += blockDim.x) kept[i] = (int)(keys[i] & 0xFFFFF);
  } else {
    for (int i = tid; i < m; i += blockDim.x) kept[i] = i;
  }
  __syncthreads();
  for (int i = tid; i < m; i += blockDim.x) kdep[i] = t.depth[kept[i]];
  __syncthreads();
  // row of kept node i: 1 + #{kept j with (depth, order) smaller}
  for (int i = tid; i < m; i += blockDim.x) {
    const int di = kdep[i];
    int c = 0;
    for (int j = 0; j < m; ++j) {
      const int dj = kdep[j];
      c += (dj < di) || (dj == di && j < i);
    }
    row_of[kept[i]] = 1 + c;
  }
  __syncthreads();
  for (int i = tid; i < m; i += blockDim.x) {
    const int nd = kept[i];
    const int r = row_of[nd];
    const int par = t.parent[nd];
    const int pr = (par < 0) ? 0 : row_of[par];
    t.v_tok[r] = t.tok[nd];
    t.v_node[r] = nd;
    t.v_logv[r] = t.logv[nd];
    t.v_parent[r] = pr;
    vpar[r] = pr;
  }
  if (tid == 0) {
    t.v_tok[0] = *root_token;
    t.v_node[0] = -1;
    t.v_logv[0] = 0.f;
    t.v_parent[0] = -1;
    vpar[0] = -1;
    t.counts[3] = 1 + m;
  }
  __syncthreads();
  build_masks(t, 1 + m, ctx, vpar);
}

__global__ __launch_bounds__(128) void tree_masks_kernel(TreeDev t, int n_rows, int ctx,
                                                        const int32_t* root, Lanes ln) {
  const int b = blockIdx.x;
  const int sh = lane_shift(ln, b);
  t = tree_lane(t, b, ln.bytes);
  ctx += sh;
  root = lane_at(root, b, ln.bytes) + sh;
  if (threadIdx.x == 0) {
    t.v_tok[0] = *root;
    t.v_parent[0] = -1;
    t.counts[3] = n_rows;
  }
  __syncthreads();
  build_masks(t, n_rows, ctx, t.v_parent);
}

// Walks the verified tree from the root: at each step the child whose token
// equals the target's greedy choice at the current row is accepted. Besides
// the device copies (acc, new_tok, cu_src) lane 0 writes the committed tokens
// into the sequence (seq_out) and, when `host` is not NULL, the length and the
// tokens into mapped host memory, then raises host[0] to `tag` after a
// system-scope fence, so the host can read the result while the stream runs on.
__global__ __launch_bounds__(64) void accept_kernel(TreeDev t, const int32_t* g, int max_depth,
                                                    int32_t* acc, int32_t* new_tok, int32_t* cu_src,
                                                    int32_t* seq_out, int32_t* host, int32_t tag,
                                                    Lanes ln, int64_t g_stride, int64_t host_stride) {
  const int lane = threadIdx.x;
  // this workgroup's sequence
  const int b = blockIdx.x;
  t = tree_lane(t, b, ln.bytes);
  g += b * g_stride;
  acc = lane_at(acc, b, ln.bytes);
  new_tok = lane_at(new_tok, b, ln.bytes);
  cu_src = lane_at(cu_src, b, ln.bytes);
  seq_out = lane_at(seq_out, b, ln.bytes) + lane_shift(ln, b);
  if (host) host += b * host_stride;
  const int n = t.counts[3];
  int cur = 0, L = 0;
  for (int step = 0; step < max_depth; ++step) {
    const int want = g[cur];
    int found = 0x7fffffff;
    for (int r = 1 + lane; r < n; r += 64)
      if (t.v_parent[r] == cur && t.v_tok[r] == want) found = min(found, r);
    found = wave_min_i(found);
    if (found == 0x7fffffff) break;
    if (lane == 0) {
      acc[2 + L] = found;
      new_tok[L] = want;
      cu_src[L + 1] = found;
      seq_out[L] = want;
      if (host) host[2 + L] = want;
    }
    cur = found;
    ++L;
  }
  if (lane == 0) {
    const int bonus = g[cur];
    acc[0] = L;
    acc[1] = bonus;
    new_tok[L] = bonus;
    cu_src[0] = 0;
    seq_out[L] = bonus;
    // rows L+1 .. max_depth of a fixed-size catch-up: valid tokens and sources
    for (int j = L + 1; j <= max_depth; ++j) {
      new_tok[j] = bonus;
      cu_src[j] = 0;
    }
    if (host) {
      host[2 + L] = bonus;
      host[1] = L;
      __threadfence_system();
      *reinterpret_cast<volatile int32_t*>(host) = tag;
    }
  }
}

}  // namespace

static bool lanes_bad(const Lanes& ln) { return ln.n < 1 || ln.n > MAX_LANES; }

hipError_t launch_tree_append(TreeDev t, TreeParams p, const int32_t* ids, const float* logp,
                              int pass, int ctx, hipStream_t st, const int32_t* ctx_len,
                              const Lanes& ln, int64_t ids_stride) {
  if (lanes_bad(ln)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tree_append_kernel, dim3(ln.n), dim3(256), 0, st, t, p, ids, logp, pass, ctx,
                     ctx_len, ln, ids_stride);
  return hipGetLastError();
}

hipError_t launch_tree_finalize(TreeDev t, TreeParams p, int ctx, const int32_t* root_token,
                                hipStream_t st, const Lanes& ln) {
  if (lanes_bad(ln)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tree_finalize_kernel, dim3(ln.n), dim3(1024), 0, st, t, p, ctx, root_token, ln);
  return hipGetLastError();
}

hipError_t launch_tree_masks(TreeDev t, int n_rows, int ctx, const int32_t* root_token,
                             hipStream_t st, const Lanes& ln) {
  if (lanes_bad(ln)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tree_masks_kernel, dim3(ln.n), dim3(128), 0, st, t, n_rows, ctx, root_token, ln);
  return hipGetLastError();
}

hipError_t launch_accept(TreeDev t, const int32_t* g, int max_depth, int32_t* acc,
                         int32_t* new_tok, int32_t* cu_src, int32_t* seq_out, int32_t* host,
                         int32_t tag, hipStream_t st, const Lanes& ln, int64_t g_stride,
                         int64_t host_stride) {
  if (lanes_bad(ln)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(accept_kernel, dim3(ln.n), dim3(64), 0, st, t, g, max_depth, acc, new_tok, cu_src,
                     seq_out, host, tag, ln, g_stride, host_stride);
  return hipGetLastError();
}
