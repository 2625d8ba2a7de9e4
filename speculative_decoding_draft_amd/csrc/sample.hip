// Sampling-mode (temperature > 0) acceptance over the verified tree and the
// prefill's sampled token.
//
// "EAGLE: Feature-Level Drafting for Faster Inference", section "Speculative
// decoding in four moves": with sampling, drafted tokens are kept while they
// pass the rejection-sampling test and the target corrects the first
// rejection; the output keeps the target's own distribution. EAGLE-2's page
// ("How it works", mask builder) applies the rule to the reranked tree. The
// tree's candidates are chosen deterministically, so each is proposed with
// probability one and the test accepts candidate x with probability p(x) / S:
// p = softmax(logits / T) at the current row, S the mass not yet rejected
// there. A rejected token leaves the distribution; children are tried in row
// order; with no child accepted the token is drawn from what is left.
//
// Random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11), key =
// the 64-bit seed, counter = (step, depth, draw, sequence), u = (word 0 >> 8)
// / 2^24; the sequence index (0 for a single sequence) gives each sequence
// of a batch its own stream.
// Decisions are taken in fp32: e = exp((l - max) / T), Z = fp64 sum of e
// rounded to fp32, p = e / Z, child test u * S < p(x). The residual walk
// accumulates e in fp64 in token order against (u * S) * Z.
//
// Two kernels: row_exp_kernel computes e for every verify row at once across
// the GPU (the row maximum is the logit of the greedy argmax the LM head
// already found) with an fp64 partial sum per 1024-token block; the
// one-workgroup walk then needs no exponentials, sums Z from the block
// partials, finds the residual's block from the block sums and scans only
// that block.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int NT = 1024;             // threads of the walk workgroup
constexpr int BLK = 1024;            // tokens per e-block (= NT: one per thread in a block scan)
constexpr int MAX_BLOCKS = 128;      // vocabularies up to 131072
constexpr int BITMAP_WORDS = MAX_BLOCKS * BLK / 32;
constexpr uint32_t RESIDUAL_DRAW = 0xFFFF;

__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint32_t hi0 = __umulhi(M0, c0), lo0 = M0 * c0;
    const uint32_t hi1 = __umulhi(M1, c2), lo1 = M1 * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return c0;
}

__device__ __forceinline__ float philox_u(uint64_t seed, uint32_t step, uint32_t depth, uint32_t draw,
                                         uint32_t lane) {
  const uint32_t w = philox_word0(step, depth, draw, lane, (uint32_t)seed, (uint32_t)(seed >> 32));
  return (float)(w >> 8) * (1.0f / 16777216.0f);
}

// e(v) = exp((l(v) - l(g)) / T) for one 1024-token block of one row (g = the
// row's argmax, so l(g) is its maximum), and the block's fp64 sum of e in a
// fixed order. Grid (blocks, rows), 256 threads x 4 consecutive tokens.
__global__ __launch_bounds__(256) void row_exp_kernel(const float* logits, const int32_t* g, int V,
                                                      float inv_t, float* ebuf, double* zpart) {
  __shared__ double red[256];
  const int b = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const float* l = logits + (int64_t)r * V;
  const float m = l[g[r]];
  const int v0 = b * BLK + 4 * tid;
  double acc = 0.0;
  float e[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int v = min(v0 + u, V - 1);
    e[u] = expf((l[v] - m) * inv_t);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (v0 + u < V) {
      ebuf[(int64_t)r * V + v0 + u] = e[u];
      acc += (double)e[u];
    }
  red[tid] = acc;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (tid < h) red[tid] += red[tid + h];
    __syncthreads();
  }
  if (tid == 0) zpart[(int64_t)r * gridDim.x + b] = red[0];
}

struct WalkLds {
  double d[NT];
  double bs[MAX_BLOCKS];          // per-block sums of e over the tokens left
  uint32_t bitmap[BITMAP_WORDS];  // rejected tokens of the current row
  int i[NT / 64];
  int children[TREE_MAXROWS];
  int ctok[TREE_MAXROWS];
  float cp[TREE_MAXROWS], cu[TREE_MAXROWS];
  int n_children, acc_row, n_removed, pick, blk;
  float z, S;
  double pre;
};

__device__ __forceinline__ bool is_removed(const WalkLds& s, int v) {
  return (s.bitmap[v >> 5] >> (v & 31)) & 1u;
}

// Loads row r's block sums and sets Z (their fixed-order sum, rounded to
// fp32); clears the bitmap.
__device__ void row_setup(const double* zpart, int r, int nb, int V, WalkLds& s) {
  const int tid = threadIdx.x;
  for (int w = tid; w < (V + 31) / 32; w += NT) s.bitmap[w] = 0u;
  if (tid < nb) s.bs[tid] = zpart[(int64_t)r * nb + tid];
  __syncthreads();
  if (tid == 0) {
    double z = 0.0;
    for (int b = 0; b < nb; ++b) z += s.bs[b];
    s.z = (float)z;
  }
  __syncthreads();
}

// The residual token of a row (e = its exponentials; the tokens in the
// bitmap removed) for the draw u: the first token, in id order, whose
// running fp64 sum of e exceeds (u * S) * Z, else the last token left with
// e > 0. Result in s.pick.
__device__ void residual_pick(const float* e, int V, int nb, float u, WalkLds& s) {
  const int tid = threadIdx.x;
  const double target = (double)(u * s.S) * (double)s.z;
  if (tid == 0) {
    // block sums over the tokens left, then the block where the walk crosses
    for (int j = 0; j < s.n_removed; ++j) {
      const int x = s.ctok[j];
      s.bs[x / BLK] -= (double)e[x];
    }
    double pre = 0.0;
    int blk = -1;
    for (int b = 0; b < nb; ++b) {
      if (pre + s.bs[b] > target) {
        blk = b;
        break;
      }
      pre += s.bs[b];
    }
    s.blk = blk;
    s.pre = pre;
    s.pick = -1;
  }
  __syncthreads();
  const int blk = s.blk;
  if (blk >= 0) {
    // scan the crossing block, one token per thread
    const int v = blk * BLK + tid;
    const bool left = v < V && !is_removed(s, v);
    const float ev = left ? e[v] : 0.f;
    s.d[tid] = (double)ev;
    __syncthreads();
    for (int o = 1; o < NT; o <<= 1) {
      const double add = tid >= o ? s.d[tid - o] : 0.0;
      __syncthreads();
      s.d[tid] += add;
      __syncthreads();
    }
    const bool cross = left && s.pre + s.d[tid] > target;
    const int first = wave_min_i(cross ? tid : NT);
    int lastv = (left && ev > 0.f) ? tid : -1;
    for (int off = 32; off >= 1; off >>= 1) lastv = max(lastv, __shfl_xor(lastv, off));
    if ((tid & 63) == 0) s.i[tid >> 6] = first;
    __syncthreads();
    if (tid == 0) {
      int f = NT;
      for (int w = 0; w < NT / 64; ++w) f = min(f, s.i[w]);
      s.pick = f < NT ? blk * BLK + f : -1;
    }
    __syncthreads();
    if ((tid & 63) == 0) s.i[tid >> 6] = lastv;
    __syncthreads();
    if (tid == 0 && s.pick < 0) {
      // rounding put the crossing past the block's scan: its last token left
      int lv = -1;
      for (int w = 0; w < NT / 64; ++w) lv = max(lv, s.i[w]);
      if (lv >= 0) s.pick = blk * BLK + lv;
    }
    __syncthreads();
  }
  // no crossing (rounding left the sum short): the last token left with e > 0
  for (int b = nb - 1; b >= 0 && s.pick < 0; --b) {
    const int v = b * BLK + tid;
    int lastv = (v < V && !is_removed(s, v) && e[v] > 0.f) ? tid : -1;
    for (int off = 32; off >= 1; off >>= 1) lastv = max(lastv, __shfl_xor(lastv, off));
    if ((tid & 63) == 0) s.i[tid >> 6] = lastv;
    __syncthreads();
    if (tid == 0) {
      int lv = -1;
      for (int w = 0; w < NT / 64; ++w) lv = max(lv, s.i[w]);
      if (lv >= 0) s.pick = b * BLK + lv;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(NT) void accept_sample_kernel(TreeDev t, const float* ebuf,
                                                           const double* zpart, int V, int nb,
                                                           uint64_t seed, uint32_t step,
                                                           uint32_t lane, int max_depth,
                                                           int32_t* acc,
                                                           int32_t* new_tok, int32_t* cu_src,
                                                           int32_t* seq_out, int32_t* host,
                                                           int32_t tag) {
  __shared__ WalkLds s;
  const int tid = threadIdx.x;
  const int n = t.counts[3];
  int cur = 0, L = 0;
  for (int depth = 0;; ++depth) {
    const float* e = ebuf + (int64_t)cur * V;
    if (tid < 64) {
      // children of `cur` in row order: rows 1 + lane and 65 + lane, by ballot
      int c = 0;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int r = 1 + tid + 64 * half;
        const bool is = depth < max_depth && r < n && t.v_parent[r] == cur;
        const uint64_t bal = __ballot(is);
        if (is) s.children[c + __popcll(bal & ((1ull << tid) - 1))] = r;
        c += __popcll(bal);
      }
      if (tid == 0) s.n_children = c;
    }
    row_setup(zpart, cur, nb, V, s);   // (its barriers also publish the children)
    const int nc = s.n_children;
    for (int j = tid; j < nc; j += NT) {
      // each child's token, probability and draw, all in parallel
      const int x = t.v_tok[s.children[j]];
      s.ctok[j] = x;
      s.cp[j] = e[x] / s.z;
      s.cu[j] = philox_u(seed, step, (uint32_t)depth, (uint32_t)j, lane);
    }
    __syncthreads();
    if (tid == 0) {
      float S = 1.f;
      int accepted = -1, nrem = 0;
      for (int j = 0; j < nc; ++j) {
        const float px = s.cp[j];
        if (s.cu[j] * S < px) {
          accepted = s.children[j];
          break;
        }
        S -= px;
        const int x = s.ctok[j];
        s.bitmap[x >> 5] |= 1u << (x & 31);
        ++nrem;
      }
      s.acc_row = accepted;
      s.S = S;
      s.n_removed = nrem;
    }
    __syncthreads();
    const int accepted = s.acc_row;
    if (accepted >= 0) {
      if (tid == 0) {
        const int x = s.ctok[s.n_removed];   // the accepted child follows the rejected ones
        acc[2 + L] = accepted;
        new_tok[L] = x;
        cu_src[L + 1] = accepted;
        seq_out[L] = x;
        if (host) host[2 + L] = x;
      }
      cur = accepted;
      ++L;
      __syncthreads();
      continue;
    }
    residual_pick(e, V, nb, philox_u(seed, step, (uint32_t)depth, RESIDUAL_DRAW, lane), s);
    if (tid == 0) {
      const int bonus = s.pick;
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
    return;
  }
}

__global__ __launch_bounds__(NT) void sample_token_kernel(const float* ebuf, const double* zpart,
                                                          int V, int nb, uint64_t seed,
                                                          uint32_t step, uint32_t lane,
                                                          int32_t* out) {
  __shared__ WalkLds s;
  row_setup(zpart, 0, nb, V, s);
  if (threadIdx.x == 0) {
    s.S = 1.f;
    s.n_removed = 0;
  }
  __syncthreads();
  residual_pick(ebuf, V, nb, philox_u(seed, step, 0u, RESIDUAL_DRAW, lane), s);
  if (threadIdx.x == 0) out[0] = s.pick;
}

}  // namespace

bool sample_vocab_ok(int V) { return V >= 1 && V <= MAX_BLOCKS * BLK; }

uint64_t sample_zpart_doubles(int rows, int V) { return (uint64_t)rows * ((V + BLK - 1) / BLK); }

hipError_t launch_row_exp(const float* logits, const int32_t* g, int rows, int V, float temperature,
                          float* ebuf, double* zpart, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (!sample_vocab_ok(V) || !(temperature > 0.f)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(row_exp_kernel, dim3((V + BLK - 1) / BLK, rows), dim3(256), 0, st, logits, g,
                     V, 1.0f / temperature, ebuf, zpart);
  return hipGetLastError();
}

hipError_t launch_accept_sample(TreeDev t, const float* ebuf, const double* zpart, int V,
                                uint64_t seed, uint32_t step, uint32_t lane, int max_depth,
                                int32_t* acc, int32_t* new_tok, int32_t* cu_src, int32_t* seq_out,
                                int32_t* host, int32_t tag, hipStream_t st) {
  if (!sample_vocab_ok(V)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(accept_sample_kernel, dim3(1), dim3(NT), 0, st, t, ebuf, zpart, V,
                     (V + BLK - 1) / BLK, seed, step, lane, max_depth, acc, new_tok, cu_src,
                     seq_out, host, tag);
  return hipGetLastError();
}

hipError_t launch_sample_token(const float* ebuf, const double* zpart, int V, uint64_t seed,
                               uint32_t step, uint32_t lane, int32_t* out, hipStream_t st) {
  if (!sample_vocab_ok(V)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sample_token_kernel, dim3(1), dim3(NT), 0, st, ebuf, zpart, V,
                     (V + BLK - 1) / BLK, seed, step, lane, out);
  return hipGetLastError();
}
