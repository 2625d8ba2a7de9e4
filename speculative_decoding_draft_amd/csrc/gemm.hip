// Skinny MFMA GEMM for decode-time projections (M <= 80 rows per pass) and
// the fused LM-head reductions. Every projection here reads each weight
// byte once per pass, so the kernel is organised around streaming W:
//  * a 512-thread workgroup owns 16*NB output columns; its 8 waves split
//    the K range and issue up to 8 steps (16 B per lane each) of W loads
//    before the first MFMA, so each CU keeps ~64 KB of weights in flight;
//  * the activation x (bf16 or fp32, a few MB at most) is read from L2 per
//    step; rows beyond M read row M-1 and are discarded;
//  * the 8 partial accumulators are summed in LDS in a fixed order; when a
//    tile is further split over workgroups (narrow N), partials go to a
//    workspace and the last workgroup to arrive sums them in split order,
//    so results are deterministic.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int NWAVES = 8;
constexpr int NTHREADS = NWAVES * WAVE;
constexpr int PREF = 8;   // W steps issued before consuming them

struct GemmArgs {
  const void* W; int64_t ldw;
  const void* X; int64_t ldx; int64_t xlo;
  int M, N, K;          // N = output columns (SwiGLU: F)
  int n_tiles, splits, steps_per_split;
  float* Y; int64_t ldy;
  void* Yt; int64_t ytlo;
  float* part; int* counters;
};

// Rows of W read by n-block b of tile `tile`.
template <int NB, int EPI>
__device__ __forceinline__ int block_row(int tile, int b, int N) {
  if (EPI == EPI_SWIGLU) {
    return (b < NB / 2) ? tile * 8 * NB + 16 * b : N + tile * 8 * NB + 16 * (b - NB / 2);
  }
  return tile * 16 * NB + 16 * b;
}

// Streams this workgroup's K range and leaves the reduced tile in
// `tile_out[n_local][m_local]` (16*NB x 16*MT floats, LDS).
template <typename T, int MT, int NB>
__device__ __forceinline__ void tile_compute(const T* __restrict__ W, int64_t ldw,
                                             const int (&wrow)[NB], const T* __restrict__ X,
                                             int64_t ldx, int64_t xlo, int M, int m0, int s_lo,
                                             int s_hi, float* red, float* tile_out) {
  using MM = Mma<T>;
  constexpr int EPL = MM::EPL, KS = MM::KSTEP;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;

  const T* wp[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) wp[b] = W + (int64_t)(wrow[b] + lr) * ldw + lg * EPL;
  const T* xp[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    int m = min(m0 + 16 * t + lr, M - 1);
    xp[t] = X + (int64_t)m * ldx + lg * EPL;
  }

  const int n = max(0, s_hi - s_lo);
  const int q = n / NWAVES, r = n % NWAVES;
  const int ws = s_lo + wave * q + min(wave, r);
  const int we = ws + q + (wave < r ? 1 : 0);

  f32x4 acc[NB][MT];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[b][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int s = ws; s < we; s += PREF) {
    const int cnt = we - s;
    uint4 wf[PREF][NB];
#pragma unroll
    for (int u = 0; u < PREF; ++u)
      if (u < cnt) {
#pragma unroll
        for (int b = 0; b < NB; ++b) wf[u][b] = ld16(wp[b] + (int64_t)(s + u) * KS);
      }
#pragma unroll
    for (int u = 0; u < PREF; ++u)
      if (u < cnt) {
        uint4 xf[MT], xl[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          xf[t] = ld16(xp[t] + (int64_t)(s + u) * KS);
          if (Opnd<T>::SPLIT) xl[t] = ld16(xp[t] + xlo + (int64_t)(s + u) * KS);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            MM::mma(wf[u][b], xf[t], acc[b][t]);
            if (Opnd<T>::SPLIT) MM::mma(wf[u][b], xl[t], acc[b][t]);
          }
      }
  }

  // fixed-order reduction of the 8 waves: (w + w+4) then ((0+1) + (2+3))
  constexpr int NV = NB * MT * 4;
  if (wave >= 4) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[((wave - 4) * NV + (b * MT + t) * 4 + j) * WAVE + lane] = acc[b][t][j];
  }
  __syncthreads();
  if (wave < 4) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float* p = &red[(wave * NV + (b * MT + t) * 4 + j) * WAVE + lane];
          *p = acc[b][t][j] + *p;
        }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < NV * WAVE; e += NTHREADS) {
    const int v = e / WAVE, ln = e % WAVE;
    const float val = (red[(0 * NV + v) * WAVE + ln] + red[(1 * NV + v) * WAVE + ln]) +
                      (red[(2 * NV + v) * WAVE + ln] + red[(3 * NV + v) * WAVE + ln]);
    const int b = v / (MT * 4), t = (v / 4) % MT, j = v % 4;
    const int nl = 16 * b + 4 * (ln >> 4) + j;
    const int ml = 16 * t + (ln & 15);
    tile_out[nl * (16 * MT) + ml] = val;
  }
  __syncthreads();
}

template <typename T, int MT, int NB, int EPI>
__global__ __launch_bounds__(NTHREADS) void gemm_kernel(GemmArgs a) {
  __shared__ float red[4 * NB * MT * 4 * WAVE];
  __shared__ float tile_out[16 * NB * 16 * MT];
  __shared__ int s_last;
  constexpr int R = 16 * NB, C = 16 * MT;

  int tile, split;
  if (a.splits == 1) {
    tile = blockIdx.x;
    split = 0;
  } else {  // the splits of one tile land on the same XCD (round-robin of 8)
    const int idx = blockIdx.x;
    split = (idx / 8) % a.splits;
    tile = (idx % 8) + 8 * (idx / (8 * a.splits));
    if (tile >= a.n_tiles) return;
  }
  const int m0 = blockIdx.y * C;
  const int rows_total = (EPI == EPI_SWIGLU) ? 2 * a.N : a.N;
  // per-lane clamping for partial blocks
  int wrow_l[NB];
  const int lr = threadIdx.x & 15;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    int r0 = block_row<NB, EPI>(tile, b, a.N);
    int lim = (EPI == EPI_SWIGLU) ? ((b < NB / 2) ? a.N : rows_total) : rows_total;
    wrow_l[b] = min(r0 + lr, lim - 1) - lr;
  }
  const int total = a.K / Mma<T>::KSTEP;
  const int s_lo = split * a.steps_per_split;
  const int s_hi = min(total, s_lo + a.steps_per_split);
  tile_compute<T, MT, NB>((const T*)a.W, a.ldw, wrow_l, (const T*)a.X, a.ldx, a.xlo, a.M, m0,
                          s_lo, s_hi, red, tile_out);

  const int mrows = min(C, a.M - m0);
  if (a.splits > 1) {
    // partial tile -> workspace [split][M][rows_total]; the last arriver sums
    for (int e = threadIdx.x; e < R * C; e += NTHREADS) {
      const int ml = e / R, nl = e % R;
      if (ml >= mrows) continue;
      const int b = nl / 16;
      const int row = block_row<NB, EPI>(tile, b, a.N) + (nl % 16);
      if (row >= rows_total) continue;
      a.part[((int64_t)split * a.M + m0 + ml) * rows_total + row] = tile_out[nl * C + ml];
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      const int prev = atomicAdd(&a.counters[blockIdx.y * a.n_tiles + tile], 1);
      s_last = (prev == a.splits - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    for (int e = threadIdx.x; e < R * C; e += NTHREADS) {
      const int ml = e / R, nl = e % R;
      if (ml >= mrows) continue;
      const int b = nl / 16;
      const int row = block_row<NB, EPI>(tile, b, a.N) + (nl % 16);
      if (row >= rows_total) continue;
      float s = 0.f;
      for (int sp = 0; sp < a.splits; ++sp)
        s += __builtin_nontemporal_load(&a.part[((int64_t)sp * a.M + m0 + ml) * rows_total + row]);
      tile_out[nl * C + ml] = s;
    }
    __syncthreads();
    if (threadIdx.x == 0) a.counters[blockIdx.y * a.n_tiles + tile] = 0;
  }

  if (EPI == EPI_SWIGLU) {
    constexpr int HALF = R / 2;
    for (int e = threadIdx.x; e < HALF * C; e += NTHREADS) {
      const int ml = e / HALF, nl = e % HALF;
      const int col = tile * HALF + nl;
      if (ml >= mrows || col >= a.N) continue;
      const float g = tile_out[nl * C + ml];
      const float u = tile_out[(nl + HALF) * C + ml];
      const float v = g / (1.0f + expf(-g)) * u;
      Opnd<T>::store((T*)a.Yt, a.ytlo, (int64_t)(m0 + ml) * a.N + col, v);
    }
  } else {
    for (int e = threadIdx.x; e < R * C; e += NTHREADS) {
      const int ml = e / R, nl = e % R;
      const int col = tile * R + nl;
      if (ml >= mrows || col >= a.N) continue;
      float* y = &a.Y[(int64_t)(m0 + ml) * a.ldy + col];
      const float v = tile_out[nl * C + ml];
      if (EPI == EPI_ADD) *y = *y + v;
      else *y = v;
    }
  }
}

// ---------------------------------------------------------------- LM head
struct HeadArgs {
  const void* W; const void* X; int64_t xlo;
  int M, V, H, k;
  float* part;      // per workgroup and row: argmax {max1, id1, max2} or topk {max, sum, k vals, k ids}
  float* logits;    // optional [M, V]
};

template <typename T, int MT, int NB, bool TOPK>
__global__ __launch_bounds__(NTHREADS) void lmhead_kernel(HeadArgs a) {
  __shared__ float red[4 * NB * MT * 4 * WAVE];
  __shared__ float tile_out[16 * NB * 16 * MT];
  constexpr int R = 16 * NB, C = 16 * MT;
  const int tile = blockIdx.x;
  const int lr = threadIdx.x & 15;
  int wrow[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) wrow[b] = min(tile * R + 16 * b + lr, a.V - 1) - lr;
  const int total = a.H / Mma<T>::KSTEP;
  tile_compute<T, MT, NB>((const T*)a.W, a.H, wrow, (const T*)a.X, a.H, a.xlo, a.M, 0, 0, total,
                          red, tile_out);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nvalid = min(R, a.V - tile * R);
  if (a.logits) {
    for (int e = threadIdx.x; e < R * C; e += NTHREADS) {
      const int ml = e / R, nl = e % R;
      if (ml < a.M && nl < nvalid)
        a.logits[(int64_t)ml * a.V + tile * R + nl] = tile_out[nl * C + ml];
    }
  }
  const int stride = TOPK ? (2 + 2 * a.k) : 3;
  for (int m = wave; m < a.M; m += NWAVES) {
    const bool ok = lane < nvalid;
    float v = ok ? tile_out[lane * C + m] : -INFINITY;
    int id = tile * R + lane;
    float* out = a.part + ((int64_t)tile * a.M + m) * stride;
    if (!TOPK) {
      // max with lowest id, then second max
      float bv = v; int bi = ok ? id : 0x7fffffff;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        float ov = __shfl_xor(bv, o); int oi = __shfl_xor(bi, o);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      float sv = (ok && id != bi) ? v : -INFINITY;
      sv = wave_max(sv);
      if (lane == 0) { out[0] = bv; out[1] = __int_as_float(bi); out[2] = sv; }
    } else {
      const float mx = wave_max(v);
      const float se = wave_sum(ok ? expf(v - mx) : 0.f);
      if (lane == 0) { out[0] = mx; out[1] = se; }
      float cur = v; int cid = ok ? id : 0x7fffffff;
      for (int i = 0; i < a.k; ++i) {
        float bv = cur; int bi = cid;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          float ov = __shfl_xor(bv, o); int oi = __shfl_xor(bi, o);
          if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
        }
        if (lane == 0) { out[2 + i] = bv; out[2 + a.k + i] = __int_as_float(bi); }
        if (cid == bi) { cur = -INFINITY; cid = 0x7fffffff; }
      }
    }
  }
}

// one workgroup per row: merge the per-tile argmax records
__global__ __launch_bounds__(256) void argmax_combine(const float* part, int n_tiles, int M,
                                                      int32_t* g, float* margin) {
  const int m = blockIdx.x;
  float b1 = -INFINITY, b2 = -INFINITY; int i1 = 0x7fffffff;
  for (int t = threadIdx.x; t < n_tiles; t += blockDim.x) {
    const float* p = part + ((int64_t)t * M + m) * 3;
    float p1 = p[0], p2 = p[2]; int pi = __float_as_int(p[1]);
    if (p1 > b1 || (p1 == b1 && pi < i1)) { b2 = fmaxf(b1, p2); b1 = p1; i1 = pi; }
    else b2 = fmaxf(b2, p1);
  }
  __shared__ float s1[256], s2[256]; __shared__ int si[256];
  s1[threadIdx.x] = b1; s2[threadIdx.x] = b2; si[threadIdx.x] = i1;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      float a1 = s1[threadIdx.x], a2 = s2[threadIdx.x]; int ai = si[threadIdx.x];
      float c1 = s1[threadIdx.x + o], c2 = s2[threadIdx.x + o]; int ci = si[threadIdx.x + o];
      if (c1 > a1 || (c1 == a1 && ci < ai)) { a2 = fmaxf(a1, c2); a1 = c1; ai = ci; }
      else a2 = fmaxf(a2, c1);
      s1[threadIdx.x] = a1; s2[threadIdx.x] = a2; si[threadIdx.x] = ai;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) { g[m] = si[0]; margin[m] = s1[0] - s2[0]; }
}

// one workgroup per row: global max, sum of exp, and the k best (val desc, id asc)
__global__ __launch_bounds__(256) void topk_combine(const float* part, int n_tiles, int M, int k,
                                                    int32_t* ids, float* logp) {
  const int m = blockIdx.x;
  const int stride = 2 + 2 * k;
  __shared__ float sred[256];
  __shared__ float s_gmax, s_lse;
  // global max
  float mx = -INFINITY;
  for (int t = threadIdx.x; t < n_tiles; t += 256) mx = fmaxf(mx, part[((int64_t)t * M + m) * stride]);
  sred[threadIdx.x] = mx;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) sred[threadIdx.x] = fmaxf(sred[threadIdx.x], sred[threadIdx.x + o]);
    __syncthreads();
  }
  if (threadIdx.x == 0) s_gmax = sred[0];
  __syncthreads();
  const float gmax = s_gmax;
  float se = 0.f;
  for (int t = threadIdx.x; t < n_tiles; t += 256) {
    const float* p = part + ((int64_t)t * M + m) * stride;
    se += p[1] * expf(p[0] - gmax);
  }
  __syncthreads();
  sred[threadIdx.x] = se;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) sred[threadIdx.x] = sred[threadIdx.x] + sred[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) s_lse = logf(sred[0]);
  __syncthreads();
  // per-thread sorted candidate list
  float lv[16]; int li[16];
  for (int i = 0; i < k; ++i) { lv[i] = -INFINITY; li[i] = 0x7fffffff; }
  for (int t = threadIdx.x; t < n_tiles; t += 256) {
    const float* p = part + ((int64_t)t * M + m) * stride;
    for (int i = 0; i < k; ++i) {
      float v = p[2 + i]; int id = __float_as_int(p[2 + k + i]);
      if (id == 0x7fffffff) break;
      // insert if better than the last
      if (v > lv[k - 1] || (v == lv[k - 1] && id < li[k - 1])) {
        int j = k - 1;
        while (j > 0 && (v > lv[j - 1] || (v == lv[j - 1] && id < li[j - 1]))) {
          lv[j] = lv[j - 1]; li[j] = li[j - 1]; --j;
        }
        lv[j] = v; li[j] = id;
      } else {
        break;  // the tile's list is sorted: nothing later can enter
      }
    }
  }
  __shared__ float hv[256]; __shared__ int hi[256], ht[256];
  int head = 0;
  for (int r = 0; r < k; ++r) {
    hv[threadIdx.x] = head < k ? lv[head] : -INFINITY;
    hi[threadIdx.x] = head < k ? li[head] : 0x7fffffff;
    ht[threadIdx.x] = threadIdx.x;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if ((int)threadIdx.x < o) {
        float c = hv[threadIdx.x + o]; int ci = hi[threadIdx.x + o];
        if (c > hv[threadIdx.x] || (c == hv[threadIdx.x] && ci < hi[threadIdx.x])) {
          hv[threadIdx.x] = c; hi[threadIdx.x] = ci; ht[threadIdx.x] = ht[threadIdx.x + o];
        }
      }
      __syncthreads();
    }
    if (threadIdx.x == 0) {
      ids[m * k + r] = hi[0];
      logp[m * k + r] = (hv[0] - gmax) - s_lse;
    }
    const int winner = ht[0];
    __syncthreads();
    if ((int)threadIdx.x == winner) ++head;
  }
}

template <typename T, int EPI>
hipError_t gemm_dispatch(const GemmPlan& p, const GemmArgs& a, hipStream_t st) {
  dim3 grid(p.splits == 1 ? p.n_tiles : ((p.n_tiles + 7) / 8) * 8 * p.splits, p.m_chunks);
#define GEMM_CASE(MT_)                                                                  \
  case MT_:                                                                             \
    hipLaunchKernelGGL((gemm_kernel<T, MT_, 2, EPI>), grid, dim3(NTHREADS), 0, st, a); \
    break;
  switch (p.mt) {
    GEMM_CASE(1) GEMM_CASE(2) GEMM_CASE(3) GEMM_CASE(4) GEMM_CASE(5)
    default: return hipErrorInvalidValue;
  }
#undef GEMM_CASE
  return hipGetLastError();
}

template <typename T, bool TOPK>
hipError_t head_dispatch(int mt, int n_tiles, const HeadArgs& a, hipStream_t st) {
#define HEAD_CASE(MT_)                                                                           \
  case MT_:                                                                                      \
    hipLaunchKernelGGL((lmhead_kernel<T, MT_, 2, TOPK>), dim3(n_tiles), dim3(NTHREADS), 0, st, a); \
    break;
  switch (mt) {
    HEAD_CASE(1) HEAD_CASE(2) HEAD_CASE(3) HEAD_CASE(4) HEAD_CASE(5)
    default: return hipErrorInvalidValue;
  }
#undef HEAD_CASE
  return hipGetLastError();
}

}  // namespace

GemmPlan gemm_plan(int M, int N_rows, int K, int dtype, int epi) {
  GemmPlan p;
  p.nb = 2;
  if (M <= 80) { p.mt = (M + 15) / 16; p.m_chunks = 1; }
  else { p.mt = 4; p.m_chunks = (M + 63) / 64; }
  const int R = 16 * p.nb;
  const int outs = (epi == EPI_SWIGLU) ? N_rows / 2 : N_rows;
  p.n_tiles = (epi == EPI_SWIGLU) ? (outs + R / 2 - 1) / (R / 2) : (outs + R - 1) / R;
  const int steps = K / (dtype == 1 ? 32 : 16);
  int s = 1;
  while (p.n_tiles * s < 256 && s < 8 && steps / (2 * s) >= NWAVES) s *= 2;
  p.splits = s;
  return p;
}

uint64_t gemm_part_floats(const GemmPlan& p, int N_rows, int M) {
  return p.splits > 1 ? (uint64_t)p.splits * M * N_rows : 0;
}

hipError_t launch_gemm(int dtype, int epi, const void* W, const void* x, int64_t xlo, int M, int N,
                       int K, float* Y, int64_t ldy, void* Yt, int64_t ytlo, float* part,
                       int* counters, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  const int rows = (epi == EPI_SWIGLU) ? 2 * N : N;
  GemmPlan p = gemm_plan(M, rows, K, dtype, epi);
  GemmArgs a;
  a.W = W; a.ldw = K; a.X = x; a.ldx = K; a.xlo = xlo; a.M = M; a.N = N; a.K = K;
  a.n_tiles = p.n_tiles; a.splits = p.splits;
  const int steps = K / (dtype == 1 ? 32 : 16);
  a.steps_per_split = (steps + p.splits - 1) / p.splits;
  a.Y = Y; a.ldy = ldy; a.Yt = Yt; a.ytlo = ytlo; a.part = part; a.counters = counters;
  if (dtype == 1) {
    switch (epi) {
      case EPI_STORE: return gemm_dispatch<bf16_t, EPI_STORE>(p, a, stream);
      case EPI_ADD: return gemm_dispatch<bf16_t, EPI_ADD>(p, a, stream);
      default: return gemm_dispatch<bf16_t, EPI_SWIGLU>(p, a, stream);
    }
  }
  switch (epi) {
    case EPI_STORE: return gemm_dispatch<float, EPI_STORE>(p, a, stream);
    case EPI_ADD: return gemm_dispatch<float, EPI_ADD>(p, a, stream);
    default: return gemm_dispatch<float, EPI_SWIGLU>(p, a, stream);
  }
}

uint64_t lmhead_part_floats(int M, int V, int k) {
  const int n_tiles = (V + 31) / 32;
  if (M > 80) M = 64;
  return (uint64_t)n_tiles * M * (k > 0 ? (2 + 2 * k) : 3);
}

hipError_t launch_lmhead_argmax(int dtype, const void* W, const void* x, int64_t xlo, int M, int V,
                                int H, float* part, int32_t* g, float* margin, float* logits,
                                hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  if (M > 80) {  // rows in passes of 64 (the weight is re-read per pass)
    const int esz = dtype == 1 ? 2 : 4;
    for (int m0 = 0; m0 < M; m0 += 64) {
      const int mc = M - m0 < 64 ? M - m0 : 64;
      hipError_t e = launch_lmhead_argmax(dtype, W, (const char*)x + (int64_t)m0 * H * esz, xlo, mc, V,
                                          H, part, g + m0, margin + m0,
                                          logits ? logits + (int64_t)m0 * V : nullptr, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  HeadArgs a{W, x, xlo, M, V, H, 0, part, logits};
  const int n_tiles = (V + 31) / 32;
  const int mt = (M + 15) / 16;
  hipError_t e = dtype == 1 ? head_dispatch<bf16_t, false>(mt, n_tiles, a, stream)
                            : head_dispatch<float, false>(mt, n_tiles, a, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(argmax_combine, dim3(M), dim3(256), 0, stream, part, n_tiles, M, g, margin);
  return hipGetLastError();
}

hipError_t launch_lmhead_topk(int dtype, const void* W, const void* x, int64_t xlo, int M, int V,
                              int H, int k, float* part, int32_t* ids, float* logp,
                              hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  if (k < 1 || k > 16) return hipErrorInvalidValue;
  if (M > 80) {
    const int esz = dtype == 1 ? 2 : 4;
    for (int m0 = 0; m0 < M; m0 += 64) {
      const int mc = M - m0 < 64 ? M - m0 : 64;
      hipError_t e = launch_lmhead_topk(dtype, W, (const char*)x + (int64_t)m0 * H * esz, xlo, mc, V,
                                        H, k, part, ids + (int64_t)m0 * k, logp + (int64_t)m0 * k,
                                        stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  HeadArgs a{W, x, xlo, M, V, H, k, part, nullptr};
  const int n_tiles = (V + 31) / 32;
  const int mt = (M + 15) / 16;
  hipError_t e = dtype == 1 ? head_dispatch<bf16_t, true>(mt, n_tiles, a, stream)
                            : head_dispatch<float, true>(mt, n_tiles, a, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_combine, dim3(M), dim3(256), 0, stream, part, n_tiles, M, k, ids, logp);
  return hipGetLastError();
}
