// Weight-streaming projections (M <= 80 activation rows per pass) and the
// fused LM-head reductions.
//
// Every projection of a decode/verify pass reads each weight byte once, so
// the kernel is built around streaming W from HBM:
//  * a workgroup of NW waves owns NW*16 consecutive weight rows (one 16-row
//    MFMA block per wave) and a K range; the K range is walked in chunks of
//    CS steps (16 bytes of W per lane per step);
//  * the activation chunk x[M, chunk] (fp32 values kept as bf16 hi + lo
//    planes, or one fp32 plane) is staged once per workgroup into LDS in an
//    XOR-swizzled layout (conflict-free 16-byte reads) and shared by all
//    waves, so x is read from L2 once per NW*16 weight rows;
//  * the next chunk's W fragments and x chunk are loaded while the current
//    chunk is multiplied (double buffering in registers and LDS);
//  * narrow outputs are split over K across workgroups; each split writes
//    its own fp32 partial plane and the consumer of the result (the residual
//    + RMSNorm kernel, or RoPE) sums the planes in a fixed order, so no
//    cross-workgroup synchronisation is needed and results are repeatable.
#include <hip/hip_ext.h>

#include "common.h"
#include "kernels.h"

namespace {

// LDS address (elements) of 16-byte chunk q of staged row r. Rows are KCH
// elements wide (C 16-byte chunks); the chunk index is XOR-swizzled with the
// row. LDS has 32 banks of 4 bytes, so a 16-byte access serves eight lanes
// per cycle: the operand reads (eight consecutive rows, one chunk) and the
// stores (consecutive chunks of one or two rows) must fall in eight
// distinct 16-byte bank groups. With C >= 8 a row spans whole bank rounds
// and chunk q ^ (r mod 8) does it; with C = 4 two rows share a round and
// q ^ ((r / 2) mod 4) does it (C = 2: q ^ ((r / 4) mod 2)).
template <typename T, int KCH>
__device__ __forceinline__ int xs_addr(int r, int q) {
  constexpr int EPL = 16 / sizeof(T);
  constexpr int C = KCH / EPL;
  constexpr int SH = C >= 8 ? 0 : C == 4 ? 1 : C == 2 ? 2 : 3;
  constexpr int SM = (C >= 8 ? 8 : C) - 1;
  return r * KCH + ((q ^ ((r >> SH) & SM)) * EPL);
}

struct ProjArgs {
  const void* W;        // [rows, K]
  const void* X;        // [M, K] operand (lo plane at X + xlo)
  int64_t xlo;
  int M, rows, K;       // rows of W (SwiGLU: 2F, gate rows then up rows)
  int F;                // SwiGLU: output columns
  int splits, steps_per_split;
  float* Y;             // EPI_PART: partial planes [split][M][ldy]
  int64_t ldy, plane;
  void* Yt;             // EPI_SWIGLU: operand [M, F] (lo plane at Yt + ytlo)
  int64_t ytlo;
  const float* rs = nullptr;   // RowScale: sums of squares, RS_SLICES per row (or none)
  int rs_h = 0;
  float rs_eps = 0.f;
};
static_assert(RS_SLICES == 4, "the projections read a row's sums of squares as one float4");

// RowScale factor of a row from its per-slice sums of squares (fixed order).
__device__ __forceinline__ float row_scale(float4 v, int H, float eps) {
  return 1.0f / sqrtf((v.x + v.y + v.z + v.w) / (float)H + eps);
}

template <typename T, int MT, int NW, int CS>
struct ProjShape {
  static constexpr int EPL = 16 / sizeof(T);
  static constexpr int KS = Mma<T>::KSTEP;              // k per step
  static constexpr int KCH = CS * KS;                   // k per chunk
  static constexpr int MP = 16 * MT;                    // staged activation rows
  static constexpr int PLANES = Opnd<T>::SPLIT ? 2 : 1;
  static constexpr int PIECES = PLANES * MP * KCH / EPL;  // 16-byte pieces per chunk
  static constexpr int NX = (PIECES + NW * 64 - 1) / (NW * 64);
  static constexpr int LDS_ELEMS = PLANES * MP * KCH;   // one buffer
};

// Loads this thread's pieces of the activation chunk starting at step s0.
template <typename T, int MT, int NW, int CS>
__device__ __forceinline__ void stage_load(const ProjArgs& a, int s0, int s_hi, uint4 (&xr)[ProjShape<T, MT, NW, CS>::NX]) {
  using S = ProjShape<T, MT, NW, CS>;
  const T* X = (const T*)a.X;
#pragma unroll
  for (int i = 0; i < S::NX; ++i) {
    const int p = min((int)threadIdx.x + i * NW * 64, S::PIECES - 1);
    const int plane = p / (S::MP * S::KCH / S::EPL);
    const int rem = p % (S::MP * S::KCH / S::EPL);
    const int row = min(rem / (S::KCH / S::EPL), a.M - 1);
    const int col = min(s0 * S::KS + (rem % (S::KCH / S::EPL)) * S::EPL, s_hi * S::KS - S::EPL);
    xr[i] = ld16(X + plane * a.xlo + (int64_t)row * a.K + col);
  }
}

template <typename T, int MT, int NW, int CS>
__device__ __forceinline__ void stage_store(T* xs, const uint4 (&xr)[ProjShape<T, MT, NW, CS>::NX]) {
  using S = ProjShape<T, MT, NW, CS>;
#pragma unroll
  for (int i = 0; i < S::NX; ++i) {
    const int p = threadIdx.x + i * NW * 64;
    if (p >= S::PIECES) break;
    const int plane = p / (S::MP * S::KCH / S::EPL);
    const int rem = p % (S::MP * S::KCH / S::EPL);
    const int row = rem / (S::KCH / S::EPL);
    const int q = rem % (S::KCH / S::EPL);
    *reinterpret_cast<uint4*>(xs + xs_addr<T, S::KCH>(plane * S::MP + row, q)) = xr[i];
  }
}

// Streams rows [row0, row0 + 16) of W over steps [s_lo, s_hi) against the
// staged activations; acc[t] holds the 16 x 16 tile of m-tile t.
template <typename T, int MT, int NW, int CS>
__device__ __forceinline__ void proj_core(const ProjArgs& a, int row0, int s_lo, int s_hi, T* xs,
                                          f32x4 (&acc)[MT]) {
  using S = ProjShape<T, MT, NW, CS>;
  using MM = Mma<T>;
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const T* wp;
  int64_t wstep;   // elements between consecutive K steps of this lane's piece
  if constexpr (Opnd<T>::SPLIT) {
    // bf16 weights are fragment-packed (see pack_frag_kernel): a full
    // 16-row block is a run of 1 KB fragments, one per K step, lane-ordered;
    // rows of a ragged last block stay row-major.
    const int rb = min(row0, a.rows - 1) >> 4;
    if ((rb + 1) * 16 <= a.rows) {
      wp = (const T*)a.W + (int64_t)rb * 16 * a.K + lane * S::EPL;
      wstep = 16 * S::KS;
    } else {
      wp = (const T*)a.W + (int64_t)min(row0 + lr, a.rows - 1) * a.K + lg * S::EPL;
      wstep = S::KS;
    }
  } else {
    wp = (const T*)a.W + (int64_t)min(row0 + lr, a.rows - 1) * a.K + lg * S::EPL;
    wstep = S::KS;
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nch = (s_hi - s_lo + CS - 1) / CS;
  uint4 wA[CS], wB[CS], xr[S::NX];
  T* xs0 = xs;
  T* xs1 = xs + S::LDS_ELEMS;

  auto load_w = [&](uint4 (&w)[CS], int c) {
#pragma unroll
    for (int u = 0; u < CS; ++u) w[u] = ld16(wp + (int64_t)min(s_lo + c * CS + u, s_hi - 1) * wstep);
  };
  auto compute = [&](const uint4 (&w)[CS], const T* x, int c) {
#pragma unroll
    for (int u = 0; u < CS; ++u) {
      if (s_lo + c * CS + u < s_hi) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const uint4 xh = *reinterpret_cast<const uint4*>(x + xs_addr<T, S::KCH>(16 * t + lr, 4 * u + lg));
          MM::mma(w[u], xh, acc[t]);
          if (Opnd<T>::SPLIT) {
            const uint4 xl = *reinterpret_cast<const uint4*>(x + xs_addr<T, S::KCH>(S::MP + 16 * t + lr, 4 * u + lg));
            MM::mma(w[u], xl, acc[t]);
          }
        }
      }
    }
  };
  if (nch <= 0) return;
  load_w(wA, 0);
  stage_load<T, MT, NW, CS>(a, s_lo, s_hi, xr);
  stage_store<T, MT, NW, CS>(xs0, xr);
  for (int c = 0; c < nch; c += 2) {
    if (c + 1 < nch) {
      stage_load<T, MT, NW, CS>(a, s_lo + (c + 1) * CS, s_hi, xr);
      load_w(wB, c + 1);
    }
    __syncthreads();
    compute(wA, xs0, c);
    if (c + 1 < nch) stage_store<T, MT, NW, CS>(xs1, xr);
    if (c + 1 >= nch) break;
    if (c + 2 < nch) {
      stage_load<T, MT, NW, CS>(a, s_lo + (c + 2) * CS, s_hi, xr);
      load_w(wA, c + 2);
    }
    __syncthreads();
    compute(wB, xs1, c + 1);
    if (c + 2 < nch) stage_store<T, MT, NW, CS>(xs0, xr);
  }
}


// bf16 version of proj_core with a software pipeline the compiler can keep
// full: chunk c is multiplied while the weight fragments of chunks c+1 and
// c+2 and the activations of chunk c+1 are in flight. Buffers form static
// rings (weights 4, activation registers 2, LDS 2) walked by a loop unrolled
// four times; loads past the last chunk re-read it (cache hits) instead of
// sitting under a branch, so every wait is a partial vmcnt and one
// LDS-only barrier per chunk orders the activation buffers.
//
// A wave owns NB consecutive 16-row weight blocks (rows row0 .. row0 +
// 16 NB): every activation fragment read from LDS feeds NB products. Many
// activation rows (a batch of verify rows, a prefill chunk) make the MFMAs
// wait on LDS reads, one 1 KB fragment per product at NB = 1; NB > 1 divides
// that traffic.
template <int MT, int NW, int CS, int NB>
__device__ __forceinline__ void proj_core_bf16(const ProjArgs& a, int row0, int s_lo, int s_hi,
                                               bf16_t* xs, f32x4 (&acc)[NB][MT]) {
  using S = ProjShape<bf16_t, MT, NW, CS>;
  constexpr int PPL = S::MP * S::KCH / S::EPL;   // 16-byte pieces per plane
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const bf16_t* W = (const bf16_t*)a.W;
  const bf16_t* X = (const bf16_t*)a.X;
  const bf16_t* wp[NB];
  int64_t wstep[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int r0 = row0 + 16 * j;
    const int rb = min(r0, a.rows - 1) >> 4;
    if ((rb + 1) * 16 <= a.rows) {   // fragment-packed block
      wp[j] = W + (int64_t)rb * 16 * a.K + lane * S::EPL;
      wstep[j] = 16 * S::KS;
    } else {                         // ragged last block: row-major rows
      wp[j] = W + (int64_t)min(r0 + lr, a.rows - 1) * a.K + lg * S::EPL;
      wstep[j] = S::KS;
    }
  }
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nch = (s_hi - s_lo + CS - 1) / CS;
  if (nch <= 0) return;
  auto xload = [&](uint4 (&xr)[S::NX], int c) {
    const int cc = min(c, nch - 1);
#pragma unroll
    for (int i = 0; i < S::NX; ++i) {
      const int p = min(tid + i * NW * 64, S::PIECES - 1);
      const int plane = p / PPL, rem = p % PPL;
      const int row = min(rem / (S::KCH / S::EPL), a.M - 1), q = rem % (S::KCH / S::EPL);
      const int col = min((s_lo + cc * CS) * S::KS + q * S::EPL, s_hi * S::KS - S::EPL);
      xr[i] = ld16(X + plane * a.xlo + (int64_t)row * a.K + col);
    }
  };
  auto wload = [&](uint4 (&w)[NB][CS], int c) {
    const int cc = min(c, nch - 1);
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int u = 0; u < CS; ++u)
        w[j][u] = ld16(wp[j] + (int64_t)min(s_lo + cc * CS + u, s_hi - 1) * wstep[j]);
  };
  // one K step, m-tiles in groups of up to four: a group's activation
  // fragments are read first, then its products are issued hi-plane first,
  // so consecutive MFMAs rarely feed one accumulator and no MFMA waits on
  // the read just before it (the group bounds the registers this takes)
  auto step = [&](const uint4 (&w)[NB][CS], const bf16_t* x, int u) {
    // (the many-row tiles, MT >= 8, are short of registers: one tile at a time)
    constexpr int G = MT < 4 ? MT : MT < 8 ? 4 : 1;
#pragma unroll
    for (int t0 = 0; t0 < MT; t0 += G) {
      uint4 xh[G], xl[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int t = t0 + g < MT ? t0 + g : MT - 1;
        xh[g] = *reinterpret_cast<const uint4*>(x + xs_addr<bf16_t, S::KCH>(16 * t + lr, 4 * u + lg));
        xl[g] = *reinterpret_cast<const uint4*>(x + xs_addr<bf16_t, S::KCH>(S::MP + 16 * t + lr, 4 * u + lg));
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
        if (t0 + g < MT)
#pragma unroll
          for (int j = 0; j < NB; ++j) Mma<bf16_t>::mma(w[j][u], xh[g], acc[j][t0 + g]);
#pragma unroll
      for (int g = 0; g < G; ++g)
        if (t0 + g < MT)
#pragma unroll
          for (int j = 0; j < NB; ++j) Mma<bf16_t>::mma(w[j][u], xl[g], acc[j][t0 + g]);
    }
  };
  auto compute = [&](const uint4 (&w)[NB][CS], const bf16_t* x, int c) {
    // a whole chunk: straight-line code (not for the many-row tiles, whose
    // registers cannot hold a second copy of the step)
    if (MT < 8 && s_lo + (c + 1) * CS <= s_hi) {
#pragma unroll
      for (int u = 0; u < CS; ++u) step(w, x, u);
    } else {
#pragma unroll
      for (int u = 0; u < CS; ++u)
        if (s_lo + c * CS + u < s_hi) step(w, x, u);
    }
  };
  uint4 w[4][NB][CS], xr[2][S::NX];
  xload(xr[0], 0);
  wload(w[0], 0);
  xload(xr[1], 1);
  wload(w[1], 1);
  stage_store<bf16_t, MT, NW, CS>(xs, xr[0]);
  lds_barrier();
  for (int c0 = 0; c0 < nch; c0 += 4) {
#define PROJ_STEP(J)                                                                  \
    {                                                                                 \
      const int c = c0 + J;                                                           \
      xload(xr[J % 2], c + 2);                                                        \
      wload(w[(J + 2) % 4], c + 2);                                                   \
      if (c < nch) compute(w[J], xs + (J % 2) * S::LDS_ELEMS, c);                     \
      stage_store<bf16_t, MT, NW, CS>(xs + ((J + 1) % 2) * S::LDS_ELEMS, xr[(J + 1) % 2]); \
      lds_barrier();                                                                  \
    }
    PROJ_STEP(0) PROJ_STEP(1) PROJ_STEP(2) PROJ_STEP(3)
#undef PROJ_STEP
  }
}

// LDS elements of a projection workgroup: the two activation buffers, or
// for SwiGLU the gate values [NW/2 * 16 * NB columns][MP] fp32 if they need
// more.
template <typename T, int MT, int NW, int CS, int NB, int EPI>
constexpr int proj_lds_elems() {
  using S = ProjShape<T, MT, NW, CS>;
  constexpr int act = 2 * S::LDS_ELEMS;
  constexpr int gate = EPI == EPI_SWIGLU ? (NW / 2) * 16 * NB * S::MP * 4 / (int)sizeof(T) : 0;
  return act > gate ? act : gate;
}

// RS: the operand rows are RMSNorm numerators and a.rs holds their sums of
// squares (RowScale); separate instantiations, so projections without it
// keep no registers for it. RS_REG: each lane holds its own rows' sums
// through the main loop (4 MT registers); RS_LDS: one float4 per thread,
// the factors published in LDS after the loop (4 registers, one barrier).
// Same-box cycles: RS_LDS keeps the eight-wave SwiGLU at 108 rows within two
// workgroups per CU (RS_REG took it from 114 to 131 registers and a second
// round of workgroups: c2 batch 4 at 432 against 447 tokens/s); at five
// m-tiles (one workgroup per CU) RS_REG measured faster (c4 gate|up 2.07
// against 2.18 ms per cycle).
enum { RS_NONE = 0, RS_REG = 1, RS_LDS = 2 };
template <typename T, int MT, int NW, int CS, int NB, int EPI, int RS = RS_NONE>
__global__ __launch_bounds__(NW * 64) void proj_kernel(ProjArgs a) {
  using S = ProjShape<T, MT, NW, CS>;
  static_assert(NB == 1 || Opnd<T>::SPLIT, "several row blocks per wave: bf16 only");
  __shared__ __attribute__((aligned(16))) T xs[proj_lds_elems<T, MT, NW, CS, NB, EPI>()];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int tile = blockIdx.x / a.splits, split = blockIdx.x % a.splits;
  const int m0 = blockIdx.y * S::MP;
  ProjArgs b = a;
  b.X = (const T*)a.X + (int64_t)m0 * a.K;
  b.M = min(S::MP, a.M - m0);
  const int total = a.K / S::KS;
  const int s_lo = split * a.steps_per_split;
  const int s_hi = min(total, s_lo + a.steps_per_split);
  // SwiGLU tiles: waves [0, NW/2) take gate rows, waves [NW/2, NW) the
  // matching up rows, so one tile yields NW/2 * 16 output columns.
  // a wave's rows: NB consecutive 16-row blocks from row0
  constexpr int WR = 16 * NB;
  int row0;
  if (EPI == EPI_SWIGLU) {
    const int half = NW / 2;
    const int col0 = tile * half * WR + (wave % half) * WR;
    row0 = (wave < half) ? col0 : a.F + col0;
  } else {
    row0 = (tile * NW + wave) * WR;
  }
  // RowScale: thread i < MP requests staged row i's sums of squares before
  // the main loop (the oldest load, so the loop's waits cover it), turns
  // them into the row's factor after it and publishes it in LDS: one float4
  // per thread through the loop instead of one per m-tile and lane, so the
  // instance keeps the registers (and workgroups per CU) of the plain one
  float4 rsv[RS == RS_REG ? MT : 1];
  rsv[0] = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (RS == RS_LDS) {
    if ((int)threadIdx.x < S::MP) rsv[0] = ld4(a.rs + RS_SLICES * min(m0 + (int)threadIdx.x, a.M - 1));
  } else if constexpr (RS == RS_REG) {
#pragma unroll
    for (int t = 0; t < MT; ++t) rsv[t] = ld4(a.rs + RS_SLICES * min(m0 + 16 * t + lr, a.M - 1));
  }
  f32x4 acc[NB][MT];
  if constexpr (Opnd<T>::SPLIT) {
    proj_core_bf16<MT, NW, CS, NB>(b, row0, s_lo, s_hi, xs, acc);
  } else {
    static_assert(NB == 1, "fp32 projections take one row block per wave");
    proj_core<T, MT, NW, CS>(b, row0, s_lo, s_hi, xs, acc[0]);
  }
  if constexpr (RS == RS_LDS) {
    __shared__ float rsf[S::MP];
    if ((int)threadIdx.x < S::MP) rsf[threadIdx.x] = row_scale(rsv[0], a.rs_h, a.rs_eps);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const float f = rsf[16 * t + lr];
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) acc[jb][t] *= f;
    }
  } else if constexpr (RS == RS_REG) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const float f = row_scale(rsv[t], a.rs_h, a.rs_eps);
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) acc[jb][t] *= f;
    }
  }

  if (EPI == EPI_SWIGLU) {
    constexpr int half = NW / 2;
    __syncthreads();   // xs is reused for the gate values
    float* gate = reinterpret_cast<float*>(xs);   // [half * WR cols][MP]
    if (wave < half) {
#pragma unroll
      for (int jb = 0; jb < NB; ++jb)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            gate[(wave * WR + 16 * jb + 4 * lg + j) * S::MP + 16 * t + lr] = acc[jb][t][j];
    }
    __syncthreads();
    if (wave >= half) {
      const int w2 = wave - half;
#pragma unroll
      for (int jb = 0; jb < NB; ++jb)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int c = w2 * WR + 16 * jb + 4 * lg + j;
            const int col = tile * half * WR + c;
            const int m = 16 * t + lr;
            if (m < b.M && col < a.F) {
              const float g = gate[c * S::MP + m];
              const float v = g / (1.0f + expf(-g)) * acc[jb][t][j];
              Opnd<T>::store((T*)a.Yt, a.ytlo, (int64_t)(m0 + m) * a.F + col, v);
            }
          }
    }
  } else {
    float* Y = a.Y + (int64_t)split * a.plane;
    // one 16-byte store per lane and m-tile (four consecutive rows) when the
    // plane allows it: scalar stores cost a measurable share of the kernel
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) {
      const int r0 = row0 + 16 * jb;
      const bool vec = (a.ldy & 3) == 0 && (a.plane & 3) == 0 && ((uintptr_t)a.Y & 15) == 0 &&
                       r0 + 16 <= a.rows;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int m = 16 * t + lr;
        if (m >= b.M) continue;
        float* yr = Y + (int64_t)(m0 + m) * a.ldy + r0 + 4 * lg;
        if (vec) {
          *reinterpret_cast<f32x4*>(yr) = acc[jb][t];
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (r0 + 4 * lg + j < a.rows) yr[j] = acc[jb][t][j];
        }
      }
    }
  }
}

// ---------------------------------------------------------------- many rows
// Split-K projection over many activation rows (a batch's verify rows, a
// prefill chunk), bf16 only. The WC * XG waves of a workgroup form a WC x XG
// grid: wave (c, g) multiplies the four 16-row weight blocks [64 c, 64 c +
// 64) of the tile by staged rows [16 MT g, 16 MT (g + 1)), so each 1 KB
// activation fragment read from LDS feeds eight products (hi and lo planes,
// four blocks; two in proj_kernel's many-row tiles) and the XG groups share
// one activation stage.
//
// The activation chunk (32 K columns of every staged row, hi and lo) goes
// from global memory straight into LDS (global_load_lds_dwordx4: lane l of
// a wave's copy lands at the wave's LDS base + 16 l), so no registers hold
// it in flight and no LDS stores are issued. Each 1 KB block of the stage is
// 16 rows x 4 chunks in the xs_addr swizzle, so lane l of block b copies
// staged row R = 16 b + l / 4 at logical chunk (l % 4) ^ ((R / 2) % 4).
// Weight fragments stream into a register ring two chunks ahead; the LDS
// reads of m-tile t + 1 are issued before the products of m-tile t.
// Measured on the 7B shapes against proj_kernel at 216-512 rows: q|k|v
// -8..-15%, o -11%, down -17..-20%. (Staging through registers instead
// spilled at MT = 8 and ran 15-25% slower; SwiGLU tiles of this shape gained
// nothing over 64-row passes.)
template <int MT, int WC, int XG>
__device__ __forceinline__ void rows_core(const ProjArgs& a, int row0, int s_lo, int s_hi, int xg,
                                          bf16_t* xs0, bf16_t* xs1, f32x4 (&acc)[4][MT]) {
  constexpr int NW = WC * XG, NB = 4, KS = 32;
  constexpr int MP = 16 * MT * XG;   // staged rows of one plane
  constexpr int NBLK = 2 * MP / 16;  // 1 KB blocks of one stage buffer
  static_assert(NBLK % NW == 0, "stage blocks must split evenly over the waves");
  constexpr int BPW = NBLK / NW;
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bf16_t* W = (const bf16_t*)a.W;
  const bf16_t* X = (const bf16_t*)a.X;
  const bf16_t* wp[NB];
  int64_t wstep[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int r0 = row0 + 16 * j;
    const int rb = min(r0, a.rows - 1) >> 4;
    if ((rb + 1) * 16 <= a.rows) {   // fragment-packed block
      wp[j] = W + (int64_t)rb * 16 * a.K + lane * 8;
      wstep[j] = 16 * KS;
    } else {                         // ragged last block: row-major rows
      wp[j] = W + (int64_t)min(r0 + lr, a.rows - 1) * a.K + lg * 8;
      wstep[j] = KS;
    }
  }
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nch = s_hi - s_lo;
  if (nch <= 0) return;
  int64_t xoff[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int R = 16 * (wave * BPW + i) + (lane >> 2);
    const int plane = R / MP;
    const int row = min(R - plane * MP, a.M - 1);
    const int q = (lane & 3) ^ ((R >> 1) & 3);
    xoff[i] = plane * a.xlo + (int64_t)row * a.K + q * 8;
  }
  // (inline assembly: the compiler then leaves the wait for these copies to
  // the explicit vmcnt below instead of draining every outstanding load
  // before each LDS read; the M0 write needs one wait state)
  auto xdma = [&](bf16_t* buf, int c) {
    const int k0 = (s_lo + min(c, nch - 1)) * KS;
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16_t*)(buf + (wave * BPW + i) * 512);
      const bf16_t* src = X + xoff[i] + k0;
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src)
                   : "memory", "m0");
    }
  };
  auto wload = [&](uint4 (&w)[NB], int c) {
    const int s = s_lo + min(c, nch - 1);
#pragma unroll
    for (int j = 0; j < NB; ++j) w[j] = ld16(wp[j] + (int64_t)s * wstep[j]);
  };
  const int xr0 = 16 * MT * xg;
  auto rd = [&](const bf16_t* x, int r) {
    return *reinterpret_cast<const uint4*>(x + xs_addr<bf16_t, KS>(r, lg));
  };
  auto compute = [&](const uint4 (&w)[NB], const bf16_t* x) {
    uint4 h[2], l[2];
    h[0] = rd(x, xr0 + lr);
    l[0] = rd(x, MP + xr0 + lr);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t + 1 < MT) {
        h[(t + 1) & 1] = rd(x, xr0 + 16 * (t + 1) + lr);
        l[(t + 1) & 1] = rd(x, MP + xr0 + 16 * (t + 1) + lr);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) Mma<bf16_t>::mma(w[j], h[t & 1], acc[j][t]);
#pragma unroll
      for (int j = 0; j < NB; ++j) Mma<bf16_t>::mma(w[j], l[t & 1], acc[j][t]);
    }
  };
  // the stage of chunk c + 1 is complete once only the NB weight loads
  // issued after it (chunk c + 2) may still be in flight; the barrier then
  // also ends every wave's reads of the buffer the next copy overwrites
  uint4 w[4][NB];
  xdma(xs0, 0);
  wload(w[0], 0);
  wload(w[1], 1);
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * NB) : "memory");
  for (int c0 = 0; c0 < nch; c0 += 4) {
#define ROWS_STEP(J)                                                           \
    {                                                                          \
      const int c = c0 + J;                                                    \
      xdma((J % 2) ? xs0 : xs1, c + 1);                                        \
      wload(w[(J + 2) % 4], c + 2);                                            \
      if (c < nch) compute(w[J], (J % 2) ? xs1 : xs0);                         \
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(NB) : "memory");   \
    }
    ROWS_STEP(0) ROWS_STEP(1) ROWS_STEP(2) ROWS_STEP(3)
#undef ROWS_STEP
  }
}

template <int MT, int WC, int XG>
__global__ __launch_bounds__(WC * XG * 64) void rows_kernel(ProjArgs a) {
  constexpr int NB = 4, MP = 16 * MT * XG, BUF = 2 * MP * 32;
  __shared__ __attribute__((aligned(1024))) bf16_t xs0[BUF];
  __shared__ __attribute__((aligned(1024))) bf16_t xs1[BUF];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int wc = wave % WC, xg = wave / WC;
  const int tile = blockIdx.x / a.splits, split = blockIdx.x % a.splits;
  const int m0 = blockIdx.y * MP;
  ProjArgs b = a;
  b.X = (const bf16_t*)a.X + (int64_t)m0 * a.K;
  b.M = min(MP, a.M - m0);
  const int total = a.K / 32;
  const int s_lo = split * a.steps_per_split;
  const int s_hi = min(total, s_lo + a.steps_per_split);
  const int xrow0 = 16 * MT * xg;
  const int row0 = (tile * WC + wc) * 16 * NB;
  f32x4 acc[NB][MT];
  rows_core<MT, WC, XG>(b, row0, s_lo, s_hi, xg, xs0, xs1, acc);
  if (a.rs) {   // RowScale (uniform); loaded here: this kernel's registers are spoken for
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const float f = row_scale(ld4(a.rs + RS_SLICES * min(m0 + xrow0 + 16 * t + lr, a.M - 1)),
                                a.rs_h, a.rs_eps);
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) acc[jb][t] *= f;
    }
  }
  float* Y = a.Y + (int64_t)split * a.plane;
#pragma unroll
  for (int jb = 0; jb < NB; ++jb) {
    const int r0 = row0 + 16 * jb;
    const bool vec = (a.ldy & 3) == 0 && (a.plane & 3) == 0 && ((uintptr_t)a.Y & 15) == 0 &&
                     r0 + 16 <= a.rows;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = xrow0 + 16 * t + lr;
      if (m >= b.M) continue;
      float* yr = Y + (int64_t)(m0 + m) * a.ldy + r0 + 4 * lg;
      if (vec) {
        *reinterpret_cast<f32x4*>(yr) = acc[jb][t];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (r0 + 4 * lg + j < a.rows) yr[j] = acc[jb][t][j];
      }
    }
  }
}

// SwiGLU over many rows, second half: the gate|up projection left S partial
// planes [S][M][2F] (gate columns, then up); this pass sums each column's
// planes in plane order and writes SiLU(g) * u as the next operand (bf16 hi
// and lo planes). Four consecutive columns per thread, 16-byte loads.
__global__ __launch_bounds__(256) void silu_mul_planes_kernel(const float* __restrict__ part, int S,
                                                              int64_t plane, int M, int F,
                                                              bf16_t* __restrict__ out, int64_t lo) {
  const int m = blockIdx.y;
  const int j = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (j >= F) return;
  const float* pr = part + (int64_t)m * 2 * F;
  float4 g = ld4(pr + j), u = ld4(pr + F + j);
  for (int s = 1; s < S; ++s) {
    const float4 a = ld4(pr + s * plane + j), b = ld4(pr + s * plane + F + j);
    g.x += a.x; g.y += a.y; g.z += a.z; g.w += a.w;
    u.x += b.x; u.y += b.y; u.z += b.z; u.w += b.w;
  }
  const float v[4] = {g.x / (1.0f + expf(-g.x)) * u.x, g.y / (1.0f + expf(-g.y)) * u.y,
                      g.z / (1.0f + expf(-g.z)) * u.z, g.w / (1.0f + expf(-g.w)) * u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) Opnd<bf16_t>::store(out, lo, (int64_t)m * F + j + e, v[e]);
}

// ---------------------------------------------------------------- packing
// Fragment packing of a bf16 matrix [rows, K] (K a multiple of 32): full
// 16-row block rb is stored as K/32 fragments of 1 KB, fragment s holding
// rows 16rb..16rb+15 x columns 32s..32s+31 in the order the 16x16x32 MFMA
// A operand is loaded (lane l = r + 16g: row 16rb + r, columns 32s + 8g ..
// 32s + 8g + 7). A block keeps its row-major byte range, so the first
// 16*nrb rows pack in place through a staging copy; one wave load then reads
// 1 KB of contiguous HBM instead of sixteen 64-byte pieces.
__global__ __launch_bounds__(256) void pack_frag_kernel(const bf16_t* __restrict__ src,
                                                        bf16_t* __restrict__ dst, int64_t pieces,
                                                        int K) {
  const int steps = K >> 5;
  for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < pieces; p += (int64_t)gridDim.x * 256) {
    const int64_t f = p >> 6;
    const int l = (int)(p & 63);
    const int64_t rb = f / steps;
    const int s = (int)(f % steps);
    const uint4 v = ld16(src + (rb * 16 + (l & 15)) * K + s * 32 + 8 * (l >> 4));
    *reinterpret_cast<uint4*>(dst + p * 8) = v;
  }
}

// ---------------------------------------------------------------- LM head
// Per-tile top-k record of the draft LM head: {max, sum of exp, k values,
// k ids}, padded to a multiple of four floats so a row's records (stored
// row-major: record (m, tile) at (m * n_tiles + tile) * rec) copy with
// 16-byte loads.
__host__ __device__ constexpr int topk_record(int k) { return (2 + 2 * k + 3) & ~3; }

struct HeadArgs {
  ProjArgs p;     // W = LM head [V, H], X = features
  int k;
  float* part;    // per tile and row: argmax {max1, id1, max2} or topk {max, sum, k vals, k ids}
  float* logits;  // optional [M, V]
};

template <typename T, int MT, int NW, int CS, bool TOPK>
__global__ __launch_bounds__(NW * 64) void lmhead_kernel(HeadArgs h) {
  using S = ProjShape<T, MT, NW, CS>;
  __shared__ __attribute__((aligned(16))) T xs[2 * S::LDS_ELEMS];
  const ProjArgs& a = h.p;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int tile = blockIdx.x;
  const int R = NW * 16;
  const int row0 = tile * R + wave * 16;
  f32x4 acc[MT];
  proj_core<T, MT, NW, CS>(a, row0, 0, a.K / S::KS, xs, acc);
  __syncthreads();
  float* vals = reinterpret_cast<float*>(xs);   // [R][MP]
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) vals[(wave * 16 + 4 * lg + j) * S::MP + 16 * t + lr] = acc[t][j];
  __syncthreads();
  const int nvalid = min(R, a.rows - tile * R);
  if (h.logits) {
    for (int e = threadIdx.x; e < R * S::MP; e += NW * 64) {
      const int m = e / R, n = e % R;
      if (m < a.M && n < nvalid) h.logits[(int64_t)m * a.rows + tile * R + n] = vals[n * S::MP + m];
    }
  }
  // each lane holds RPL of the tile's R vocabulary rows: lane + 64 * u
  constexpr int RPL = (NW * 16) / 64;
  static_assert(RPL * 64 == NW * 16, "tile rows must be a multiple of the wave width");
  static_assert(NW * 16 * S::MP * 4 <= (int)sizeof(xs), "row values must fit the staging buffer");
  const int stride = TOPK ? topk_record(h.k) : 3;
  for (int m = wave; m < a.M; m += NW) {
    float v[RPL];
    int id[RPL];
#pragma unroll
    for (int u = 0; u < RPL; ++u) {
      const int n = lane + 64 * u;
      const bool ok = n < nvalid;
      v[u] = ok ? vals[n * S::MP + m] : -INFINITY;
      id[u] = ok ? tile * R + n : 0x7fffffff;
    }
    float* out = TOPK ? h.part + ((int64_t)m * gridDim.x + tile) * stride
                      : h.part + ((int64_t)tile * a.M + m) * stride;
    if (!TOPK) {
      float bv = v[0];
      int bi = id[0];
#pragma unroll
      for (int u = 1; u < RPL; ++u)
        if (v[u] > bv || (v[u] == bv && id[u] < bi)) { bv = v[u]; bi = id[u]; }
      int bl = lane;
      wave_argmax(bv, bi, bl);
      float lv = -INFINITY;
#pragma unroll
      for (int u = 0; u < RPL; ++u)
        if (id[u] != bi) lv = fmaxf(lv, v[u]);
      const float sv = wave_max(lv);
      if (lane == 0) { out[0] = bv; out[1] = __int_as_float(bi); out[2] = sv; }
    } else {
      float lm = v[0];
#pragma unroll
      for (int u = 1; u < RPL; ++u) lm = fmaxf(lm, v[u]);
      const float mx = wave_max(lm);
      float le = 0.f;
#pragma unroll
      for (int u = 0; u < RPL; ++u) le += (id[u] != 0x7fffffff) ? expf(v[u] - mx) : 0.f;
      const float se = wave_sum(le);
      if (lane == 0) { out[0] = mx; out[1] = se; }
      for (int i = 0; i < h.k; ++i) {
        // this lane's best remaining candidate, then the wave's
        float bv = v[0];
        int bi = id[0];
#pragma unroll
        for (int u = 1; u < RPL; ++u)
          if (v[u] > bv || (v[u] == bv && id[u] < bi)) { bv = v[u]; bi = id[u]; }
        int bl = lane;
        wave_argmax(bv, bi, bl);
        if (lane == 0) { out[2 + i] = bv; out[2 + h.k + i] = __int_as_float(bi); }
#pragma unroll
        for (int u = 0; u < RPL; ++u)
          if (id[u] == bi) { v[u] = -INFINITY; id[u] = 0x7fffffff; }
      }
    }
  }
}

// one workgroup per row: merge the per-tile argmax records
__global__ __launch_bounds__(256) void argmax_combine(const float* part, int n_tiles, int M,
                                                      int32_t* g, float* margin) {
  const int m = blockIdx.x;
  float b1 = -INFINITY, b2 = -INFINITY;
  int i1 = 0x7fffffff;
  for (int t = threadIdx.x; t < n_tiles; t += blockDim.x) {
    const float* p = part + ((int64_t)t * M + m) * 3;
    const float p1 = p[0], p2 = p[2];
    const int pi = __float_as_int(p[1]);
    if (p1 > b1 || (p1 == b1 && pi < i1)) { b2 = fmaxf(b1, p2); b1 = p1; i1 = pi; }
    else b2 = fmaxf(b2, p1);
  }
  __shared__ float s1[256], s2[256];
  __shared__ int si[256];
  s1[threadIdx.x] = b1; s2[threadIdx.x] = b2; si[threadIdx.x] = i1;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      float a1 = s1[threadIdx.x], a2 = s2[threadIdx.x];
      int ai = si[threadIdx.x];
      const float c1 = s1[threadIdx.x + o], c2 = s2[threadIdx.x + o];
      const int ci = si[threadIdx.x + o];
      if (c1 > a1 || (c1 == a1 && ci < ai)) { a2 = fmaxf(a1, c2); a1 = c1; ai = ci; }
      else a2 = fmaxf(a2, c1);
      s1[threadIdx.x] = a1; s2[threadIdx.x] = a2; si[threadIdx.x] = ai;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) { g[m] = si[0]; margin[m] = s1[0] - s2[0]; }
}

// One workgroup of four waves per row: the global max and log-sum-exp over
// the vocabulary tiles, then the k best (val desc, id asc) merged from the
// tiles' sorted lists. The row's records are first copied to LDS with
// 16-byte loads, sixteen in flight per thread (in segments when they exceed
// the 96 KB buffer; a 128k vocabulary's 1002 tiles of top-8 records fit in
// one). A threshold T, the k-th largest of the tile maxima, bounds the
// merge: k distinct values are >= T, so no value below T is among the k
// best, and since every tile list is sorted a tile stops at its first
// candidate under T. Each thread keeps its best candidates in registers as
// sorted 64-bit (value desc, id asc) keys (bubble insertion with static
// indices); each wave pops its k best with wave-wide 64-bit DPP maxima, and
// wave 0 merges the four lists.
__global__ __launch_bounds__(256) void topk_combine(const float* part, int n_tiles, int M, int k,
                                                    int32_t* ids, float* logp) {
  constexpr int KMAX = 16, BUF = 24576, NT = 256, NWV = NT / 64;
  __shared__ __attribute__((aligned(16))) float buf[BUF];
  __shared__ float s_red[2 * NWV];
  __shared__ uint64_t s_key[NWV * KMAX];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rec = topk_record(k), seg = BUF / rec;
  const float* row = part + (int64_t)m * n_tiles * rec;
  auto stage = [&](int t0, int nt) {
    __syncthreads();   // earlier reads of buf are done
    const float4* src = reinterpret_cast<const float4*>(row + (int64_t)t0 * rec);
    float4* dst = reinterpret_cast<float4*>(buf);
    const int n4 = nt * rec / 4;
    for (int i0 = 0; i0 < n4; i0 += NT * 16) {
      // all sixteen loads are issued before the first store: threads past
      // the end re-copy the last piece (same value, same place) instead of
      // branching, so no load is sunk into a conditional store
      float4 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = src[min(i0 + NT * u + tid, n4 - 1)];
#pragma unroll
      for (int u = 0; u < 16; ++u) dst[min(i0 + NT * u + tid, n4 - 1)] = v[u];
    }
    __syncthreads();
  };
  // this thread's best candidates as (value desc, id asc) keys, sorted
  constexpr uint64_t NONE = 0;   // below every real key
  uint64_t lk[KMAX];
  auto reset = [&]() {
#pragma unroll
    for (int i = 0; i < KMAX; ++i) lk[i] = NONE;
  };
  auto insert = [&](uint64_t key) {
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      if (i < k) {
        const uint64_t cur = lk[i];
        lk[i] = key > cur ? key : cur;
        key = key > cur ? cur : key;
      }
    }
  };
  // k rounds of a wave-wide maximum over the lanes' list heads; the lane
  // holding it (keys are unique) pops it; emit(r, key)
  auto pop_k = [&](auto&& emit) {
    for (int r = 0; r < k; ++r) {
      const uint64_t best = wave_max_u64(lk[0]);
      emit(r, best);
      if (lk[0] == best && best != NONE) {
#pragma unroll
        for (int i = 0; i + 1 < KMAX; ++i) lk[i] = lk[i + 1];
        lk[KMAX - 1] = NONE;
      }
    }
  };
  // every wave's k best go to LDS; wave 0 then holds them one per lane
  // (4k <= 64) and pops the k best of the workgroup
  auto merge_waves = [&](auto&& emit) {
    pop_k([&](int r, uint64_t key) {
      if (lane == 0) s_key[wave * KMAX + r] = key;
    });
    __syncthreads();
    if (wave == 0) {
      reset();
      const int w = lane / KMAX, r = lane % KMAX;
      if (r < k) lk[0] = s_key[w * KMAX + r];
      pop_k(emit);
    }
    __syncthreads();
  };
  // pass 1: the global max and the threshold T from the tile maxima
  reset();
  float mx = -INFINITY;
  for (int t0 = 0; t0 < n_tiles; t0 += seg) {
    const int nt = min(seg, n_tiles - t0);
    stage(t0, nt);
    for (int t = tid; t < nt; t += NT) {
      const float v = buf[t * rec];
      mx = fmaxf(mx, v);
      insert(vid_key(v, t0 + t));
    }
  }
  mx = wave_max(mx);
  if (lane == 0) s_red[wave] = mx;
  merge_waves([&](int r, uint64_t key) {
    if (r == k - 1 && lane == 0) s_red[NWV] = vid_value(key);
  });
  const float gmax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const float thr = s_red[NWV];
  // pass 2: sum of exp and the k best among candidates >= T
  reset();
  float se = 0.f;
  for (int t0 = 0; t0 < n_tiles; t0 += seg) {
    const int nt = min(seg, n_tiles - t0);
    if (n_tiles > seg) stage(t0, nt);   // a single segment is still staged
    for (int t = tid; t < nt; t += NT) {
      const float* p = buf + t * rec;
      se += p[1] * expf(p[0] - gmax);
      for (int c = 0; c < k; ++c) {
        const float cv = p[2 + c];
        const int ci = __float_as_int(p[2 + k + c]);
        if (ci == 0x7fffffff || cv < thr) break;   // tile lists are sorted
        insert(vid_key(cv, ci));
      }
    }
  }
  se = wave_sum(se);
  __syncthreads();   // s_red reads above are done
  if (lane == 0) s_red[wave] = se;
  __syncthreads();
  const float lse = logf((s_red[0] + s_red[1]) + (s_red[2] + s_red[3]));
  merge_waves([&](int r, uint64_t key) {
    if (lane == 0) {
      ids[m * k + r] = vid_id(key);
      logp[m * k + r] = (vid_value(key) - gmax) - lse;
    }
  });
}

// ---------------------------------------------------------------- dispatch
// Launch shape per m-tile count and kernel kind (partial-plane projection,
// SwiGLU, LM head): waves per workgroup and steps per staged chunk. Small
// chunks keep the LDS footprint low so several workgroups share a CU, which
// the weight stream needs more than a deep per-wave prefetch (measured on
// the 7B shapes).
constexpr int KIND_HEAD = 3;
template <int MT, int KIND> struct Cfg { static constexpr int NW = 8, CS = 4, NB = 1; };
template <> struct Cfg<1, EPI_PART> { static constexpr int NW = 4, CS = 4, NB = 1; };
template <> struct Cfg<1, EPI_SWIGLU> { static constexpr int NW = 8, CS = 4, NB = 1; };
template <> struct Cfg<1, KIND_HEAD> { static constexpr int NW = 8, CS = 8, NB = 1; };
template <> struct Cfg<2, EPI_PART> { static constexpr int NW = 8, CS = 2, NB = 1; };
template <> struct Cfg<2, EPI_SWIGLU> { static constexpr int NW = 8, CS = 2, NB = 1; };
template <> struct Cfg<3, EPI_PART> { static constexpr int NW = 4, CS = 2, NB = 1; };
template <> struct Cfg<3, EPI_SWIGLU> { static constexpr int NW = 8, CS = 2, NB = 1; };
template <> struct Cfg<4, EPI_PART> { static constexpr int NW = 8, CS = 2, NB = 1; };
template <> struct Cfg<4, EPI_SWIGLU> { static constexpr int NW = 8, CS = 2, NB = 1; };
template <> struct Cfg<5, EPI_PART> { static constexpr int NW = 8, CS = 2, NB = 1; };
template <> struct Cfg<5, EPI_SWIGLU> { static constexpr int NW = 8, CS = 2, NB = 1; };

template <int KIND>
int waves_t(int mt) {
  switch (mt) {
    case 1: return Cfg<1, KIND>::NW;
    case 2: return Cfg<2, KIND>::NW;
    case 3: return Cfg<3, KIND>::NW;
    case 4: return Cfg<4, KIND>::NW;
    default: return Cfg<5, KIND>::NW;
  }
}
template <int KIND>
int chunk_t(int mt) {
  switch (mt) {
    case 1: return Cfg<1, KIND>::CS;
    case 2: return Cfg<2, KIND>::CS;
    case 3: return Cfg<3, KIND>::CS;
    case 4: return Cfg<4, KIND>::CS;
    default: return Cfg<5, KIND>::CS;
  }
}
int waves_for(int mt, int kind) {
  return kind == EPI_SWIGLU ? waves_t<EPI_SWIGLU>(mt) : kind == KIND_HEAD ? waves_t<KIND_HEAD>(mt) : waves_t<EPI_PART>(mt);
}
int chunk_for(int mt, int kind) {
  return kind == EPI_SWIGLU ? chunk_t<EPI_SWIGLU>(mt) : kind == KIND_HEAD ? chunk_t<KIND_HEAD>(mt) : chunk_t<EPI_PART>(mt);
}

// One dispatch of proj_kernel<T, MT, NW, CS, NB, EPI, RS>, with RS chosen by
// whether the projection scales its rows (bf16 only).
template <typename T, int MT, int NW, int CS, int NB, int EPI>
hipError_t proj_dispatch(const ProjArgs& a, dim3 grid, dim3 block, hipStream_t st, const KTiming* tm) {
  if constexpr (Opnd<T>::SPLIT) {
    if (a.rs) {
      constexpr int R = MT >= 5 ? RS_REG : RS_LDS;
      if (tm)
        hipExtLaunchKernelGGL((proj_kernel<T, MT, NW, CS, NB, EPI, R>), grid, block, 0, st, tm->start, tm->stop, 0, a);
      else
        hipLaunchKernelGGL((proj_kernel<T, MT, NW, CS, NB, EPI, R>), grid, block, 0, st, a);
      return hipGetLastError();
    }
  } else {
    if (a.rs) return hipErrorInvalidValue;
  }
  if (tm)
    hipExtLaunchKernelGGL((proj_kernel<T, MT, NW, CS, NB, EPI>), grid, block, 0, st, tm->start, tm->stop, 0, a);
  else
    hipLaunchKernelGGL((proj_kernel<T, MT, NW, CS, NB, EPI>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <typename T, int MT, int EPI>
hipError_t launch_proj_mt(const ProjArgs& a, int tiles, int m_chunks, hipStream_t st, const KTiming* tm) {
  constexpr int NW = Cfg<MT, EPI>::NW, CS = Cfg<MT, EPI>::CS;
  constexpr int NB = Opnd<T>::SPLIT ? Cfg<MT, EPI>::NB : 1;
  return proj_dispatch<T, MT, NW, CS, NB, EPI>(a, dim3(tiles * a.splits, m_chunks), dim3(NW * 64), st, tm);
}

// SwiGLU with six or fourteen waves (48 or 112 output columns per
// workgroup) in place of eight, for FFN widths whose eight-wave grid leaves
// CUs idle or spills into a second round: F = 11008 takes 230 workgroups
// (eight waves: 172; measured 8-11% faster at 7, 27 and 61 rows) and F =
// 28672 takes 256 (eight waves: 448; 9% faster at 61 rows).
template <typename T, int MT, int NW>
hipError_t launch_swiglu_w(const ProjArgs& a, int tiles, hipStream_t st, const KTiming* tm) {
  constexpr int CS = (NW == 6 && MT == 2) ? 4 : 2;
  return proj_dispatch<T, MT, NW, CS, 1, EPI_SWIGLU>(a, dim3(tiles), dim3(NW * 64), st, tm);
}

template <typename T, int EPI>
hipError_t launch_proj_t(int mt, const ProjArgs& a, int tiles, int m_chunks, hipStream_t st,
                         const KTiming* tm, int nw) {
  if constexpr (EPI == EPI_SWIGLU) {
    if (nw == 6 || nw == 14) {
      if (m_chunks != 1) return hipErrorInvalidValue;
      if (nw == 6) {
        switch (mt) {
          case 1: return launch_swiglu_w<T, 1, 6>(a, tiles, st, tm);
          case 2: return launch_swiglu_w<T, 2, 6>(a, tiles, st, tm);
          case 3: return launch_swiglu_w<T, 3, 6>(a, tiles, st, tm);
          case 4: return launch_swiglu_w<T, 4, 6>(a, tiles, st, tm);
          case 5: return launch_swiglu_w<T, 5, 6>(a, tiles, st, tm);
          default: return hipErrorInvalidValue;
        }
      }
      switch (mt) {   // fourteen waves leave 128 registers per lane: up to four m-tiles
        case 1: return launch_swiglu_w<T, 1, 14>(a, tiles, st, tm);
        case 2: return launch_swiglu_w<T, 2, 14>(a, tiles, st, tm);
        case 3: return launch_swiglu_w<T, 3, 14>(a, tiles, st, tm);
        case 4: return launch_swiglu_w<T, 4, 14>(a, tiles, st, tm);
        default: return hipErrorInvalidValue;
      }
    }
  }
  if constexpr (EPI == EPI_PART) {
    if (nw == 6) {   // the six-wave shape of gemm_plan (two or four m-tiles, one m-chunk)
      if ((mt != 2 && mt != 4) || m_chunks != 1) return hipErrorInvalidValue;
      const dim3 grid(tiles * a.splits), block(6 * 64);
      return mt == 2 ? proj_dispatch<T, 2, 6, 2, 1, EPI_PART>(a, grid, block, st, tm)
                     : proj_dispatch<T, 4, 6, 2, 1, EPI_PART>(a, grid, block, st, tm);
    }
  }
  switch (mt) {
    case 1: return launch_proj_mt<T, 1, EPI>(a, tiles, m_chunks, st, tm);
    case 2: return launch_proj_mt<T, 2, EPI>(a, tiles, m_chunks, st, tm);
    case 3: return launch_proj_mt<T, 3, EPI>(a, tiles, m_chunks, st, tm);
    case 4: return launch_proj_mt<T, 4, EPI>(a, tiles, m_chunks, st, tm);
    case 5: return launch_proj_mt<T, 5, EPI>(a, tiles, m_chunks, st, tm);
    default: return hipErrorInvalidValue;
  }
}

// rows_kernel with four wave columns (256 weight rows per tile) and two
// row groups (16 MT * 2 rows per m-chunk)
template <int MT>
hipError_t launch_rows_mt(const ProjArgs& a, int tiles, int m_chunks, hipStream_t st, const KTiming* tm) {
  const dim3 grid(tiles * a.splits, m_chunks), block(8 * 64);
  if (tm)
    hipExtLaunchKernelGGL((rows_kernel<MT, 4, 2>), grid, block, 0, st, tm->start, tm->stop, 0, a);
  else
    hipLaunchKernelGGL((rows_kernel<MT, 4, 2>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <typename T, bool TOPK, int MT, int NW = Cfg<MT, KIND_HEAD>::NW, int CS = Cfg<MT, KIND_HEAD>::CS>
hipError_t launch_head_mt(const HeadArgs& h, int tiles, hipStream_t st) {
  hipLaunchKernelGGL((lmhead_kernel<T, MT, NW, CS, TOPK>), dim3(tiles), dim3(NW * 64), 0, st, h);
  return hipGetLastError();
}

// LM-head tiles. Every workgroup stages all of the call's activation rows
// over the full hidden width, so these reads grow with the number of
// workgroups and of distinct rows. Up to HEAD_FEW_ROWS rows they mostly hit
// in the vector cache and four-wave tiles of 64 vocabulary rows with deep
// chunks stream the weight best; above that, eight-wave tiles of 128
// vocabulary rows halve the activation reads per weight byte and the merge's
// per-tile records.
constexpr int HEAD_FEW_ROWS = 4;

template <typename T, bool TOPK>
hipError_t launch_head_t(int mt, const HeadArgs& h, int tiles, hipStream_t st) {
  switch (mt) {
    case 1: return h.p.M <= HEAD_FEW_ROWS ? launch_head_mt<T, TOPK, 1, 4, 16>(h, tiles, st)
                                          : launch_head_mt<T, TOPK, 1>(h, tiles, st);
    case 2: return launch_head_mt<T, TOPK, 2>(h, tiles, st);
    case 3: return launch_head_mt<T, TOPK, 3>(h, tiles, st);
    case 4: return launch_head_mt<T, TOPK, 4>(h, tiles, st);
    default: return launch_head_mt<T, TOPK, 5>(h, tiles, st);
  }
}

int head_rows(int M) { return M <= HEAD_FEW_ROWS ? 64 : 16 * waves_for(M > 64 ? 5 : (M + 15) / 16, KIND_HEAD); }

}  // namespace

GemmPlan gemm_plan(int M, int N_rows, int K, int dtype, int epi) {
  GemmPlan p;
  if (dtype == 1 && epi == EPI_PART && (M > 128 || (M > 80 && (N_rows >= 8192 || K >= 8192)))) {
    // rows_kernel (above 128 rows; from 81 rows for wide or deep shapes, the
    // 4096 x 4096 one measured faster in 64-row passes there): 256 weight
    // rows per tile; split K until the grid covers three quarters of the
    // CUs, keeping >= 16 steps per split. m-chunks of 256 rows when that
    // takes at most four splits (more measured slower), else of 128 rows
    // (more m-chunks for narrow outputs)
    p.xg = 2;
    p.nb = 4;
    p.nw = 8;
    p.n_tiles = (N_rows + 255) / 256;
    const int steps = K / 32;
    auto splits_for = [&](int m_chunks, int cap) {
      int s = 1;
      while (s < cap && p.n_tiles * m_chunks * s * 4 < 3 * 256 && steps / (2 * s) >= 16) s *= 2;
      return s;
    };
    const int mc8 = (M + 255) / 256, s8 = splits_for(mc8, 4);
    if (M > 128 && p.n_tiles * mc8 * s8 * 4 >= 3 * 256) {
      p.mt = 8;
      p.m_chunks = mc8;
      // several 256-row chunks whose unsplit grid already covers most CUs
      // (the gate|up shapes at 512 rows) run unsplit: measured 3-10% faster,
      // and the consumer sums one plane
      p.splits = mc8 >= 2 && p.n_tiles * mc8 >= 160 ? 1 : s8;
    } else {
      p.mt = 4;
      p.m_chunks = (M + 127) / 128;
      p.splits = splits_for(p.m_chunks, 16);
    }
    return p;
  }
  if (M <= 80) {
    p.mt = (M + 15) / 16;
  } else {
    p.mt = 4;   // passes of 64 rows
  }
  p.m_chunks = (M + 16 * p.mt - 1) / (16 * p.mt);
  p.nw = waves_for(p.mt, epi);
  p.nb = 1;
  const int rows_per_tile = 16 * p.nw * p.nb;
  if (epi == EPI_SWIGLU) {
    const int F = N_rows / 2;
    p.n_tiles = (F + rows_per_tile / 2 - 1) / (rows_per_tile / 2);
    p.splits = 1;
    // one pass of row tiles: of six, eight and fourteen waves take the
    // largest grid that still fits one workgroup per CU (eight if none does)
    if (p.m_chunks == 1 && p.mt <= 5 && p.nb == 1 && p.nw == 8) {
      int best = p.n_tiles <= 256 ? p.n_tiles : 0;
      for (int w : {6, 14}) {
        if (w == 14 && p.mt > 4) continue;
        const int t = (F + 8 * w - 1) / (8 * w);
        if (t <= 256 && t > best) {
          best = t;
          p.nw = w;
          p.n_tiles = t;
        }
      }
    }
  } else {
    // bf16, two or four m-tiles, an output whose 96-row tiles number
    // 96-128: six waves and two splits (192-256 workgroups of long
    // pipelines, two partial planes for the consumer). The q|k|v projection:
    // 20.8 us against 22.5 (eight waves, eight splits) at 27 rows, 26.0
    // against 28.6 (eight waves, two splits) at 61; narrower outputs (o,
    // down) stay faster with eight waves.
    if (dtype == 1 && (p.mt == 2 || p.mt == 4) && p.m_chunks == 1 && N_rows % 96 == 0 &&
        N_rows / 96 >= 96 && N_rows / 96 <= 128 && K / 32 >= 64) {
      p.nw = 6;
      p.n_tiles = N_rows / 96;
      p.splits = 2;
      return p;
    }
    p.n_tiles = (N_rows + rows_per_tile - 1) / rows_per_tile;
    const int steps = K / (dtype == 1 ? 32 : 16);
    // Split K as little as keeps each workgroup's pipeline long (>= 8 chunks
    // at one or two m-tiles, 16 above), then widen until the grid covers
    // every CU, and cap it at four workgroups per CU: each split adds an
    // [M, N] fp32 plane of HBM writes (measured on the 7B shapes).
    const int cs = chunk_for(p.mt, epi);
    const int chunks = (steps + cs - 1) / cs;
    const int target = p.mt <= 2 ? 8 : p.mt < 8 ? 16 : 32;
    int s = 1;
    while (s < 16 && chunks / (2 * s) >= target) s *= 2;
    if (p.mt < 8)   // the many-row tiles keep the MFMAs busy without a wider grid
      while (p.n_tiles * s < 256 && s < 16 && chunks / (2 * s) >= 4) s *= 2;
    while (p.n_tiles * s > 1024 && s > 1) s /= 2;
    // Four or more m-tiles (49-80 rows): one round of workgroups, the
    // largest split count (any integer) that keeps the grid within 256.
    // A second partial round measured slower at these heavier workgroups
    // (q|k|v at 65 rows: 5 splits 20.6 us against 8 splits 24.1; the 70B
    // down at 61 rows: 4 splits 100 us against 16 splits 106); at one or two
    // m-tiles several workgroups per CU hide more latency and win.
    if (p.mt >= 4 && p.n_tiles * s > 256) s = std::max(1, 256 / p.n_tiles);
    p.splits = s;
  }
  return p;
}

uint64_t gemm_part_floats(const GemmPlan& p, int N_rows, int M) {
  return (uint64_t)p.splits * M * N_rows;
}

bool swiglu_by_planes(int dtype, int M) { return dtype == 1 && M > 128; }

hipError_t launch_gemm(int dtype, int epi, const void* W, const void* x, int64_t xlo, int M, int N,
                       int K, float* Y, int64_t ldy, void* Yt, int64_t ytlo, int splits_out[1],
                       hipStream_t stream, const KTiming* tm, RowScale rsc) {
  if (M <= 0) return hipSuccess;
  if (epi == EPI_SWIGLU && swiglu_by_planes(dtype, M)) {
    // many rows: gate|up as one split-K projection (rows_kernel) into the
    // caller's partial-plane scratch Y, then SiLU(g) * u into Yt. Measured
    // against 64-row passes of the fused kernel: -17..-24% at 256-512 rows
    // on the 7B and 8B FFN shapes.
    if (!Y || (N & 3)) return hipErrorInvalidValue;
    int S = 1;
    hipError_t e = launch_gemm(dtype, EPI_PART, W, x, xlo, M, 2 * N, K, Y, 2 * N, nullptr, 0, &S,
                               stream, tm, rsc);
    if (e != hipSuccess) return e;
    const dim3 grid((N / 4 + 255) / 256, M);
    hipLaunchKernelGGL(silu_mul_planes_kernel, grid, dim3(256), 0, stream, Y, S, (int64_t)M * 2 * N, M,
                       N, (bf16_t*)Yt, ytlo);
    if (splits_out) splits_out[0] = S;
    return hipGetLastError();
  }
  const int rows = (epi == EPI_SWIGLU) ? 2 * N : N;
  GemmPlan p = gemm_plan(M, rows, K, dtype, epi);
  ProjArgs a;
  a.W = W; a.X = x; a.xlo = xlo; a.M = M; a.rows = rows; a.K = K; a.F = N;
  a.splits = p.splits;
  const int steps = K / (dtype == 1 ? 32 : 16);
  a.steps_per_split = (steps + p.splits - 1) / p.splits;
  a.Y = Y; a.ldy = ldy; a.plane = (int64_t)M * ldy;
  a.Yt = Yt; a.ytlo = ytlo;
  a.rs = rsc.ss; a.rs_h = rsc.H; a.rs_eps = rsc.eps;
  if (rsc.ss && rsc.H <= 0) return hipErrorInvalidValue;
  if (splits_out) splits_out[0] = p.splits;
  if (p.xg == 2)
    return p.mt == 8 ? launch_rows_mt<8>(a, p.n_tiles, p.m_chunks, stream, tm)
                     : launch_rows_mt<4>(a, p.n_tiles, p.m_chunks, stream, tm);
  if (dtype == 1) {
    return epi == EPI_SWIGLU ? launch_proj_t<bf16_t, EPI_SWIGLU>(p.mt, a, p.n_tiles, p.m_chunks, stream, tm, p.nw)
                             : launch_proj_t<bf16_t, EPI_PART>(p.mt, a, p.n_tiles, p.m_chunks, stream, tm, p.nw);
  }
  return epi == EPI_SWIGLU ? launch_proj_t<float, EPI_SWIGLU>(p.mt, a, p.n_tiles, p.m_chunks, stream, tm, p.nw)
                           : launch_proj_t<float, EPI_PART>(p.mt, a, p.n_tiles, p.m_chunks, stream, tm, p.nw);
}

uint64_t lmhead_part_floats(int M, int V, int k) {
  if (M > 80) M = 64;
  const int n_tiles = (V + head_rows(M) - 1) / head_rows(M);
  return (uint64_t)n_tiles * M * (k > 0 ? topk_record(k) : 3);
}

static hipError_t head_launch(int dtype, bool topk, const void* W, const void* x, int64_t xlo, int M, int V,
                              int H, int k, float* part, float* logits, int* n_tiles_out,
                              hipStream_t stream) {
  HeadArgs h;
  h.p.W = W; h.p.X = x; h.p.xlo = xlo; h.p.M = M; h.p.rows = V; h.p.K = H; h.p.F = 0;
  h.p.splits = 1; h.p.steps_per_split = H / (dtype == 1 ? 32 : 16);
  h.p.Y = nullptr; h.p.ldy = 0; h.p.plane = 0; h.p.Yt = nullptr; h.p.ytlo = 0;
  h.k = k; h.part = part; h.logits = logits;
  const int mt = (M + 15) / 16;
  const int tiles = (V + head_rows(M) - 1) / head_rows(M);
  *n_tiles_out = tiles;
  if (dtype == 1)
    return topk ? launch_head_t<bf16_t, true>(mt, h, tiles, stream) : launch_head_t<bf16_t, false>(mt, h, tiles, stream);
  return topk ? launch_head_t<float, true>(mt, h, tiles, stream) : launch_head_t<float, false>(mt, h, tiles, stream);
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
  int tiles = 0;
  hipError_t e = head_launch(dtype, false, W, x, xlo, M, V, H, 0, part, logits, &tiles, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(argmax_combine, dim3(M), dim3(256), 0, stream, part, tiles, M, g, margin);
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
  int tiles = 0;
  hipError_t e = head_launch(dtype, true, W, x, xlo, M, V, H, k, part, nullptr, &tiles, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_combine, dim3(M), dim3(256), 0, stream, part, tiles, M, k, ids, logp);
  return hipGetLastError();
}

hipError_t launch_pack_frag(const void* src, void* dst, int64_t n_blocks, int K, hipStream_t st) {
  if (n_blocks <= 0) return hipSuccess;
  if (K <= 0 || K % 32) return hipErrorInvalidValue;
  const int64_t pieces = n_blocks * (K / 32) * 64;
  const int64_t want = (pieces + 255) / 256;
  const int grid = (int)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(pack_frag_kernel, dim3(grid), dim3(256), 0, st, (const bf16_t*)src, (bf16_t*)dst,
                     pieces, K);
  return hipGetLastError();
}
