// Attention over a paged KV cache with an ancestry bitmask, plus the small
// per-row kernels around it (embedding, RMSNorm, RoPE + KV append, draft
// input assembly, row gathers, KV compaction).
//
// bf16 attention (head_dim 128) has three forms, all with the same per-block
// arithmetic: per 32-key block a wave computes S^T = K Q^T and O^T += V^T P^T
// on 16x16x32 bf16 MFMA; keys are read in an order that makes each lane's 8
// scores exactly the P^T operand of the PV product, so P never leaves
// registers. Q, K, V and P are carried as bf16 hi + lo parts (three
// products; lo*lo dropped), which keeps ~16 mantissa bits. A chunk's K (hi
// and lo planes, XOR-swizzled rows) and V^T (hi and lo) are staged in LDS
// once and shared by every query row of the KV head that reads it.
//  - attn_bf16_kernel: one workgroup of four waves per (64-key chunk, KV
//    head, group of (query head, 16-row block) pairs); every chunk's loads
//    go out at once, each chunk leaves a (max, sum, O) partial per row and
//    head, and attn_combine_kernel merges them. For few rows per sequence
//    (static-tree verify, draft passes), where latency bounds the launch.
//  - attn_split_kernel: one workgroup of eight waves per (KV head, key
//    split, row group) walks the chunks of its split; the query rows of a GQA
//    group are packed densely into 16-row tiles. For many rows per sequence
//    (dynamic-tree verify), where the KV stream bounds the launch.
//  - attn_flash_kernel: causal prefill rows (no tree keys), one pass over
//    the keys per (KV head, row block), no partials.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int CHUNK = 64;     // keys per attention workgroup

// Pages hold a power-of-two number of slots (the launchers check it), so
// slot -> (page, offset) is a shift and a mask, not an integer division.
__device__ __forceinline__ int page_shift(const KVView& v) { return __ffs(v.page) - 1; }

template <typename T>
__device__ __forceinline__ T* kv_ptr(const KVView& v, int slot, int sel, int h) {
  const int sh = page_shift(v);
  const int pg = v.page_table[slot >> sh];
  return (T*)v.base + (int64_t)pg * v.page_elems +
         ((int64_t)(sel * v.n_kv + h) * v.page + (slot & (v.page - 1))) * v.d;
}

// Element i of cache row `slot` in plane `sel` of KV head h. A page holds,
// per plane and KV head, `page` rows of d elements; bf16 caches keep their V
// planes (sel 2 and 3) transposed within the page: d rows of `page` slots,
// so the V^T operand of the attention products is a contiguous run of
// slots in memory.
template <typename T>
__device__ __forceinline__ T* kv_elem(const KVView& v, int slot, int sel, int h, int i) {
  const int sh = page_shift(v);
  T* pl = (T*)v.base + (int64_t)v.page_table[slot >> sh] * v.page_elems +
          (int64_t)(sel * v.n_kv + h) * v.page * v.d;
  if (sizeof(T) == 2 && sel >= 2) return pl + (int64_t)i * v.page + (slot & (v.page - 1));
  return pl + (int64_t)(slot & (v.page - 1)) * v.d + i;
}

// K (which = 0) or V (which = 1) element of one cache row.
template <typename T> struct KVStore;
template <> struct KVStore<float> {
  __device__ static void put(const KVView& v, int slot, int which, int h, int i, float x) {
    *kv_elem<float>(v, slot, which, h, i) = x;
  }
};
template <> struct KVStore<bf16_t> {
  __device__ static void put(const KVView& v, int slot, int which, int h, int i, float x) {
    const bf16_t hi = f32_to_bf16(x);
    *kv_elem<bf16_t>(v, slot, 2 * which, h, i) = hi;
    *kv_elem<bf16_t>(v, slot, 2 * which + 1, h, i) = f32_to_bf16(x - bf16_to_f32(hi));
  }
};

// bf16 key chunks start on page boundaries (pages hold a power-of-two
// number of slots, at least CHUNK), so a chunk lies in one page and its V^T
// rows are aligned runs of CHUNK slots; keys of the first chunk below
// pre_lo are masked like any key a row does not see.
__device__ __forceinline__ int chunk_base(int pre_lo) { return pre_lo & ~(CHUNK - 1); }

// 16-byte piece p of a chunk's V^T (hi and lo planes, 128 dimensions):
// plane p / 1024, dimension (p / 8) % 128, slots 8 (p % 8) .. + 7 of the
// chunk that starts at slot k0 of page pg.
__device__ __forceinline__ const bf16_t* vt_piece(const KVView& kv, int pg, int hk, int k0, int p) {
  constexpr int D = 128;
  const int plane = p / (D * 8), dim = (p / 8) % D, kg = p % 8;
  return (const bf16_t*)kv.base + (int64_t)pg * kv.page_elems +
         ((int64_t)((2 + plane) * kv.n_kv + hk) * D + dim) * kv.page + (k0 & (kv.page - 1)) + 8 * kg;
}
// Stores piece p into the staged V^T (rows padded to `VP` elements). Only
// chunk slots [lo, hi) hold keys (the chunk's keys from pre_lo to the
// launch's last key); the others are written as zeros, so whatever a cache
// holds there never meets a zero probability (0 * NaN would be NaN).
template <int VP>
__device__ __forceinline__ void vt_put(bf16_t (&vt)[2][128][VP], int p, uint4 v, int lo, int hi) {
  const int plane = p / 1024, dim = (p / 8) % 128, kg = p % 8;
  const int a = lo - 8 * kg, b = hi - 8 * kg;   // this piece keeps elements [a, b)
  if (a > 0 || b < 8) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t m0 = (2 * j >= a && 2 * j < b) ? 0xffffu : 0u;
      const uint32_t m1 = (2 * j + 1 >= a && 2 * j + 1 < b) ? 0xffff0000u : 0u;
      w[j] &= m0 | m1;
    }
    v = uint4{w[0], w[1], w[2], w[3]};
  }
  *reinterpret_cast<uint4*>(&vt[plane][dim][8 * kg]) = v;
}

__device__ __forceinline__ bool row_sees(const RowVis& rv, int prehi, uint64_t m0, uint64_t m1,
                                         int key) {
  if (key >= rv.pre_lo && key < prehi) return true;
  const int j = key - rv.tree_base;
  if (j < 0 || j >= rv.n_tree) return false;
  return ((j < 64 ? (m0 >> j) : (m1 >> (j - 64))) & 1ull) != 0;
}

// Sequence b of a multi-sequence launch: row range, per-row inputs, cache
// and key positions (see Lanes).
__device__ __forceinline__ RowVis lane_vis(const RowVis& v, const Lanes& ln, int lane) {
  RowVis r = v;
  const int o = lane_shift(ln, lane);
  r.tree_base += o;
  r.key_end += o;
  r.prehi = (const int32_t*)((const char*)v.prehi + lane * ln.bytes);
  r.mask = (const uint64_t*)((const char*)v.mask + lane * ln.bytes);
  return r;
}
template <typename T>
__device__ __forceinline__ KVView lane_kv(const KVView& v, int lane) {
  KVView r = v;
  r.base = (T*)v.base + lane * v.lane_elems;
  return r;
}

// Max and sum of a value with the lane 16 or 32 away (the score rows of one
// MFMA tile are spread over the four 16-lane rows of the wave). gfx950's
// permlane swaps exchange whole 16-lane rows in registers, where __shfl_xor
// makes a round trip through the LDS crossbar; each lane ends with its own
// value and its partner's, in some order, and max / + are commutative, so
// the results equal the shuffle versions bit for bit.
__device__ __forceinline__ float xrow16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xrow32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xrow16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xrow32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct AttnArgs {
  const bf16_t* q; int64_t qlo;
  KVView kv;
  RowVis vis;
  int M, nq, group;
  int ppg;   // (query head, row block) pairs per workgroup
  float scale;
  float* opart;
  float* mlpart;
  Lanes ln;
  int n_groups;   // pair groups per sequence: blockIdx.z = sequence * n_groups + group
};

// 16-byte column c of a staged K row of key index `key`: XOR-swizzled so the
// 16 keys read by one MFMA operand load fall in distinct LDS banks.
__device__ __forceinline__ int k_swz(int key) { return (key & 3) | ((key >> 1) & 12); }

__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a) {
  constexpr int D = 128, CK = CHUNK, VP = CK + 8;   // V^T row pitch (elements)
  __shared__ uint4 ks[2][CK][16];                  // K hi/lo: [key][16-byte column ^ swz]
  __shared__ __attribute__((aligned(16))) bf16_t vt[2][D][VP];   // V^T hi/lo
  const int chunk = blockIdx.x, hk = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, g = lane >> 4;
  // this workgroup's sequence: its rows r0 .. r0 + Ml - 1 of the launch's Mt
  const int seq = blockIdx.z / a.n_groups, grp = blockIdx.z - seq * a.n_groups;
  const int Mt = a.M, Ml = a.ln.n > 1 ? a.ln.rows : a.M, r0 = seq * Ml;
  const RowVis vis = lane_vis(a.vis, a.ln, seq);
  const KVView kv = lane_kv<bf16_t>(a.kv, seq);
  const int k0 = chunk_base(vis.pre_lo) + chunk * CK;
  if (k0 >= vis.key_end) return;   // a shorter sequence: uniform over the workgroup
  const int k1 = min(vis.key_end, k0 + CK);

  // ---- stage the chunk (keys past k1 repeat the last key; they are masked).
  // Every load of this thread is issued before the first LDS store, so the
  // workgroup waits for one memory latency instead of one per piece.
  static_assert(2 * CK * 16 == 8 * 256 && 2 * (CK / 2) * 16 == 4 * 256, "staging assumes 256 threads");
  // The chunk lies in one KV page: its page-table entry is read once, up
  // front, so no KV address waits on a per-element table load.
  const int pgsz = kv.page, pg = kv.page_table[k0 >> page_shift(kv)];
  auto kvp = [&](int key, int plane) {
    return (const bf16_t*)kv.base + (int64_t)pg * kv.page_elems +
           ((int64_t)(plane * kv.n_kv + hk) * pgsz + (key & (pgsz - 1))) * D;
  };
  // (query head, row block) pairs; fewer pairs than waves: split keys
  // pairs of this workgroup: group blockIdx.z of a.ppg (query head, row
  // block) pairs; a GQA head with many pairs and few chunks spreads its pairs
  // over several workgroups
  const int nrb = (Ml + 15) / 16, pbase = grp * a.ppg;
  const int P = min(a.ppg, a.group * nrb - pbase);
  int kw = 1;
  while (P * kw * 2 <= 4 && kw * 2 <= CK / 32) kw *= 2;
  const int kg = wave / P;                 // key group of this wave (kw > 1)
  const int nblk = CK / 32 / kw;           // 32-key blocks per key group
  const int pr0 = kw > 1 ? wave % P : wave, pstep = kw > 1 ? P : 4;
  const bool active = pr0 < P && kg < kw;
  // the query fragments and ancestry masks of this wave's next pair; the first
  // pair's are requested here, before the chunk, so both latencies overlap
  uint4 qf[4], ql[4];
  int prehi = 0;
  uint64_t mk0 = 0, mk1 = 0;
  auto load_pair = [&](int pr) {
    const int h = hk * a.group + (pbase + pr) / nrb, rb = (pbase + pr) % nrb;
    const int rowc = min(rb * 16 + lr, Ml - 1);
    const bf16_t* qp = a.q + ((int64_t)(r0 + rowc) * a.nq + h) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qf[s] = ld16(qp + 32 * s);
      ql[s] = ld16(qp + a.qlo + 32 * s);
    }
    prehi = vis.prehi[rowc];
    mk0 = vis.mask[2 * rowc];
    mk1 = vis.mask[2 * rowc + 1];
  };
  if (active) load_pair(pr0);
  uint4 kr[8], vr[8];
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int i = tid + 256 * it;
    const int plane = i / (CK * 16), key = (i / 16) % CK, c = i % 16;
    kr[it] = ld16(kvp(min(k0 + key, k1 - 1), plane) + 8 * c);
  }
#pragma unroll
  for (int it = 0; it < 8; ++it) vr[it] = ld16(vt_piece(kv, pg, hk, k0, tid + 256 * it));
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int i = tid + 256 * it;
    const int plane = i / (CK * 16), key = (i / 16) % CK, c = i % 16;
    ks[plane][key][c ^ k_swz(key)] = kr[it];
  }
#pragma unroll
  for (int it = 0; it < 8; ++it) vt_put(vt, tid + 256 * it, vr[it], vis.pre_lo - k0, k1 - k0);
  __syncthreads();

  float m_keep = -INFINITY, l_keep = 0.f;
  f32x4 o[8];
  int pair_keep = -1;
  for (int pr = pr0; active && pr < P; pr += pstep) {
    const int h = hk * a.group + (pbase + pr) / nrb, rb = (pbase + pr) % nrb;
    const int row = rb * 16 + lr;
    float m_run = -INFINITY, l_run = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int pmin = wave_min_i(prehi);   // smallest visible-prefix end of the pair's rows
    for (int bi = 0; bi < nblk; ++bi) {
      const int kb0 = (kg * nblk + bi) * 32;   // block start within the chunk
      f32x4 sc[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int key = kb0 + 8 * (lr >> 2) + 4 * hh + (lr & 3);
        const int sw = k_swz(key);
        sc[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {  // (K_hi + K_lo)(Q_hi + Q_lo), lo*lo dropped
          const uint4 kf = ks[0][key][(4 * s + g) ^ sw];
          const uint4 kl = ks[1][key][(4 * s + g) ^ sw];
          Mma<bf16_t>::mma(kf, qf[s], sc[hh]);
          Mma<bf16_t>::mma(kf, ql[s], sc[hh]);
          Mma<bf16_t>::mma(kl, qf[s], sc[hh]);
        }
      }
      float p[8];
      float bm = -INFINITY;
      if (k0 + kb0 >= vis.pre_lo && k0 + kb0 + 32 <= min(pmin, k1)) {
        // every key of the block is in every row's visible prefix
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p[i] = sc[i >> 2][i & 3] * a.scale;
          bm = fmaxf(bm, p[i]);
        }
      } else {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = k0 + kb0 + 8 * g + 4 * hh + e;
            const bool ok = key < k1 && row_sees(vis, prehi, mk0, mk1, key);
            p[4 * hh + e] = ok ? sc[hh][e] * a.scale : -INFINITY;
            bm = fmaxf(bm, p[4 * hh + e]);
          }
      }
      bm = xrow16_max(bm);
      bm = xrow32_max(bm);
      const float m_new = fmaxf(m_run, bm);
      float alpha = 1.f, ps = 0.f;
      if (m_new != -INFINITY) {
        alpha = exp2f(m_run - m_new);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p[i] = exp2f(p[i] - m_new);
          ps += p[i];
        }
        m_run = m_new;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = 0.f;
      }
      ps = xrow16_sum(ps);
      ps = xrow32_sum(ps);
      l_run = l_run * alpha + ps;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] *= alpha;
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ph[j] = pack_bf16x2(p[2 * j], p[2 * j + 1]);
        pl[j] = pack_bf16x2(p[2 * j] - bf16_lo_f(ph[j]), p[2 * j + 1] - bf16_hi_f(ph[j]));
      }
      const uint4 phi = uint4{ph[0], ph[1], ph[2], ph[3]};
      const uint4 plo = uint4{pl[0], pl[1], pl[2], pl[3]};
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {  // (V_hi + V_lo)(P_hi + P_lo), lo*lo dropped
        const uint4 va = *reinterpret_cast<const uint4*>(&vt[0][16 * dt + lr][kb0 + 8 * g]);
        const uint4 val = *reinterpret_cast<const uint4*>(&vt[1][16 * dt + lr][kb0 + 8 * g]);
        Mma<bf16_t>::mma(va, phi, o[dt]);
        Mma<bf16_t>::mma(va, plo, o[dt]);
        Mma<bf16_t>::mma(val, phi, o[dt]);
      }
    }
    if (kw == 1) {
      if (row < Ml) {
        float* op = a.opart + (((int64_t)chunk * Mt + r0 + row) * a.nq + h) * D;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int e = 0; e < 4; ++e) op[16 * dt + 4 * g + e] = o[dt][e];
        if (g == 0) {
          float* ml = a.mlpart + (((int64_t)chunk * Mt + r0 + row) * a.nq + h) * 2;
          ml[0] = m_run;
          ml[1] = l_run;
        }
      }
    } else {
      m_keep = m_run;
      l_keep = l_run;
      pair_keep = pr;
    }
    if (pr + pstep < P) load_pair(pr + pstep);
  }
  if (kw == 1) return;   // uniform across the workgroup

  // ---- merge the key groups of each pair through LDS (reuses the K area)
  __syncthreads();
  float* mo = reinterpret_cast<float*>(&ks[0][0][0]);     // [wave][16 rows][128]
  float* mm = reinterpret_cast<float*>(&vt[0][0][0]);     // [wave][16 rows][2]
  static_assert(4 * 16 * D * 4 <= (int)sizeof(ks), "merge buffer must fit");
  if (pair_keep >= 0) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) mo[(wave * 16 + lr) * D + 16 * dt + 4 * g + e] = o[dt][e];
    if (g == 0) {
      mm[(wave * 16 + lr) * 2] = m_keep;
      mm[(wave * 16 + lr) * 2 + 1] = l_keep;
    }
  }
  __syncthreads();
  if (pair_keep >= 0 && kg == 0) {
    const int h = hk * a.group + (pbase + pair_keep) / nrb, rb = (pbase + pair_keep) % nrb;
    const int row = rb * 16 + lr;
    float gm = -INFINITY;
    for (int k = 0; k < kw; ++k) gm = fmaxf(gm, mm[((wave + k * P) * 16 + lr) * 2]);
    float lsum = 0.f, wk[4];
    for (int k = 0; k < kw; ++k) {
      const float mk = mm[((wave + k * P) * 16 + lr) * 2];
      wk[k] = mk == -INFINITY ? 0.f : exp2f(mk - gm);
      lsum += wk[k] * mm[((wave + k * P) * 16 + lr) * 2 + 1];
    }
    if (row < Ml) {
      float* op = a.opart + (((int64_t)chunk * Mt + r0 + row) * a.nq + h) * D;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int dd = 16 * dt + 4 * g + e;
          float acc = 0.f;
          for (int k = 0; k < kw; ++k) acc += wk[k] * mo[((wave + k * P) * 16 + lr) * D + dd];
          op[dd] = acc;
        }
      if (g == 0) {
        float* ml = a.mlpart + (((int64_t)chunk * Mt + r0 + row) * a.nq + h) * 2;
        ml[0] = gm;
        ml[1] = lsum;
      }
    }
  }
}

// Causal attention over many rows with no tree keys (prefill chunks and the
// draft catch-up over them), in flash form: one workgroup per
// (KV head, block of 16 RB query rows) walks the key chunks from the visible
// prefix start to its rows' last visible key. Each chunk's K and V^T (hi
// and lo) are staged in LDS in attn_bf16_kernel's layout while the next
// chunk's loads are in flight; every wave keeps the running max, sum and O
// of its (query head, 16-row block) pairs over its half of each chunk's keys
// in registers, with the same MFMA products and log2-unit online softmax as
// attn_bf16_kernel; the two halves merge in LDS and the normalized rows are
// written once: no per-chunk partials in memory and no merge kernel. A row sees
// key k iff pre_lo <= k < prehi[row]. Workgroups are dispatched to the 8
// XCDs round-robin by index, so the index is mapped to put every row block
// of a KV head on one XCD: they walk the same keys at about the same time
// and read them from that XCD's L2 instead of each from memory.
struct FlashArgs {
  const bf16_t* q; int64_t qlo;
  KVView kv;
  RowVis vis;
  int M, nq, group;
  int rb;       // 16-row blocks per workgroup
  float scale;  // log2 units
  bf16_t* out; int64_t olo;
};

template <int PW>   // (query head, row block) pairs per wave
__global__ __launch_bounds__(512) void attn_flash_kernel(FlashArgs a) {
  // Eight waves: wave w takes pair slot w % 4 and the key half w / 4 of every
  // chunk (32 of its 64 keys), so two waves share each SIMD; the halves keep
  // their own running (max, sum, O) and are merged through LDS at the end.
  constexpr int D = 128, CK = CHUNK, VP = CK + 8, NT = 512;
  __shared__ uint4 ks[2][CK][16];
  __shared__ __attribute__((aligned(16))) bf16_t vt[2][D][VP];
  __shared__ int kend_sh;
  const RowVis& vis = a.vis;
  const KVView& kv = a.kv;
  int hk, rbi;
  if ((kv.n_kv & 7) == 0) {
    const int hpx = kv.n_kv >> 3, j = blockIdx.x >> 3;
    hk = (blockIdx.x & 7) * hpx + j % hpx;
    rbi = j / hpx;
  } else {
    hk = blockIdx.x % kv.n_kv;
    rbi = blockIdx.x / kv.n_kv;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = wave & 3, kh = wave >> 2;
  const int lr = lane & 15, g = lane >> 4;
  const int row_lo = rbi * 16 * a.rb;
  const int nrows = min(16 * a.rb, a.M - row_lo);
  // the block's last visible key: the largest prehi over its rows
  if (tid < 64) {
    int e = tid < nrows ? vis.prehi[row_lo + tid] : 0;
    e = max(e, __shfl_xor(e, 1));
    e = max(e, __shfl_xor(e, 2));
    e = max(e, __shfl_xor(e, 4));
    e = max(e, __shfl_xor(e, 8));
    e = max(e, __shfl_xor(e, 16));
    e = max(e, __shfl_xor(e, 32));
    if (tid == 0) kend_sh = min(e, vis.key_end);
  }
  __syncthreads();
  const int kend = kend_sh;
  const int cb = chunk_base(vis.pre_lo);
  const int nch = kend > vis.pre_lo ? (kend - cb + CK - 1) / CK : 0;

  // this wave's pairs: p = slot + 4 i, head j = p / rb, row block p % rb
  const int npairs = a.group * a.rb;
  uint4 qf[PW][4], ql[PW][4];
  int prehi[PW], pmin[PW];
  float m_run[PW], l_run[PW];
  f32x4 o[PW][8];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int p = min(slot + 4 * i, npairs - 1);
    const int h = hk * a.group + p / a.rb;
    const int rowc = min(row_lo + 16 * (p % a.rb) + lr, a.M - 1);
    const bf16_t* qp = a.q + ((int64_t)rowc * a.nq + h) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qf[i][s] = ld16(qp + 32 * s);
      ql[i][s] = ld16(qp + a.qlo + 32 * s);
    }
    prehi[i] = vis.prehi[rowc];
    pmin[i] = wave_min_i(prehi[i]);
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int pgsz = kv.page, psh = page_shift(kv);
  uint4 kr[4], vr[4];
  int v_lo = 0, v_hi = 0;   // the staged chunk's key slots
  // loads of chunk c into registers (keys past the chunk's end repeat its
  // last key; they are masked); the chunk lies in one KV page
  auto load_chunk = [&](int c) {
    const int k0 = cb + c * CK, k1 = min(kend, k0 + CK);
    const int pg = kv.page_table[k0 >> psh];
    auto kvp = [&](int key, int plane) {
      return (const bf16_t*)kv.base + (int64_t)pg * kv.page_elems +
             ((int64_t)(plane * kv.n_kv + hk) * pgsz + (key & (pgsz - 1))) * D;
    };
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int i = tid + NT * it;
      const int plane = i / (CK * 16), key = (i / 16) % CK, c16 = i % 16;
      kr[it] = ld16(kvp(min(k0 + key, k1 - 1), plane) + 8 * c16);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) vr[it] = ld16(vt_piece(kv, pg, hk, k0, tid + NT * it));
    v_lo = vis.pre_lo - k0;
    v_hi = k1 - k0;
  };
  auto store_chunk = [&]() {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int i = tid + NT * it;
      const int plane = i / (CK * 16), key = (i / 16) % CK, c16 = i % 16;
      ks[plane][key][c16 ^ k_swz(key)] = kr[it];
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) vt_put(vt, tid + NT * it, vr[it], v_lo, v_hi);
  };

  if (nch > 0) {
    load_chunk(0);
    store_chunk();
  }
  __syncthreads();
  const int kb0 = 32 * kh;   // this wave's 32 keys of every chunk
  for (int c = 0; c < nch; ++c) {
    const int k0 = cb + c * CK, k1 = min(kend, k0 + CK);
    if (c + 1 < nch) load_chunk(c + 1);
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      if (slot + 4 * i >= npairs) continue;   // uniform over the wave
      // the two 16-key halves accumulate in turn (two independent MFMA
      // chains; each half's order is attn_bf16_kernel's)
      f32x4 sc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < 4; ++s) {  // (K_hi + K_lo)(Q_hi + Q_lo), lo*lo dropped
        uint4 kf[2], kl[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int key = kb0 + 8 * (lr >> 2) + 4 * hh + (lr & 3);
          kf[hh] = ks[0][key][(4 * s + g) ^ k_swz(key)];
          kl[hh] = ks[1][key][(4 * s + g) ^ k_swz(key)];
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) Mma<bf16_t>::mma(kf[hh], qf[i][s], sc[hh]);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) Mma<bf16_t>::mma(kf[hh], ql[i][s], sc[hh]);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) Mma<bf16_t>::mma(kl[hh], qf[i][s], sc[hh]);
      }
      float p[8];
      float bm = -INFINITY;
      if (k0 + kb0 >= vis.pre_lo && k0 + kb0 + 32 <= min(pmin[i], k1)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = sc[e >> 2][e & 3] * a.scale;
          bm = fmaxf(bm, p[e]);
        }
      } else {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = k0 + kb0 + 8 * g + 4 * hh + e;
            const bool ok = key >= vis.pre_lo && key < k1 && key < prehi[i];
            p[4 * hh + e] = ok ? sc[hh][e] * a.scale : -INFINITY;
            bm = fmaxf(bm, p[4 * hh + e]);
          }
      }
      bm = xrow16_max(bm);
      bm = xrow32_max(bm);
      const float m_new = fmaxf(m_run[i], bm);
      float alpha = 1.f, ps = 0.f;
      if (m_new != -INFINITY) {
        alpha = exp2f(m_run[i] - m_new);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = exp2f(p[e] - m_new);
          ps += p[e];
        }
        m_run[i] = m_new;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = 0.f;
      }
      ps = xrow16_sum(ps);
      ps = xrow32_sum(ps);
      l_run[i] = l_run[i] * alpha + ps;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[i][dt] *= alpha;
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ph[j] = pack_bf16x2(p[2 * j], p[2 * j + 1]);
        pl[j] = pack_bf16x2(p[2 * j] - bf16_lo_f(ph[j]), p[2 * j + 1] - bf16_hi_f(ph[j]));
      }
      const uint4 phi = uint4{ph[0], ph[1], ph[2], ph[3]};
      const uint4 plo = uint4{pl[0], pl[1], pl[2], pl[3]};
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {  // (V_hi + V_lo)(P_hi + P_lo), lo*lo dropped
        const uint4 v0 = *reinterpret_cast<const uint4*>(&vt[0][16 * dt + lr][kb0 + 8 * g]);
        const uint4 v1 = *reinterpret_cast<const uint4*>(&vt[1][16 * dt + lr][kb0 + 8 * g]);
        Mma<bf16_t>::mma(v0, phi, o[i][dt]);
        Mma<bf16_t>::mma(v0, plo, o[i][dt]);
        Mma<bf16_t>::mma(v1, phi, o[i][dt]);
      }
    }
    __syncthreads();   // every wave is done with this chunk's LDS
    if (c + 1 < nch) {
      store_chunk();
      __syncthreads();
    }
  }
  // merge the two key halves of each pair (the K area holds the second
  // half's O, the V area its max and sum), then write the normalized rows
  float* mo = reinterpret_cast<float*>(&ks[0][0][0]);   // [slot][16 rows][128]
  float* mm = reinterpret_cast<float*>(&vt[0][0][0]);   // [slot][16 rows][2]
  static_assert(4 * 16 * D * 4 <= (int)sizeof(ks), "merge buffer must fit");
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int p = slot + 4 * i;
    const bool has = p < npairs;   // uniform over the wave
    if (kh == 1 && has) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) mo[(slot * 16 + lr) * D + 16 * dt + 4 * g + e] = o[i][dt][e];
      if (g == 0) {
        mm[(slot * 16 + lr) * 2] = m_run[i];
        mm[(slot * 16 + lr) * 2 + 1] = l_run[i];
      }
    }
    __syncthreads();
    if (kh == 0 && has) {
      const int h = hk * a.group + p / a.rb;
      const int row = row_lo + 16 * (p % a.rb) + lr;
      const float m1 = mm[(slot * 16 + lr) * 2], l1 = mm[(slot * 16 + lr) * 2 + 1];
      const float mx = fmaxf(m_run[i], m1);
      const float w0 = m_run[i] == -INFINITY ? 0.f : exp2f(m_run[i] - mx);
      const float w1 = m1 == -INFINITY ? 0.f : exp2f(m1 - mx);
      const float l = w0 * l_run[i] + w1 * l1;
      const float inv = l > 0.f ? 1.f / l : 0.f;
      if (row < a.M) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int dd = 16 * dt + 4 * g + e;
            const float v = (w0 * o[i][dt][e] + w1 * mo[(slot * 16 + lr) * D + dd]) * inv;
            Opnd<bf16_t>::store(a.out, a.olo, ((int64_t)row * a.nq + h) * D + dd, v);
          }
      }
    }
    __syncthreads();
  }
}

// Tree-masked attention for verify and draft rows (and short catch-ups), in
// split form: one workgroup of eight waves per (KV head, key split, row
// group) walks the 64-key chunks of its split with the flash kernel's chunk
// pipeline (K and V^T hi/lo staged in LDS, the next chunk's loads in flight
// meanwhile) and the same MFMA products and log2-unit online softmax. The
// query rows of one KV head -- its `group` query heads times the sequence's
// rows -- are packed densely into 16-row tiles (query row qr = j * rows + r
// for query head j of the group and row r), so a GQA group's rows fill the
// MFMA tiles instead of each head padding its rows to 16. A row group holds
// up to 4 * PW tiles; wave w takes tile slot w % 4 (PW tiles each) and the
// key half w / 4 of every chunk, and the halves merge through LDS. When no
// sequence of the launch splits its keys the normalized rows are written as
// the next projection's operand; otherwise each split leaves one (max, sum,
// O) partial per row and query head in attn_bf16_kernel's chunk layout for
// attn_combine_kernel. The split
// count depends only on the sequence's own key count, tiles and KV heads, so
// a sequence gets the same bits alone or in a batch. Workgroup indices are
// mapped so that the row groups of one (KV head, split) share an XCD and
// read its keys from that XCD's L2.
struct SplitArgs {
  const bf16_t* q; int64_t qlo;
  KVView kv;
  RowVis vis;
  Lanes ln;
  int M, nq, group;
  int ntile;                  // 16-row tiles per (sequence, KV head)
  int tpg;                    // tiles per row group
  int rg;                     // row groups per (sequence, KV head)
  int smax;                   // splits in the grid (the largest over sequences)
  int splits[MAX_LANES];      // sequence b's split count
  float scale;                // log2 units
  bf16_t* out; int64_t olo;   // one split: the normalized output operand
  float* opart; float* mlpart;  // several: partials [split][M][nq][D], [split][M][nq][2]
};

// Most key chunks one workgroup of attn_split_kernel walks (its page list
// sits in LDS); the launcher raises the split count to keep within it.
constexpr int ATTN_SPLIT_CHUNKS = 1024;

template <int PW>
__global__ __launch_bounds__(512) void attn_split_kernel(SplitArgs a) {
  constexpr int D = 128, CK = CHUNK, NT = 512;
  // two chunk buffers, filled straight from the cache (see copy_chunk): K
  // hi/lo as [key][16-byte column ^ k_swz(key)] and V^T hi/lo as
  // [dimension][8-slot group ^ (dimension mod 8)]; the XOR swizzles keep
  // the operand reads free of bank conflicts
  __shared__ uint4 ks[2][2][CK][16];
  __shared__ uint4 vs[2][2][D][8];
  __shared__ int pgs[ATTN_SPLIT_CHUNKS];   // page of each of this workgroup's chunks
  const int seq = blockIdx.z;
  int S = 1;
#pragma unroll
  for (int i = 0; i < MAX_LANES; ++i) S = i == seq ? a.splits[i] : S;
  // workgroup -> (unit = KV head * smax + split, row group)
  const int U = a.kv.n_kv * a.smax;
  int unit, rgi;
  if ((U & 7) == 0) {
    const int w = blockIdx.x, j = w >> 3;
    unit = (w & 7) + 8 * (j / a.rg);
    rgi = j % a.rg;
  } else {
    unit = blockIdx.x / a.rg;
    rgi = blockIdx.x % a.rg;
  }
  const int hk = unit / a.smax, sp = unit % a.smax;
  if (sp >= S) return;   // a sequence with fewer splits: uniform over the workgroup
  const RowVis vis = lane_vis(a.vis, a.ln, seq);
  const KVView kv = lane_kv<bf16_t>(a.kv, seq);
  const int Ml = a.ln.n > 1 ? a.ln.rows : a.M, r0 = seq * Ml;
  const int nqr = a.group * Ml;   // query rows of this KV head
  const int cb = chunk_base(vis.pre_lo);
  const int nch = (vis.key_end - cb + CK - 1) / CK;
  const int c_lo = (int)((int64_t)sp * nch / S), c_hi = (int)((int64_t)(sp + 1) * nch / S);
  const int kend = vis.key_end;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = wave & 3, kh = wave >> 2;
  const int lr = lane & 15, g = lane >> 4;
  const int t0 = rgi * a.tpg, ntg = min(a.tpg, a.ntile - t0);   // this group's tiles

  const int pgsz = kv.page, psh = page_shift(kv);
  for (int i = tid; i < c_hi - c_lo; i += NT) pgs[i] = kv.page_table[(cb + (c_lo + i) * CK) >> psh];
  uint4 qf[PW][4], ql[PW][4];
  int prehi[PW], pmin[PW], rowr[PW], headj[PW];
  bool valid[PW];
  uint64_t mk0[PW], mk1[PW];
  float m_run[PW], l_run[PW];
  f32x4 o[PW][8];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int t = t0 + min(slot + 4 * i, max(ntg - 1, 0));
    const int qr = 16 * t + lr;
    valid[i] = slot + 4 * i < ntg && qr < nqr;
    const int qc = min(qr, nqr - 1);
    headj[i] = qc / Ml;
    rowr[i] = qc - headj[i] * Ml;
    const int h = hk * a.group + headj[i];
    const bf16_t* qp = a.q + ((int64_t)(r0 + rowr[i]) * a.nq + h) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qf[i][s] = ld16(qp + 32 * s);
      ql[i][s] = ld16(qp + a.qlo + 32 * s);
    }
    prehi[i] = vis.prehi[rowr[i]];
    mk0[i] = vis.n_tree > 0 ? vis.mask[2 * rowr[i]] : 0ull;
    mk1[i] = vis.n_tree > 0 ? vis.mask[2 * rowr[i] + 1] : 0ull;
    pmin[i] = wave_min_i(prehi[i]);
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Chunks are copied from the cache straight into LDS: wave w issues 1 KB
  // blocks 8w .. 8w + 7 of the chunk's 64 (0-31: the K planes, four keys a
  // block; 32-63: the V^T planes, eight dimensions a block), each lane
  // reading the 16 bytes that belong at lane * 16 of its block under the
  // swizzles. The copies are asm (global_load_lds_dwordx4 writes no
  // register) and are waited for with explicit vmcnt counts, so one chunk
  // is in flight while the previous one is multiplied: the compiler's own
  // wait tracking cannot see them, and every load it tracks (the query rows,
  // the masks, the page entries) is complete before the first copy.
  auto lds_u32 = [](const void* p) {
    return (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(uintptr_t)(__attribute__((address_space(3))) const void*)p);
  };
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto copy_chunk = [&](int c, int b) {
    const int ko = (cb + c * CK) & (pgsz - 1);
    const bf16_t* pb = (const bf16_t*)kv.base + (int64_t)pgs[c - c_lo] * kv.page_elems;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = wave_u * 8 + j;
      uint32_t lds;
      const bf16_t* src;
      if (q < 32) {
        const int plane = q >> 4, key = 4 * (q & 15) + (lane >> 4);
        lds = lds_u32(&ks[b][plane][4 * (q & 15)][0]);
        src = pb + ((int64_t)(plane * kv.n_kv + hk) * pgsz + ko + key) * D + 8 * ((lane & 15) ^ k_swz(key));
      } else {
        const int qv = q - 32, plane = qv >> 4, dim = 8 * (qv & 15) + (lane >> 3);
        lds = lds_u32(&vs[b][plane][8 * (qv & 15)][0]);
        src = pb + ((int64_t)((2 + plane) * kv.n_kv + hk) * D + dim) * pgsz + ko + 8 * ((lane & 7) ^ (dim & 7));
      }
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src)
                   : "memory", "m0");
    }
  };
  // V^T slots of chunk c outside [pre_lo, kend) (the first chunk's below
  // pre_lo, the last chunk's past the last key) are set to zero once the
  // copy has landed: a cache may hold anything there, and 0 * NaN is NaN
  auto clear_vt = [&](int c, int b) {
    const int k0 = cb + c * CK;
    const int lo = vis.pre_lo - k0, hi = min(kend, k0 + CK) - k0;
    if (lo <= 0 && hi >= CK) return;   // uniform
    if (tid < 2 * D) {
      const int plane = tid / D, dim = tid % D;
#pragma unroll
      for (int col = 0; col < 8; ++col) {
        const int kg = col ^ (dim & 7);
        const int x = lo - 8 * kg, y = hi - 8 * kg;   // keep elements [x, y)
        if (x <= 0 && y >= 8) continue;
        uint4 v = vs[b][plane][dim][col];
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t m0 = (2 * e >= x && 2 * e < y) ? 0xffffu : 0u;
          const uint32_t m1 = (2 * e + 1 >= x && 2 * e + 1 < y) ? 0xffff0000u : 0u;
          w[e] &= m0 | m1;
        }
        vs[b][plane][dim][col] = uint4{w[0], w[1], w[2], w[3]};
      }
    }
    lds_barrier();
  };
  __syncthreads();                     // pgs
  __builtin_amdgcn_s_waitcnt(0xF70);   // vmcnt(0): every tracked load is done
  if (c_lo < c_hi) copy_chunk(c_lo, 0);
  const int kb0 = 32 * kh;   // this wave's 32 keys of every chunk
  // per chunk: S^T = K Q^T for the wave's tiles (each K fragment read from
  // LDS once for all of them), masking and the online softmax, then
  // O^T += V^T P^T (each V^T fragment read once)
  auto compute = [&](int c, int b) {
    const int k0 = cb + c * CK, k1 = min(kend, k0 + CK);
    f32x4 sc[PW][2];
#pragma unroll
    for (int i = 0; i < PW; ++i) sc[i][0] = sc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {  // (K_hi + K_lo)(Q_hi + Q_lo), lo*lo dropped
      uint4 kf[2], kl[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int key = kb0 + 8 * (lr >> 2) + 4 * hh + (lr & 3);
        kf[hh] = ks[b][0][key][(4 * s + g) ^ k_swz(key)];
        kl[hh] = ks[b][1][key][(4 * s + g) ^ k_swz(key)];
      }
#pragma unroll
      for (int i = 0; i < PW; ++i) {
        if (slot + 4 * i >= ntg) continue;   // uniform over the wave
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) Mma<bf16_t>::mma(kf[hh], qf[i][s], sc[i][hh]);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) Mma<bf16_t>::mma(kf[hh], ql[i][s], sc[i][hh]);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) Mma<bf16_t>::mma(kl[hh], qf[i][s], sc[i][hh]);
      }
    }
    uint4 phi[PW], plo[PW];
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      phi[i] = plo[i] = uint4{0u, 0u, 0u, 0u};
      if (slot + 4 * i >= ntg) continue;
      float p[8];
      float bm = -INFINITY;
      if (k0 + kb0 >= vis.pre_lo && k0 + kb0 + 32 <= min(pmin[i], k1)) {
        // every key of the block is in every row's visible prefix
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = sc[i][e >> 2][e & 3] * a.scale;
          bm = fmaxf(bm, p[e]);
        }
      } else {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = k0 + kb0 + 8 * g + 4 * hh + e;
            const bool ok = key < k1 && row_sees(vis, prehi[i], mk0[i], mk1[i], key);
            p[4 * hh + e] = ok ? sc[i][hh][e] * a.scale : -INFINITY;
            bm = fmaxf(bm, p[4 * hh + e]);
          }
      }
      bm = xrow16_max(bm);
      bm = xrow32_max(bm);
      const float m_new = fmaxf(m_run[i], bm);
      float alpha = 1.f, ps = 0.f;
      if (m_new != -INFINITY) {
        alpha = exp2f(m_run[i] - m_new);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = exp2f(p[e] - m_new);
          ps += p[e];
        }
        m_run[i] = m_new;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = 0.f;
      }
      ps = xrow16_sum(ps);
      ps = xrow32_sum(ps);
      l_run[i] = l_run[i] * alpha + ps;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[i][dt] *= alpha;
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ph[j] = pack_bf16x2(p[2 * j], p[2 * j + 1]);
        pl[j] = pack_bf16x2(p[2 * j] - bf16_lo_f(ph[j]), p[2 * j + 1] - bf16_hi_f(ph[j]));
      }
      phi[i] = uint4{ph[0], ph[1], ph[2], ph[3]};
      plo[i] = uint4{pl[0], pl[1], pl[2], pl[3]};
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {  // (V_hi + V_lo)(P_hi + P_lo), lo*lo dropped
      const int vr = 16 * dt + lr, vc = ((kb0 >> 3) + g) ^ (vr & 7);
      const uint4 v0 = vs[b][0][vr][vc];
      const uint4 v1 = vs[b][1][vr][vc];
#pragma unroll
      for (int i = 0; i < PW; ++i) {
        if (slot + 4 * i >= ntg) continue;
        Mma<bf16_t>::mma(v0, phi[i], o[i][dt]);
        Mma<bf16_t>::mma(v0, plo[i], o[i][dt]);
        Mma<bf16_t>::mma(v1, phi[i], o[i][dt]);
      }
    }
  };

  // chunk c + 1 is copied while chunk c is multiplied; each wave waits for
  // its own copies of chunk c (eight blocks younger than them may be in
  // flight), and the barrier makes every wave's copies visible
  for (int c = c_lo; c < c_hi; ++c) {
    const int b = (c - c_lo) & 1;
    if (c + 1 < c_hi) {
      copy_chunk(c + 1, b ^ 1);
      asm volatile("s_waitcnt vmcnt(8)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    clear_vt(c, b);
    compute(c, b);
    lds_barrier();   // every wave is done with buffer b before chunk c + 2 overwrites it
  }
  // merge the two key halves of each tile (the K area holds the second
  // half's O, the V area its max and sum), then write the rows
  float* mo = reinterpret_cast<float*>(&ks[0][0][0][0]);   // [slot][16 rows][128]
  float* mm = reinterpret_cast<float*>(&vs[0][0][0][0]);   // [slot][16 rows][2]
  static_assert(4 * 16 * D * 4 <= (int)sizeof(ks), "merge buffer must fit");
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const bool has = slot + 4 * i < ntg;   // uniform over the wave
    if (kh == 1 && has) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) mo[(slot * 16 + lr) * D + 16 * dt + 4 * g + e] = o[i][dt][e];
      if (g == 0) {
        mm[(slot * 16 + lr) * 2] = m_run[i];
        mm[(slot * 16 + lr) * 2 + 1] = l_run[i];
      }
    }
    __syncthreads();
    if (kh == 0 && has) {
      const int h = hk * a.group + headj[i];
      const int row = r0 + rowr[i];
      const float m1 = mm[(slot * 16 + lr) * 2], l1 = mm[(slot * 16 + lr) * 2 + 1];
      const float mx = fmaxf(m_run[i], m1);
      const float w0 = m_run[i] == -INFINITY ? 0.f : exp2f(m_run[i] - mx);
      const float w1 = m1 == -INFINITY ? 0.f : exp2f(m1 - mx);
      const float l = w0 * l_run[i] + w1 * l1;
      if (valid[i]) {
        if (a.smax == 1) {
          const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int dd = 16 * dt + 4 * g + e;
              const float v = (w0 * o[i][dt][e] + w1 * mo[(slot * 16 + lr) * D + dd]) * inv;
              Opnd<bf16_t>::store(a.out, a.olo, ((int64_t)row * a.nq + h) * D + dd, v);
            }
        } else {
          const int64_t rec = ((int64_t)sp * a.M + row) * a.nq + h;
          float* op = a.opart + rec * D;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v[e] = w0 * o[i][dt][e] + w1 * mo[(slot * 16 + lr) * D + 16 * dt + 4 * g + e];
            *reinterpret_cast<f32x4*>(op + 16 * dt + 4 * g) = v;
          }
          if (g == 0) {
            a.mlpart[rec * 2] = mx;
            a.mlpart[rec * 2 + 1] = l;
          }
        }
      }
    }
    __syncthreads();
  }
}

constexpr int ATTN_MAX_CHUNKS = 2048;

// Merges the per-chunk (max, sum, O) partials of one (row, head): the chunk
// weights exp(m_c - max) are computed once into LDS, then each thread sums
// its output element over the chunks in chunk order, eight loads in flight.
// Key chunks of each sequence of a launch.
struct LaneChunks {
  int rows;                // rows per sequence (every row is sequence 0's when n == 1)
  int n;
  int chunks[MAX_LANES];
};

template <typename T>
__global__ __launch_bounds__(128) void attn_combine_kernel(const float* opart, const float* mlpart,
                                                           LaneChunks lc, int M, int nq, int d,
                                                           T* out, int64_t lo) {
  __shared__ float sw[ATTN_MAX_CHUNKS];
  __shared__ float red[4];
  const int r = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seq = lc.n > 1 ? r / lc.rows : 0;
  int n_chunks = 0;
#pragma unroll
  for (int i = 0; i < MAX_LANES; ++i) n_chunks = i == seq ? lc.chunks[i] : n_chunks;
  const int64_t cs = (int64_t)M * nq;   // (row, head) records per chunk
  const float* ml0 = mlpart + ((int64_t)r * nq + h) * 2;
  float mx = -INFINITY;
  for (int c = tid; c < n_chunks; c += 128) mx = fmaxf(mx, ml0[c * cs * 2]);
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  const float gm = fmaxf(red[0], red[1]);
  float den = 0.f;
  for (int c = tid; c < n_chunks; c += 128) {
    const float m_c = ml0[c * cs * 2], l_c = ml0[c * cs * 2 + 1];
    const float w = l_c == 0.f ? 0.f : exp2f(m_c - gm);
    sw[c] = w;
    den += w * l_c;
  }
  den = wave_sum(den);
  __syncthreads();   // red[0..1] read above; sw complete below
  if (lane == 0) red[2 + wave] = den;
  __syncthreads();
  den = red[2] + red[3];
  const float* o0 = opart + ((int64_t)r * nq + h) * d;
  for (int j = tid; j < d; j += 128) {
    float num = 0.f;
    int c = 0;
    for (; c + 8 <= n_chunks; c += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = o0[(c + u) * cs * d + j];
#pragma unroll
      for (int u = 0; u < 8; ++u) num += sw[c + u] * v[u];
    }
    for (; c < n_chunks; ++c) num += sw[c] * o0[c * cs * d + j];
    Opnd<T>::store(out, lo, ((int64_t)r * nq + h) * d + j, num / den);
  }
}

// fp32 path: one 64-lane wave per (row, head), keys in order, online softmax.
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* q, KVView kv_all, RowVis vis_all,
                                                      Lanes ln, int M, int nq, int group, int d,
                                                      float scale, float* out) {
  const int r = blockIdx.x, h = blockIdx.y, hk = h / group;
  const int lane = threadIdx.x;
  const int seq = ln.n > 1 ? r / ln.rows : 0, j = ln.n > 1 ? r - seq * ln.rows : r;
  const RowVis vis = lane_vis(vis_all, ln, seq);
  const KVView kv = lane_kv<float>(kv_all, seq);
  const int prehi = vis.prehi[j];
  const uint64_t mk0 = vis.mask[2 * j], mk1 = vis.mask[2 * j + 1];
  const float* qr = q + ((int64_t)r * nq + h) * d;
  float qv[4], ov[4] = {0.f, 0.f, 0.f, 0.f};
  const int nper = (d + 63) / 64;
  for (int i = 0; i < nper; ++i) qv[i] = (lane + 64 * i < d) ? qr[lane + 64 * i] : 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  for (int key = vis.pre_lo; key < vis.key_end; ++key) {
    if (!row_sees(vis, prehi, mk0, mk1, key)) continue;
    const float* kp = kv_ptr<float>(kv, key, 0, hk);
    const float* vp = kv_ptr<float>(kv, key, 1, hk);
    float part = 0.f;
    for (int i = 0; i < nper; ++i)
      if (lane + 64 * i < d) part += qv[i] * kp[lane + 64 * i];
    const float s = wave_sum(part) * scale;
    const float m_new = fmaxf(m_run, s);
    const float alpha = expf(m_run - m_new);
    const float pexp = expf(s - m_new);
    l_run = l_run * alpha + pexp;
    for (int i = 0; i < nper; ++i)
      if (lane + 64 * i < d) ov[i] = ov[i] * alpha + pexp * vp[lane + 64 * i];
    m_run = m_new;
  }
  for (int i = 0; i < nper; ++i)
    if (lane + 64 * i < d) out[((int64_t)r * nq + h) * d + lane + 64 * i] = ov[i] / l_run;
}

// ---------------------------------------------------------------- rows
// Four consecutive elements of a weight row as floats (bf16: one 8-byte load).
template <typename T> __device__ __forceinline__ float4 ld4e(const T* p);
template <> __device__ __forceinline__ float4 ld4e<float>(const float* p) { return ld4(p); }
template <> __device__ __forceinline__ float4 ld4e<bf16_t>(const bf16_t* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return make_float4(bf16_lo_f(w.x), bf16_hi_f(w.x), bf16_lo_f(w.y), bf16_hi_f(w.y));
}

template <typename T>
__global__ void embed_kernel(const T* E, int H, const int32_t* tok, float* h, Lanes ln) {
  const int r = blockIdx.x;
  const int b = ln.n > 1 ? r / ln.rows : 0, j = r - b * (ln.n > 1 ? ln.rows : 0);
  const T* e = E + (int64_t)lane_at(tok, b, ln.bytes)[j] * H;
  float* d = h + (int64_t)r * H;
  if (H % 4 == 0) {   // four elements per thread and step (uniform)
    for (int i = 4 * threadIdx.x; i < H; i += 4 * blockDim.x)
      *reinterpret_cast<float4*>(d + i) = ld4e(e + i);
    return;
  }
  for (int i = threadIdx.x; i < H; i += blockDim.x) d[i] = Elem<T>::to_f(e[i]);
}

__device__ __forceinline__ float block_sum_256(float v, float* sh) {
  // fixed-order block reduction (256 threads)
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) sh[threadIdx.x] = sh[threadIdx.x] + sh[threadIdx.x + o];
    __syncthreads();
  }
  const float s = sh[0];
  __syncthreads();
  return s;
}

// One workgroup of 1024 threads per row; thread t owns float4 groups t + 1024 u.
// h <- (set ? 0 : h) + sum of the S partial planes; then either the RMS-normalised
// row times gain (to out_t, and to out_f if given) or h itself is written as an operand.
template <typename T, int NV>
__global__ __launch_bounds__(1024) void resnorm_kernel(float* h, int H, const float* part, int S,
                                                       int64_t plane, int set, const float* gain,
                                                       float eps, T* out_t, int64_t lo, float* out_f) {
  __shared__ float sh[16];
  const int r = blockIdx.x;
  const int n4 = H / 4;
  float* x = h + (int64_t)r * H;
  const float* p[NV];
  bool ok[NV];
  float4 v[NV], g[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int j = threadIdx.x + 1024 * u;
    ok[u] = j < n4;
    p[u] = part + (int64_t)r * H + 4 * j;
  }
  // the gain is requested with the row's first loads, not after the block
  // reduction: a load issued behind the barrier would be one more memory
  // round trip on the kernel's critical path
  if (gain) {
#pragma unroll
    for (int u = 0; u < NV; ++u) g[u] = ld4(gain + 4 * min((int)threadIdx.x + 1024 * u, n4 - 1));
  }
  if (S > 0) {
    // the residual row is requested before the partial planes so the two
    // loads overlap
#pragma unroll
    for (int u = 0; u < NV; ++u)
      v[u] = (set || !ok[u]) ? make_float4(0.f, 0.f, 0.f, 0.f) : ld4(x + 4 * (threadIdx.x + 1024 * u));
    float4 acc[NV];
    plane_sums<NV>(p, ok, S, plane, acc);
#pragma unroll
    for (int u = 0; u < NV; ++u) add4(v[u], acc[u]);
  } else {
#pragma unroll
    for (int u = 0; u < NV; ++u)
      v[u] = (set || !ok[u]) ? make_float4(0.f, 0.f, 0.f, 0.f) : ld4(x + 4 * (threadIdx.x + 1024 * u));
  }
  const int64_t rb = (int64_t)r * H;
  if (S > 0 || set) {
#pragma unroll
    for (int u = 0; u < NV; ++u)
      if (ok[u]) *reinterpret_cast<float4*>(x + 4 * (threadIdx.x + 1024 * u)) = v[u];
  }
  if (!gain) {
#pragma unroll
    for (int u = 0; u < NV; ++u)
      if (ok[u]) opnd_store4(out_t, lo, rb + 4 * (threadIdx.x + 1024 * u), v[u]);
    return;
  }
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < NV; ++u) ss += v[u].x * v[u].x + v[u].y * v[u].y + v[u].z * v[u].z + v[u].w * v[u].w;
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < 16; ++w) tot += sh[w];   // fixed order: identical in every thread
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    if (!ok[u]) continue;
    const int i = 4 * (threadIdx.x + 1024 * u);
    const float4 y = make_float4(v[u].x * inv * g[u].x, v[u].y * inv * g[u].y, v[u].z * inv * g[u].z,
                                 v[u].w * inv * g[u].w);
    if (out_f) *reinterpret_cast<float4*>(out_f + rb + i) = y;
    opnd_store4(out_t, lo, rb + i, y);
  }
}

// resnorm_kernel's residual update with the normalization split over
// RS_SLICES workgroups per row: workgroup (r, sl) of H / (4 RS_SLICES)
// threads owns columns [sl H / RS_SLICES, (sl + 1) H / RS_SLICES) of row r,
// four per thread. It writes h, the operand gain * h (the RMSNorm numerator)
// and the slice's sum of squares to ss[RS_SLICES r + sl]; the projection
// that consumes the operand multiplies its output rows by the RMSNorm
// factor (RowScale). One workgroup per row pulls all of a row's partial
// planes through one CU; RS_SLICES workgroups share them.
template <typename T>
__global__ __launch_bounds__(1024) void resnorm_slice_kernel(float* h, int H, const float* part, int S,
                                                             int64_t plane, int set,
                                                             const float* gain, T* out_t, int64_t lo,
                                                             float* ss) {
  __shared__ float red[16];
  const int r = blockIdx.x, sl = blockIdx.y;
  const int c = 4 * (sl * (int)blockDim.x + (int)threadIdx.x);   // < H: the grid tiles the row
  const int64_t rc = (int64_t)r * H + c;
  float* x = h + rc;
  // the gain with the row's loads: none waits behind the reduction
  const float4 g = gain ? ld4(gain + c) : make_float4(1.f, 1.f, 1.f, 1.f);
  float4 v = set ? make_float4(0.f, 0.f, 0.f, 0.f) : ld4(x);
  if (S > 0) {
    const float* p[1] = {part + rc};
    const bool ok[1] = {true};
    float4 acc[1];
    plane_sums<1>(p, ok, S, plane, acc);
    add4(v, acc[0]);
  }
  if (S > 0 || set) *reinterpret_cast<float4*>(x) = v;
  if (!gain) {
    opnd_store4(out_t, lo, rc, v);
    return;
  }
  opnd_store4(out_t, lo, rc, make_float4(v.x * g.x, v.y * g.y, v.z * g.z, v.w * g.w));
  float s2 = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  s2 = wave_sum(s2);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s2;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < (int)blockDim.x / 64; ++w) t += red[w];   // fixed order
    ss[RS_SLICES * r + sl] = t;
  }
}

// dst[r, :W] (+)= sum of the S partial planes; grid (rows, W / 1024 rounded up), 256 threads
// each owning 4 consecutive columns.
__global__ __launch_bounds__(256) void sum_planes_kernel(const float* part, int S, int64_t plane, int W,
                                                         float* dst, int add) {
  const int r = blockIdx.x;
  const int c = 4 * (blockIdx.y * 256 + threadIdx.x);
  if (c >= W) return;
  const int64_t o = (int64_t)r * W + c;
  if ((W & 3) == 0) {
    const float* p[1] = {part + o};
    const bool ok[1] = {true};
    float4 acc[1];
    plane_sums<1>(p, ok, S, plane, acc);
    if (add) add4(acc[0], ld4(dst + o));
    *reinterpret_cast<float4*>(dst + o) = acc[0];
  } else {
    for (int e = 0; e < 4 && c + e < W; ++e) {
      float acc = part[o + e];
      for (int s = 1; s < S; ++s) acc += part[(int64_t)s * plane + o + e];
      dst[o + e] = add ? dst[o + e] + acc : acc;
    }
  }
}

// Sums the split-K planes of the fused q|k|v projection, applies the rotary
// embedding (rotate-half pairing) to q and k, writes q as an operand and k, v
// into the cache slot of each row. Workgroups [0, M n_qk): one row and 1024 / d
// consecutive q or k heads of it. The rest: 32 dimensions of one V head over
// a block of rb = 32 rows of one sequence, so that the transposed V planes of
// a bf16 cache are written by consecutive lanes at consecutive slots.
template <typename T>
__global__ __launch_bounds__(256) void rope_kv_kernel(const float* qkv, int S, int64_t plane, int nq,
                                                      int nkv, int d, const int32_t* pos,
                                                      const int32_t* slot,
                                                      const float* cos_t, const float* sin_t,
                                                      T* q_out, int64_t qlo, KVView kv_all,
                                                      Lanes ln, int M, int n_qk, int rb) {
  // q/k workgroups use the first 1024 floats; V workgroups rb rows of dg
  // floats at a pitch of dg + 1 (the transposed reads fall in distinct banks)
  __shared__ float xs[32 * 33];
  const int width = (nq + 2 * nkv) * d;
  const int half = d / 2;
  if ((int)blockIdx.x >= M * n_qk) {
    // ---- dimensions [i0, i0 + dg) of V head h over block blk of rb rows
    // of one sequence (rb * dg <= 1024: one float4 of each plane per thread,
    // its planes' loads in one round)
    const int dg = min(32, d), ndg = d / dg;
    int vb = blockIdx.x - M * n_qk;
    const int i0 = (vb % ndg) * dg;
    vb /= ndg;
    const int h = vb % nkv, blk = vb / nkv;
    const int rps = ln.n > 1 ? ln.rows : M;   // rows per sequence
    const int bps = (rps + rb - 1) / rb;
    const int seq = blk / bps, j0 = (blk % bps) * rb, nr = min(rb, rps - j0);
    const int r0 = seq * rps + j0;
    const int32_t* sl = (const int32_t*)((const char*)slot + seq * ln.bytes);
    const KVView kv = lane_kv<T>(kv_all, seq);
    const int col0 = (nq + nkv + h) * d + i0;
    // the cache slots of this thread's stores are requested with the plane
    // loads (rb * dg <= 1024: at most four stores per thread)
    int slt[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = min((int)threadIdx.x + 256 * k, nr * dg - 1);
      slt[k] = sl[j0 + (sizeof(T) == 2 ? e % nr : e / dg)];
    }
    {
      const int e = 4 * threadIdx.x;
      const bool ok[1] = {e < nr * dg};
      const int ec = ok[0] ? e : 0;
      const float* pp[1] = {qkv + (int64_t)(r0 + ec / dg) * width + col0 + ec % dg};
      float4 acc[1];
      plane_sums<1>(pp, ok, S, plane, acc);
      if (ok[0]) {
        float* x = xs + (e / dg) * (dg + 1) + e % dg;
        x[0] = acc[0].x; x[1] = acc[0].y; x[2] = acc[0].z; x[3] = acc[0].w;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // bf16: consecutive lanes on consecutive rows (slots) of one dimension
      // of the transposed V planes; fp32: along the row
      const int e = (int)threadIdx.x + 256 * k;
      if (e >= nr * dg) break;
      const int rr = sizeof(T) == 2 ? e % nr : e / dg, i = sizeof(T) == 2 ? e / nr : e % dg;
      KVStore<T>::put(kv, slt[k], 1, h, i0 + i, xs[rr * (dg + 1) + i]);
    }
    return;
  }
  // ---- one row, q or k heads [h0, h0 + nh)
  const int r = blockIdx.x / n_qk, grp = blockIdx.x % n_qk;
  // the row's sequence: its position / slot entries and its cache
  const int seq = ln.n > 1 ? r / ln.rows : 0, j = ln.n > 1 ? r - seq * ln.rows : r;
  pos = (const int32_t*)((const char*)pos + seq * ln.bytes);
  slot = (const int32_t*)((const char*)slot + seq * ln.bytes);
  const KVView kv = lane_kv<T>(kv_all, seq);
  const int hpw = 1024 / d;
  const int h0 = grp * hpw;
  const int nh = min(hpw, nq + nkv - h0);
  // the row's position and slot, then its cos / sin entries, are requested
  // while the plane loads are in flight, not behind the barrier; when half
  // divides 256 every pair this thread rotates has the same i
  const int pj = pos[j], sl = slot[j];
  const float* c = cos_t + (int64_t)pj * half;
  const float* s = sin_t + (int64_t)pj * half;
  const bool one_i = 256 % half == 0;
  const int it = (int)threadIdx.x % half;
  const float ci = one_i ? c[it] : 0.f, si = one_i ? s[it] : 0.f;
  {
    const int e = 4 * threadIdx.x;
    const bool ok[1] = {e < nh * d};
    const float* p[1] = {qkv + (int64_t)r * width + h0 * d + e};
    float4 acc[1];
    plane_sums<1>(p, ok, S, plane, acc);
    if (ok[0]) *reinterpret_cast<float4*>(xs + e) = acc[0];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < nh * half; idx += 256) {
    const int lh = idx / half, i = idx % half;
    const int head = h0 + lh;
    const float* src = xs + lh * d;
    const float x1 = src[i], x2 = src[i + half];
    const float cc = one_i ? ci : c[i], ss = one_i ? si : s[i];
    const float y1 = x1 * cc - x2 * ss;
    const float y2 = x2 * cc + x1 * ss;
    if (head < nq) {
      const int64_t base = ((int64_t)r * nq + head) * d;
      Opnd<T>::store(q_out, qlo, base + i, y1);
      Opnd<T>::store(q_out, qlo, base + i + half, y2);
    } else {
      KVStore<T>::put(kv, sl, 0, head - nq, i, y1);
      KVStore<T>::put(kv, sl, 0, head - nq, i + half, y2);
    }
  }
}

template <typename T>
__global__ void draft_input_e1_kernel(const T* E, const int32_t* tok, const float* feat,
                                      const int32_t* idx, int H, T* x, int64_t lo, Lanes ln,
                                      int64_t feat_stride, int64_t idx_bytes) {
  const int r = blockIdx.x;
  const int b = ln.n > 1 ? r / ln.rows : 0, j = r - b * (ln.n > 1 ? ln.rows : 0);
  const T* e = E + (int64_t)lane_at(tok, b, ln.bytes)[j] * H;
  const float* f = feat + b * feat_stride + (int64_t)lane_at(idx, b, idx_bytes)[j] * H;
  const int64_t row = (int64_t)r * 2 * H;
  if constexpr (Opnd<T>::SPLIT) {
    // bf16 (H a multiple of 8): eight elements per thread and step, one
    // 16-byte embedding load and two 16-byte feature loads
    for (int i = threadIdx.x * 8; i < H; i += blockDim.x * 8) {
      const uint4 ev = ld16(e + i);
      const float4 f0 = ld4(f + i), f1 = ld4(f + i + 4);
      const uint32_t w[4] = {ev.x, ev.y, ev.z, ev.w};
      float4 e0, e1;
      e0.x = __uint_as_float(w[0] << 16); e0.y = __uint_as_float(w[0] & 0xffff0000u);
      e0.z = __uint_as_float(w[1] << 16); e0.w = __uint_as_float(w[1] & 0xffff0000u);
      e1.x = __uint_as_float(w[2] << 16); e1.y = __uint_as_float(w[2] & 0xffff0000u);
      e1.z = __uint_as_float(w[3] << 16); e1.w = __uint_as_float(w[3] & 0xffff0000u);
      opnd_store4(x, lo, row + i, e0);
      opnd_store4(x, lo, row + i + 4, e1);
      opnd_store4(x, lo, row + H + i, f0);
      opnd_store4(x, lo, row + H + i + 4, f1);
    }
  } else {
    for (int i = threadIdx.x; i < H; i += blockDim.x) {
      Opnd<T>::store(x, lo, row + i, Elem<T>::to_f(e[i]));
      Opnd<T>::store(x, lo, row + H + i, f[i]);
    }
  }
}

// E3 draft input of one row: x = RMSNorm([E[t]; g]) * gain over the 2H-wide
// concatenation (operand), h = g. Thread t owns float4 groups t + 256 u of
// each half; all of its loads (embedding, feature, both gain halves) go
// out in one round, and the row's sum of squares is one wave reduction
// plus a four-way sum in LDS.
template <typename T, int NV>
__global__ __launch_bounds__(256) void draft_input_e3_kernel(const T* E, const int32_t* tok,
                                                             const float* feat, const int32_t* idx,
                                                             const float* gain, float eps, int H,
                                                             T* x, int64_t lo, float* h, Lanes ln,
                                                             int64_t feat_stride, int64_t idx_bytes) {
  __shared__ float sh[4];
  const int r = blockIdx.x;
  const int b = ln.n > 1 ? r / ln.rows : 0, j = r - b * (ln.n > 1 ? ln.rows : 0);
  const T* e = E + (int64_t)lane_at(tok, b, ln.bytes)[j] * H;
  const float* f = feat + b * feat_stride + (int64_t)lane_at(idx, b, idx_bytes)[j] * H;
  const int n4 = H / 4;
  float4 ev[NV], fv[NV], ge[NV], gf[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int q = 4 * min((int)threadIdx.x + 256 * u, n4 - 1);   // past the end: a repeat, not used
    ev[u] = ld4e(e + q);
    fv[u] = ld4(f + q);
    ge[u] = ld4(gain + q);
    gf[u] = ld4(gain + H + q);
  }
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < NV; ++u)
    if ((int)threadIdx.x + 256 * u < n4)
      ss += ev[u].x * ev[u].x + ev[u].y * ev[u].y + ev[u].z * ev[u].z + ev[u].w * ev[u].w +
            fv[u].x * fv[u].x + fv[u].y * fv[u].y + fv[u].z * fv[u].z + fv[u].w * fv[u].w;
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float inv = 1.0f / sqrtf(((sh[0] + sh[1]) + (sh[2] + sh[3])) / (float)(2 * H) + eps);
  const int64_t row = (int64_t)r * 2 * H;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int g4 = (int)threadIdx.x + 256 * u;
    if (g4 >= n4) continue;
    const int q = 4 * g4;
    opnd_store4(x, lo, row + q,
                make_float4(ev[u].x * inv * ge[u].x, ev[u].y * inv * ge[u].y, ev[u].z * inv * ge[u].z,
                            ev[u].w * inv * ge[u].w));
    opnd_store4(x, lo, row + H + q,
                make_float4(fv[u].x * inv * gf[u].x, fv[u].y * inv * gf[u].y, fv[u].z * inv * gf[u].z,
                            fv[u].w * inv * gf[u].w));
    *reinterpret_cast<float4*>(h + (int64_t)r * H + q) = fv[u];
  }
}

__global__ void gather_f32_kernel(const float* src, int64_t ld, const int32_t* idx, int W, float* dst) {
  const int r = blockIdx.x;
  const float* s = src + (int64_t)idx[r] * ld;
  for (int i = threadIdx.x; i < W; i += blockDim.x) dst[(int64_t)r * W + i] = s[i];
}

template <typename T>
__global__ void gather_t_kernel(const T* src, int64_t ld, int64_t src_lo, const int32_t* idx, int W,
                                T* dst, int64_t dst_lo) {
  const int r = blockIdx.x;
  const T* s = src + (int64_t)idx[r] * ld;
  for (int i = threadIdx.x; i < W; i += blockDim.x) {
    dst[(int64_t)r * W + i] = s[i];
    if (Opnd<T>::SPLIT) dst[dst_lo + (int64_t)r * W + i] = s[src_lo + i];
  }
}

// Row b: sequence b's root row (row b * src_rows + acc_b[0]) of the fp32
// rows src_f and of the operand rows src_t (width W each).
// gather_t_kernel in 16-byte pieces (widths, pitches and plane offsets in
// whole pieces, 16-byte aligned buffers): eight pieces of each plane in
// flight per thread; threads past the end repeat the last piece (same value,
// same place) so no load waits behind a conditional store.
template <typename T>
__global__ __launch_bounds__(256) void gather_t16_kernel(const T* src, int64_t ld, int64_t src_lo,
                                                         const int32_t* idx, int W, T* dst,
                                                         int64_t dst_lo) {
  constexpr int EPV = 16 / sizeof(T);
  constexpr int PL = Opnd<T>::SPLIT ? 2 : 1;
  const int r = blockIdx.x;
  const T* s = src + (int64_t)idx[r] * ld;
  T* d = dst + (int64_t)r * W;
  const int nv = W / EPV;
  for (int i0 = 0; i0 < nv; i0 += 256 * 8) {
    uint4 v[8][PL];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = min(i0 + 256 * u + (int)threadIdx.x, nv - 1) * EPV;
#pragma unroll
      for (int pl = 0; pl < PL; ++pl) v[u][pl] = *reinterpret_cast<const uint4*>(s + pl * src_lo + i);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = min(i0 + 256 * u + (int)threadIdx.x, nv - 1) * EPV;
#pragma unroll
      for (int pl = 0; pl < PL; ++pl) *reinterpret_cast<uint4*>(d + pl * dst_lo + i) = v[u][pl];
    }
  }
}

template <typename T>
__global__ void gather_roots_kernel(const float* src_f, const T* src_t, int64_t src_lo, int src_rows,
                                    const int32_t* acc, int W, float* dst_f, int64_t dst_stride,
                                    T* dst_t, int64_t dst_lo, Lanes ln) {
  const int b = blockIdx.x;
  const int64_t row = (int64_t)b * src_rows + lane_at(acc, b, ln.bytes)[0];
  constexpr int EPV = 16 / sizeof(T);
  if (W % EPV == 0 && dst_stride % 4 == 0 && src_lo % EPV == 0 && dst_lo % EPV == 0) {
    // 16-byte pieces (uniform): the fp32 row, then the operand planes
    for (int i = 4 * threadIdx.x; i < W; i += 4 * blockDim.x)
      *reinterpret_cast<float4*>(dst_f + b * dst_stride + i) = ld4(src_f + row * W + i);
    for (int i = EPV * threadIdx.x; i < W; i += EPV * blockDim.x) {
      *reinterpret_cast<uint4*>(dst_t + (int64_t)b * W + i) = *reinterpret_cast<const uint4*>(src_t + row * W + i);
      if (Opnd<T>::SPLIT)
        *reinterpret_cast<uint4*>(dst_t + dst_lo + (int64_t)b * W + i) =
            *reinterpret_cast<const uint4*>(src_t + src_lo + row * W + i);
    }
    return;
  }
  for (int i = threadIdx.x; i < W; i += blockDim.x) {
    dst_f[b * dst_stride + i] = src_f[row * W + i];
    dst_t[(int64_t)b * W + i] = src_t[row * W + i];
    if (Opnd<T>::SPLIT) dst_t[dst_lo + (int64_t)b * W + i] = src_t[src_lo + row * W + i];
  }
}

template <typename T>
__global__ void store_feat_kernel(const float* h, int H, T* dst, int64_t ldd, int64_t lo) {
  const int r = blockIdx.x;
  for (int i = threadIdx.x; i < H; i += blockDim.x)
    Opnd<T>::store(dst, lo, (int64_t)r * ldd + i, h[(int64_t)r * H + i]);
}

__global__ void rows_causal_kernel(int first, int M, int32_t* pos, int32_t* slot, int32_t* prehi,
                                   uint64_t* mask, Lanes ln) {
  const int b = blockIdx.y;
  first += lane_shift(ln, b);
  pos = lane_at(pos, b, ln.bytes);
  slot = lane_at(slot, b, ln.bytes);
  prehi = lane_at(prehi, b, ln.bytes);
  mask = lane_at(mask, b, ln.bytes);
  for (int r = threadIdx.x + blockIdx.x * blockDim.x; r < M; r += blockDim.x * gridDim.x) {
    pos[r] = first + r;
    slot[r] = first + r;
    prehi[r] = first + r + 1;
    mask[2 * r] = 0;
    mask[2 * r + 1] = 0;
  }
}

// Moves the K/V rows of the accepted path (tree slots ctx + path[j]) to
// slots ctx + 1 + j in every layer. Each thread owns one element of one
// (layer, kv head) and reads all sources before writing any destination,
// since a destination may be an earlier source.
template <typename T>
__global__ void kv_compact_kernel(KVView v, int64_t layer_elems, const int32_t* Lp,
                                  const int32_t* path, int ctx, int planes, Lanes ln) {
  const int layer = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  Lp = lane_at(Lp, b, ln.bytes);
  path = lane_at(path, b, ln.bytes);
  ctx += lane_shift(ln, b);
  const int L = *Lp;
  if (L <= 0) return;
  KVView lv = v;
  lv.base = (T*)v.base + (int64_t)layer * layer_elems + b * v.lane_elems;
  for (int e = threadIdx.x; e < planes * v.d; e += blockDim.x) {
    const int sel = e / v.d, i = e % v.d;
    T vals[EAGLE_COMPACT_MAX];
    for (int j = 0; j < L; ++j) vals[j] = *kv_elem<T>(lv, ctx + path[j], sel, h, i);
    for (int j = 0; j < L; ++j) *kv_elem<T>(lv, ctx + 1 + j, sel, h, i) = vals[j];
  }
}

}  // namespace

int attn_chunk_keys() { return CHUNK; }
int attn_max_chunks() { return ATTN_MAX_CHUNKS; }

uint64_t attn_part_floats(int max_chunks, int M, int nq, int d) {
  return (uint64_t)max_chunks * M * nq * (d + 2);
}

#define DT_DISPATCH(dtype, KERNEL_CALL_BF16, KERNEL_CALL_F32) \
  do {                                                        \
    if ((dtype) == 1) { KERNEL_CALL_BF16; } else { KERNEL_CALL_F32; } \
  } while (0)

static bool kv_page_bad(const KVView& v) { return v.page <= 0 || (v.page & (v.page - 1)) != 0; }

static bool lanes_bad(const Lanes& ln, int M) {
  return ln.n < 1 || ln.n > MAX_LANES || (ln.n > 1 && ln.rows * ln.n != M);
}

hipError_t launch_embed(int dtype, const void* E, int H, const int32_t* tok, int M, float* h,
                        hipStream_t st, const Lanes& ln) {
  if (M <= 0) return hipSuccess;
  if (lanes_bad(ln, M)) return hipErrorInvalidValue;
  DT_DISPATCH(dtype,
              hipLaunchKernelGGL(embed_kernel<bf16_t>, dim3(M), dim3(256), 0, st, (const bf16_t*)E, H, tok, h, ln),
              hipLaunchKernelGGL(embed_kernel<float>, dim3(M), dim3(256), 0, st, (const float*)E, H, tok, h, ln));
  return hipGetLastError();
}

hipError_t launch_resnorm(int dtype, float* h, int H, int M, const float* part, int S,
                          int64_t plane, int set, const float* gain, float eps, void* out_t,
                          int64_t lo, float* out_f, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (H % 4 != 0 || H > 4 * 4096) return hipErrorInvalidValue;
  const int nv = (H / 4 + 1023) / 1024;
#define RN(NV)                                                                                   \
  DT_DISPATCH(dtype,                                                                             \
              hipLaunchKernelGGL((resnorm_kernel<bf16_t, NV>), dim3(M), dim3(1024), 0, st, h, H, \
                                 part, S, plane, set, gain, eps, (bf16_t*)out_t, lo, out_f),     \
              hipLaunchKernelGGL((resnorm_kernel<float, NV>), dim3(M), dim3(1024), 0, st, h, H,  \
                                 part, S, plane, set, gain, eps, (float*)out_t, lo, out_f))
  switch (nv) {
    case 1: RN(1); break;
    case 2: RN(2); break;
    case 3: RN(3); break;
    default: RN(4); break;
  }
#undef RN
  return hipGetLastError();
}

bool resnorm_slices_fit(int H) { return H > 0 && H % (64 * RS_SLICES * 4) == 0 && H <= 16384; }

hipError_t launch_resnorm_slices(int dtype, float* h, int H, int M, const float* part, int S,
                                 int64_t plane, int set, const float* gain, void* out_t, int64_t lo,
                                 float* ss, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (!resnorm_slices_fit(H) || (gain && !ss)) return hipErrorInvalidValue;
  const dim3 grid(M, RS_SLICES), block(H / (4 * RS_SLICES));
  DT_DISPATCH(dtype,
              hipLaunchKernelGGL(resnorm_slice_kernel<bf16_t>, grid, block, 0, st, h, H, part, S, plane, set, gain, (bf16_t*)out_t, lo, ss),
              hipLaunchKernelGGL(resnorm_slice_kernel<float>, grid, block, 0, st, h, H, part, S, plane, set, gain, (float*)out_t, lo, ss));
  return hipGetLastError();
}

hipError_t launch_sum_planes(const float* part, int S, int64_t plane, int M, int W, float* dst,
                             int add, hipStream_t st) {
  if (M <= 0 || W <= 0) return hipSuccess;
  hipLaunchKernelGGL(sum_planes_kernel, dim3(M, (W + 1023) / 1024), dim3(256), 0, st, part, S, plane,
                     W, dst, add);
  return hipGetLastError();
}

hipError_t launch_rope_kv(int dtype, const float* qkv, int S, int64_t plane, int M, int nq, int nkv,
                          int d, const int32_t* pos, const int32_t* slot, const float* cos_t,
                          const float* sin_t, void* q_out, int64_t qlo, KVView kv, hipStream_t st,
                          const Lanes& ln) {
  if (kv_page_bad(kv)) return hipErrorInvalidValue;
  if (M <= 0) return hipSuccess;
  if (ln.n < 1 || ln.n > MAX_LANES || (ln.n > 1 && ln.rows * ln.n != M)) return hipErrorInvalidValue;
  if (d < 4 || d > 1024 || 1024 % d != 0 || ((nq + 2 * nkv) * d) % 4 != 0) return hipErrorInvalidValue;
  const int hpw = 1024 / d;
  const int n_qk = (nq + nkv + hpw - 1) / hpw;               // q/k workgroups per row
  const int dg = std::min(32, d), rb = 32;                   // dims and rows per V workgroup
  const int rps = ln.n > 1 ? ln.rows : M;
  const int n_v = (d / dg) * nkv * ln.n * ((rps + rb - 1) / rb);
  const dim3 grid(M * n_qk + n_v);
  DT_DISPATCH(dtype,
              hipLaunchKernelGGL(rope_kv_kernel<bf16_t>, grid, dim3(256), 0, st, qkv, S, plane, nq, nkv, d, pos, slot, cos_t, sin_t, (bf16_t*)q_out, qlo, kv, ln, M, n_qk, rb),
              hipLaunchKernelGGL(rope_kv_kernel<float>, grid, dim3(256), 0, st, qkv, S, plane, nq, nkv, d, pos, slot, cos_t, sin_t, (float*)q_out, qlo, kv, ln, M, n_qk, rb));
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, const void* q, int64_t qlo, KVView kv, RowVis vis, int M,
                            int nq, int d, float scale, float* opart, float* mlpart, void* out_t,
                            int64_t olo, hipStream_t st, const Lanes& ln) {
  if (kv_page_bad(kv)) return hipErrorInvalidValue;
  if (M <= 0) return hipSuccess;
  if (ln.n < 1 || ln.n > MAX_LANES || (ln.n > 1 && ln.rows * ln.n != M)) return hipErrorInvalidValue;
  const int group = nq / kv.n_kv;
  // every sequence needs at least one key; the grid covers the longest
  LaneChunks lc{ln.n > 1 ? ln.rows : M, ln.n, {}};
  int n_chunks = 0;
  for (int b = 0; b < ln.n; ++b) {
    // bf16 chunks start on page boundaries (chunk_base); fp32 rows walk keys from pre_lo
    const int c0 = dtype == 1 ? (vis.pre_lo & ~(CHUNK - 1)) : vis.pre_lo;
    const int c = (vis.key_end + ln.off[b] - c0 + CHUNK - 1) / CHUNK;
    if (c <= 0) return hipErrorInvalidValue;
    lc.chunks[b] = c;
    n_chunks = std::max(n_chunks, c);
  }
  if (dtype == 1) {
    if (d != 128) return hipErrorInvalidValue;
    if (n_chunks > ATTN_MAX_CHUNKS || kv.page < CHUNK || kv.page % CHUNK) return hipErrorInvalidValue;
    if (vis.n_tree == 0 && ln.n == 1 && M >= 32 && group <= 8) {
      // causal rows without tree keys (prefill chunks): flash form, 16 rb
      // rows per workgroup, at least four (head, row block) pairs
      const int rb = group >= 4 ? 1 : 4 / group;
      FlashArgs f{(const bf16_t*)q, qlo, kv, vis, M, nq, group, rb, scale * 1.4426950408889634f,
                  (bf16_t*)out_t, olo};
      const dim3 grid((M + 16 * rb - 1) / (16 * rb) * kv.n_kv);
      if (group * rb > 4)
        hipLaunchKernelGGL(attn_flash_kernel<2>, grid, dim3(512), 0, st, f);
      else
        hipLaunchKernelGGL(attn_flash_kernel<1>, grid, dim3(512), 0, st, f);
      return hipGetLastError();
    }
    if (lc.rows < 48) {
      // few rows per sequence (a static tree's verify, every draft pass):
      // one workgroup per (64-key chunk, KV head) so every chunk's loads go
      // out at once -- these launches are bound by memory latency, and a
      // walk over several chunks per workgroup measured slower here; then
      // the chunk combine. Split a head's (query head, row block) pairs over
      // more workgroups only while the grid is short of two workgroups per
      // CU: every extra group stages the chunk again.
      const int pairs = group * ((lc.rows + 15) / 16);   // per sequence
      const int wgs = n_chunks * kv.n_kv * ln.n;
      const int want = (512 + wgs - 1) / wgs;
      int n_groups = std::max(1, std::min((pairs + 3) / 4, want));
      const int ppg = (pairs + n_groups - 1) / n_groups;
      n_groups = (pairs + ppg - 1) / ppg;
      AttnArgs a{(const bf16_t*)q, qlo, kv, vis, M, nq, group, ppg, scale * 1.4426950408889634f,
                 opart, mlpart, ln, n_groups};
      hipLaunchKernelGGL(attn_bf16_kernel, dim3(n_chunks, kv.n_kv, n_groups * ln.n), dim3(256), 0,
                         st, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(attn_combine_kernel<bf16_t>, dim3(M, nq), dim3(128), 0, st, opart, mlpart,
                         lc, M, nq, d, (bf16_t*)out_t, olo);
      return hipGetLastError();
    }
    // many rows per sequence (dynamic-tree verify passes): the split form.
    // Query rows of a KV head packed into 16-row tiles, up to four tiles per
    // row group (balanced; one per wave slot), and each sequence's key chunks
    // split so the grid holds at most 256 workgroups (the kernel runs one per
    // CU: a 257th would wait for a second round), at least two chunks per
    // split. Scores are taken in log2 units (scale * log2 e) so the softmax
    // uses the native exp2; maxima in mlpart are in the same units.
    const int ntile = (group * lc.rows + 15) / 16;
    const int rg = (ntile + 3) / 4, tpg = (ntile + rg - 1) / rg;
    const int units = kv.n_kv * rg;
    SplitArgs sa{(const bf16_t*)q, qlo, kv, vis, ln, M, nq, group, ntile, tpg, rg, 1, {},
                 scale * 1.4426950408889634f, (bf16_t*)out_t, olo, opart, mlpart};
    for (int b = 0; b < ln.n; ++b) {
      const int want = 256 / units;   // one 512-thread workgroup per CU
      sa.splits[b] = std::max(1, std::min(want, lc.chunks[b] / 2));
      sa.splits[b] = std::max(sa.splits[b], (lc.chunks[b] + ATTN_SPLIT_CHUNKS - 1) / ATTN_SPLIT_CHUNKS);
      lc.chunks[b] = sa.splits[b];
      sa.smax = std::max(sa.smax, sa.splits[b]);
    }
    const dim3 grid(kv.n_kv * sa.smax * rg, 1, ln.n);
    hipLaunchKernelGGL(attn_split_kernel<1>, grid, dim3(512), 0, st, sa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || sa.smax == 1) return e;
    hipLaunchKernelGGL(attn_combine_kernel<bf16_t>, dim3(M, nq), dim3(128), 0, st, opart, mlpart,
                       lc, M, nq, d, (bf16_t*)out_t, olo);
  } else {
    if (d > 256) return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_f32_kernel, dim3(M, nq), dim3(64), 0, st, (const float*)q, kv, vis, ln,
                       M, nq, group, d, scale, (float*)out_t);
  }
  return hipGetLastError();
}

hipError_t launch_draft_input_e1(int dtype, const void* E, const int32_t* tok, const float* feat,
                                 const int32_t* idx, int M, int H, void* x, int64_t lo,
                                 hipStream_t st, const Lanes& ln, int64_t feat_stride,
                                 int64_t idx_bytes) {
  if (M <= 0) return hipSuccess;
  if (lanes_bad(ln, M)) return hipErrorInvalidValue;
  DT_DISPATCH(dtype,
              hipLaunchKernelGGL(draft_input_e1_kernel<bf16_t>, dim3(M), dim3(256), 0, st, (const bf16_t*)E, tok, feat, idx, H, (bf16_t*)x, lo, ln, feat_stride, idx_bytes),
              hipLaunchKernelGGL(draft_input_e1_kernel<float>, dim3(M), dim3(256), 0, st, (const float*)E, tok, feat, idx, H, (float*)x, lo, ln, feat_stride, idx_bytes));
  return hipGetLastError();
}

hipError_t launch_draft_input_e3(int dtype, const void* E, const int32_t* tok, const float* feat,
                                 const int32_t* idx, const float* gain, float eps, int M, int H,
                                 void* x, int64_t lo, float* h, hipStream_t st, const Lanes& ln,
                                 int64_t feat_stride, int64_t idx_bytes) {
  if (M <= 0) return hipSuccess;
  if (lanes_bad(ln, M)) return hipErrorInvalidValue;
  // float4 groups: H a multiple of 4 (and of the 16-byte feature rows), at most 8 groups per
  // thread and half
  if (H % 4 != 0 || H > 8 * 1024 || feat_stride % 4 != 0) return hipErrorInvalidValue;
  const int nv = (H / 4 + 255) / 256;
#define E3(NV)                                                                                        \
  DT_DISPATCH(dtype,                                                                                  \
              hipLaunchKernelGGL((draft_input_e3_kernel<bf16_t, NV>), dim3(M), dim3(256), 0, st,      \
                                 (const bf16_t*)E, tok, feat, idx, gain, eps, H, (bf16_t*)x, lo, h,   \
                                 ln, feat_stride, idx_bytes),                                         \
              hipLaunchKernelGGL((draft_input_e3_kernel<float, NV>), dim3(M), dim3(256), 0, st,       \
                                 (const float*)E, tok, feat, idx, gain, eps, H, (float*)x, lo, h, ln, \
                                 feat_stride, idx_bytes))
  if (nv <= 1) E3(1);
  else if (nv <= 2) E3(2);
  else if (nv <= 4) E3(4);
  else E3(8);
#undef E3
  return hipGetLastError();
}

hipError_t launch_gather_roots(int dtype, const float* src_f, const void* src_t, int64_t src_lo,
                               int src_rows, const int32_t* acc, int W, float* dst_f,
                               int64_t dst_stride, void* dst_t, int64_t dst_lo, const Lanes& ln,
                               hipStream_t st) {
  if (ln.n < 1 || ln.n > MAX_LANES || src_rows < 1) return hipErrorInvalidValue;
  DT_DISPATCH(dtype,
              hipLaunchKernelGGL(gather_roots_kernel<bf16_t>, dim3(ln.n), dim3(256), 0, st, src_f, (const bf16_t*)src_t, src_lo, src_rows, acc, W, dst_f, dst_stride, (bf16_t*)dst_t, dst_lo, ln),
              hipLaunchKernelGGL(gather_roots_kernel<float>, dim3(ln.n), dim3(256), 0, st, src_f, (const float*)src_t, src_lo, src_rows, acc, W, dst_f, dst_stride, (float*)dst_t, dst_lo, ln));
  return hipGetLastError();
}

hipError_t launch_gather_f32(const float* src, int64_t ld, const int32_t* idx, int M, int W,
                             float* dst, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_f32_kernel, dim3(M), dim3(256), 0, st, src, ld, idx, W, dst);
  return hipGetLastError();
}

hipError_t launch_gather_t(int dtype, const void* src, int64_t ld, int64_t src_lo, const int32_t* idx,
                           int M, int W, void* dst, int64_t dst_lo, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  const int epv = dtype == 1 ? 8 : 4;
  const bool vec = W % epv == 0 && ld % epv == 0 && src_lo % epv == 0 && dst_lo % epv == 0 &&
                   ((uintptr_t)src & 15) == 0 && ((uintptr_t)dst & 15) == 0;
  if (vec) {
    DT_DISPATCH(dtype,
                hipLaunchKernelGGL(gather_t16_kernel<bf16_t>, dim3(M), dim3(256), 0, st, (const bf16_t*)src, ld, src_lo, idx, W, (bf16_t*)dst, dst_lo),
                hipLaunchKernelGGL(gather_t16_kernel<float>, dim3(M), dim3(256), 0, st, (const float*)src, ld, src_lo, idx, W, (float*)dst, dst_lo));
    return hipGetLastError();
  }
  DT_DISPATCH(dtype,
              hipLaunchKernelGGL(gather_t_kernel<bf16_t>, dim3(M), dim3(256), 0, st, (const bf16_t*)src, ld, src_lo, idx, W, (bf16_t*)dst, dst_lo),
              hipLaunchKernelGGL(gather_t_kernel<float>, dim3(M), dim3(256), 0, st, (const float*)src, ld, src_lo, idx, W, (float*)dst, dst_lo));
  return hipGetLastError();
}

hipError_t launch_store_feat(int dtype, const float* h, int H, int M, void* dst, int64_t ldd,
                             int64_t lo, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  DT_DISPATCH(dtype,
              hipLaunchKernelGGL(store_feat_kernel<bf16_t>, dim3(M), dim3(256), 0, st, h, H, (bf16_t*)dst, ldd, lo),
              hipLaunchKernelGGL(store_feat_kernel<float>, dim3(M), dim3(256), 0, st, h, H, (float*)dst, ldd, lo));
  return hipGetLastError();
}

hipError_t launch_rows_causal(int first, int M, int32_t* pos, int32_t* slot, int32_t* prehi,
                              uint64_t* mask, hipStream_t st, const Lanes& ln) {
  if (M <= 0) return hipSuccess;
  if (ln.n < 1 || ln.n > MAX_LANES) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rows_causal_kernel, dim3((M + 255) / 256, ln.n), dim3(256), 0, st, first, M, pos,
                     slot, prehi, mask, ln);
  return hipGetLastError();
}

hipError_t launch_kv_compact(int dtype, KVView layer0, int64_t layer_elems, int n_layers,
                             const int32_t* L, const int32_t* path, int ctx, hipStream_t st,
                             const Lanes& ln) {
  if (kv_page_bad(layer0)) return hipErrorInvalidValue;
  if (ln.n < 1 || ln.n > MAX_LANES) return hipErrorInvalidValue;
  DT_DISPATCH(dtype,
              hipLaunchKernelGGL(kv_compact_kernel<bf16_t>, dim3(n_layers, layer0.n_kv, ln.n), dim3(512), 0, st, layer0, layer_elems, L, path, ctx, 4, ln),
              hipLaunchKernelGGL(kv_compact_kernel<float>, dim3(n_layers, layer0.n_kv, ln.n), dim3(256), 0, st, layer0, layer_elems, L, path, ctx, 2, ln));
  return hipGetLastError();
}
