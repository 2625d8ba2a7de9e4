// Shared device definitions of the gfx950 kernels: element types, rounding,
// MFMA fragments, small warp helpers. Host-visible launcher prototypes live
// in kernels.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;                       // raw bfloat16 bits
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

#define WAVE 64
#define EAGLE_COMPACT_MAX 16   // longest accepted path (= max draft depth)

// ---------------------------------------------------------------- rounding
__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// Round-to-nearest-even fp32 -> bf16 with the gfx950 conversion instruction
// (v_cvt_pk_bf16_f32; the same bits as adding 0x7fff plus the lsb to the
// fp32 pattern and truncating, for finite inputs).
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}
// Two values in one 32-bit word, element a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_hw v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Element type T of weights / KV / matrix operands: float or bf16_t.
template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static float load(const float* p) { return *p; }
  __device__ static float to_f(float v) { return v; }
  __device__ static float from_f(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  __device__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ static float to_f(bf16_t v) { return bf16_to_f32(v); }
  __device__ static bf16_t from_f(float v) { return f32_to_bf16(v); }
};

// Activation operands of the matrix cores. fp32 configs keep one fp32 plane.
// bf16 configs keep each value v as two bf16 planes, hi = bf16(v) and
// lo = bf16(v - hi), the lo plane `lo` elements after the hi plane: 16
// significant bits, and hi*w + lo*w on the bf16 MFMA gives the product of
// the fp32 activation with a bf16 weight to that precision.
template <typename T> struct Opnd;
template <> struct Opnd<float> {
  static constexpr bool SPLIT = false;
  __device__ static void store(float* p, int64_t, int64_t i, float v) { p[i] = v; }
};
template <> struct Opnd<bf16_t> {
  static constexpr bool SPLIT = true;
  __device__ static void store(bf16_t* p, int64_t lo, int64_t i, float v) {
    const bf16_t h = f32_to_bf16(v);
    p[i] = h;
    p[lo + i] = f32_to_bf16(v - bf16_to_f32(h));
  }
};

// Four consecutive operand values from element i (i a multiple of 4).
__device__ __forceinline__ void opnd_store4(float* p, int64_t, int64_t i, float4 v) {
  *reinterpret_cast<float4*>(p + i) = v;
}
__device__ __forceinline__ void opnd_store4(bf16_t* p, int64_t lo, int64_t i, float4 v) {
  const float f[4] = {v.x, v.y, v.z, v.w};
  uint32_t hw[2], lw[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    hw[e] = pack_bf16x2(f[2 * e], f[2 * e + 1]);
    lw[e] = pack_bf16x2(f[2 * e] - bf16_lo_f(hw[e]), f[2 * e + 1] - bf16_hi_f(hw[e]));
  }
  *reinterpret_cast<uint2*>(p + i) = make_uint2(hw[0], hw[1]);
  *reinterpret_cast<uint2*>(p + lo + i) = make_uint2(lw[0], lw[1]);
}

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void add4(float4& a, const float4& b) {
  a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
}

// Sums of split-K partial planes: acc[u] = sum over s ascending of p[u][s * plane],
// with NV * B independent 16-byte loads in flight per thread.
template <int NV>
__device__ __forceinline__ void plane_sums(const float* const (&p)[NV], const bool (&ok)[NV], int S,
                                           int64_t plane, float4 (&acc)[NV]) {
  constexpr int B = NV >= 8 ? 1 : 8 / NV;
#pragma unroll
  for (int u = 0; u < NV; ++u) acc[u] = ok[u] ? ld4(p[u]) : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 1; s0 < S; s0 += B) {
    float4 t[B][NV];
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int u = 0; u < NV; ++u)
        t[b][u] = (ok[u] && s0 + b < S) ? ld4(p[u] + (int64_t)(s0 + b) * plane)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int u = 0; u < NV; ++u)
        if (s0 + b < S) add4(acc[u], t[b][u]);
  }
}

// ---------------------------------------------------------------- MFMA
// One "step" is 16 bytes per lane along K: 8 bf16 or 4 fp32 elements.
// 16x16 tiles: lane l owns row (l & 15) of the A operand and column (l & 15)
// of the B operand; lane group (l >> 4) owns a 16-byte slice of K. The
// result D[i][j] sits in lane j + 16*(i/4), element i%4. Within a step, K
// may be permuted arbitrarily as long as A and B use the same permutation.
template <typename T> struct Mma;
template <> struct Mma<bf16_t> {
  static constexpr int EPL = 8;          // elements per lane per step
  static constexpr int KSTEP = 32;       // K covered by one step (4 lane groups)
  __device__ __forceinline__ static void mma(const uint4& a, const uint4& b, f32x4& c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static constexpr int EPL = 4;
  static constexpr int KSTEP = 16;
  // four 16x16x4 MFMAs; element e of every lane covers k = 4*(l>>4) + e
  __device__ __forceinline__ static void mma(const uint4& a, const uint4& b, f32x4& c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
};

// Workgroup barrier that waits only for this wave's LDS operations: global
// loads still in flight (weights, cache chunks being copied) stay in flight
// across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// ---------------------------------------------------------------- reductions
// Wave-wide reductions: four DPP steps combine the 16 lanes of each row (quad
// xor 1, quad xor 2, half-row mirror, row mirror: every pairing joins two
// disjoint groups, so each lane of a row ends with the row's value), then the
// four row values are read into scalar registers and combined. DPP moves are
// register-to-register; a __shfl_xor chain goes through the LDS crossbar
// (ds_bpermute) with a round trip per step. Results are wave-uniform.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(x)));
}
constexpr int DPP_QUAD_XOR1 = 0xB1, DPP_QUAD_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141,
              DPP_MIRROR = 0x140;
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<DPP_QUAD_XOR1>(v);
  v += dpp_f<DPP_QUAD_XOR2>(v);
  v += dpp_f<DPP_HALF_MIRROR>(v);
  v += dpp_f<DPP_MIRROR>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<DPP_QUAD_XOR1>(v));
  v = fmaxf(v, dpp_f<DPP_QUAD_XOR2>(v));
  v = fmaxf(v, dpp_f<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp_f<DPP_MIRROR>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dpp_i<DPP_QUAD_XOR1>(v));
  v = min(v, dpp_i<DPP_QUAD_XOR2>(v));
  v = min(v, dpp_i<DPP_HALF_MIRROR>(v));
  v = min(v, dpp_i<DPP_MIRROR>(v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Wave-wide argmax of (v desc, id asc, src asc): every lane passes its
// candidate and gets the winner back (wave-uniform). src breaks exact ties
// (e.g. empty candidates) so the order is total and all lanes agree.
__device__ __forceinline__ bool argmax_better(float ov, int oi, int os, float v, int i, int s) {
  return ov > v || (ov == v && (oi < i || (oi == i && os < s)));
}
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& v, int& i, int& s) {
  const float ov = dpp_f<CTRL>(v);
  const int oi = dpp_i<CTRL>(i), os = dpp_i<CTRL>(s);
  if (argmax_better(ov, oi, os, v, i, s)) { v = ov; i = oi; s = os; }
}
__device__ __forceinline__ void wave_argmax(float& v, int& i, int& s) {
  argmax_step<DPP_QUAD_XOR1>(v, i, s);
  argmax_step<DPP_QUAD_XOR2>(v, i, s);
  argmax_step<DPP_HALF_MIRROR>(v, i, s);
  argmax_step<DPP_MIRROR>(v, i, s);
  float bv = lane_f(v, 0);
  int bi = __builtin_amdgcn_readlane(i, 0), bs = __builtin_amdgcn_readlane(s, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float rv = lane_f(v, 16 * r);
    const int ri = __builtin_amdgcn_readlane(i, 16 * r), rs = __builtin_amdgcn_readlane(s, 16 * r);
    if (argmax_better(rv, ri, rs, bv, bi, bs)) { bv = rv; bi = ri; bs = rs; }
  }
  v = bv;
  i = bi;
  s = bs;
}

// Total order of floats as unsigned keys (ascending float -> ascending key).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// (value desc, id asc) as one 64-bit key, larger = better: candidates then
// compare with one 64-bit comparison, and a wave-wide maximum takes four DPP
// steps on the two halves.
__device__ __forceinline__ uint64_t vid_key(float v, int id) {
  return ((uint64_t)float_key(v) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)id);
}
// key 0 is below every real key (no candidate): value -inf, id 0x7fffffff
__device__ __forceinline__ float vid_value(uint64_t k) {
  return k ? key_float((uint32_t)(k >> 32)) : -INFINITY;
}
__device__ __forceinline__ int vid_id(uint64_t k) {
  return k ? (int)(0xFFFFFFFFu - (uint32_t)k) : 0x7fffffff;
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
  const uint32_t lo = (uint32_t)dpp_i<CTRL>((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)dpp_i<CTRL>((int)(uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t lane_u64(uint64_t x, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  uint64_t o;
  o = dpp_u64<DPP_QUAD_XOR1>(x); x = o > x ? o : x;
  o = dpp_u64<DPP_QUAD_XOR2>(x); x = o > x ? o : x;
  o = dpp_u64<DPP_HALF_MIRROR>(x); x = o > x ? o : x;
  o = dpp_u64<DPP_MIRROR>(x); x = o > x ? o : x;
  const uint64_t a = lane_u64(x, 0), b = lane_u64(x, 16), c = lane_u64(x, 32), d = lane_u64(x, 48);
  const uint64_t ab = a > b ? a : b, cd = c > d ? c : d;
  return ab > cd ? ab : cd;
}
