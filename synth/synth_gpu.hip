// Device-side twin of synth.c: fills a device buffer with the same seeded
// values, bit for bit (integer hashing plus one correctly rounded fp64
// multiply and one round-to-nearest conversion). Input generation only; it
// lets the harness materialise multi-GB synthetic weights directly in HBM.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

__host__ __device__ static inline uint64_t mix(uint64_t x) {
  uint64_t z = x + GOLDEN;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

__device__ static inline uint32_t lanesum(uint64_t h) {
  return (uint32_t)(h & 0xFFFF) + (uint32_t)((h >> 16) & 0xFFFF) +
         (uint32_t)((h >> 32) & 0xFFFF) + (uint32_t)(h >> 48);
}

__device__ static inline float elem(uint64_t key, uint64_t i) {
  const double C = 0x1.91530bd7c536ep-22;  // 0.02*sqrt(1.5)/65536
  uint32_t s = lanesum(mix(key + 2 * i)) + lanesum(mix(key + 2 * i + 1));
  return (float)((double)((int64_t)s - 262140) * C);
}

__global__ void fill_f32(uint64_t key, uint64_t offset, uint64_t n, float* out) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = elem(key, offset + i);
}

__global__ void fill_bf16(uint64_t key, uint64_t offset, uint64_t n, uint16_t* out) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    float f = elem(key, offset + i);
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    out[i] = (uint16_t)(u >> 16);
  }
}

__global__ void fill_const_f32(uint64_t n, float v, float* out) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = v;
}

extern "C" {
// dtype 0 = fp32, 1 = bf16. Returns a hipError_t value (0 = success).
int synth_gpu_fill(uint64_t seed, uint64_t stream_id, uint64_t offset, uint64_t n,
                   int dtype, void* dst, void* stream) {
  if (n == 0) return 0;
  if (dst == nullptr) return (int)hipErrorInvalidValue;
  uint64_t key = mix(seed ^ (stream_id * GOLDEN));
  int blocks = (int)((n + 255) / 256);
  if (blocks > 65536) blocks = 65536;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == 0)
    fill_f32<<<blocks, 256, 0, s>>>(key, offset, n, (float*)dst);
  else
    fill_bf16<<<blocks, 256, 0, s>>>(key, offset, n, (uint16_t*)dst);
  return (int)hipGetLastError();
}

int synth_gpu_fill_const_f32(uint64_t n, float v, void* dst, void* stream) {
  if (n == 0) return 0;
  if (dst == nullptr) return (int)hipErrorInvalidValue;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 65536) blocks = 65536;
  fill_const_f32<<<blocks, 256, 0, (hipStream_t)stream>>>(n, v, (float*)dst);
  return (int)hipGetLastError();
}
}
