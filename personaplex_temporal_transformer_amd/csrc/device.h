// Device helpers shared by the libpp kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pp {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

struct bf16_t {
  uint16_t bits;
};

// bfloat16 -> float32 is exact: the bfloat16 bits are the upper half of the float.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float32 -> bfloat16, round to nearest, ties to even (values here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Storage-type helpers for weights / cache elements (float or bfloat16).
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPerChunk = 4;  // elements per 16-byte chunk
  __device__ static __forceinline__ void widen(u32x4 c, float* out) {
    out[0] = __uint_as_float(c.x); out[1] = __uint_as_float(c.y);
    out[2] = __uint_as_float(c.z); out[3] = __uint_as_float(c.w);
  }
  __device__ static __forceinline__ float load1(const float* p) { return *p; }
  __device__ static __forceinline__ void store1(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kPerChunk = 8;
  __device__ static __forceinline__ void widen(u32x4 c, float* out) {
    out[0] = bf16_lo(c.x); out[1] = bf16_hi(c.x); out[2] = bf16_lo(c.y); out[3] = bf16_hi(c.y);
    out[4] = bf16_lo(c.z); out[5] = bf16_hi(c.z); out[6] = bf16_lo(c.w); out[7] = bf16_hi(c.w);
  }
  __device__ static __forceinline__ float load1(const bf16_t* p) { return bf16_to_f32(p->bits); }
  __device__ static __forceinline__ void store1(bf16_t* p, float v) { p->bits = f32_to_bf16(v); }
};

// 16-byte streaming load (weights are read exactly once per step).
__device__ __forceinline__ u32x4 load_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Butterfly sum over the 64 lanes of a wave; every lane gets the total. The order of
// additions is fixed, so results are bit-reproducible.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}
// Sum over aligned groups of `width` lanes (width a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = W / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Block-wide sum for 256-thread blocks; `scratch` holds >= 4 floats of shared memory.
__device__ __forceinline__ float block_sum_256(float v, float* scratch) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) scratch[wid] = v;
  __syncthreads();
  return (scratch[0] + scratch[1]) + (scratch[2] + scratch[3]);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

}  // namespace pp
