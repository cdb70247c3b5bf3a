// Device helpers shared by the libpp kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pp {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// 8 bfloat16 values (one 16-byte chunk) as float16: each bfloat16 is the top half of a
// float32; the packed conversion is exact for values inside float16's normal range
// (bfloat16 has the shorter significand).
__device__ __forceinline__ f16x8 bf16x8_to_f16(u32x4 w) {
  f16x8 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const auto p = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w[k] << 16), __uint_as_float(w[k] & 0xffff0000u));
    r[2 * k] = (_Float16)p[0];
    r[2 * k + 1] = (_Float16)p[1];
  }
  return r;
}

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

// float32 -> float16 bits, round to nearest even (the hardware conversion).
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// float32 -> float16 bits, round to nearest even, saturated to +-65504.
__device__ __forceinline__ uint16_t f32_to_f16_sat(float f) {
  return f32_to_f16(fminf(fmaxf(f, -65504.f), 65504.f));
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

// Buffer loads: a resource over [base, base + bytes) makes lanes whose offset is out of
// range read zeros without touching memory, so range guards need no branches (loads
// stay straight-line and the compiler's waits stay precise).
constexpr int kBufOutOfRange = 0x7ffffff0;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load16_stream(__amdgpu_buffer_rsrc_t r, int byte_offset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, 2 /* non-temporal */);
}

// 16 bytes per lane from a buffer into LDS: lane i's bytes land at LDS byte address
// lds_base + 16*i (lds_base is wave-uniform, passed through M0). Issued from inline
// assembly so that the compiler does not add a wait on these loads before every LDS read
// (it cannot tell the pipeline stages apart); the kernel waits for them explicitly with
// an explicit s_waitcnt. No other instruction in these kernels uses M0.
__device__ __forceinline__ void lds_dma16(u32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_base) : "memory");
}

// Buffer resource words for [base, base + bytes): raw addressing, no stride, reads past
// the end return zero.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

// LDS byte address of a __shared__ object (the low half of its generic address).
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// DPP lane moves inside a row of 16 lanes (no LDS traffic).
__device__ __forceinline__ float dpp_xor1(float v) {  // quad_perm [1,0,3,2]
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float v) {  // quad_perm [2,3,0,1]
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_half_mirror(float v) {  // lane i <-> 7 - i within 8
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_mirror(float v) {  // lane i <-> 15 - i within 16
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
}

// Sum over aligned groups of W lanes (W = 8, 16, 32 or 64); every lane of a group gets
// the same bits: each step adds two partial sums that are already equal across the lanes
// involved, and float addition is commutative. The order is fixed, so results are
// reproducible run to run.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(W == 8 || W == 16 || W == 32 || W == 64, "group width");
  v += dpp_xor1(v);
  v += dpp_xor2(v);
  v += dpp_half_mirror(v);
  if (W >= 16) v += dpp_mirror(v);
  if (W >= 32) v += __shfl_xor(v, 16, kWave);
  if (W >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}
__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Workgroup barrier for LDS communication only: waits for this wave's LDS operations,
// not for its outstanding global loads (a full __syncthreads() also drains the global
// load counter, which would stall prefetched weight streams). The memory clobber keeps
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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

// 2^x with the hardware exponential (exp2(-inf) = 0); used where x <= 0 (softmax weights).
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pp
