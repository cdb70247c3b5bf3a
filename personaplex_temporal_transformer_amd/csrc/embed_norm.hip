// Embedding sum and row RMSNorm kernels.
//
// Embedding sum: "PersonaPlex native LM audit", section 3 'Input embedding sum' -- the
// frame's input is the plain sum of one row from each of the 17 stream tables (text,
// 8 agent audio, 8 user audio); ID -1 contributes an exact zero vector.
// RMSNorm: same page, section 3 'One of the 32 temporal blocks' -- float32 arithmetic,
// x * alpha / sqrt(mean(x^2) + eps), no mean subtraction.
#include <cmath>

#include "device.h"
#include "frag_layout.h"
#include "internal.h"

namespace pp {

// One thread owns one 16-byte chunk of the output row's table rows (8 bfloat16 or 4
// float32 features) of one frame; blocks of 64 threads, so a decode frame spreads over
// D / 512 (bfloat16) workgroups. It loads the chunk of every stream's row first (all in
// flight together), then adds them in stream order 0..n-1 in float32 -- a fixed order,
// so the result is reproducible. An ID of -1 leaves the running sum untouched.
constexpr int kEmbedThreads = 64;

// NSLOT table slots are read (17 for the model's text + 16 audio streams, else kMaxStreams).
template <typename WT, bool DEVIDS, int NSLOT>
__global__ __launch_bounds__(kEmbedThreads) __attribute__((amdgpu_waves_per_eu(1, 4)))
void k_embed_sum(EmbedArgs a) {
  constexpr int EPC = Elem<WT>::kPerChunk;
  const int row = blockIdx.y;
  const int d = (blockIdx.x * kEmbedThreads + threadIdx.x) * EPC;
  if (a.state && row == 0 && blockIdx.x == 0) {
    if (threadIdx.x == 0) a.state[0] = a.pos;
    for (int i = threadIdx.x; a.rope && i < a.dh; i += kEmbedThreads) a.rope[i] = a.rope_cs[i];
  }
  if (d >= a.D) return;
  // Every row load is issued before the first is used, with no branch around any of them
  // (a load under a branch makes the compiler wait for all earlier loads, which turned the
  // 17 row reads into 17 memory round trips). The host fills the slots past n_streams with
  // the text table and ID -1; every slot past n_streams, and every ID -1, reads row 0 of its
  // table and is dropped by a select, so a dropped term adds nothing (not even 0 * inf).
  const int n = a.n_streams;
  u32x4 raw[NSLOT];
  bool keep[NSLOT];
#pragma unroll
  for (int k = 0; k < NSLOT; ++k) {
    const int id = DEVIDS ? a.ids_dev[(size_t)row * n + (k < n ? k : n - 1)] : a.ids_arg[k];
    raw[k] = load16(static_cast<const WT*>(a.tables[k]) + (size_t)((k < n && id > 0) ? id : 0) * a.D + d);
    keep[k] = (!DEVIDS || k < n) && id >= 0;
  }
  // keeps the scheduler from pulling each sum step up behind its own load
  __builtin_amdgcn_sched_barrier(0);
  float acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
#pragma unroll
  for (int k = 0; k < NSLOT; ++k) {
    float v[EPC];
    Elem<WT>::widen(raw[k], v);
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = keep[k] ? acc[e] + v[e] : acc[e];
  }
  float* o = a.out + (size_t)row * a.D + d;
#pragma unroll
  for (int e = 0; e < EPC; e += 4) *reinterpret_cast<f32x4*>(o + e) = f32x4{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
}

hipError_t launch_embed(const EmbedArgs& a, bool bf16, hipStream_t s) {
  const int epc = bf16 ? 8 : 4;
  if (a.D % epc) return hipErrorInvalidValue;
  dim3 grid((a.D / epc + kEmbedThreads - 1) / kEmbedThreads, a.rows);
  if (a.n_streams < 1 || a.n_streams > kMaxStreams) return hipErrorInvalidValue;
  const auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(kEmbedThreads), 0, s, a); };
  constexpr int kModelStreams = 17;
  const bool few = a.n_streams <= kModelStreams;
  if (bf16 && a.ids_dev) few ? go(k_embed_sum<bf16_t, true, kModelStreams>) : go(k_embed_sum<bf16_t, true, kMaxStreams>);
  else if (bf16) few ? go(k_embed_sum<bf16_t, false, kModelStreams>) : go(k_embed_sum<bf16_t, false, kMaxStreams>);
  else if (a.ids_dev) few ? go(k_embed_sum<float, true, kModelStreams>) : go(k_embed_sum<float, true, kMaxStreams>);
  else few ? go(k_embed_sum<float, false, kModelStreams>) : go(k_embed_sum<float, false, kMaxStreams>);
  return hipGetLastError();
}

// One block per row; float32 statistics; writes float32 and/or float16 output (the
// float16 rows are the activation operand of the prefill's matrix products, row-major, or
// with f16_frag set of the batched decode's skinny products, in their fragment order).
__global__ __launch_bounds__(kBlock) void k_rmsnorm_rows(const float* __restrict__ x,
                                                         const float* __restrict__ alpha, float eps,
                                                         int D, float* __restrict__ out_f32,
                                                         uint16_t* __restrict__ out_f16, int f16_frag, float f16_scale) {
  __shared__ float red[4];
  const float* xr = x + (size_t)blockIdx.x * D;
  auto emit = [&](int i, f32x4 y) {
    if (out_f32) *reinterpret_cast<f32x4*>(out_f32 + (size_t)blockIdx.x * D + i) = y;
    if (out_f16) {
      const f32x4 z = y * f16_scale;   // a power of two: the float16 operand's scale
      const uint32_t lo = (uint32_t)f32_to_f16(z.x) | ((uint32_t)f32_to_f16(z.y) << 16);
      const uint32_t hi = (uint32_t)f32_to_f16(z.z) | ((uint32_t)f32_to_f16(z.w) << 16);
      // four consecutive k (i % 4 == 0) stay within one 8-value fragment run
      const size_t oi = f16_frag ? frag_act_index((int)blockIdx.x, i, D) : (size_t)blockIdx.x * D + i;
      *reinterpret_cast<uint2*>(out_f16 + oi) = make_uint2(lo, hi);
    }
  };
  // Rows of up to kBlock * 16 values stay in registers between the sum of squares and the
  // scaling, with the scales loaded alongside (one memory round trip instead of two); the
  // per-thread sums run over the same elements in the same order either way.
  constexpr int NV = 4;
  float ss = 0.f;
  if (D <= kBlock * 4 * NV) {
    f32x4 v[NV], al[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int i = (threadIdx.x + j * kBlock) * 4;
      v[j] = i < D ? *reinterpret_cast<const f32x4*>(xr + i) : f32x4{0.f, 0.f, 0.f, 0.f};
      al[j] = i < D ? *reinterpret_cast<const f32x4*>(alpha + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if ((threadIdx.x + j * kBlock) * 4 < D) ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
    const float r = 1.0f / sqrtf(block_sum_256(ss, red) / (float)D + eps);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int i = (threadIdx.x + j * kBlock) * 4;
      if (i < D) emit(i, (v[j] * r) * al[j]);
    }
    return;
  }
  for (int i = threadIdx.x * 4; i < D; i += kBlock * 4) {
    f32x4 v = *reinterpret_cast<const f32x4*>(xr + i);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  const float r = 1.0f / sqrtf(block_sum_256(ss, red) / (float)D + eps);
  for (int i = threadIdx.x * 4; i < D; i += kBlock * 4) {
    f32x4 v = *reinterpret_cast<const f32x4*>(xr + i);
    f32x4 al = *reinterpret_cast<const f32x4*>(alpha + i);
    emit(i, (v * r) * al);
  }
}

hipError_t launch_rmsnorm_rows(const float* x, const float* alpha, float eps, int D, int rows,
                               float* out_f32, void* out_f16, bool f16_frag, hipStream_t s, int f16_exp) {
  if (f16_frag && D % 32) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_rmsnorm_rows, dim3(rows), dim3(kBlock), 0, s, x, alpha, eps, D, out_f32,
                     static_cast<uint16_t*>(out_f16), f16_frag ? 1 : 0, std::ldexp(1.0f, -f16_exp));
  return hipGetLastError();
}

}  // namespace pp
