// Depth-loop glue kernels: per-call setup and per-position code selection + input.
//
// "PersonaPlex native LM audit", section 4: position q's input is the temporal-to-depth
// projection of h plus an embedding -- the depth text table at the selected text token
// for q = 0, otherwise table q-1 at the code selected for position q-1. The code of a
// position is the supplied one where provided, else the model's choice: the argmax of
// that position's logits (lowest index on ties), or -- for the generator, section 7 'One
// exact generator step' -- a temperature / top-k draw with that position's uniform.
#include "device.h"
#include "internal.h"
#include "sample.h"

namespace pp {

__global__ __launch_bounds__(kBlock) void k_depth_setup(DepthSetupArgs a) {
  for (int i = threadIdx.x; i < a.d_temporal; i += kBlock) a.h_dst[i] = a.h_src[i];
  if (threadIdx.x == 0) {
    a.ctrl->text = a.text_token;
    a.ctrl->temperature = 0.f;
    a.ctrl->top_k = 1;
  }
  if (threadIdx.x < a.n_steps) {
    a.ctrl->forced[threadIdx.x] = a.forced[threadIdx.x];
    a.ctrl->u[threadIdx.x] = 0.0;
  }
}

hipError_t launch_depth_setup(const DepthSetupArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_depth_setup, dim3(1), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

// One block. For q > 0 it fixes the code of position q-1; for q < n_steps it forms z.
// The reads that do not depend on the selection -- the logits row (kSelPer values per
// thread cover up to 2048 logits) and this position's projection row (kZPer values per
// thread, d_model up to 1024) -- are issued together first, unconditionally (clamped
// indices), so the greedy selection and z cost two memory round trips: logits, then the
// chosen embedding row. Longer rows take loops.
constexpr int kSelPer = 8, kZPer = 4;

// (value, index) of the larger value, the lower index on equal values
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

template <typename WT>
__global__ __launch_bounds__(kBlock) void k_depth_select(DepthSelectArgs a) {
  __shared__ float bv[kBlock / 64];
  __shared__ int bi[kBlock / 64];
  __shared__ SampleLds sl;
  __shared__ int code_s;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const bool sel = a.q > 0, fits = a.n_out <= kSelPer * kBlock;
  const float* lg = a.logits + (size_t)(sel ? a.q - 1 : 0) * a.n_out;
  float lv[kSelPer];
#pragma unroll
  for (int j = 0; j < kSelPer; ++j) {
    const int i = j * kBlock + tid;
    lv[j] = lg[i < a.n_out ? i : a.n_out - 1];
  }
  const bool zrow = a.q < a.n_steps, zfits = a.D <= kZPer * kBlock;
  const float* c = a.c_all + (size_t)(zrow ? a.q : 0) * a.D;
  float cv[kZPer];
#pragma unroll
  for (int j = 0; j < kZPer; ++j) {
    const int d = j * kBlock + tid;
    cv[j] = c[d < a.D ? d : a.D - 1];
  }
  if (sel) {
    const DepthCtrl* ct = a.ctrl;
    const int forced = ct->forced[a.q - 1];
    if (forced >= 0) {
      if (tid == 0) code_s = forced;
    } else if (ct->top_k > 1 && ct->temperature > 0.f) {
      const int pick = block_sample_top_k<kBlock, kDepthSampleMaxOut / kBlock>(lg, a.n_out, ct->temperature,
                                                                             ct->top_k, ct->u[a.q - 1], sl);
      if (tid == 0) code_s = pick;
    } else {
      // greedy: each thread's first maximum in index order, then the block's (lowest index
      // among equal maxima; a row with no value above -inf selects 0)
      float best = -INFINITY;
      int idx = 0x7fffffff;
      if (fits) {
#pragma unroll
        for (int j = 0; j < kSelPer; ++j) {
          const int i = j * kBlock + tid;
          if (i < a.n_out && lv[j] > best) { best = lv[j]; idx = i; }
        }
      } else {
        for (int i = tid; i < a.n_out; i += kBlock) {
          const float v = lg[i];
          if (v > best) { best = v; idx = i; }
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) argmax_merge(best, idx, __shfl_xor(best, o), __shfl_xor(idx, o));
      if (lane == 0) { bv[wid] = best; bi[wid] = idx; }
      __syncthreads();
      if (tid == 0) {
        float v = bv[0];
        int i = bi[0];
        for (int w = 1; w < kBlock / 64; ++w) argmax_merge(v, i, bv[w], bi[w]);
        code_s = i == 0x7fffffff ? 0 : i;
      }
    }
    __syncthreads();
    if (tid == 0) a.codes[a.q - 1] = code_s;
  }
  if (!zrow) return;
  const WT* e = a.q == 0 ? static_cast<const WT*>(a.text_emb) + (size_t)a.ctrl->text * a.D
                         : static_cast<const WT*>(a.audio_emb[a.q - 1]) + (size_t)code_s * a.D;
  if (zfits) {
    float ev[kZPer];
#pragma unroll
    for (int j = 0; j < kZPer; ++j) {
      const int d = j * kBlock + tid;
      ev[j] = Elem<WT>::load1(e + (d < a.D ? d : a.D - 1));
    }
#pragma unroll
    for (int j = 0; j < kZPer; ++j) {
      const int d = j * kBlock + tid;
      if (d < a.D) a.z[d] = cv[j] + ev[j];
    }
  } else {
    for (int d = tid; d < a.D; d += kBlock) a.z[d] = c[d] + Elem<WT>::load1(e + d);
  }
}

hipError_t launch_depth_select(const DepthSelectArgs& a, bool bf16, hipStream_t s) {
  if (bf16) hipLaunchKernelGGL(k_depth_select<bf16_t>, dim3(1), dim3(kBlock), 0, s, a);
  else hipLaunchKernelGGL(k_depth_select<float>, dim3(1), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace pp
