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
template <typename WT>
__global__ __launch_bounds__(kBlock) void k_depth_select(DepthSelectArgs a) {
  __shared__ float bv[kBlock];
  __shared__ int bi[kBlock];
  __shared__ SampleLds sl;
  __shared__ int code_s;
  const int tid = threadIdx.x;
  if (a.q > 0) {
    const DepthCtrl* c = a.ctrl;
    const int forced = c->forced[a.q - 1];
    const float* lg = a.logits + (size_t)(a.q - 1) * a.n_out;
    if (forced >= 0) {
      if (tid == 0) code_s = forced;
    } else if (c->top_k > 1 && c->temperature > 0.f) {
      const int pick = block_sample_top_k<kBlock, kDepthSampleMaxOut / kBlock>(lg, a.n_out, c->temperature,
                                                                             c->top_k, c->u[a.q - 1], sl);
      if (tid == 0) code_s = pick;
    } else {
      float best = -INFINITY;
      int idx = 0x7fffffff;
      for (int i = tid; i < a.n_out; i += kBlock) {
        const float v = lg[i];
        if (v > best) { best = v; idx = i; }   // strict: the first maximum in this thread's order
      }
      bv[tid] = best;
      bi[tid] = idx;
      __syncthreads();
      for (int w = kBlock / 2; w > 0; w >>= 1) {
        if (tid < w) {
          const float v2 = bv[tid + w];
          const int i2 = bi[tid + w];
          if (v2 > bv[tid] || (v2 == bv[tid] && i2 < bi[tid])) { bv[tid] = v2; bi[tid] = i2; }
        }
        __syncthreads();
      }
      if (tid == 0) code_s = bi[0] == 0x7fffffff ? 0 : bi[0];
    }
    __syncthreads();
    if (tid == 0) a.codes[a.q - 1] = code_s;
  }
  if (a.q >= a.n_steps) return;
  const WT* e = a.q == 0 ? static_cast<const WT*>(a.text_emb) + (size_t)a.ctrl->text * a.D
                         : static_cast<const WT*>(a.audio_emb[a.q - 1]) + (size_t)code_s * a.D;
  const float* c = a.c_all + (size_t)a.q * a.D;
  for (int d = tid; d < a.D; d += kBlock) a.z[d] = c[d] + Elem<WT>::load1(e + d);
}

hipError_t launch_depth_select(const DepthSelectArgs& a, bool bf16, hipStream_t s) {
  if (bf16) hipLaunchKernelGGL(k_depth_select<bf16_t>, dim3(1), dim3(kBlock), 0, s, a);
  else hipLaunchKernelGGL(k_depth_select<float>, dim3(1), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace pp
