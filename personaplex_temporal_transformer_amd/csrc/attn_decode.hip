// Decode attention over the temporal ring: one query per head against every visible key.
//
// "PersonaPlex native LM audit", section 3: ordinary multi-head attention (32 query, key
// and value heads of 128), scale 1/sqrt(d_head), softmax, no dropout; the declared mask
// admits keys with 0 <= query_pos - key_pos < context. Keys in the ring were rotated at
// their own positions when written, so nothing is rotated here. With the frame at
// position p written into slot p mod C first, the visible keys are exactly the slots
// 0 .. min(p+1, C)-1 (softmax does not depend on the order of keys).
//
// Split-K over keys: block (s, h) handles an equal share of head h's keys, so H x S
// blocks stream the K and V bytes once, 16 bytes per lane, and each forms a float32
// partial (o, max, sum). Scores are carried in base-2 units (q is pre-scaled by
// log2(e) / sqrt(d_head)), so every exponential is one exp2 and the partial max is in
// those units: softmax weights 2^(s - m) equal e^(s' - m') for the natural-unit scores.
// The S partials of a head are merged in split order -- a fixed order, so results are
// bit-reproducible -- in the W_O GEMV's prologue, or by a small combine kernel for more
// than 8 splits and for batched steps. A batched step with one split per head writes its
// float16 output from the attention blocks themselves.
#include "attn_body.h"
#include "frag_layout.h"

namespace pp {

// Block (s, h) of the split-K decode attention (see attn_body.h).
template <typename KT, int DH, int NB, int NT>
__global__ __launch_bounds__(NT) void k_attn_decode(AttnDecodeArgs a) {
  if (blockIdx.z > 0) {  // session b of a batched step
    const size_t b = blockIdx.z;
    a.q += b * a.H * DH;
    a.k = static_cast<const KT*>(a.k) + b * a.kv_bstride;
    a.v = static_cast<const KT*>(a.v) + b * a.kv_bstride;
    a.part_o += b * a.H * a.S * DH;
    a.part_ml += b * a.H * a.S * 2;
  }
  attn_body<KT, DH, NB, NT>(a, blockIdx.x, blockIdx.y, (int)blockIdx.z);
}

// Merge the S partials (o_s, m_s, l_s) of head h in split order:
// o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s with M = max_s m_s (base-2 units).
// All partials of the head are first loaded into LDS in one parallel round.
template <int DH>
__global__ __launch_bounds__(kBlock) void k_attn_combine(AttnDecodeArgs a) {
  __shared__ float po[kMaxAttnSplits * DH], pml[kMaxAttnSplits * 2];
  const int h = blockIdx.x, t = threadIdx.x;
  const size_t b = blockIdx.y;   // session (batched step)
  const float* part_o = a.part_o + b * a.H * a.S * DH;
  const float* part_ml = a.part_ml + b * a.H * a.S * 2;
  for (int i = t; i < a.S * DH; i += kBlock) po[i] = part_o[(size_t)h * a.S * DH + i];
  for (int i = t; i < a.S * 2; i += kBlock) pml[i] = part_ml[(size_t)h * a.S * 2 + i];
  __syncthreads();
  if (t >= DH) return;
  float M = -INFINITY;
  for (int i = 0; i < a.S; ++i) M = fmaxf(M, pml[2 * i]);
  float L = 0.f, o = 0.f;
  for (int i = 0; i < a.S; ++i) {
    const float mi = pml[2 * i];
    if (mi == -INFINITY) continue;  // empty split
    const float w = exp2_fast(mi - M);
    L += w * pml[2 * i + 1];
    o += w * po[i * DH + t];
  }
  if (a.out16) a.out16[frag_act_index((int)b, h * DH + t, a.H * DH)] = f32_to_f16_sat(o / L * ldexpf(1.0f, -a.o16_exp));
  else a.out[b * a.H * DH + h * DH + t] = o / L;
}

hipError_t launch_attn_decode(const AttnDecodeArgs& a, bool bf16, int dh, hipStream_t s) {
  const int nb = a.batch > 1 ? a.batch : 1;
  if (a.S < 1 || a.S > kMaxAttnSplits) return hipErrorInvalidValue;
  const dim3 grid(a.S, a.H, nb);
  if (bf16 && dh == 128) hipLaunchKernelGGL((k_attn_decode<bf16_t, 128, 6, 512>), grid, dim3(512), 0, s, a);
  else if (bf16 && dh == 64) hipLaunchKernelGGL((k_attn_decode<bf16_t, 64, 6, 512>), grid, dim3(512), 0, s, a);
  else if (!bf16 && dh == 128) hipLaunchKernelGGL((k_attn_decode<float, 128, 6, 512>), grid, dim3(512), 0, s, a);
  else if (!bf16 && dh == 64) hipLaunchKernelGGL((k_attn_decode<float, 64, 6, 512>), grid, dim3(512), 0, s, a);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.combine || (a.S == 1 && a.out16)) return e;   // one split: written directly
  if (dh == 128) hipLaunchKernelGGL((k_attn_combine<128>), dim3(a.H, nb), dim3(kBlock), 0, s, a);
  else hipLaunchKernelGGL((k_attn_combine<64>), dim3(a.H, nb), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace pp
