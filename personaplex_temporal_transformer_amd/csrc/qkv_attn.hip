// Fused decode kernel: RMSNorm + QKV + RoPE + ring append, then split-K attention.
//
// "PersonaPlex native LM audit", section 3 ('One of the 32 temporal blocks'): the first
// half of a block, u = RMSNorm(x), [q, k, v] = W_QKV u, RoPE on q and k, k and v into the
// ring slot of the frame, then attention of q over the visible keys. Attention of head h
// needs only head h's q, k and v rows, so it does not need the whole QKV product: each
// workgroup first computes its share of the QKV rows (published with agent-scope stores)
// and adds the number of rows it wrote for each head to that head's counter; it then
// issues the ring loads of its attention split (head blockIdx / S, split blockIdx % S)
// and waits only for its own head's counter. One launch instead of two: the attention's
// ring streaming starts while other workgroups are still finishing their QKV rows.
//
// Requirements (checked on the host): bfloat16 weights, d_model 4096 (eight 16-byte
// chunks per lane), d_head 128, at most 8 splits (merged in the W_O prologue), grid =
// H * S workgroups, one per CU at most, so that every workgroup is resident while others
// wait for it.
#include "attn_body.h"
#include "gemv_kernel.h"

namespace pp {

template <int NB>
__global__ __launch_bounds__(kGemvWaves * 64) void k_qkv_attn(GemvArgs g, AttnDecodeArgs at, QkvAttnFuse f) {
  extern __shared__ float xs[];
  gemv_body<bf16_t, 2, 8, true, PRO_RMSNORM, EPI_QKV, false, true, 2, true>(g, xs, blockIdx.x, gridDim.x);
  // every wave's stores have completed before the block's rows are counted
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int r0 = 2 * (int)((long long)blockIdx.x * g.n_groups / gridDim.x);
    const int r1 = 2 * (int)((long long)(blockIdx.x + 1) * g.n_groups / gridDim.x);
    for (int r = r0; r < r1;) {
      const int w = r % g.D, head = w / g.dh;
      const int e = r - w % g.dh + g.dh < r1 ? r - w % g.dh + g.dh : r1;  // end of this head's run
      __hip_atomic_fetch_add(f.cnt + head, (unsigned long long)(e - r), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      r = e;
    }
  }
  const long long seq = f.seq >= 0 ? f.seq : g.state[1];
  const AttnFuse af{f.cnt, (unsigned long long)(3 * g.dh) * (unsigned long long)seq, f.err};
  attn_body<bf16_t, 128, NB, kGemvWaves * 64, true>(at, (int)blockIdx.x % at.S, (int)blockIdx.x / at.S, af);
}

bool qkv_attn_supported(bool bf16, int D, int dh, int H, int S, int n_cu) {
  return bf16 && D == 4096 && dh == 128 && S <= 8 && H * S <= n_cu && H * S <= 3 * D / 2;
}

hipError_t launch_qkv_attn(const GemvArgs& g, const AttnDecodeArgs& at, const QkvAttnFuse& f, hipStream_t s) {
  const int nb = at.H * at.S;
  if (g.n_groups != 3 * g.D / 2 || g.K != g.D || at.S < 1) return hipErrorInvalidValue;
  const size_t lds = (size_t)2 * kGemvWaves * 64 * 4 * sizeof(float);  // x staging, as gemv_body's XR = 2
  hipLaunchKernelGGL(k_qkv_attn<6>, dim3(nb), dim3(kGemvWaves * 64), lds, s, g, at, f);
  return hipGetLastError();
}

}  // namespace pp
