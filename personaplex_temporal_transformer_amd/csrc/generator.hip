// Generator frame kernels: the delayed-code ring around the temporal step and the depth
// loop, and the standalone row sampler.
//
// "PersonaPlex native LM audit", 'Generator delayed-code cache' and section 7 'One exact
// generator step': an integer ring of n_streams x C slots (C = maximum delay + 3) with a
// provided flag per entry. At cursor s, supplied codes of stream k go to slot
// (s + delay_k) mod C and are marked provided; the first call only fills slot 0 with the
// initial tokens (where nothing was supplied); later calls read the temporal input from
// slot (s-1) mod C, select into slot s mod C (supplied entries win over samples), clear
// the consumed slot's flags and, once s exceeds the maximum delay, emit stream k from
// slot (s - max_delay + delay_k) mod C.
//
// One thread per stream in the ring kernels: each stream's ring row is touched by its
// own thread only, so they need no synchronisation.
#include "device.h"
#include "internal.h"
#include "sample.h"

namespace pp {

__global__ __launch_bounds__(64) void k_gen_prepare(GenPrepArgs a) {
  const int k = threadIdx.x;
  if (k >= a.n) return;
  GenState* g = a.g;
  if (a.provided[k] >= 0) {
    const int slot = (int)((a.s + a.delays[k]) % a.C);
    g->tok[k][slot] = a.provided[k];
    g->prov[k][slot] = 1;
  }
  if (a.s == 0) {
    if (!g->prov[k][0]) g->tok[k][0] = a.initial[k];
    return;
  }
  const int src = (int)((a.s - 1) % a.C), tgt = (int)(a.s % a.C);
  g->ids[k] = g->tok[k][src];
  const int sup = g->prov[k][tgt] ? g->tok[k][tgt] : -1;
  if (k == 0) {
    g->text_forced = sup;
    g->u_text = a.u[0];
    a.dctrl->temperature = a.audio_temperature;
    a.dctrl->top_k = a.audio_top_k;
  } else {
    a.dctrl->forced[k - 1] = sup;
    a.dctrl->u[k - 1] = a.u[k];
  }
}

hipError_t launch_gen_prepare(const GenPrepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_gen_prepare, dim3(1), dim3(64), 0, s, a);
  return hipGetLastError();
}

// The frame's text selection: the supplied text of the target slot, else a draw from
// the text logits. It conditions depth position 0.
__global__ __launch_bounds__(kGenTextThreads) void k_gen_text(GenTextArgs a) {
  __shared__ SampleLds sl;
  GenState* g = a.g;
  const int sup = g->text_forced;
  int pick = sup;
  if (sup < 0) pick = block_sample_top_k<kGenTextThreads, kGenTextPer>(a.logits, a.n, a.temperature, a.top_k,
                                                                          g->u_text, sl);
  if (threadIdx.x == 0) {
    a.dctrl->text = pick;
    g->chosen[0] = pick;
  }
}

hipError_t launch_gen_text(const GenTextArgs& a, hipStream_t s) {
  if (a.n < 1 || a.n > kGenTextThreads * kGenTextPer) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_gen_text, dim3(1), dim3(kGenTextThreads), 0, s, a);
  return hipGetLastError();
}

__global__ __launch_bounds__(64) void k_gen_finish(GenFinishArgs a) {
  const int k = threadIdx.x;
  if (k >= a.n) return;
  GenState* g = a.g;
  const int src = (int)((a.s - 1) % a.C), tgt = (int)(a.s % a.C);
  const int c = k == 0 ? g->chosen[0] : a.codes[k - 1];
  g->chosen[k] = c;
  if (!g->prov[k][tgt]) g->tok[k][tgt] = c;
  g->prov[k][src] = 0;
  if (a.out && a.s > a.max_delay) a.out[k] = g->tok[k][(int)((a.s - a.max_delay + a.delays[k]) % a.C)];
}

hipError_t launch_gen_finish(const GenFinishArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_gen_finish, dim3(1), dim3(64), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- standalone sampler
template <int NT, int PER>
__global__ __launch_bounds__(NT) void k_sample_rows(const float* __restrict__ logits, int n, float temperature,
                                                    int top_k, const double* __restrict__ u, int32_t* out) {
  __shared__ SampleLds sl;
  const int r = blockIdx.x;
  const int pick = block_sample_top_k<NT, PER>(logits + (size_t)r * n, n, temperature, top_k, u ? u[r] : 0.0, sl);
  if (threadIdx.x == 0) out[r] = pick;
}

hipError_t launch_sample_rows(const float* logits, int rows, int n, float temperature, int top_k,
                              const double* u, int32_t* out, hipStream_t s) {
  if (rows < 1 || n < 1 || top_k > kMaxTopK) return hipErrorInvalidValue;
  if (n <= 256 * 8)
    hipLaunchKernelGGL((k_sample_rows<256, 8>), dim3(rows), dim3(256), 0, s, logits, n, temperature, top_k, u, out);
  else if (n <= 1024 * 8)
    hipLaunchKernelGGL((k_sample_rows<1024, 8>), dim3(rows), dim3(1024), 0, s, logits, n, temperature, top_k, u, out);
  else if (n <= 1024 * 32)
    hipLaunchKernelGGL((k_sample_rows<1024, 32>), dim3(rows), dim3(1024), 0, s, logits, n, temperature, top_k, u, out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pp
