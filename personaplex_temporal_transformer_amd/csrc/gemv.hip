// GEMV launch by prologue/epilogue kind; the kernels live in gemv_kernel.h and are
// instantiated one kind per source file (gemv_<kind>.hip).
#include "internal.h"

namespace pp {

// Explicitly instantiated, one kind per gemv_<kind>.hip.
template <int PRO, int EPI>
hipError_t launch_gemv_kind(int rb, bool bf16, const GemvArgs& a, int blocks, hipStream_t s);

hipError_t launch_gemv(int pro, int epi, bool bf16, int rows_per_group, const GemvArgs& a,
                       int blocks, hipStream_t s) {
  if (a.n_groups <= 0) return hipSuccess;
  if (blocks <= 0 || blocks > a.n_groups) blocks = a.n_groups;
  const int rb = rows_per_group;
  if (pro == PRO_RMSNORM && epi == EPI_QKV) return launch_gemv_kind<PRO_RMSNORM, EPI_QKV>(rb, bf16, a, blocks, s);
  if (pro == PRO_COPY && epi == EPI_RESID) return launch_gemv_kind<PRO_COPY, EPI_RESID>(rb, bf16, a, blocks, s);
  if (pro == PRO_RMSNORM && epi == EPI_SWIGLU) return launch_gemv_kind<PRO_RMSNORM, EPI_SWIGLU>(rb, bf16, a, blocks, s);
  if (pro == PRO_RMSNORM && epi == EPI_STORE) return launch_gemv_kind<PRO_RMSNORM, EPI_STORE>(rb, bf16, a, blocks, s);
  if (pro == PRO_COPY && epi == EPI_STORE) return launch_gemv_kind<PRO_COPY, EPI_STORE>(rb, bf16, a, blocks, s);
  if (pro == PRO_RMSNORM && epi == EPI_DEPTH_QKV) return launch_gemv_kind<PRO_RMSNORM, EPI_DEPTH_QKV>(rb, bf16, a, blocks, s);
  if (pro == PRO_DEPTH_ATTN && epi == EPI_RESID) return launch_gemv_kind<PRO_DEPTH_ATTN, EPI_RESID>(rb, bf16, a, blocks, s);
  if (pro == PRO_ATTN_MERGE && epi == EPI_RESID) return launch_gemv_kind<PRO_ATTN_MERGE, EPI_RESID>(rb, bf16, a, blocks, s);
  if (pro == PRO_LAYERNORM && epi == EPI_STORE) return launch_gemv_kind<PRO_LAYERNORM, EPI_STORE>(rb, bf16, a, blocks, s);
  return hipErrorInvalidValue;
}

}  // namespace pp
