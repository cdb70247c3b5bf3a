// GEMV instantiation: PRO_ATTN_MERGE prologue, EPI_RESID epilogue.
#include "gemv_kernel.h"

namespace pp {
template hipError_t launch_gemv_kind<PRO_ATTN_MERGE, EPI_RESID>(int, bool, const GemvArgs&, int, hipStream_t);
}  // namespace pp
