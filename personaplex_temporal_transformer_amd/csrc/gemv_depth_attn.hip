// GEMV instantiation: PRO_DEPTH_ATTN prologue, EPI_RESID epilogue.
#include "gemv_kernel.h"

namespace pp {
template hipError_t launch_gemv_kind<PRO_DEPTH_ATTN, EPI_RESID>(int, bool, const GemvArgs&, int, hipStream_t);
}  // namespace pp
