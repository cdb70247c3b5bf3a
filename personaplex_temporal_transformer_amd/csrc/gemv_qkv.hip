// GEMV instantiation: PRO_RMSNORM prologue, EPI_QKV epilogue.
#include "gemv_kernel.h"

namespace pp {
template hipError_t launch_gemv_kind<PRO_RMSNORM, EPI_QKV>(int, bool, const GemvArgs&, int, hipStream_t);
}  // namespace pp
