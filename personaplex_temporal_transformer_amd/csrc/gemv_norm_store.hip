// GEMV instantiation: PRO_RMSNORM prologue, EPI_STORE epilogue.
#include "gemv_kernel.h"

namespace pp {
template hipError_t launch_gemv_kind<PRO_RMSNORM, EPI_STORE>(int, bool, const GemvArgs&, int, hipStream_t);
}  // namespace pp
