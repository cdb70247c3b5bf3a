// GEMV instantiation: PRO_LAYERNORM prologue, EPI_STORE epilogue (memory-reader queries).
#include "gemv_kernel.h"

namespace pp {
template hipError_t launch_gemv_kind<PRO_LAYERNORM, EPI_STORE>(int, bool, const GemvArgs&, int, hipStream_t);
}  // namespace pp
