// Full-sequence (prefill) path of the temporal model: workspace and launch order.
#include <hip/hip_runtime.h>

#include <string>

#include "internal.h"
#include "model.h"
#include "pp.h"

using namespace pp;

pp_status pp_model::alloc_prefill() {
  const int T = max_T > 0 ? max_T : 0;
  const int ns = cfg.n_audio + 1;
  size_t bytes = 0;
  auto take = [&](size_t n) { size_t off = bytes; bytes += (n + 255) / 256 * 256; return off; };
  const size_t oid = take(sizeof(int32_t) * (size_t)(T > 0 ? T : 1) * ns);
  if (hipMalloc(&pws, bytes) != hipSuccess) return pp_fail(PP_E_HIP, "hipMalloc of prefill workspace failed");
  ids_dev = reinterpret_cast<int32_t*>(static_cast<char*>(pws) + oid);
  return PP_OK;
}

void pp_model::free_prefill() {
  if (pws) (void)hipFree(pws);
  pws = nullptr;
}

extern "C" pp_status pp_temporal_prefill(pp_model* m, pp_kv* kv, const int32_t* ids_host, int32_t T,
                                         float* h_out_dev, void* stream) {
  if (!m || !kv || !ids_host || !h_out_dev) return pp_fail(PP_E_ARG, "NULL argument");
  (void)T;
  (void)stream;
  return pp_fail(PP_E_ARG, "prefill is not available in this build");
}
