// Depth transformer ("depformer") host side.
#include <hip/hip_runtime.h>

#include "model.h"
#include "pp.h"

extern "C" pp_status pp_depformer_create(const pp_depth_config* cfg, const pp_depth_weights* w,
                                         pp_depformer** out) {
  (void)cfg; (void)w;
  if (out) *out = nullptr;
  return pp_fail(PP_E_ARG, "depformer is not available in this build");
}
extern "C" pp_status pp_depformer_destroy(pp_depformer* d) {
  (void)d;
  return pp_fail(PP_E_ARG, "depformer is not available in this build");
}
extern "C" pp_status pp_depformer_step(pp_depformer* d, const float* h_dev, const int32_t* text_token_host,
                                       const int32_t* forced_host, int32_t batch, int32_t* codes_dev,
                                       float* logits_dev, void* stream) {
  (void)d; (void)h_dev; (void)text_token_host; (void)forced_host; (void)batch; (void)codes_dev;
  (void)logits_dev; (void)stream;
  return pp_fail(PP_E_ARG, "depformer is not available in this build");
}
