// Generator frame host side: validation, device state and the launch order of one call.
//
// One call at cursor s ("PersonaPlex native LM audit", section 7 'One exact generator
// step'), with every integer of the ring kept on the device:
//   prepare  place supplied codes, fill slot 0 at s = 0, gather the temporal input and
//            the depth control words (supplied targets, draws, sampling rule)
//   temporal embedding sum from the device IDs, the block stack (graph), final norm
//            straight into the depformer's h, text head
//   text     supplied text or a temperature / top-k draw -> depth position 0's token
//   depth    the depformer's frame (graph); each position draws unless supplied
//   finish   selections into the unsupplied target entries, clear the consumed flags,
//            gather the aligned output
#include <hip/hip_runtime.h>

#include <string>

#include "internal.h"
#include "model.h"
#include "pp.h"

using namespace pp;

struct pp_generator {
  pp_model* m = nullptr;
  pp_kv* kv = nullptr;
  pp_depformer* d = nullptr;
  pp_generator_config cfg{};
  int n = 17, C = 4, max_delay = 1;
  void* ws = nullptr;
  GenState* g = nullptr;
  float* text_logits = nullptr;
  long long s = 0;
  ~pp_generator() {
    if (ws) (void)hipFree(ws);
  }
};

extern "C" pp_status pp_generator_create(pp_model* m, pp_kv* kv, pp_depformer* d, const pp_generator_config* cfg,
                                         pp_generator** out) {
  if (!out) return pp_fail(PP_E_ARG, "out is NULL");
  *out = nullptr;
  if (!m || !kv || !d || !cfg) return pp_fail(PP_E_ARG, "NULL argument");
  if (kv->m != m) return pp_fail(PP_E_ARG, "kv ring belongs to another model");
  if (kv->B != 1) return pp_fail(PP_E_ARG, "the generator needs a batch-1 KV ring");
  if (!m->text_head) return pp_fail(PP_E_ARG, "the model has no text head");
  const pp_temporal_config& tc = m->cfg;
  const pp_depth_config& dc = d->cfg;
  const int n = cfg->n_streams;
  if (n != tc.n_audio + 1 || n != dc.n_steps + 1 || n > kMaxStreams)
    return pp_fail(PP_E_ARG, "n_streams must equal the model's n_audio + 1 and the depformer's n_steps + 1");
  if (dc.d_temporal != tc.d_model) return pp_fail(PP_E_ARG, "depformer d_temporal differs from the model's d_model");
  if (dc.text_vocab != tc.text_vocab) return pp_fail(PP_E_ARG, "text vocab of model and depformer differ");
  int max_delay = 0;
  for (int k = 0; k < n; ++k) {
    if (cfg->delays[k] < 0 || cfg->delays[k] > kGenMaxRing - 3)
      return pp_fail(PP_E_ARG, "stream " + std::to_string(k) + ": delay outside [0, " +
                                   std::to_string(kGenMaxRing - 3) + "]");
    max_delay = cfg->delays[k] > max_delay ? cfg->delays[k] : max_delay;
  }
  if (cfg->text_initial < 0 || cfg->text_initial >= tc.text_vocab || cfg->audio_initial < 0 ||
      cfg->audio_initial >= tc.audio_vocab)
    return pp_fail(PP_E_ID, "initial token outside its table");
  if (cfg->text_top_k > kMaxTopK || cfg->audio_top_k > kMaxTopK) return pp_fail(PP_E_ARG, "top_k above 1024");
  if (tc.text_vocab - 1 > kGenTextThreads * kGenTextPer) return pp_fail(PP_E_ARG, "text head above 32768 classes");
  if (cfg->audio_top_k > 1 && cfg->audio_temperature > 0.f && dc.n_out > kDepthSampleMaxOut)
    return pp_fail(PP_E_ARG, "sampled depth selection needs n_out <= 2048");

  pp_generator* g = new pp_generator();
  g->m = m;
  g->kv = kv;
  g->d = d;
  g->cfg = *cfg;
  g->n = n;
  g->max_delay = max_delay;
  g->C = max_delay + 3;
  const size_t state_bytes = (sizeof(GenState) + 255) / 256 * 256;
  const size_t bytes = state_bytes + sizeof(float) * (size_t)(tc.text_vocab - 1);
  if (hipMalloc(&g->ws, bytes) != hipSuccess || hipMemset(g->ws, 0, bytes) != hipSuccess) {
    delete g;
    return pp_fail(PP_E_HIP, "hipMalloc of the generator state failed");
  }
  g->g = static_cast<GenState*>(g->ws);
  g->text_logits = reinterpret_cast<float*>(static_cast<char*>(g->ws) + state_bytes);
  *out = g;
  return PP_OK;
}

extern "C" pp_status pp_generator_info(const pp_generator* g, int64_t* cursor, uint64_t* state_bytes) {
  if (!g) return pp_fail(PP_E_ARG, "generator is NULL");
  if (cursor) *cursor = g->s;
  if (state_bytes) *state_bytes = sizeof(GenState);
  return PP_OK;
}

extern "C" pp_status pp_generator_store(const pp_generator* g, void* dst_dev, void* stream) {
  if (!g || !dst_dev) return pp_fail(PP_E_ARG, "NULL argument");
  const hipError_t e = hipMemcpyAsync(dst_dev, g->g, sizeof(GenState), hipMemcpyDeviceToDevice,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("pp_generator_store: ") + hipGetErrorString(e));
  return PP_OK;
}

extern "C" pp_status pp_generator_restore(pp_generator* g, const void* src_dev, int64_t cursor, void* stream) {
  if (!g || !src_dev) return pp_fail(PP_E_ARG, "NULL argument");
  if (cursor < 0) return pp_fail(PP_E_ARG, "negative cursor");
  const hipError_t e = hipMemcpyAsync(g->g, src_dev, sizeof(GenState), hipMemcpyDeviceToDevice,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("pp_generator_restore: ") + hipGetErrorString(e));
  g->s = cursor;
  return PP_OK;
}

extern "C" pp_status pp_generator_destroy(pp_generator* g) {
  if (!g) return pp_fail(PP_E_ARG, "generator is NULL");
  delete g;
  return PP_OK;
}

extern "C" pp_status pp_generator_step(pp_generator* g, const int32_t* provided_host, const double* uniforms_host,
                                       int32_t* out_dev, int32_t* has_output_host, void* stream) {
  if (!g || !has_output_host) return pp_fail(PP_E_ARG, "NULL argument");
  const pp_temporal_config& tc = g->m->cfg;
  const pp_depth_config& dc = g->d->cfg;
  const pp_generator_config& c = g->cfg;
  GenPrepArgs pa{};
  pa.g = g->g;
  pa.dctrl = g->d->ctrl;
  pa.s = g->s;
  pa.n = g->n;
  pa.C = g->C;
  pa.audio_temperature = c.audio_temperature;
  pa.audio_top_k = c.audio_top_k;
  for (int k = 0; k < g->n; ++k) {
    const int32_t p = provided_host ? provided_host[k] : -1;
    const int32_t lim = k == 0 ? tc.text_vocab : dc.n_out;
    if (p < -1 || p >= lim)
      return pp_fail(PP_E_ID, "stream " + std::to_string(k) + ": supplied code " + std::to_string(p) +
                                  " outside [-1, " + std::to_string(lim) + ")");
    const double u = uniforms_host ? uniforms_host[k] : 0.0;
    if (!(u >= 0.0 && u < 1.0)) return pp_fail(PP_E_ARG, "uniform draw outside [0, 1)");
    pa.provided[k] = p;
    pa.delays[k] = c.delays[k];
    pa.initial[k] = k == 0 ? c.text_initial : c.audio_initial;
    pa.u[k] = u;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_gen_prepare(pa, st);
  if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("generator prepare: ") + hipGetErrorString(e));
  *has_output_host = 0;
  if (g->s == 0) {
    g->s = 1;
    return PP_OK;
  }
  pp_status ps = g->m->decode(g->kv, nullptr, g->g->ids, g->d->h, g->text_logits, st);
  if (ps) return ps;
  GenTextArgs ta{g->g, g->d->ctrl, g->text_logits, tc.text_vocab - 1, c.text_temperature, c.text_top_k};
  if ((e = launch_gen_text(ta, st)) != hipSuccess)
    return pp_fail(PP_E_HIP, std::string("generator text: ") + hipGetErrorString(e));
  if ((ps = g->d->run(st))) return ps;
  GenFinishArgs fa{};
  fa.g = g->g;
  fa.codes = g->d->codes;
  fa.out = out_dev;
  for (int k = 0; k < g->n; ++k) fa.delays[k] = c.delays[k];
  fa.s = g->s;
  fa.n = g->n;
  fa.C = g->C;
  fa.max_delay = g->max_delay;
  if ((e = launch_gen_finish(fa, st)) != hipSuccess)
    return pp_fail(PP_E_HIP, std::string("generator finish: ") + hipGetErrorString(e));
  *has_output_host = (out_dev && g->s > g->max_delay) ? 1 : 0;
  g->s += 1;
  return PP_OK;
}

extern "C" pp_status pp_generator_inspect(const pp_generator* g, int32_t* inputs_dev, int32_t* chosen_dev,
                                          float* text_logits_dev, float* depth_logits_dev, void* stream) {
  if (!g) return pp_fail(PP_E_ARG, "generator is NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t ns = sizeof(int32_t) * g->n;
  hipError_t e = hipSuccess;
  if (inputs_dev) e = hipMemcpyAsync(inputs_dev, g->g->ids, ns, hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess && chosen_dev) e = hipMemcpyAsync(chosen_dev, g->g->chosen, ns, hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess && text_logits_dev)
    e = hipMemcpyAsync(text_logits_dev, g->text_logits, sizeof(float) * (g->m->cfg.text_vocab - 1),
                       hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess && depth_logits_dev)
    e = hipMemcpyAsync(depth_logits_dev, g->d->logits, sizeof(float) * g->d->cfg.n_steps * g->d->cfg.n_out,
                       hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("generator inspect: ") + hipGetErrorString(e));
  return PP_OK;
}

extern "C" pp_status pp_sample_top_k(const float* logits_dev, int32_t rows, int32_t n, float temperature,
                                     int32_t top_k, const double* uniforms_dev, int32_t* out_dev, void* stream) {
  if (!logits_dev || !out_dev) return pp_fail(PP_E_ARG, "NULL argument");
  if (rows < 1 || n < 1 || n > 32768) return pp_fail(PP_E_ARG, "rows must be >= 1 and n in [1, 32768]");
  if (top_k > kMaxTopK) return pp_fail(PP_E_ARG, "top_k above 1024");
  int n_cu = 0;
  pp_status ps = pp_device_check(&n_cu);
  if (ps) return ps;
  hipError_t e = launch_sample_rows(logits_dev, rows, n, temperature, top_k, uniforms_dev, out_dev,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("sample: ") + hipGetErrorString(e));
  return PP_OK;
}
