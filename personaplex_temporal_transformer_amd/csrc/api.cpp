// C ABI of libpp (declared in include/pp.h): argument and ID validation, workspace and
// KV-ring ownership, and the launch order of one decode step / prefill / depth frame.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "internal.h"
#include "model.h"
#include "pp.h"

using namespace pp;

// ------------------------------------------------------------------ errors

static thread_local std::string g_err;

pp_status pp_fail(pp_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

extern "C" const char* pp_last_error(void) { return g_err.c_str(); }

pp_status pp_device_check(int* n_cu) {
  int dev = -1, count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count == 0)
    return pp_fail(PP_E_DEVICE, "no HIP device visible");
  if (hipGetDevice(&dev) != hipSuccess) return pp_fail(PP_E_DEVICE, "no current HIP device");
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return pp_fail(PP_E_DEVICE, "hipGetDeviceProperties failed");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return pp_fail(PP_E_DEVICE, std::string("libpp is built for gfx950; current device is ") +
                                    prop.gcnArchName);
  *n_cu = prop.multiProcessorCount;
  return PP_OK;
}

// ------------------------------------------------------------------ temporal model

// Split-K factor of the decode attention: about one workgroup per CU over all heads.
static int auto_splits(int n_cu, int H) {
  const int S = (n_cu + H - 1) / H;
  return S < 1 ? 1 : (S > kMaxAttnSplits ? kMaxAttnSplits : S);
}

static pp_status validate_temporal_config(const pp_temporal_config* c) {
  if (!c) return pp_fail(PP_E_ARG, "config is NULL");
  if (c->wdtype != PP_F32 && c->wdtype != PP_BF16) return pp_fail(PP_E_DTYPE, "wdtype must be PP_F32 or PP_BF16");
  if (c->n_layers < 1 || c->d_model < 8 || c->n_heads < 1 || c->context < 1 || c->d_ff < 8)
    return pp_fail(PP_E_ARG, "non-positive dimension in config");
  if (c->d_head != 64 && c->d_head != 128) return pp_fail(PP_E_ARG, "d_head must be 64 or 128");
  if (c->n_heads * c->d_head != c->d_model) return pp_fail(PP_E_ARG, "d_model != n_heads * d_head");
  if (c->d_model % 8 || c->d_ff % 8) return pp_fail(PP_E_ARG, "d_model and d_ff must be multiples of 8");
  if (c->d_model > 12288 || c->d_ff > 12288) return pp_fail(PP_E_ARG, "d_model/d_ff above 12288 unsupported");
  if (c->n_audio < 0 || c->n_audio + 1 > kMaxStreams) return pp_fail(PP_E_ARG, "n_audio out of range");
  if (c->text_vocab < 2 || c->audio_vocab < 1) return pp_fail(PP_E_ARG, "vocab sizes must be positive");
  if (!(c->rope_theta > 0) || !(c->eps >= 0)) return pp_fail(PP_E_ARG, "rope_theta must be > 0, eps >= 0");
  return PP_OK;
}

extern "C" pp_status pp_temporal_create(const pp_temporal_config* cfg, const pp_temporal_weights* w,
                                        int32_t max_batch, int32_t max_prefill_T, pp_model** out) {
  if (!out) return pp_fail(PP_E_ARG, "out is NULL");
  *out = nullptr;
  pp_status st = validate_temporal_config(cfg);
  if (st) return st;
  if (!w) return pp_fail(PP_E_ARG, "weights are NULL");
  if (max_batch < 1 || max_batch > kSgemmMaxBatch) return pp_fail(PP_E_ARG, "max_batch must be in [1, 64]");
  if (max_batch > 1 && cfg->wdtype != PP_BF16)
    return pp_fail(PP_E_ARG, "batched decode (max_batch > 1) needs bf16 weights");
  if (max_batch > 1 && (cfg->d_model % 32 || cfg->d_ff % 32 || (cfg->text_vocab - 1) % 16))
    return pp_fail(PP_E_ARG, "batched decode needs d_model % 32, d_ff % 32 and the text head rows % 16 == 0");
  if (max_prefill_T < 0 || max_prefill_T > cfg->context)
    return pp_fail(PP_E_CAPACITY, "max_prefill_T must be in [0, context]");
  int n_cu = 0;
  if ((st = pp_device_check(&n_cu))) return st;
  const int L = cfg->n_layers;
  if (!w->text_emb || !w->out_norm || (cfg->n_audio > 0 && !w->audio_emb) || !w->norm1 || !w->norm2 ||
      !w->w_qkv || !w->w_o || !w->w_in || !w->w_out)
    return pp_fail(PP_E_ARG, "a required weight pointer is NULL");
  for (int i = 0; i < cfg->n_audio; ++i)
    if (!w->audio_emb[i]) return pp_fail(PP_E_ARG, "audio_emb[" + std::to_string(i) + "] is NULL");
  for (int l = 0; l < L; ++l)
    if (!w->norm1[l] || !w->norm2[l] || !w->w_qkv[l] || !w->w_o[l] || !w->w_in[l] || !w->w_out[l])
      return pp_fail(PP_E_ARG, "layer " + std::to_string(l) + " has a NULL weight");

  pp_model* m = new pp_model();
  m->cfg = *cfg;
  m->bf16 = cfg->wdtype == PP_BF16;
  m->n_cu = n_cu;
  (void)hipGetDevice(&m->device);
  m->text_emb = w->text_emb;
  m->audio_emb.assign(w->audio_emb, w->audio_emb + cfg->n_audio);
  m->norm1.assign(w->norm1, w->norm1 + L);
  m->norm2.assign(w->norm2, w->norm2 + L);
  m->w_qkv.assign(w->w_qkv, w->w_qkv + L);
  m->w_o.assign(w->w_o, w->w_o + L);
  m->w_in.assign(w->w_in, w->w_in + L);
  m->w_out.assign(w->w_out, w->w_out + L);
  m->out_norm = w->out_norm;
  m->text_head = w->text_head;
  m->max_batch = max_batch;
  m->max_T = max_prefill_T;
  m->use_graph = true;
  m->gemv_blocks = n_cu;   // one 8-wave GEMV workgroup per CU
  m->wout_rb = cfg->d_model % 2 == 0 ? 2 : 1;

  const int D = cfg->d_model, F = cfg->d_ff, H = cfg->n_heads, dh = cfg->d_head;
  // attention splits: about one block per CU over all heads (at most kMaxAttnSplits)
  m->S = m->S_auto = auto_splits(n_cu, H);
  st = m->alloc_decode(D, F, H, dh);
  if (!st && m->bf16 && (max_prefill_T > 0 || max_batch > 1)) st = m->compute_f16_scales();
  if (!st) st = m->alloc_prefill();
  if (!st && max_batch > 1) st = m->pack_batched();
  if (st) {
    delete m;
    return st;
  }
  *out = m;
  return PP_OK;
}

pp_status pp_model::alloc_decode(int D, int F, int H, int dh) {
  size_t bytes = 0;
  auto take = [&](size_t n) { size_t off = bytes; bytes += (n + 255) / 256 * 256; return off; };
  const size_t ox = take(sizeof(float) * D), oq = take(sizeof(float) * D), oo = take(sizeof(float) * D);
  // batch-1 partials for any split count pp_temporal_set_attn_splits may choose
  const size_t os = take(sizeof(float) * F), op = take(sizeof(float) * (size_t)H * kMaxAttnSplits * dh);
  const size_t oml = take(sizeof(float) * (size_t)H * kMaxAttnSplits * 2);
  const size_t ost = take(sizeof(long long) * 4);
  const size_t orp = take(sizeof(float) * dh);
  // batched decode: per-session residuals, queries, float16 activations, attention partials
  const size_t nb = max_batch > 1 ? (size_t)max_batch : 0;
  const size_t nb16 = (nb + 15) / 16 * 16;   // float16 operands in whole 16-session fragment tiles
  const size_t obx = take(sizeof(float) * nb * D), obq = take(sizeof(float) * nb * D);
  const size_t obu = take(2 * nb16 * D), obo = take(2 * nb16 * D), obs = take(2 * nb16 * F);
  const size_t obp = take(sizeof(float) * nb * H * S_auto * dh), obm = take(sizeof(float) * nb * H * S_auto * 2);
  if (hipMalloc(&ws, bytes) != hipSuccess) return pp_fail(PP_E_HIP, "hipMalloc of decode workspace failed");
  if (hipMemset(ws, 0, bytes) != hipSuccess) return pp_fail(PP_E_HIP, "hipMemset of decode workspace failed");
  char* b = static_cast<char*>(ws);
  x = reinterpret_cast<float*>(b + ox);
  q = reinterpret_cast<float*>(b + oq);
  o = reinterpret_cast<float*>(b + oo);
  s = reinterpret_cast<float*>(b + os);
  part_o = reinterpret_cast<float*>(b + op);
  part_ml = reinterpret_cast<float*>(b + oml);
  state = reinterpret_cast<long long*>(b + ost);
  rope = reinterpret_cast<float*>(b + orp);
  db = DecodeBufs{x, q, o, s, part_o, part_ml, state, rope};
  if (nb) {
    bx = reinterpret_cast<float*>(b + obx);
    bq = reinterpret_cast<float*>(b + obq);
    bu16 = reinterpret_cast<uint16_t*>(b + obu);
    bo16 = reinterpret_cast<uint16_t*>(b + obo);
    bs16 = reinterpret_cast<uint16_t*>(b + obs);
    bpart_o = reinterpret_cast<float*>(b + obp);
    bpart_ml = reinterpret_cast<float*>(b + obm);
  }
  return PP_OK;
}

// Batched decode reads every matrix from a copy in the skinny products' fragment order
// (csrc/sgemm.hip): one allocation holding all layers' W_QKV, W_O, W_in, W_out and the
// text head, packed once here.
pp_status pp_model::pack_batched() {
  const pp_temporal_config& c = cfg;
  const size_t D = c.d_model, F = c.d_ff, L = c.n_layers, V = c.text_vocab - 1;
  const size_t per_layer = (3 * D * D + D * D + 2 * F * D + D * F) * 2;
  const size_t bytes = L * per_layer + (text_head ? V * D * 2 : 0);
  if (hipMalloc(&pk_ws, bytes) != hipSuccess) return pp_fail(PP_E_HIP, "hipMalloc of the packed weights failed");
  char* p = static_cast<char*>(pk_ws);
  hipError_t e = hipSuccess;
  for (size_t l = 0; l < L && e == hipSuccess; ++l) {
    const F16Exps& fe = f16e[l];
    pk_qkv.push_back(p);
    e = launch_sgemm_pack(w_qkv[l], p, (int)(3 * D), (int)D, 0, false, fe.w_qkv, nullptr);
    p += 3 * D * D * 2;
    pk_o.push_back(p);
    if (e == hipSuccess) e = launch_sgemm_pack(w_o[l], p, (int)D, (int)D, 0, false, fe.w_o, nullptr);
    p += D * D * 2;
    pk_in.push_back(p);
    if (e == hipSuccess) e = launch_sgemm_pack(w_in[l], p, (int)F, (int)D, (int)F, true, fe.w_in, nullptr);
    p += 2 * F * D * 2;
    pk_out.push_back(p);
    if (e == hipSuccess) e = launch_sgemm_pack(w_out[l], p, (int)D, (int)F, 0, false, fe.w_out, nullptr);
    p += D * F * 2;
  }
  if (e == hipSuccess && text_head) {
    pk_head = p;
    e = launch_sgemm_pack(text_head, p, (int)V, (int)D, 0, false, f16e_whead, nullptr);
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("packing weights for batched decode: ") + hipGetErrorString(e));
  return PP_OK;
}

pp_model::~pp_model() {
  for (hipEvent_t e : trace_ev) (void)hipEventDestroy(e);
  free_prefill();
  if (ws) (void)hipFree(ws);
  if (pk_ws) (void)hipFree(pk_ws);
  if (ids_pinned) (void)hipHostFree(ids_pinned);
  if (ids_event) (void)hipEventDestroy(ids_event);
}

extern "C" pp_status pp_temporal_destroy(pp_model* m) {
  if (!m) return pp_fail(PP_E_ARG, "model is NULL");
  delete m;
  return PP_OK;
}

extern "C" pp_status pp_temporal_set_graph(pp_model* m, int32_t enable) {
  if (!m) return pp_fail(PP_E_ARG, "model is NULL");
  m->use_graph = enable != 0;
  return PP_OK;
}

extern "C" pp_status pp_temporal_set_attn_splits(pp_model* m, int32_t splits) {
  if (!m) return pp_fail(PP_E_ARG, "model is NULL");
  if (splits < 0 || splits > kMaxAttnSplits)
    return pp_fail(PP_E_ARG, "splits outside [0, " + std::to_string(kMaxAttnSplits) + "]");
  const int S = splits == 0 ? m->S_auto : splits;
  if (S != m->S) {
    m->S = S;
    ++m->graph_gen;   // captured graphs hold the old launch shape
  }
  return PP_OK;
}

// ------------------------------------------------------------------ KV ring

extern "C" pp_status pp_kv_alloc(const pp_model* m, int32_t batch, pp_kv** out) {
  if (!m || !out) return pp_fail(PP_E_ARG, "NULL argument");
  *out = nullptr;
  if (batch < 1 || batch > m->max_batch) return pp_fail(PP_E_ARG, "batch outside [1, max_batch]");
  const pp_temporal_config& c = m->cfg;
  const size_t esz = m->bf16 ? 2 : 4;
  const size_t bytes = (size_t)c.n_layers * 2 * batch * c.n_heads * c.context * c.d_head * esz;
  pp_kv* kv = new pp_kv();
  kv->m = const_cast<pp_model*>(m);
  kv->B = batch;
  kv->bytes = bytes;
  if (hipMalloc(&kv->ring, bytes) != hipSuccess) {
    delete kv;
    return pp_fail(PP_E_HIP, "hipMalloc of the KV ring (" + std::to_string(bytes) + " bytes) failed");
  }
  *out = kv;
  return PP_OK;
}

pp_kv::~pp_kv() {
  if (exec) (void)hipGraphExecDestroy(exec);
  if (graph) (void)hipGraphDestroy(graph);
  if (ring) (void)hipFree(ring);
}

extern "C" pp_status pp_kv_free(pp_kv* kv) {
  if (!kv) return pp_fail(PP_E_ARG, "kv is NULL");
  delete kv;
  return PP_OK;
}

extern "C" pp_status pp_kv_reset(pp_kv* kv) {
  if (!kv) return pp_fail(PP_E_ARG, "kv is NULL");
  kv->pos = 0;
  return PP_OK;
}

extern "C" pp_status pp_kv_info(const pp_kv* kv, int64_t* position, uint64_t* bytes) {
  if (!kv) return pp_fail(PP_E_ARG, "kv is NULL");
  if (position) *position = kv->pos;
  if (bytes) *bytes = kv->bytes;
  return PP_OK;
}

extern "C" pp_status pp_kv_load(pp_kv* kv, const void* src_dev, int32_t n_frames, void* stream) {
  if (!kv || !src_dev) return pp_fail(PP_E_ARG, "NULL argument");
  const pp_temporal_config& c = kv->m->cfg;
  if (n_frames < 1 || n_frames > c.context) return pp_fail(PP_E_CAPACITY, "n_frames outside [1, context]");
  const size_t esz = kv->m->bf16 ? 2 : 4;
  const size_t rows = (size_t)c.n_layers * 2 * kv->B * c.n_heads;
  const size_t w = (size_t)n_frames * c.d_head * esz;
  hipError_t e = hipMemcpy2DAsync(kv->ring, (size_t)c.context * c.d_head * esz, src_dev, w, w, rows,
                                  hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("pp_kv_load: ") + hipGetErrorString(e));
  kv->pos = n_frames;
  return PP_OK;
}

extern "C" pp_status pp_kv_store(const pp_kv* kv, void* dst_dev, void* stream) {
  if (!kv || !dst_dev) return pp_fail(PP_E_ARG, "NULL argument");
  hipError_t e = hipMemcpyAsync(dst_dev, kv->ring, kv->bytes, hipMemcpyDeviceToDevice,
                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("pp_kv_store: ") + hipGetErrorString(e));
  return PP_OK;
}

extern "C" pp_status pp_kv_restore(pp_kv* kv, const void* src_dev, int64_t position, void* stream) {
  if (!kv || !src_dev) return pp_fail(PP_E_ARG, "NULL argument");
  if (position < 0) return pp_fail(PP_E_ARG, "negative position");
  hipError_t e = hipMemcpyAsync(kv->ring, src_dev, kv->bytes, hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("pp_kv_restore: ") + hipGetErrorString(e));
  kv->pos = position;
  return PP_OK;
}

// ------------------------------------------------------------------ embedding

pp_status pp_model::check_ids(const int32_t* ids, size_t frames) const {
  const int ns = cfg.n_audio + 1;
  for (size_t f = 0; f < frames; ++f)
    for (int k = 0; k < ns; ++k) {
      const int32_t id = ids[f * ns + k];
      const int32_t vocab = k == 0 ? cfg.text_vocab : cfg.audio_vocab;
      if (id < -1 || id >= vocab)
        return pp_fail(PP_E_ID, "frame " + std::to_string(f) + " stream " + std::to_string(k) + ": ID " +
                                    std::to_string(id) + " outside [-1, " + std::to_string(vocab) + ")");
    }
  return PP_OK;
}

void pp_model::embed_tables(EmbedArgs& a) const {
  // slots past the model's streams read the text table with ID -1 (dropped), so the kernel
  // loads every slot with no branch
  for (int k = 0; k < kMaxStreams; ++k) {
    a.tables[k] = text_emb;
    a.ids_arg[k] = -1;
  }
  for (int i = 0; i < cfg.n_audio; ++i) a.tables[i + 1] = audio_emb[i];
  a.n_streams = cfg.n_audio + 1;
  a.D = cfg.d_model;
}

pp_status pp_model::stage_ids(const int32_t* ids_host, size_t n, hipStream_t s) {
  // IDs go through a pinned buffer owned by the model; the event guards its reuse.
  if (n > ids_frames * (size_t)(cfg.n_audio + 1))
    return pp_fail(PP_E_CAPACITY, "more IDs than the model's ID region holds (" + std::to_string(ids_frames) +
                                      " frames: max_prefill_T x max_batch)");
  if (n > ids_cap) {
    if (ids_pinned) {
      (void)hipEventSynchronize(ids_event);
      (void)hipHostFree(ids_pinned);
    }
    ids_pinned = nullptr;
    if (hipHostMalloc(reinterpret_cast<void**>(&ids_pinned), n * sizeof(int32_t)) != hipSuccess)
      return pp_fail(PP_E_HIP, "hipHostMalloc of the ID staging buffer failed");
    ids_cap = n;
  }
  if (!ids_event && hipEventCreateWithFlags(&ids_event, hipEventDisableTiming) != hipSuccess)
    return pp_fail(PP_E_HIP, "hipEventCreate failed");
  (void)hipEventSynchronize(ids_event);
  std::memcpy(ids_pinned, ids_host, n * sizeof(int32_t));
  hipError_t e = hipMemcpyAsync(ids_dev, ids_pinned, n * sizeof(int32_t), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipEventRecord(ids_event, s);
  if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("staging IDs: ") + hipGetErrorString(e));
  return PP_OK;
}

extern "C" pp_status pp_embed_sum(const pp_model* mc, const int32_t* ids_host, int32_t batch, int32_t T,
                                  float* x_out_dev, void* stream) {
  pp_model* m = const_cast<pp_model*>(mc);
  if (!m || !ids_host || !x_out_dev) return pp_fail(PP_E_ARG, "NULL argument");
  if (batch < 1 || batch > m->max_batch || T < 1) return pp_fail(PP_E_ARG, "batch or T out of range");
  const size_t frames = (size_t)batch * T;
  // sizes first: the IDs are read only once the call is known to fit
  if (frames > 1 && frames > m->ids_frames)
    return pp_fail(PP_E_CAPACITY, "batch*T exceeds max_prefill_T x max_batch frames");
  pp_status st = m->check_ids(ids_host, frames);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  EmbedArgs a{};
  m->embed_tables(a);
  a.out = x_out_dev;
  a.rows = (int)frames;
  if (frames == 1) {
    for (int k = 0; k < a.n_streams; ++k) a.ids_arg[k] = ids_host[k];
  } else {
    if ((st = m->stage_ids(ids_host, frames * a.n_streams, s))) return st;
    a.ids_dev = m->ids_dev;
  }
  hipError_t e = launch_embed(a, m->bf16, s);
  if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("embed: ") + hipGetErrorString(e));
  return PP_OK;
}

// ------------------------------------------------------------------ decode step

// pos_arg: the frame's position, passed by value to the kernels of a direct launch; -1
// when the launches are captured into a graph, whose kernels read it from `state`.
hipError_t pp_model::enqueue_layers(pp_kv* kv, hipStream_t s, bool traced, long long pos_arg,
                                     const DecodeBufs& b) {
  const pp_temporal_config& c = cfg;
  const int D = c.d_model, F = c.d_ff, H = c.n_heads, dh = c.d_head, C = c.context;
  const size_t esz = bf16 ? 2 : 4;
  const size_t per_kv = (size_t)kv->B * H * C * dh * esz;
  hipError_t e = hipSuccess;
  for (int l = 0; l < c.n_layers && e == hipSuccess; ++l) {
    char* kbase = static_cast<char*>(kv->ring) + (size_t)(2 * l) * per_kv;
    char* vbase = kbase + per_kv;

    GemvArgs g{};
    g.W = w_qkv[l]; g.x = b.x; g.alpha = norm1[l]; g.eps = (float)c.eps; g.K = D;
    g.n_groups = 3 * D / 2; g.out = b.q; g.D = D; g.dh = dh; g.C = C; g.kc = kbase; g.vc = vbase;
    g.state = b.state; g.pos = pos_arg; g.rope = b.rope;
    AttnDecodeArgs at{};
    at.q = b.q; at.k = kbase; at.v = vbase; at.state = b.state; at.pos = pos_arg; at.C = C; at.H = H; at.S = S;
    at.scale = 1.0f / std::sqrt((float)dh); at.part_o = b.part_o; at.part_ml = b.part_ml; at.out = b.o;
    const bool merge_in_wo = S <= 8 && D <= 4096;
    at.combine = merge_in_wo ? 0 : 1;
    e = launch_gemv(PRO_RMSNORM, EPI_QKV, bf16, 2, g, gemv_blocks, s);
    if (e == hipSuccess) e = launch_attn_decode(at, bf16, dh, s);
    if (e != hipSuccess) break;

    GemvArgs go{};
    go.W = w_o[l]; go.x = b.o; go.K = D; go.n_groups = D / 2; go.out = b.x;
    go.po = b.part_o; go.pml = b.part_ml; go.pS = S; go.adh = dh;
    e = launch_gemv(merge_in_wo ? PRO_ATTN_MERGE : PRO_COPY, EPI_RESID, bf16, 2, go, gemv_blocks, s);
    if (e != hipSuccess) break;

    const bool tr = traced && l == trace_layer && trace_used + 2 <= trace_ev.size();
    if (tr) (void)hipEventRecord(trace_ev[trace_used], s);
    GemvArgs gi{};
    gi.W = w_in[l]; gi.x = b.x; gi.alpha = norm2[l]; gi.eps = (float)c.eps; gi.K = D;
    gi.n_groups = F; gi.out = b.s; gi.F = F;
    e = launch_gemv(PRO_RMSNORM, EPI_SWIGLU, bf16, 2, gi, gemv_blocks, s);
    for (int r = 1; tr && r < trace_repeat && e == hipSuccess; ++r)
      e = launch_gemv(PRO_RMSNORM, EPI_SWIGLU, bf16, 2, gi, gemv_blocks, s);
    if (tr) {
      (void)hipEventRecord(trace_ev[trace_used + 1], s);
      trace_used += 2;
    }
    if (e != hipSuccess) break;

    GemvArgs gw{};
    gw.W = w_out[l]; gw.x = b.s; gw.K = F; gw.n_groups = D / wout_rb; gw.out = b.x;
    e = launch_gemv(PRO_COPY, EPI_RESID, bf16, wout_rb, gw, gemv_blocks, s);
    if (e == hipSuccess) e = enqueue_reader(l, s, b);
  }
  return e;
}

pp_status pp_model::run_layers(pp_kv* kv, hipStream_t s) {
  const bool traced = trace_layer >= 0;
  if (!use_graph || traced) {
    hipError_t e = kv->B > 1 ? enqueue_layers_batched(kv, s, kv->pos) : enqueue_layers(kv, s, traced, kv->pos, db);
    if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("decode launch: ") + hipGetErrorString(e));
    return PP_OK;
  }
  if (!kv->exec || kv->exec_model_gen != graph_gen) {
    if (kv->exec) (void)hipGraphExecDestroy(kv->exec);
    if (kv->graph) (void)hipGraphDestroy(kv->graph);
    kv->exec = nullptr;
    kv->graph = nullptr;
    hipStream_t cap;
    if (hipStreamCreateWithFlags(&cap, hipStreamNonBlocking) != hipSuccess)
      return pp_fail(PP_E_HIP, "hipStreamCreate for graph capture failed");
    hipError_t e = hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal);
    if (e == hipSuccess) {
      hipError_t le = kv->B > 1 ? enqueue_layers_batched(kv, cap, -1) : enqueue_layers(kv, cap, false, -1, db);
      e = hipStreamEndCapture(cap, &kv->graph);
      if (le != hipSuccess) e = le;
    }
    if (e == hipSuccess) e = hipGraphInstantiate(&kv->exec, kv->graph, nullptr, nullptr, 0);
    (void)hipStreamDestroy(cap);
    if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("decode graph capture: ") + hipGetErrorString(e));
    kv->exec_model_gen = graph_gen;
  }
  hipError_t e = hipGraphLaunch(kv->exec, s);
  if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("decode graph launch: ") + hipGetErrorString(e));
  return PP_OK;
}

extern "C" pp_status pp_temporal_decode_step(pp_model* m, pp_kv* kv, const int32_t* ids_host,
                                             float* h_out_dev, float* text_logits_dev, void* stream) {
  if (!m || !kv || !ids_host || !h_out_dev) return pp_fail(PP_E_ARG, "NULL argument");
  if (kv->m != m) return pp_fail(PP_E_ARG, "kv ring belongs to another model");
  pp_status st = m->check_ids(ids_host, (size_t)kv->B);
  if (st) return st;
  return m->decode(kv, ids_host, nullptr, h_out_dev, text_logits_dev, static_cast<hipStream_t>(stream));
}

// One decode frame. The IDs come from the host (ids_host, already validated) or from
// device memory (ids_dev: the generator's ring, whose entries are valid by construction).
pp_status pp_model::decode(pp_kv* kv, const int32_t* ids_host, const int32_t* ids_dev, float* h_out_dev,
                           float* text_logits_dev, hipStream_t s) {
  if (text_logits_dev && !text_head) return pp_fail(PP_E_ARG, "text logits requested but the model has no text head");
  if (kv->B > 1) {
    if (readers.visible > 0) return pp_fail(PP_E_ARG, "memory readers run in batch-1 decode only");
    return decode_batched(kv, ids_host, h_out_dev, text_logits_dev, s);
  }
  return decode_one(kv, ids_host, ids_dev, h_out_dev, text_logits_dev, s, db, true);
}

// One batch-1 frame with the step's intermediates in `b`. graph: replay / capture the layer
// stack as a HIP graph when the model is in graph mode (the model's own buffers only);
// otherwise every kernel is launched directly with the position passed by value.
pp_status pp_model::decode_one(pp_kv* kv, const int32_t* ids_host, const int32_t* ids_dev, float* h_out_dev,
                               float* text_logits_dev, hipStream_t s, const DecodeBufs& b, bool graph) {
  const pp_temporal_config& c = cfg;

  EmbedArgs a{};
  embed_tables(a);
  if (ids_dev) {
    a.ids_dev = ids_dev;
  } else {
    for (int k = 0; k < a.n_streams; ++k) a.ids_arg[k] = ids_host[k];
  }
  a.out = b.x;
  a.rows = 1;
  a.state = b.state;
  a.pos = kv->pos;
  a.rope = b.rope;
  a.dh = c.d_head;
  // RoPE angles pos * theta^(-2j/d_head) formed in float64 on the host
  for (int j = 0; j < c.d_head / 2; ++j) {
    const double ang = (double)kv->pos * std::exp(-std::log(c.rope_theta) * (2.0 * j) / (double)c.d_head);
    a.rope_cs[2 * j] = (float)std::cos(ang);
    a.rope_cs[2 * j + 1] = (float)std::sin(ang);
  }
  hipError_t e = launch_embed(a, bf16, s);
  if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("embed: ") + hipGetErrorString(e));

  if (graph) {
    pp_status st = run_layers(kv, s);
    if (st) return st;
  } else if ((e = enqueue_layers(kv, s, false, kv->pos, b)) != hipSuccess) {
    return pp_fail(PP_E_HIP, std::string("decode launch: ") + hipGetErrorString(e));
  }

  e = launch_rmsnorm_rows(b.x, out_norm, (float)c.eps, c.d_model, 1, h_out_dev, nullptr, false, s);
  if (e == hipSuccess && text_logits_dev) {
    GemvArgs g{};
    g.W = text_head; g.x = b.x; g.alpha = out_norm; g.eps = (float)c.eps; g.K = c.d_model;
    g.n_groups = (c.text_vocab - 1) / 2; g.out = text_logits_dev;
    if ((c.text_vocab - 1) % 2 == 0) {
      e = launch_gemv(PRO_RMSNORM, EPI_STORE, bf16, 2, g, gemv_blocks, s);
    } else {
      return pp_fail(PP_E_ARG, "text head rows must be even");
    }
  }
  if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("final norm / text head: ") + hipGetErrorString(e));
  kv->pos += 1;
  return PP_OK;
}

// ------------------------------------------------------------------ batched decode

// B sessions at one position: every weight byte streamed once per step serves all of
// them (skinny float16 matrix-core products, csrc/sgemm.hip); attention runs per session
// over its own ring. pos_arg as in enqueue_layers.
hipError_t pp_model::enqueue_layers_batched(pp_kv* kv, hipStream_t s, long long pos_arg) {
  const pp_temporal_config& c = cfg;
  const int D = c.d_model, F = c.d_ff, H = c.n_heads, dh = c.d_head, C = c.context, B = kv->B;
  const size_t per_kv = (size_t)B * H * C * dh * 2;
  const long long bstride = (long long)H * C * dh;
  // attention splits: about one block per CU over the B x H heads (one split once the
  // sessions fill the grid, whose blocks then write the head outputs themselves)
  const int Sb = std::max(1, std::min(S_auto, (n_cu + H * B - 1) / (H * B)));
  hipError_t e = hipSuccess;
  for (int l = 0; l < c.n_layers && e == hipSuccess; ++l) {
    char* kbase = static_cast<char*>(kv->ring) + (size_t)(2 * l) * per_kv;
    char* vbase = kbase + per_kv;
    const F16Exps& fe = f16e[l];
    // up to kSgemmNormMaxBatch sessions the QKV and W_in products form the row norm in
    // their prologue; beyond, one row-norm launch writes their float16 activations
    const bool fold = B <= kSgemmNormMaxBatch && D <= kSgemmNormMaxK;
    if (!fold && (e = launch_rmsnorm_rows(bx, norm1[l], (float)c.eps, D, B, nullptr, bu16, true, s, fe.u1)) != hipSuccess)
      break;
    SgemmArgs g{};
    g.act = bu16; g.W = pk_qkv[l]; g.B = B; g.K = D; g.N = 3 * D; g.acc_exp = fe.u1 + fe.w_qkv;
    if (fold) {
      g.xin = bx; g.alpha = norm1[l]; g.eps = (float)c.eps; g.act_exp = fe.u1;
    }
    g.q_out = bq; g.kc = kbase; g.vc = vbase; g.kv_bstride = bstride; g.rope = rope; g.state = state;
    g.pos = pos_arg; g.D = D; g.dh = dh; g.C = C;
    g.n_cu = n_cu;
    if ((e = launch_sgemm(SEPI_QKV, g, s)) != hipSuccess) break;
    AttnDecodeArgs at{};
    at.q = bq; at.k = kbase; at.v = vbase; at.state = state; at.pos = pos_arg; at.C = C; at.H = H; at.S = Sb;
    at.scale = 1.0f / std::sqrt((float)dh); at.part_o = bpart_o; at.part_ml = bpart_ml; at.combine = 1;
    at.batch = B; at.kv_bstride = bstride; at.out16 = bo16; at.o16_exp = fe.v;
    if ((e = launch_attn_decode(at, true, dh, s)) != hipSuccess) break;
    SgemmArgs go{};
    go.act = bo16; go.W = pk_o[l]; go.B = B; go.K = D; go.N = D; go.x = bx; go.acc_exp = fe.v + fe.w_o;
    go.n_cu = n_cu;
    if ((e = launch_sgemm(SEPI_RESID, go, s)) != hipSuccess) break;
    if (!fold && (e = launch_rmsnorm_rows(bx, norm2[l], (float)c.eps, D, B, nullptr, bu16, true, s, fe.u2)) != hipSuccess)
      break;
    SgemmArgs gi{};
    gi.act = bu16; gi.W = pk_in[l]; gi.B = B; gi.K = D; gi.N = F; gi.F = F; gi.s_out = bs16;
    gi.acc_exp = fe.u2 + fe.w_in; gi.s16_exp = fe.s;
    if (fold) {
      gi.xin = bx; gi.alpha = norm2[l]; gi.eps = (float)c.eps; gi.act_exp = fe.u2;
    }
    gi.n_cu = n_cu;
    if ((e = launch_sgemm(SEPI_SWIGLU, gi, s)) != hipSuccess) break;
    SgemmArgs gw{};
    gw.act = bs16; gw.W = pk_out[l]; gw.B = B; gw.K = F; gw.N = D; gw.x = bx; gw.acc_exp = fe.s + fe.w_out;
    gw.n_cu = n_cu;
    e = launch_sgemm(SEPI_RESID, gw, s);
  }
  return e;
}

pp_status pp_model::decode_batched(pp_kv* kv, const int32_t* ids_host, float* h_out_dev, float* text_logits_dev,
                                   hipStream_t s) {
  const pp_temporal_config& c = cfg;
  const int B = kv->B, D = c.d_model;
  if (!ids_host) return pp_fail(PP_E_ARG, "batched decode takes host IDs");
  EmbedArgs a{};
  embed_tables(a);
  pp_status st = stage_ids(ids_host, (size_t)B * a.n_streams, s);
  if (st) return st;
  a.ids_dev = ids_dev;
  a.out = bx;
  a.rows = B;
  a.state = state;
  a.pos = kv->pos;
  a.rope = rope;
  a.dh = c.d_head;
  for (int j = 0; j < c.d_head / 2; ++j) {
    const double ang = (double)kv->pos * std::exp(-std::log(c.rope_theta) * (2.0 * j) / (double)c.d_head);
    a.rope_cs[2 * j] = (float)std::cos(ang);
    a.rope_cs[2 * j + 1] = (float)std::sin(ang);
  }
  hipError_t e = launch_embed(a, bf16, s);
  if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("embed: ") + hipGetErrorString(e));
  if ((st = run_layers(kv, s))) return st;
  e = launch_rmsnorm_rows(bx, out_norm, (float)c.eps, D, B, h_out_dev, text_logits_dev ? bu16 : nullptr, true, s,
                          f16e_uout);
  if (e == hipSuccess && text_logits_dev) {
    SgemmArgs g{};
    g.act = bu16; g.W = pk_head; g.B = B; g.K = D; g.N = c.text_vocab - 1; g.out = text_logits_dev;
    g.acc_exp = f16e_uout + f16e_whead;
    g.n_cu = n_cu;
    e = launch_sgemm(SEPI_STORE, g, s);
  }
  if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("final norm / text head: ") + hipGetErrorString(e));
  kv->pos += 1;
  return PP_OK;
}

// ------------------------------------------------------------------ kernel timing

extern "C" pp_status pp_temporal_trace(pp_model* m, int32_t layer, int32_t repeat) {
  if (!m) return pp_fail(PP_E_ARG, "model is NULL");
  if (layer >= m->cfg.n_layers) return pp_fail(PP_E_ARG, "layer out of range");
  if (repeat < 1 || repeat > 64) return pp_fail(PP_E_ARG, "repeat outside [1, 64]");
  if (layer >= 0 && m->trace_ev.empty()) {
    m->trace_ev.resize(4096);
    for (auto& ev : m->trace_ev)
      if (hipEventCreate(&ev) != hipSuccess) return pp_fail(PP_E_HIP, "hipEventCreate failed");
  }
  m->trace_layer = layer < 0 ? -1 : layer;
  m->trace_repeat = repeat;
  m->trace_used = 0;
  return PP_OK;
}

extern "C" pp_status pp_temporal_trace_read(pp_model* m, int64_t* count, double* mean_us) {
  if (!m || !count || !mean_us) return pp_fail(PP_E_ARG, "NULL argument");
  double tot = 0;
  int64_t n = 0;
  for (size_t i = 0; i + 1 < m->trace_used; i += 2) {
    float ms = 0;
    if (hipEventSynchronize(m->trace_ev[i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, m->trace_ev[i], m->trace_ev[i + 1]) != hipSuccess)
      return pp_fail(PP_E_HIP, "reading trace events failed");
    tot += ms;
    ++n;
  }
  *count = n * m->trace_repeat;
  *mean_us = n ? tot * 1000.0 / ((double)n * m->trace_repeat) : 0.0;
  m->trace_used = 0;
  return PP_OK;
}
