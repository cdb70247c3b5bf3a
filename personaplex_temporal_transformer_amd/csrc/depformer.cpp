// Depth transformer ("depformer") host side: validation, workspace, launch order, graph.
//
// Launch order of one frame ("PersonaPlex native LM audit", section 4):
//   setup (copy h, write the text token and forced codes into device control words)
//   in_proj: all n_steps temporal-to-depth projections in one GEMV over the stacked rows
//   for q in 0 .. n_steps-1:
//     select(q): code of q-1 (forced or argmax), z = c_q + embedding
//     for each layer m: RMSNorm+QKV slice (K, V -> depth cache row q);
//                       depth attention + W_O slice + residual;
//                       RMSNorm + W_in[m][q] + SiLU product; W_out[m][q] + residual
//     head[q] -> logits_q
//   select(n_steps): code of the last position
#include <hip/hip_runtime.h>

#include <cmath>
#include <string>
#include <vector>

#include "internal.h"
#include "model.h"
#include "pp.h"

using namespace pp;

static pp_status validate_depth_config(const pp_depth_config* c) {
  if (!c) return pp_fail(PP_E_ARG, "config is NULL");
  if (c->wdtype != PP_F32 && c->wdtype != PP_BF16) return pp_fail(PP_E_DTYPE, "wdtype must be PP_F32 or PP_BF16");
  if (c->n_layers < 1 || c->d_model < 8 || c->n_heads < 1 || c->d_head < 1 || c->d_ff < 8 || c->n_steps < 1 ||
      c->window < 1 || c->n_out < 2 || c->d_temporal < 8 || c->text_vocab < 1 || c->audio_vocab < 1)
    return pp_fail(PP_E_ARG, "non-positive dimension in depth config");
  if (c->n_heads * c->d_head != c->d_model) return pp_fail(PP_E_ARG, "d_model != n_heads * d_head");
  if (c->n_heads > 32 || c->n_steps > 32 || c->d_head > 128)
    return pp_fail(PP_E_ARG, "n_heads, n_steps <= 32 and d_head <= 128 required");
  if (c->d_model % 8 || c->d_ff % 8 || c->d_temporal % 8 || c->n_out % 2)
    return pp_fail(PP_E_ARG, "d_model, d_ff, d_temporal must be multiples of 8 and n_out even");
  if (c->d_model > 2048 || c->d_ff > 12288 || c->d_temporal > 12288)
    return pp_fail(PP_E_ARG, "d_model above 2048 or d_ff/d_temporal above 12288 unsupported");
  if (c->n_out > c->audio_vocab) return pp_fail(PP_E_ARG, "n_out exceeds the audio embedding rows");
  return PP_OK;
}

extern "C" pp_status pp_depformer_create(const pp_depth_config* cfg, const pp_depth_weights* w,
                                         pp_depformer** out) {
  if (!out) return pp_fail(PP_E_ARG, "out is NULL");
  *out = nullptr;
  pp_status st = validate_depth_config(cfg);
  if (st) return st;
  if (!w || !w->in_proj || !w->text_emb || (cfg->n_steps > 1 && !w->audio_emb) || !w->w_qkv || !w->w_o ||
      !w->w_in || !w->w_out || !w->norm1 || !w->norm2 || !w->head)
    return pp_fail(PP_E_ARG, "a required weight pointer is NULL");
  const int S = cfg->n_steps, L = cfg->n_layers;
  for (int q = 0; q < S; ++q)
    if (!w->in_proj[q] || !w->head[q] || (q < S - 1 && !w->audio_emb[q]))
      return pp_fail(PP_E_ARG, "step " + std::to_string(q) + " has a NULL weight");
  for (int m = 0; m < L; ++m) {
    if (!w->w_qkv[m] || !w->w_o[m] || !w->norm1[m] || !w->norm2[m])
      return pp_fail(PP_E_ARG, "layer " + std::to_string(m) + " has a NULL weight");
    for (int q = 0; q < S; ++q)
      if (!w->w_in[m * S + q] || !w->w_out[m * S + q])
        return pp_fail(PP_E_ARG, "layer " + std::to_string(m) + " step " + std::to_string(q) + " has a NULL FFN weight");
  }
  int n_cu = 0;
  if ((st = pp_device_check(&n_cu))) return st;

  pp_depformer* d = new pp_depformer();
  d->cfg = *cfg;
  d->bf16 = cfg->wdtype == PP_BF16;
  d->n_cu = n_cu;
  d->in_proj.assign(w->in_proj, w->in_proj + S);
  d->audio_emb.assign(w->audio_emb, w->audio_emb + (S > 1 ? S - 1 : 0));
  d->w_qkv.assign(w->w_qkv, w->w_qkv + L);
  d->w_o.assign(w->w_o, w->w_o + L);
  d->w_in.assign(w->w_in, w->w_in + L * S);
  d->w_out.assign(w->w_out, w->w_out + L * S);
  d->head.assign(w->head, w->head + S);
  d->norm1.assign(w->norm1, w->norm1 + L);
  d->norm2.assign(w->norm2, w->norm2 + L);
  d->text_emb = w->text_emb;
  d->gemv_blocks = n_cu;
  d->qkv_blocks = d->attn_blocks = d->ffn_blocks = n_cu;
  d->use_graph = true;

  const int D = cfg->d_model, F = cfg->d_ff, H = cfg->n_heads, dh = cfg->d_head;
  size_t bytes = 0;
  auto take = [&](size_t n) { size_t off = bytes; bytes += (n + 255) / 256 * 256; return off; };
  const size_t oh = take(4 * (size_t)cfg->d_temporal), oc = take(4 * (size_t)S * D), oz = take(4 * (size_t)D);
  const size_t oq = take(4 * (size_t)D), os = take(4 * (size_t)F), okv = take(4 * (size_t)L * 2 * H * S * dh);
  const size_t ol = take(4 * (size_t)S * cfg->n_out), ocd = take(4 * (size_t)S), oct = take(sizeof(DepthCtrl));
  if (hipMalloc(&d->ws, bytes) != hipSuccess || hipMemset(d->ws, 0, bytes) != hipSuccess) {
    delete d;
    return pp_fail(PP_E_HIP, "hipMalloc of the depformer workspace failed");
  }
  char* b = static_cast<char*>(d->ws);
  d->h = reinterpret_cast<float*>(b + oh);
  d->c_all = reinterpret_cast<float*>(b + oc);
  d->z = reinterpret_cast<float*>(b + oz);
  d->q = reinterpret_cast<float*>(b + oq);
  d->s = reinterpret_cast<float*>(b + os);
  d->kv = reinterpret_cast<float*>(b + okv);
  d->logits = reinterpret_cast<float*>(b + ol);
  d->codes = reinterpret_cast<int32_t*>(b + ocd);
  d->ctrl = reinterpret_cast<DepthCtrl*>(b + oct);
  *out = d;
  return PP_OK;
}

extern "C" pp_status pp_depformer_destroy(pp_depformer* d) {
  if (!d) return pp_fail(PP_E_ARG, "depformer is NULL");
  delete d;
  return PP_OK;
}

hipError_t pp_depformer::enqueue(hipStream_t st) {
  const pp_depth_config& c = cfg;
  const int D = c.d_model, F = c.d_ff, H = c.n_heads, dh = c.d_head, S = c.n_steps, L = c.n_layers;
  const size_t esz = bf16 ? 2 : 4;
  hipError_t e;

  GemvArgs gp{};
  for (int qq = 0; qq < S; ++qq) gp.mats[qq] = in_proj[qq];
  gp.rows_per_mat = D;
  gp.x = h;
  gp.K = c.d_temporal;
  gp.n_groups = S * D / 2;
  gp.out = c_all;
  if ((e = launch_gemv(PRO_COPY, EPI_STORE, bf16, 2, gp, gemv_blocks, st)) != hipSuccess) return e;

  DepthSelectArgs sa{};
  sa.c_all = c_all;
  sa.text_emb = text_emb;
  for (int qq = 0; qq + 1 < S; ++qq) sa.audio_emb[qq] = audio_emb[qq];
  sa.ctrl = ctrl;
  sa.logits = logits;
  sa.codes = codes;
  sa.z = z;
  sa.D = D;
  sa.n_out = c.n_out;
  sa.n_steps = S;

  for (int qs = 0; qs < S; ++qs) {
    sa.q = qs;
    if ((e = launch_depth_select(sa, bf16, st)) != hipSuccess) return e;
    for (int m = 0; m < L; ++m) {
      float* kc = kv + (size_t)(2 * m) * H * S * dh;
      float* vc = kc + (size_t)H * S * dh;

      GemvArgs g{};
      g.W = static_cast<const char*>(w_qkv[m]) + (size_t)qs * 3 * D * D * esz;
      g.x = z; g.alpha = norm1[m]; g.eps = (float)c.eps; g.K = D; g.n_groups = 3 * D / 2;
      g.out = q; g.D = D; g.dh = dh; g.C = S; g.kc = kc; g.vc = vc; g.slot_override = qs;
      if ((e = launch_gemv(PRO_RMSNORM, EPI_DEPTH_QKV, bf16, 2, g, qkv_blocks, st)) != hipSuccess) return e;

      GemvArgs go{};
      go.W = static_cast<const char*>(w_o[m]) + (size_t)qs * D * D * esz;
      go.K = D; go.n_groups = D / 2; go.out = z;
      go.aq = q; go.ak = kc; go.av = vc; go.aH = H; go.adh = dh; go.acap = S; go.aq_pos = qs;
      go.awin = c.window; go.ascale = 1.0f / std::sqrt((float)dh);
      if ((e = launch_gemv(PRO_DEPTH_ATTN, EPI_RESID, bf16, 2, go, attn_blocks, st)) != hipSuccess) return e;

      GemvArgs gi{};
      gi.W = w_in[m * S + qs]; gi.x = z; gi.alpha = norm2[m]; gi.eps = (float)c.eps; gi.K = D;
      gi.n_groups = F; gi.out = s; gi.F = F;
      if ((e = launch_gemv(PRO_RMSNORM, EPI_SWIGLU, bf16, 2, gi, ffn_blocks, st)) != hipSuccess) return e;

      GemvArgs gw{};
      gw.W = w_out[m * S + qs]; gw.x = s; gw.K = F; gw.n_groups = D / 2; gw.out = z;
      if ((e = launch_gemv(PRO_COPY, EPI_RESID, bf16, 2, gw, ffn_blocks, st)) != hipSuccess) return e;
    }
    GemvArgs gh{};
    gh.W = head[qs]; gh.x = z; gh.K = D; gh.n_groups = c.n_out / 2; gh.out = logits + (size_t)qs * c.n_out;
    if ((e = launch_gemv(PRO_COPY, EPI_STORE, bf16, 2, gh, gemv_blocks, st)) != hipSuccess) return e;
  }
  sa.q = S;
  return launch_depth_select(sa, bf16, st);
}

extern "C" pp_status pp_depformer_step(pp_depformer* d, const float* h_dev, const int32_t* text_token_host,
                                       const int32_t* forced_host, int32_t batch, int32_t* codes_dev,
                                       float* logits_dev, void* stream) {
  if (!d || !h_dev || !text_token_host || !codes_dev) return pp_fail(PP_E_ARG, "NULL argument");
  if (batch != 1) return pp_fail(PP_E_ARG, "batch must be 1");
  const pp_depth_config& c = d->cfg;
  if (text_token_host[0] < 0 || text_token_host[0] >= c.text_vocab)
    return pp_fail(PP_E_ID, "text token " + std::to_string(text_token_host[0]) + " outside [0, text_vocab)");
  DepthSetupArgs sa{};
  sa.h_src = h_dev;
  sa.h_dst = d->h;
  sa.d_temporal = c.d_temporal;
  sa.ctrl = d->ctrl;
  sa.text_token = text_token_host[0];
  sa.n_steps = c.n_steps;
  for (int q = 0; q < c.n_steps; ++q) {
    const int32_t f = forced_host ? forced_host[q] : -1;
    if (f < -1 || f >= c.n_out)
      return pp_fail(PP_E_ID, "forced code " + std::to_string(f) + " at position " + std::to_string(q) +
                                  " outside [-1, n_out)");
    sa.forced[q] = f;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_depth_setup(sa, st);
  if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("depth setup: ") + hipGetErrorString(e));
  pp_status ps = d->run(st);
  if (ps) return ps;
  e = hipMemcpyAsync(codes_dev, d->codes, sizeof(int32_t) * c.n_steps, hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess && logits_dev)
    e = hipMemcpyAsync(logits_dev, d->logits, sizeof(float) * c.n_steps * c.n_out, hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("depformer step: ") + hipGetErrorString(e));
  return PP_OK;
}

// The frame's launches after the control words and h are in place: directly, or as one
// graph captured on first use and replayed (its kernels read everything per-frame from
// device memory).
pp_status pp_depformer::run(hipStream_t st) {
  hipError_t e;
  if (!use_graph) {
    e = enqueue(st);
  } else {
    if (!exec) {
      hipStream_t cap;
      if (hipStreamCreateWithFlags(&cap, hipStreamNonBlocking) != hipSuccess)
        return pp_fail(PP_E_HIP, "hipStreamCreate for graph capture failed");
      e = hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal);
      if (e == hipSuccess) {
        hipError_t le = enqueue(cap);
        e = hipStreamEndCapture(cap, &graph);
        if (le != hipSuccess) e = le;
      }
      if (e == hipSuccess) e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
      (void)hipStreamDestroy(cap);
      if (e != hipSuccess) {
        if (graph) (void)hipGraphDestroy(graph);
        graph = nullptr;
        exec = nullptr;
        return pp_fail(PP_E_HIP, std::string("depformer graph capture: ") + hipGetErrorString(e));
      }
    }
    e = hipGraphLaunch(exec, st);
  }
  if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("depformer launch: ") + hipGetErrorString(e));
  return PP_OK;
}

extern "C" pp_status pp_depformer_set_graph(pp_depformer* d, int32_t enable) {
  if (!d) return pp_fail(PP_E_ARG, "depformer is NULL");
  d->use_graph = enable != 0;
  return PP_OK;
}
