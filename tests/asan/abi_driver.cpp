// Host-side sanitizer driver for libpp: every entry point of pp.h, on small models with
// random weights, including the error paths (bad handles, IDs, sizes, capacities), so that
// the library's host code (validation, handle lifetimes, workspace carving, graph capture,
// staging buffers) runs under AddressSanitizer. Built against a library whose host code is
// instrumented (the device code is not); results are checked only for status codes and
// finiteness -- numerical parity is the GPU tests' business.
//
// Exit status 0 and a final "abi_driver: ok" line mean every check passed; ASan aborts the
// process on the first memory error it finds.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "pp.h"

static int g_fail = 0;
#define EXPECT(cond)                                                          \
  do {                                                                        \
    if (!(cond)) {                                                            \
      std::printf("FAILED %s:%d: %s (%s)\n", __FILE__, __LINE__, #cond, pp_last_error()); \
      ++g_fail;                                                               \
    }                                                                         \
  } while (0)
#define OK(call) EXPECT((call) == PP_OK)

static unsigned long long g_rng = 0x9E3779B97F4A7C15ull;
static float urand() {   // uniform in [-1, 1)
  g_rng = g_rng * 6364136223846793005ull + 1442695040888963407ull;
  return (float)((g_rng >> 40) & 0xFFFFFF) / 8388608.0f - 1.0f;
}
static uint16_t to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static std::vector<void*> g_allocs;
static void* dev_bf16(size_t n, float scale) {
  std::vector<uint16_t> h(n);
  for (auto& v : h) v = to_bf16(scale * urand());
  void* p = nullptr;
  if (hipMalloc(&p, n * 2) != hipSuccess || hipMemcpy(p, h.data(), n * 2, hipMemcpyHostToDevice) != hipSuccess) {
    std::printf("FAILED: device allocation\n");
    std::exit(2);
  }
  g_allocs.push_back(p);
  return p;
}
static float* dev_f32(size_t n, float base, float scale) {
  std::vector<float> h(n);
  for (auto& v : h) v = base + scale * urand();
  void* p = nullptr;
  if (hipMalloc(&p, n * 4) != hipSuccess || hipMemcpy(p, h.data(), n * 4, hipMemcpyHostToDevice) != hipSuccess) {
    std::printf("FAILED: device allocation\n");
    std::exit(2);
  }
  g_allocs.push_back(p);
  return static_cast<float*>(p);
}
static void* dev_zero(size_t bytes) {
  void* p = nullptr;
  if (hipMalloc(&p, bytes) != hipSuccess || hipMemset(p, 0, bytes) != hipSuccess) std::exit(2);
  g_allocs.push_back(p);
  return p;
}

int main() {
  // ---- host-only error paths (no device needed)
  EXPECT(pp_temporal_create(nullptr, nullptr, 1, 0, nullptr) == PP_E_ARG);
  EXPECT(pp_kv_free(nullptr) == PP_E_ARG);
  EXPECT(pp_temporal_destroy(nullptr) == PP_E_ARG);
  EXPECT(pp_temporal_decode_step(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == PP_E_ARG);
  EXPECT(pp_temporal_decode_step_noalloc(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == PP_E_ARG);
  EXPECT(pp_depformer_step(nullptr, nullptr, nullptr, nullptr, 1, nullptr, nullptr, nullptr) == PP_E_ARG);
  EXPECT(pp_generator_step(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == PP_E_ARG);
  EXPECT(pp_last_error() != nullptr);

  int n_dev = 0;
  if (hipGetDeviceCount(&n_dev) != hipSuccess || n_dev == 0) {
    std::printf("abi_driver: no GPU; host-only checks %s\n", g_fail ? "FAILED" : "ok");
    return g_fail ? 1 : 0;
  }

  // ---- a tiny bf16 temporal model: 2 blocks, d_model 256, 4 heads x 64, d_ff 256
  pp_temporal_config c{};
  c.n_layers = 2; c.d_model = 256; c.n_heads = 4; c.d_head = 64; c.d_ff = 256; c.context = 48;
  c.text_vocab = 33; c.audio_vocab = 17; c.n_audio = 16; c.wdtype = PP_BF16; c.rope_theta = 1e4; c.eps = 1e-8;
  const int D = c.d_model, F = c.d_ff, L = c.n_layers, ns = c.n_audio + 1;
  std::vector<const void*> audio, qkv, wo, win, wout;
  std::vector<const float*> n1, n2;
  for (int i = 0; i < c.n_audio; ++i) audio.push_back(dev_bf16((size_t)c.audio_vocab * D, 0.02f));
  for (int l = 0; l < L; ++l) {
    qkv.push_back(dev_bf16((size_t)3 * D * D, 0.02f));
    wo.push_back(dev_bf16((size_t)D * D, 0.02f));
    win.push_back(dev_bf16((size_t)2 * F * D, 0.02f));
    wout.push_back(dev_bf16((size_t)D * F, 0.02f));
    n1.push_back(dev_f32(D, 1.0f, 0.02f));
    n2.push_back(dev_f32(D, 1.0f, 0.02f));
  }
  pp_temporal_weights w{};
  w.text_emb = dev_bf16((size_t)c.text_vocab * D, 0.02f);
  w.audio_emb = audio.data(); w.norm1 = n1.data(); w.norm2 = n2.data();
  w.w_qkv = qkv.data(); w.w_o = wo.data(); w.w_in = win.data(); w.w_out = wout.data();
  w.out_norm = dev_f32(D, 1.0f, 0.02f);
  w.text_head = dev_bf16((size_t)(c.text_vocab - 1) * D, 0.02f);

  pp_model* m = nullptr;
  pp_temporal_config bad = c;
  bad.d_head = 96;
  EXPECT(pp_temporal_create(&bad, &w, 1, 0, &m) == PP_E_ARG && m == nullptr);
  EXPECT(pp_temporal_create(&c, &w, 1, c.context + 1, &m) == PP_E_CAPACITY);
  OK(pp_temporal_create(&c, &w, 4, 32, &m));

  std::vector<int32_t> ids((size_t)4 * 64 * ns);   // room for the capacity-error calls' declared sizes
  for (size_t i = 0; i < ids.size(); ++i) {
    const int k = (int)(i % ns);
    ids[i] = (int32_t)(((g_rng = g_rng * 6364136223846793005ull + 1) >> 33) % (k == 0 ? c.text_vocab : c.audio_vocab));
    if (i % 19 == 0) ids[i] = -1;
  }
  float* h = static_cast<float*>(dev_zero(sizeof(float) * 4 * 64 * D));
  float* lg = static_cast<float*>(dev_zero(sizeof(float) * 4 * (c.text_vocab - 1)));
  hipStream_t st = nullptr;
  OK(hipStreamCreate(&st) == hipSuccess ? PP_OK : PP_E_HIP);

  // embedding sums, including the batch x T capacity edge
  OK(pp_embed_sum(m, ids.data(), 4, 32, h, st));
  EXPECT(pp_embed_sum(m, ids.data(), 4, 33, h, st) == PP_E_CAPACITY);
  EXPECT(pp_embed_sum(m, ids.data(), 5, 1, h, st) == PP_E_ARG);
  std::vector<int32_t> bad_ids(ids.begin(), ids.begin() + ns);
  bad_ids[3] = -2;
  EXPECT(pp_embed_sum(m, bad_ids.data(), 1, 1, h, st) == PP_E_ID);

  // batch-1 decode: graph and direct, text head, the allocation-free step, splits
  pp_kv* kv = nullptr;
  OK(pp_kv_alloc(m, 1, &kv));
  int64_t pos = -1;
  uint64_t kv_bytes = 0;
  OK(pp_kv_info(kv, &pos, &kv_bytes));
  EXPECT(pos == 0 && kv_bytes == (uint64_t)L * 2 * c.n_heads * c.context * c.d_head * 2);
  for (int t = 0; t < 6; ++t) OK(pp_temporal_decode_step(m, kv, &ids[(size_t)t * ns], h, lg, st));
  OK(pp_temporal_set_graph(m, 0));
  for (int t = 6; t < 9; ++t) OK(pp_temporal_decode_step(m, kv, &ids[(size_t)t * ns], h, nullptr, st));
  OK(pp_temporal_set_attn_splits(m, 3));
  OK(pp_temporal_set_graph(m, 1));
  OK(pp_temporal_decode_step(m, kv, &ids[0], h, nullptr, st));
  EXPECT(pp_temporal_set_attn_splits(m, 65) == PP_E_ARG);
  OK(pp_temporal_set_attn_splits(m, 0));
  for (int t = 0; t < 3; ++t) OK(pp_temporal_decode_step_noalloc(m, kv, &ids[(size_t)t * ns], h, lg, st));
  EXPECT(pp_temporal_decode_step(m, kv, bad_ids.data(), h, nullptr, st) == PP_E_ID);
  OK(pp_temporal_trace(m, 1, 4));
  OK(pp_temporal_decode_step(m, kv, &ids[0], h, nullptr, st));
  int64_t cnt = 0;
  double us = 0;
  OK(pp_temporal_trace_read(m, &cnt, &us));
  EXPECT(cnt == 4 && us > 0);
  OK(pp_temporal_trace(m, -1, 1));

  // ring snapshot / restore / load / reset, prefill and chunks past the ring's end
  void* snap = dev_zero(kv_bytes);
  OK(pp_kv_store(kv, snap, st));
  OK(pp_kv_info(kv, &pos, nullptr));
  OK(pp_kv_restore(kv, snap, pos, st));
  OK(pp_kv_reset(kv));
  OK(pp_temporal_prefill(m, kv, ids.data(), 32, h, st));
  OK(pp_temporal_prefill(m, kv, ids.data(), 30, h, st));      // wraps the 48-slot ring
  EXPECT(pp_temporal_prefill(m, kv, ids.data(), 33, h, st) == PP_E_CAPACITY);
  OK(pp_temporal_prefill_embedded(m, kv, h, 16, h + (size_t)32 * D, st));
  OK(pp_kv_load(kv, snap, 40, st));
  EXPECT(pp_kv_load(kv, snap, c.context + 1, st) == PP_E_CAPACITY);

  // batched decode over 4 sessions
  pp_kv* kv4 = nullptr;
  OK(pp_kv_alloc(m, 4, &kv4));
  pp_kv* kv_bad = nullptr;
  EXPECT(pp_kv_alloc(m, 5, &kv_bad) == PP_E_ARG && kv_bad == nullptr);
  for (int t = 0; t < 5; ++t) OK(pp_temporal_decode_step(m, kv4, &ids[(size_t)t * 4 * ns], h, lg, st));
  EXPECT(pp_temporal_decode_step_noalloc(m, kv4, ids.data(), h, nullptr, st) == PP_E_ARG);
  EXPECT(pp_temporal_prefill(m, kv4, ids.data(), 4, h, st) == PP_E_ARG);

  // memory readers
  pp_reader_config rc{};
  rc.n_readers = 1; rc.blocks[0] = 1; rc.mem_dim = 64; rc.max_slots = 8; rc.ln_eps = 1e-5;
  pp_reader_weights rw{};
  rw.ln_w = dev_f32(D, 1.0f, 0.02f); rw.ln_b = dev_f32(D, 0.0f, 0.02f);
  rw.w_q = dev_bf16((size_t)D * D, 0.02f); rw.b_q = dev_f32(D, 0.0f, 0.02f);
  rw.w_k = dev_bf16((size_t)D * 64, 0.02f); rw.b_k = dev_f32(D, 0.0f, 0.02f);
  rw.w_v = dev_bf16((size_t)D * 64, 0.02f); rw.b_v = dev_f32(D, 0.0f, 0.02f);
  rw.w_o = dev_bf16((size_t)D * D, 0.02f); rw.b_o = dev_f32(D, 0.0f, 0.02f);
  OK(pp_readers_attach(m, &rc, &rw));
  void* mem = dev_bf16((size_t)8 * 64, 1.0f);
  OK(pp_readers_write(m, mem, 0, 8, st));
  EXPECT(pp_readers_write(m, mem, 4, 8, st) == PP_E_CAPACITY);
  OK(pp_readers_set_visible(m, 5));
  OK(pp_temporal_decode_step(m, kv, &ids[0], h, nullptr, st));
  EXPECT(pp_temporal_decode_step_noalloc(m, kv, &ids[0], h, nullptr, st) == PP_E_ARG);
  OK(pp_readers_set_visible(m, 0));

  // depth transformer and the generator frame
  pp_depth_config dc{};
  dc.n_layers = 2; dc.d_model = 128; dc.n_heads = 4; dc.d_head = 32; dc.d_ff = 96; dc.n_steps = 16; dc.window = 8;
  dc.text_vocab = c.text_vocab; dc.audio_vocab = c.audio_vocab; dc.n_out = 16; dc.d_temporal = D;
  dc.wdtype = PP_BF16; dc.eps = 1e-8;
  std::vector<const void*> inp, demb, dqkv, dwo, dwin, dwout, head;
  std::vector<const float*> dn1, dn2;
  for (int q = 0; q < dc.n_steps; ++q) {
    inp.push_back(dev_bf16((size_t)dc.d_model * D, 0.02f));
    head.push_back(dev_bf16((size_t)dc.n_out * dc.d_model, 0.02f));
    if (q < dc.n_steps - 1) demb.push_back(dev_bf16((size_t)dc.audio_vocab * dc.d_model, 0.02f));
  }
  for (int l = 0; l < dc.n_layers; ++l) {
    dqkv.push_back(dev_bf16((size_t)dc.n_steps * 3 * dc.d_model * dc.d_model, 0.02f));
    dwo.push_back(dev_bf16((size_t)dc.n_steps * dc.d_model * dc.d_model, 0.02f));
    dn1.push_back(dev_f32(dc.d_model, 1.0f, 0.02f));
    dn2.push_back(dev_f32(dc.d_model, 1.0f, 0.02f));
    for (int q = 0; q < dc.n_steps; ++q) {
      dwin.push_back(dev_bf16((size_t)2 * dc.d_ff * dc.d_model, 0.02f));
      dwout.push_back(dev_bf16((size_t)dc.d_model * dc.d_ff, 0.02f));
    }
  }
  pp_depth_weights dw{};
  dw.in_proj = inp.data(); dw.text_emb = dev_bf16((size_t)dc.text_vocab * dc.d_model, 0.02f);
  dw.audio_emb = demb.data(); dw.w_qkv = dqkv.data(); dw.w_o = dwo.data(); dw.w_in = dwin.data();
  dw.w_out = dwout.data(); dw.norm1 = dn1.data(); dw.norm2 = dn2.data(); dw.head = head.data();
  pp_depformer* dep = nullptr;
  OK(pp_depformer_create(&dc, &dw, &dep));
  int32_t* codes = static_cast<int32_t*>(dev_zero(sizeof(int32_t) * dc.n_steps));
  float* dlog = static_cast<float*>(dev_zero(sizeof(float) * dc.n_steps * dc.n_out));
  const int32_t tok = 5;
  std::vector<int32_t> forced(dc.n_steps, -1);
  OK(pp_depformer_step(dep, h, &tok, nullptr, 1, codes, dlog, st));
  forced[3] = 7;
  OK(pp_depformer_step(dep, h, &tok, forced.data(), 1, codes, nullptr, st));
  forced[4] = dc.n_out;
  EXPECT(pp_depformer_step(dep, h, &tok, forced.data(), 1, codes, nullptr, st) == PP_E_ID);
  OK(pp_depformer_set_graph(dep, 0));
  OK(pp_depformer_step(dep, h, &tok, nullptr, 1, codes, nullptr, st));

  pp_generator_config gc{};
  gc.n_streams = ns;
  for (int k = 0; k < ns; ++k) gc.delays[k] = (k == 0 || k == 9) ? 0 : 1;
  gc.text_initial = c.text_vocab - 1; gc.audio_initial = c.audio_vocab - 1;
  gc.text_temperature = 0.7f; gc.text_top_k = 25; gc.audio_temperature = 0.8f; gc.audio_top_k = 8;
  pp_generator* gen = nullptr;
  OK(pp_kv_reset(kv));
  OK(pp_generator_create(m, kv, dep, &gc, &gen));
  int32_t* out = static_cast<int32_t*>(dev_zero(sizeof(int32_t) * ns));
  std::vector<double> u(ns, 0.25);
  std::vector<int32_t> prov(ns, -1);
  int32_t has = 0;
  for (int s = 0; s < 4; ++s) OK(pp_generator_step(gen, prov.data(), u.data(), out, &has, st));
  int64_t cur = 0;
  uint64_t gbytes = 0;
  OK(pp_generator_info(gen, &cur, &gbytes));
  EXPECT(cur == 4 && gbytes > 0);
  void* gsnap = dev_zero(gbytes);
  OK(pp_generator_store(gen, gsnap, st));
  OK(pp_generator_step(gen, nullptr, nullptr, out, &has, st));
  OK(pp_generator_restore(gen, gsnap, cur, st));
  prov[2] = c.audio_vocab + 5;
  EXPECT(pp_generator_step(gen, prov.data(), u.data(), out, &has, st) == PP_E_ID);
  OK(pp_generator_inspect(gen, out, nullptr, nullptr, nullptr, st));
  double* ud = static_cast<double*>(dev_zero(sizeof(double) * 2));
  OK(pp_sample_top_k(lg, 1, c.text_vocab - 1, 0.7f, 5, ud, out, st));
  EXPECT(pp_sample_top_k(lg, 1, 0, 0.7f, 5, ud, out, st) == PP_E_ARG);

  OK(hipStreamSynchronize(st) == hipSuccess ? PP_OK : PP_E_HIP);
  std::vector<float> hh(D);
  OK(hipMemcpy(hh.data(), h, sizeof(float) * D, hipMemcpyDeviceToHost) == hipSuccess ? PP_OK : PP_E_HIP);
  for (float v : hh) EXPECT(std::isfinite(v));

  OK(pp_generator_destroy(gen));
  OK(pp_depformer_destroy(dep));
  OK(pp_kv_free(kv4));
  OK(pp_kv_free(kv));
  OK(pp_temporal_destroy(m));
  (void)hipStreamDestroy(st);
  for (void* p : g_allocs) (void)hipFree(p);
  std::printf("abi_driver: %s\n", g_fail ? "FAILED" : "ok");
  return g_fail ? 1 : 0;
}
