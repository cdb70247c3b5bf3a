// Memory readers of the temporal stack: attachment, memory rows, visibility.
//
// "Current sequence memory: one writer, four readers" (PersonaPlex + Inkling page),
// section 6: a reader after temporal block l adds
//   W_O softmax-attention(W_Q LayerNorm(z) + b_Q; memory keys, values) + b_O
// to the residual stream z; with no visible memory row it adds nothing. The keys and
// values of the memory rows are formed when rows are written (csrc/reader.hip); each
// decode step runs, after the reader's block: the LayerNorm + query GEMV (bias via the
// GEMV's additive input), the ring attention kernel over the visible rows, and the output
// GEMV adding into the residual stream (bias likewise).
#include <hip/hip_runtime.h>

#include <cmath>
#include <string>

#include "internal.h"
#include "model.h"
#include "pp.h"

using namespace pp;

pp_model::ReaderSet::~ReaderSet() {
  if (ws) (void)hipFree(ws);
}

extern "C" pp_status pp_readers_attach(pp_model* m, const pp_reader_config* cfg, const pp_reader_weights* w) {
  if (!m || !cfg || !w) return pp_fail(PP_E_ARG, "NULL argument");
  if (m->readers.n > 0) return pp_fail(PP_E_ARG, "readers are already attached");
  const pp_temporal_config& c = m->cfg;
  const int n = cfg->n_readers;
  if (n < 1 || n > 8) return pp_fail(PP_E_ARG, "n_readers must be in [1, 8]");
  if (cfg->mem_dim < 16 || cfg->mem_dim % 16) return pp_fail(PP_E_ARG, "mem_dim must be a positive multiple of 16");
  if (cfg->max_slots < 1) return pp_fail(PP_E_ARG, "max_slots must be >= 1");
  if (c.d_model % 64) return pp_fail(PP_E_ARG, "readers need d_model % 64 == 0");
  if (!(cfg->ln_eps >= 0)) return pp_fail(PP_E_ARG, "ln_eps must be >= 0");
  for (int i = 0; i < n; ++i) {
    if (cfg->blocks[i] < 0 || cfg->blocks[i] >= c.n_layers) return pp_fail(PP_E_ARG, "reader block out of range");
    for (int j = 0; j < i; ++j)
      if (cfg->blocks[j] == cfg->blocks[i]) return pp_fail(PP_E_ARG, "two readers after one block");
    const pp_reader_weights& r = w[i];
    if (!r.ln_w || !r.ln_b || !r.w_q || !r.b_q || !r.w_k || !r.b_k || !r.w_v || !r.b_v || !r.w_o || !r.b_o)
      return pp_fail(PP_E_ARG, "reader " + std::to_string(i) + " has a NULL weight");
  }
  const size_t esz = m->bf16 ? 2 : 4;
  const size_t per = (size_t)c.n_heads * cfg->max_slots * c.d_head * esz;
  pp_model::ReaderSet& rs = m->readers;
  if (hipMalloc(&rs.ws, 2 * per * n) != hipSuccess) return pp_fail(PP_E_HIP, "hipMalloc of the reader keys/values failed");
  for (int i = 0; i < n; ++i) {
    pp_model::Reader r{};
    r.block = cfg->blocks[i];
    r.w = w[i];
    r.K = static_cast<char*>(rs.ws) + 2 * per * i;
    r.V = static_cast<char*>(r.K) + per;
    rs.r.push_back(r);
  }
  rs.n = n;
  rs.mem_dim = cfg->mem_dim;
  rs.max_slots = cfg->max_slots;
  rs.eps = cfg->ln_eps;
  rs.visible = 0;
  ++m->graph_gen;
  return PP_OK;
}

extern "C" pp_status pp_readers_write(pp_model* m, const void* mem_dev, int32_t slot0, int32_t n, void* stream) {
  if (!m || !mem_dev) return pp_fail(PP_E_ARG, "NULL argument");
  pp_model::ReaderSet& rs = m->readers;
  if (rs.n == 0) return pp_fail(PP_E_ARG, "no readers attached");
  if (slot0 < 0 || n < 0 || (long long)slot0 + n > rs.max_slots)
    return pp_fail(PP_E_CAPACITY, "memory rows outside [0, max_slots)");
  const pp_temporal_config& c = m->cfg;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (const pp_model::Reader& r : rs.r) {
    ReaderKvArgs a{};
    a.mem = mem_dev; a.n = n; a.slot0 = slot0; a.mem_dim = rs.mem_dim; a.D = c.d_model; a.dh = c.d_head;
    a.max_slots = rs.max_slots;
    a.W = r.w.w_k; a.bias = r.w.b_k; a.out = r.K;
    hipError_t e = launch_reader_kv(a, m->bf16, s);
    if (e == hipSuccess) {
      a.W = r.w.w_v; a.bias = r.w.b_v; a.out = r.V;
      e = launch_reader_kv(a, m->bf16, s);
    }
    if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("reader keys/values: ") + hipGetErrorString(e));
  }
  return PP_OK;
}

extern "C" pp_status pp_readers_set_visible(pp_model* m, int32_t n_visible) {
  if (!m) return pp_fail(PP_E_ARG, "model is NULL");
  pp_model::ReaderSet& rs = m->readers;
  if (rs.n == 0) return pp_fail(PP_E_ARG, "no readers attached");
  if (n_visible < 0 || n_visible > rs.max_slots) return pp_fail(PP_E_CAPACITY, "n_visible outside [0, max_slots]");
  if (n_visible != rs.visible) {
    rs.visible = n_visible;
    ++m->graph_gen;   // the captured decode graph holds the count by value
  }
  return PP_OK;
}

// The reader after block l, if any and if some memory row is visible (decode, batch 1).
hipError_t pp_model::enqueue_reader(int l, hipStream_t s, const DecodeBufs& b) {
  if (readers.visible <= 0) return hipSuccess;
  const pp_temporal_config& c = cfg;
  const int D = c.d_model, H = c.n_heads, dh = c.d_head;
  for (const Reader& r : readers.r) {
    if (r.block != l) continue;
    GemvArgs gq{};
    gq.W = r.w.w_q; gq.x = b.x; gq.alpha = r.w.ln_w; gq.beta = r.w.ln_b; gq.eps = (float)readers.eps;
    gq.K = D; gq.n_groups = D / 2; gq.out = b.q; gq.add = r.w.b_q;
    hipError_t e = launch_gemv(PRO_LAYERNORM, EPI_STORE, bf16, 2, gq, gemv_blocks, s);
    if (e != hipSuccess) return e;
    const bool merge_in_wo = S <= 8 && D <= 4096;
    AttnDecodeArgs at{};
    at.q = b.q; at.k = r.K; at.v = r.V; at.state = b.state; at.pos = readers.visible - 1; at.C = readers.max_slots;
    at.H = H; at.S = S; at.scale = 1.0f / std::sqrt((float)dh); at.part_o = b.part_o; at.part_ml = b.part_ml;
    at.out = b.o; at.combine = merge_in_wo ? 0 : 1;
    if ((e = launch_attn_decode(at, bf16, dh, s)) != hipSuccess) return e;
    GemvArgs go{};
    go.W = r.w.w_o; go.x = b.o; go.K = D; go.n_groups = D / 2; go.out = b.x; go.add = r.w.b_o;
    go.po = b.part_o; go.pml = b.part_ml; go.pS = S; go.adh = dh;
    return launch_gemv(merge_in_wo ? PRO_ATTN_MERGE : PRO_COPY, EPI_RESID, bf16, 2, go, gemv_blocks, s);
  }
  return hipSuccess;
}
