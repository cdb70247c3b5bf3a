// Full-sequence (prefill) path of the temporal model: workspace and launch order.
//
// "PersonaPlex native LM audit", section 3: every block of the temporal transformer
// applied to T frames at positions p0..p0+T-1 at once, K and V of every frame left in the
// ring so that decoding continues at position p0+T. From position 0 the frames attend
// among themselves (keys read from the ring); a chunk at p0 > 0 (prompt replay into a
// live ring, section 9 'Startup prompt and clock facts') also attends to the history
// still inside each query's context window. Its keys could be overwritten by the chunk's
// own ring writes, so per layer the history is first gathered from the ring into a
// contiguous key space, the chunk's K and V are written there as well as to the ring, and
// the attention runs over that key space.
#include <hip/hip_runtime.h>

#include <cmath>
#include <string>
#include <vector>

#include "internal.h"
#include "model.h"
#include "pp.h"

using namespace pp;

pp_status pp_model::alloc_prefill() {
  const size_t T = max_T > 0 ? (size_t)max_T : 1;
  const size_t D = cfg.d_model, F = cfg.d_ff, dh = cfg.d_head;
  const size_t esz = bf16 ? 2 : 4;
  const int ns = cfg.n_audio + 1;
  size_t bytes = 0;
  auto take = [&](size_t n) { size_t off = bytes; bytes += (n + 255) / 256 * 256; return off; };
  // host IDs staged for one call: a prefill (T frames), a batched step (max_batch frames) or
  // an embedding sum over batch x T frames (up to max_T x max_batch)
  const size_t id_frames = max_T > 0 ? T * (size_t)max_batch : (size_t)max_batch;
  ids_frames = id_frames;
  const size_t oid = take(sizeof(int32_t) * id_frames * ns);
  size_t ox = 0, ou = 0, oq = 0, oa = 0, og = 0, orope = 0, ovt = 0, okx = 0, ovx = 0, osplit = 0;
  // key space of a chunk: up to context + 15 history keys (start rounded to 16) + T
  x_pitch = (int)((T + cfg.context + 16 + 63) / 64 * 64);
  vt_pitch = x_pitch;
  const size_t H = cfg.n_heads;
  if (max_T > 0) {
    ox = take(sizeof(float) * T * D);
    ou = take(esz * T * D);
    oq = take(esz * T * D);
    oa = take(esz * T * D);
    og = take(esz * T * F);
    orope = take(sizeof(float) * T * dh);
    okx = take(esz * H * x_pitch * dh);
    if (bf16) ovt = take(2 * H * dh * vt_pitch);
    else ovx = take(esz * H * x_pitch * dh);
    if (bf16) {
      // split-K partials of the W_O / W_out / W_in products of short chunks: up to 8
      // splits of 256 x 4096 residual rows, 2 of 256 x 2 d_ff W_in rows at full size
      psplit_bytes = (size_t)64 << 20;
      osplit = take(psplit_bytes);
    }
  }
  if (hipMalloc(&pws, bytes) != hipSuccess) return pp_fail(PP_E_HIP, "hipMalloc of prefill workspace failed");
  if (max_T > 0 && bf16) {
    // the matrix-core products take float16 operands: one float16 copy of every matrix,
    // w * 2^-e with e per matrix (f16e), converted once here (13.15 GB at full size)
    const size_t L = cfg.n_layers;
    const size_t per_layer = (3 * D * D + D * D + 2 * F * D + D * F) * 2;
    if (hipMalloc(&pf16_ws, L * per_layer) != hipSuccess)
      return pp_fail(PP_E_HIP, "hipMalloc of the prefill float16 weights failed");
    char* p = static_cast<char*>(pf16_ws);
    hipError_t e = hipSuccess;
    auto conv = [&](const void* src, size_t n, int w_exp, std::vector<const void*>& dst) {
      dst.push_back(p);
      if (e == hipSuccess) e = launch_bf16_to_f16(src, p, n, w_exp, nullptr);
      p += n * 2;
    };
    for (size_t l = 0; l < L; ++l) {
      conv(w_qkv[l], 3 * D * D, f16e[l].w_qkv, f16_qkv);
      conv(w_o[l], D * D, f16e[l].w_o, f16_o);
      conv(w_in[l], 2 * F * D, f16e[l].w_in, f16_in);
      conv(w_out[l], D * F, f16e[l].w_out, f16_out);
    }
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("converting prefill weights: ") + hipGetErrorString(e));
  }
  char* b = static_cast<char*>(pws);
  ids_dev = reinterpret_cast<int32_t*>(b + oid);
  if (max_T > 0) {
    px = reinterpret_cast<float*>(b + ox);
    pu = b + ou;
    pq = b + oq;
    pa = b + oa;
    pg = b + og;
    prope = reinterpret_cast<float*>(b + orope);
    pkx = b + okx;
    if (bf16) {
      psplit = reinterpret_cast<float*>(b + osplit);
      pvt = b + ovt;
      // columns outside a chunk's keys are read by the attention (as zero-weighted
      // values): keep them finite
      if (hipMemset(pvt, 0, 2 * H * dh * vt_pitch) != hipSuccess)
        return pp_fail(PP_E_HIP, "hipMemset of the prefill V copy failed");
    } else {
      pvx = b + ovx;
    }
  }
  return PP_OK;
}

void pp_model::free_prefill() {
  if (pws) (void)hipFree(pws);
  pws = nullptr;
  if (pf16_ws) (void)hipFree(pf16_ws);
  pf16_ws = nullptr;
}

static pp_status hip_fail(const char* what, hipError_t e) {
  return pp_fail(PP_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// The prefill of T frames whose first-layer inputs are the embedding sums of ids_host, or
// (ids_host == nullptr) given as x_dev [T][d_model] float32 (cached summed embeddings).
static pp_status prefill_impl(pp_model* m, pp_kv* kv, const int32_t* ids_host, const float* x_dev, int32_t T,
                              float* h_out_dev, void* stream) {
  if (!m || !kv || (!ids_host && !x_dev) || !h_out_dev) return pp_fail(PP_E_ARG, "NULL argument");
  if (kv->m != m) return pp_fail(PP_E_ARG, "kv ring belongs to another model");
  if (kv->B != 1) return pp_fail(PP_E_ARG, "prefill needs a batch-1 ring");
  if (m->readers.visible > 0) return pp_fail(PP_E_ARG, "memory readers run in batch-1 decode only");
  const pp_temporal_config& c = m->cfg;
  if (T < 1 || T > c.context || T > m->max_T)
    return pp_fail(PP_E_CAPACITY, "T must be in [1, min(context, max_prefill_T)]");
  const int D = c.d_model, F = c.d_ff, H = c.n_heads, dh = c.d_head, C = c.context;
  if (m->bf16) {
    if (D % 128 || F % 64) return pp_fail(PP_E_ARG, "bf16 prefill needs d_model % 128 == 0 and d_ff % 64 == 0");
    if (dh != 64 && dh != 128) return pp_fail(PP_E_ARG, "bf16 prefill needs d_head 64 or 128");
  } else if (dh != 64 && dh != 128) {
    return pp_fail(PP_E_ARG, "prefill needs d_head 64 or 128");
  }
  pp_status st = ids_host ? m->check_ids(ids_host, (size_t)T * kv->B) : PP_OK;
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = m->bf16;
  const long long p0 = kv->pos;
  // key space of the chunk: key index j is position q0 + j; the queries start at koff
  const int koff = p0 == 0 ? 0 : (int)(((p0 < C - 1 ? p0 : C - 1) + 15) / 16 * 16);
  const long long q0 = p0 - koff;
  int jlo = koff - (int)(p0 < (long long)C - 1 ? p0 : (long long)C - 1);   // the oldest key some query sees
  if (jlo < 0) jlo = 0;

  hipError_t e = hipSuccess;
  if (ids_host) {
    EmbedArgs a{};
    m->embed_tables(a);
    a.out = m->px;
    a.rows = T;
    if ((st = m->stage_ids(ids_host, (size_t)T * a.n_streams, s))) return st;
    a.ids_dev = m->ids_dev;
    e = launch_embed(a, bf, s);
    if (e != hipSuccess) return hip_fail("prefill embed", e);
  } else {
    e = hipMemcpyAsync(m->px, x_dev, sizeof(float) * (size_t)T * D, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_fail("prefill input copy", e);
  }
  e = launch_rope_rows(m->prope, T, p0, dh, std::log(c.rope_theta), s);
  if (e != hipSuccess) return hip_fail("prefill rope table", e);

  const size_t esz = bf ? 2 : 4;
  const size_t per_kv = (size_t)kv->B * H * C * dh * esz;
  float* u32 = bf ? nullptr : static_cast<float*>(m->pu);
  void* u16 = bf ? m->pu : nullptr;
  for (int l = 0; l < c.n_layers; ++l) {
    char* kbase = static_cast<char*>(kv->ring) + (size_t)(2 * l) * per_kv;
    char* vbase = kbase + per_kv;
    const F16Exps fe = bf ? m->f16e[l] : F16Exps{};   // float16 operand scales (zero: none)
    if (koff > 0) {
      GatherArgs ga{};
      ga.k16_exp = fe.k; ga.vt_exp = fe.v;
      ga.kring = kbase; ga.vring = vbase; ga.kx = m->pkx; ga.vx = m->pvx; ga.vt = m->pvt;
      ga.x_pitch = m->x_pitch; ga.vt_pitch = m->vt_pitch; ga.C = C; ga.H = H; ga.dh = dh;
      ga.q0 = q0; ga.jlo = jlo; ga.jhi = koff;
      e = launch_gather_history(ga, bf, s);
      if (e != hipSuccess) return hip_fail("prefill history gather", e);
    }
    e = launch_rmsnorm_rows(m->px, m->norm1[l], (float)c.eps, D, T, u32, u16, false, s, fe.u1);
    if (e != hipSuccess) return hip_fail("prefill norm1", e);

    GemmArgs g{};
    g.A = m->pu; g.B = bf ? m->f16_qkv[l] : m->w_qkv[l]; g.M = T; g.N = 3 * D; g.K = D;
    g.q_out = m->pq; g.kc = kbase; g.vc = vbase; g.rope = m->prope;
    g.D = D; g.dh = dh; g.C = C; g.p0 = (int)(p0 % C);
    g.acc_exp = fe.u1 + fe.w_qkv; g.q16_exp = fe.q; g.k16_exp = fe.k; g.vt_exp = fe.v;
    g.vt = m->pvt; g.vt_pitch = m->vt_pitch;
    if (koff > 0 || bf) {   // the bf16-weight path's attention always reads float16 K from the key space
      g.kx = m->pkx; g.vx = bf ? nullptr : m->pvx; g.x_pitch = m->x_pitch; g.xoff = koff;
    }
    e = launch_gemm(GEPI_QKV, bf, g, m->n_cu, s);
    if (e != hipSuccess) return hip_fail("prefill QKV", e);

    AttnPrefillArgs at{};
    at.q = m->pq; at.vt = m->pvt; at.vt_pitch = m->vt_pitch; at.out = m->pa;
    if (koff > 0 || bf) {
      at.k = m->pkx; at.v = m->pvx; at.k_pitch = m->x_pitch;
    } else {
      at.k = kbase; at.v = vbase; at.k_pitch = C;
    }
    // scores of the scaled float16 Q and K copies: the scale gains 2^(q + k)
    at.T = T; at.H = H; at.C = C; at.koff = koff; at.jlo = jlo;
    at.scale = (float)std::ldexp(1.0 / std::sqrt((double)dh), fe.q + fe.k);
    at.part = m->psplit; at.part_bytes = m->psplit_bytes; at.n_cu = m->n_cu;
    e = launch_attn_prefill(at, bf, dh, s);
    if (e != hipSuccess) return hip_fail("prefill attention", e);

    GemmArgs go{};
    go.A = m->pa; go.B = bf ? m->f16_o[l] : m->w_o[l]; go.M = T; go.N = D; go.K = D; go.x = m->px;
    go.acc_exp = fe.v + fe.w_o;
    go.part = m->psplit; go.part_bytes = m->psplit_bytes;
    e = launch_gemm(GEPI_RESID, bf, go, m->n_cu, s);
    if (e != hipSuccess) return hip_fail("prefill W_O", e);

    e = launch_rmsnorm_rows(m->px, m->norm2[l], (float)c.eps, D, T, u32, u16, false, s, fe.u2);
    if (e != hipSuccess) return hip_fail("prefill norm2", e);

    GemmArgs gi{};
    gi.A = m->pu; gi.B = bf ? m->f16_in[l] : m->w_in[l]; gi.M = T; gi.N = F; gi.K = D; gi.F = F; gi.s_out = m->pg;
    gi.acc_exp = fe.u2 + fe.w_in; gi.s16_exp = fe.s;
    gi.part = m->psplit; gi.part_bytes = m->psplit_bytes;
    e = launch_gemm(GEPI_SWIGLU, bf, gi, m->n_cu, s);
    if (e != hipSuccess) return hip_fail("prefill W_in", e);

    GemmArgs gw{};
    gw.A = m->pg; gw.B = bf ? m->f16_out[l] : m->w_out[l]; gw.M = T; gw.N = D; gw.K = F; gw.x = m->px;
    gw.acc_exp = fe.s + fe.w_out; gw.tag = 1;
    gw.part = m->psplit; gw.part_bytes = m->psplit_bytes;
    e = launch_gemm(GEPI_RESID, bf, gw, m->n_cu, s);
    if (e != hipSuccess) return hip_fail("prefill W_out", e);
  }
  e = launch_rmsnorm_rows(m->px, m->out_norm, (float)c.eps, D, T, h_out_dev, nullptr, false, s);
  if (e != hipSuccess) return hip_fail("prefill final norm", e);
  kv->pos = p0 + T;
  return PP_OK;
}

extern "C" pp_status pp_temporal_prefill(pp_model* m, pp_kv* kv, const int32_t* ids_host, int32_t T,
                                         float* h_out_dev, void* stream) {
  if (!ids_host) return pp_fail(PP_E_ARG, "NULL argument");
  return prefill_impl(m, kv, ids_host, nullptr, T, h_out_dev, stream);
}

extern "C" pp_status pp_temporal_prefill_embedded(pp_model* m, pp_kv* kv, const float* x_dev, int32_t T,
                                                  float* h_out_dev, void* stream) {
  if (!x_dev) return pp_fail(PP_E_ARG, "NULL argument");
  return prefill_impl(m, kv, nullptr, x_dev, T, h_out_dev, stream);
}
