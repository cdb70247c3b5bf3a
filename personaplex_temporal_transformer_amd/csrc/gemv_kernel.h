// Matrix-vector kernels for batch-1 decode (template; each gemv_*.hip instantiates one
// prologue/epilogue kind so that the kinds compile in parallel): y = W x with W [rows][K] row-major.
//
// At batch 1 every weight byte is used once per step, so these kernels are bound by HBM
// bandwidth, not by arithmetic: each wave streams whole rows with 16-byte non-temporal
// loads (a wave reads 1 KB contiguous per load instruction), keeps several rows and
// chunks in flight, and reduces each row with a fixed-order butterfly. The input vector
// is staged once per workgroup in LDS (float32), optionally RMS-normalised on the way.
//
// Fused prologue / epilogues follow "PersonaPlex native LM audit", section 3 ('One of
// the 32 temporal blocks', 'Positions, attention mask and final text head'):
//   PRO_RMSNORM  x <- alpha * x / sqrt(mean(x^2) + eps) in float32
//   PRO_LAYERNORM  x <- alpha * (x - mean(x)) / sqrt(mean((x - mean(x))^2) + eps) + beta
//                (the memory readers' query norm, "Current sequence memory: one writer,
//                four readers", section 6; two workgroup reductions, mean first)
//   PRO_ATTN_MERGE  x <- merge of the decode-attention split partials (online-softmax
//                rescaling by 2^(m_s - max m), the maxima being in base-2 units, divided
//                by the merged sum)
//   PRO_DEPTH_ATTN  x <- softmax attention of the depth query over this frame's depth
//                cache (no RoPE; window 0 <= q - q' < win), recomputed by each workgroup
//                ("PersonaPlex native LM audit", section 4, 'One depth block at position q')
//   EPI_QKV      rows Q|K|V of in_proj; RoPE on adjacent pairs (2j, 2j+1) of Q and K at
//                the frame's absolute position with omega_j = theta^(-2j/d_head) (the
//                per-position cos/sin table is formed in float64 by the embedding kernel);
//                Q -> float32 buffer, K (rotated) and V (raw) -> ring slot pos mod C
//                (section 6, temporal attention cache)
//   EPI_SWIGLU   ActivationGating: rows i (g) and F+i (z) of linear_in give SiLU(g) * z
//   EPI_RESID    residual add into the float32 stream
//   EPI_DEPTH_QKV  depth block QKV slice: q -> buffer, K and V -> depth cache row q
#pragma once

#include "device.h"
#include "internal.h"

namespace pp {

template <int RB, int EPI>
__device__ __forceinline__ int row_of(const GemvArgs& a, int g, int r) {
  if (EPI == EPI_SWIGLU) {
    constexpr int P = RB / 2;
    return r < P ? g * P + r : a.F + g * P + (r - P);
  }
  return g * RB + r;
}

// pos: the frame's position and ropes: its cos/sin table in LDS (EPI_QKV; read in the
// prologue, ahead of the weight loads, so the epilogue does not wait on global memory).
template <typename WT, int RB, int EPI>
__device__ __forceinline__ void epilogue(const GemvArgs& a, int g, const float (&acc)[RB], const float (&res)[RB],
                                         long long pos, const float* ropes) {
  if (EPI == EPI_STORE) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int row = g * RB + r;
      a.out[row] = acc[r] + (a.add ? a.add[row] : 0.f);
    }
  } else if (EPI == EPI_RESID) {
#pragma unroll
    for (int r = 0; r < RB; ++r) a.out[g * RB + r] = res[r] + (acc[r] + (a.add ? a.add[g * RB + r] : 0.f));
  } else if (EPI == EPI_SWIGLU) {
    constexpr int P = RB / 2;
#pragma unroll
    for (int p = 0; p < P; ++p) a.out[g * P + p] = silu(acc[p]) * acc[P + p];
  } else if (EPI == EPI_QKV) {
    const int slot = (int)(pos % a.C);
#pragma unroll
    for (int p = 0; p < RB / 2; ++p) {
      const int row = g * RB + 2 * p;
      const int sec = row / a.D;             // 0 = Q, 1 = K, 2 = V
      const int w = row - sec * a.D;
      const int head = w / a.dh, d = w - head * a.dh;
      float y0 = acc[2 * p], y1 = acc[2 * p + 1];
      if (sec < 2) {
        const float c = ropes[d], s = ropes[d + 1];
        const float r0 = y0 * c - y1 * s, r1 = y0 * s + y1 * c;
        y0 = r0;
        y1 = r1;
      }
      if (sec == 0) {
        a.out[w] = y0;
        a.out[w + 1] = y1;
      } else {
        WT* base = static_cast<WT*>(sec == 1 ? a.kc : a.vc) + ((size_t)head * a.C + slot) * a.dh + d;
        Elem<WT>::store1(base, y0);
        Elem<WT>::store1(base + 1, y1);
      }
    }
  } else if (EPI == EPI_DEPTH_QKV) {
    const int slot = a.slot_override;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int row = g * RB + r;
      const int sec = row / a.D;
      const int w = row - sec * a.D;
      const int head = w / a.dh, d = w - head * a.dh;
      if (sec == 0)
        a.out[w] = acc[r];
      else
        (static_cast<float*>(sec == 1 ? a.kc : a.vc))[((size_t)head * a.C + slot) * a.dh + d] = acc[r];
    }
  }
}

// Depth attention for every head into x (element i stored at xpos(i)): scores
// q.k * scale over the keys of positions [aq_pos - awin + 1, aq_pos] (clipped at 0),
// softmax with max subtraction, then the weighted sum of values. Wave w takes heads w,
// w + nw, ... two at a time (head pairs w + 2p*nw, w + (2p+1)*nw), issuing both heads' q,
// K and V reads before either head's reductions, so the pair costs one memory latency;
// lane l holds head dimensions l and l + 64 (d_head <= 128), so every q, K and V read is a
// coalesced row segment. Keys go in batches of 8 (one batch for the usual window of 8) whose
// K and V reads are all issued together; each score is a wave-wide sum (every lane gets the
// same bits) and the softmax runs online across batches. Per head the arithmetic and its
// order do not depend on the pairing.
template <class XPos>
__device__ void depth_attention(const GemvArgs& a, float* x, XPos xpos) {
  constexpr int KB = 8, HP = 2;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int k0 = a.aq_pos - a.awin + 1 > 0 ? a.aq_pos - a.awin + 1 : 0;
  const int nk = a.aq_pos - k0 + 1;
  const int dh = a.adh;
  const bool on0 = lane < dh, on1 = lane + 64 < dh;
  for (int hb = w; hb < a.aH; hb += HP * nw) {
    bool hv[HP];
    const float* kh[HP];
    const float* vh[HP];
    float q0[HP], q1[HP], m[HP], l[HP], o0[HP], o1[HP];
#pragma unroll
    for (int u = 0; u < HP; ++u) {
      const int h = hb + u * nw;
      hv[u] = h < a.aH;
      const int hc = hv[u] ? h : hb;  // a missing second head reads the first one's rows
      const float* qh = a.aq + hc * dh;
      kh[u] = a.ak + ((size_t)hc * a.acap + k0) * dh;
      vh[u] = a.av + ((size_t)hc * a.acap + k0) * dh;
      q0[u] = on0 ? qh[lane] : 0.f;
      q1[u] = on1 ? qh[lane + 64] : 0.f;
      m[u] = -INFINITY;
      l[u] = o0[u] = o1[u] = 0.f;
    }
    for (int jb = 0; jb < nk; jb += KB) {
      float kv0[HP][KB], kv1[HP][KB], vv0[HP][KB], vv1[HP][KB];
#pragma unroll
      for (int u = 0; u < HP; ++u)
#pragma unroll
        for (int b = 0; b < KB; ++b) {
          const int j = jb + b;
          const bool ok = j < nk;
          kv0[u][b] = ok && on0 ? kh[u][j * dh + lane] : 0.f;
          kv1[u][b] = ok && on1 ? kh[u][j * dh + lane + 64] : 0.f;
          vv0[u][b] = ok && on0 ? vh[u][j * dh + lane] : 0.f;
          vv1[u][b] = ok && on1 ? vh[u][j * dh + lane + 64] : 0.f;
        }
#pragma unroll
      for (int u = 0; u < HP; ++u) {
        float sc[KB];
        float mb = -INFINITY;
#pragma unroll
        for (int b = 0; b < KB; ++b) {
          sc[b] = -INFINITY;
          if (jb + b < nk) {
            sc[b] = wave_sum(q0[u] * kv0[u][b] + q1[u] * kv1[u][b]) * a.ascale;
            mb = fmaxf(mb, sc[b]);
          }
        }
        const float mn = fmaxf(m[u], mb);                          // finite: the batch has >= 1 key
        const float r = m[u] == -INFINITY ? 0.f : expf(m[u] - mn);  // rescale of the earlier batches
        l[u] *= r;
        o0[u] *= r;
        o1[u] *= r;
#pragma unroll
        for (int b = 0; b < KB; ++b) {
          if (jb + b < nk) {
            const float p = expf(sc[b] - mn);
            l[u] += p;
            o0[u] += p * vv0[u][b];
            o1[u] += p * vv1[u][b];
          }
        }
        m[u] = mn;
      }
    }
#pragma unroll
    for (int u = 0; u < HP; ++u) {
      if (!hv[u]) continue;
      const int h = hb + u * nw;
      const float inv = 1.0f / l[u];
      if (on0) x[xpos(h * dh + lane)] = o0[u] * inv;
      if (on1) x[xpos(h * dh + lane + 64)] = o1[u] * inv;
    }
  }
}

// The depth attention's usual shape (at most two heads per wave, a window of at most 8
// keys, d_head <= 64) in two halves: depth_attn_request issues every q, K and V read of the
// wave's heads with no branch around any of them (rows past the window and lanes past
// d_head read a valid clamped address, and their values are masked), so a caller can
// request its weights behind them and wait for the attention's rows alone (loads complete
// in order); depth_attn_finish then does what depth_attention does for one batch of keys,
// with the same arithmetic in the same order per head.
constexpr int kDepthFastKeys = 8;
struct DepthRows {
  float q[2], k[2][kDepthFastKeys], v[2][kDepthFastKeys];
};

__device__ __forceinline__ bool depth_attn_fast(const GemvArgs& a, int nw) {
  return a.aH <= 2 * nw && a.awin <= kDepthFastKeys && a.adh <= 64;
}

__device__ __forceinline__ void depth_attn_request(const GemvArgs& a, DepthRows& r) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int k0 = a.aq_pos - a.awin + 1 > 0 ? a.aq_pos - a.awin + 1 : 0;
  const int nk = a.aq_pos - k0 + 1;
  const int dh = a.adh;
  const int lc = lane < dh ? lane : 0;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int h = w + u * nw;
    const int hc = h < a.aH ? h : 0;
    r.q[u] = a.aq[hc * dh + lc];
    const size_t base = ((size_t)hc * a.acap + k0) * dh + lc;
#pragma unroll
    for (int b = 0; b < kDepthFastKeys; ++b) {
      const size_t j = (size_t)(b < nk ? b : nk - 1) * dh;
      r.k[u][b] = a.ak[base + j];
      r.v[u][b] = a.av[base + j];
    }
  }
}

template <class XPos>
__device__ __forceinline__ void depth_attn_finish(const GemvArgs& a, const DepthRows& r, float* x, XPos xpos) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int k0 = a.aq_pos - a.awin + 1 > 0 ? a.aq_pos - a.awin + 1 : 0;
  const int nk = a.aq_pos - k0 + 1;
  const int dh = a.adh;
  const bool on = lane < dh;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int h = w + u * nw;
    if (h >= a.aH) continue;
    const float q = on ? r.q[u] : 0.f;
    float sc[kDepthFastKeys];
    float mb = -INFINITY;
#pragma unroll
    for (int b = 0; b < kDepthFastKeys; ++b) {
      // the product and the scaled score are each rounded, as in depth_attention (left
      // contractible, the product would fuse into the first cross-lane addition and the
      // scaling into the softmax's subtraction)
      float t;
      {
#pragma clang fp contract(off)
        const float prod = q * r.k[u][b];
        t = wave_sum(prod) * a.ascale;
      }
      sc[b] = b < nk ? t : -INFINITY;
      mb = fmaxf(mb, sc[b]);
    }
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int b = 0; b < kDepthFastKeys; ++b) {
      if (b < nk) {
        const float p = expf(sc[b] - mb);
        l += p;
        o += p * r.v[u][b];
      }
    }
    if (on) x[xpos(h * dh + lane)] = o * (1.0f / l);
  }
}

constexpr int kGemvWaves = 8;                 // waves per GEMV workgroup

// Rows are processed in groups of RB rows; a lane streams 16-byte chunks c = p*64*U +
// u*64 + lane (u < U) of each row in pass p, so a wave reads 1 KB contiguous per load.
// Block b owns the contiguous groups [b*G/nb, (b+1)*G/nb) -- equal shares, so a grid of
// one block per CU is balanced -- and wave w takes groups w, w+NW, w+2NW, ... of them.
//
// Latency hiding: x is loaded first, then the first item's weights, and x is staged in
// LDS while those weights are in flight (global loads complete in order, and the LDS-only
// barrier does not wait for them). In the loop, as soon as a buffer has been consumed
// it is refilled with the item two steps ahead, so two items of weights are in flight.
// ONEPASS (a row fits in one pass of U chunks per lane): each lane then keeps its slice
// of x in registers; otherwise x is read from LDS per pass.
// MM: rows come from the pointer table a.mats (several matrices, rows_per_mat each);
// FULL: every pass covers whole chunks (K / chunk is a multiple of 64*U), no guards.
//
// Block `blk` of `nblk` takes its share of the row groups; `xs` is the LDS copy of x.
template <typename WT, int RB, int U, bool ONEPASS, int PRO, int EPI, bool MM, bool FULL, int XR>
__device__ __forceinline__ void gemv_body(const GemvArgs& a, float* xs, int blk, int nblk) {
  constexpr int NW = kGemvWaves, NT = NW * 64;
  __shared__ float red[NW];
  __shared__ float red2[PRO == PRO_LAYERNORM ? NW : 1];
  __shared__ float ropes[EPI == EPI_QKV ? 256 : 1];
  constexpr int EPC = Elem<WT>::kPerChunk;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int K = a.K;
  const int nch = K / EPC;
  const int np = ONEPASS ? 1 : (nch + kWave * U - 1) / (kWave * U);
  const int gb0 = (int)((long long)blk * a.n_groups / nblk);
  const int gb1 = (int)((long long)(blk + 1) * a.n_groups / nblk);
  // LDS copy of x, quarter-chunk planes: float4 e of chunk c at (e * NCP + c) * 4, so the
  // lanes of a wave (consecutive chunks) read consecutive 16-byte words, conflict-free.
  constexpr int NCP = XR * NT * 4 / EPC;  // chunks per plane (padded)
  auto xq_index = [&](int c, int e) { return (e * NCP + c) * 4; };

  // ---- weights of one (group, pass) item; the residual rows of a group are read
  // before its weights (EPI_RESID), so waiting for them never waits for later weights
  auto issue = [&](u32x4 (&buf)[RB][U], float (&res)[RB], int gg, int pp) {
    if (EPI == EPI_RESID && pp == 0) {
#pragma unroll
      for (int r = 0; r < RB; ++r) res[r] = a.out[gg * RB + r];
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int row = row_of<RB, EPI>(a, gg, r);
      const char* rp;
      if constexpr (MM)
        rp = static_cast<const char*>(a.mats[row / a.rows_per_mat]) + (size_t)(row % a.rows_per_mat) * K * sizeof(WT);
      else
        rp = static_cast<const char*>(a.W) + (size_t)row * K * sizeof(WT);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = pp * kWave * U + u * kWave + lane;
        if (FULL)
          buf[r][u] = load_stream(rp + (size_t)c * 16);
        else
          buf[r][u] = c < nch ? load_stream(rp + (size_t)c * 16) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto next_g = [&](int gg, int pp) { return pp + 1 < np ? gg : gg + NW; };
  auto next_p = [&](int pp) { return pp + 1 < np ? pp + 1 : 0; };

  int ga = gb0 + wid, pa = 0;
  int gb = next_g(ga, pa), pb = next_p(pa);
  const int g_first = ga < gb1 ? ga : gb1 - 1;  // a valid group of this block (blocks <= groups)
  u32x4 wa[RB][U], wb[RB][U];
  float ra[RB], rb[RB];
  float xr[ONEPASS ? U : 1][EPC];
  long long pos = a.pos;

  if constexpr (PRO == PRO_ATTN_MERGE) {
    // x = merged attention output. Thread t merges dims [8t, 8t+8) of one head from up to
    // 8 split partials; the partials are loaded (clamped, unconditional) before the first
    // item's weights, then merged and staged in LDS while the weights are in flight.
    constexpr int SM = 8;
    const int dh = a.adh;
    const int d0 = tid * 8 < K ? tid * 8 : K - 8;
    const int hh = d0 / dh, dd = d0 - hh * dh;
    f32x4 ov[SM][2];
    float mv[SM], lv[SM];
#pragma unroll
    for (int sp = 0; sp < SM; ++sp) {
      const int sc = sp < a.pS ? sp : a.pS - 1;
      const float* o = a.po + ((size_t)hh * a.pS + sc) * dh + dd;
      ov[sp][0] = *reinterpret_cast<const f32x4*>(o);
      ov[sp][1] = *reinterpret_cast<const f32x4*>(o + 4);
      const float* ml = a.pml + ((size_t)hh * a.pS + sc) * 2;
      mv[sp] = ml[0];
      lv[sp] = ml[1];
    }
    // partials, then the first weights, then the merge: waiting for the partials does not
    // wait for the weights, and the weights are in flight during the merge
    __builtin_amdgcn_sched_barrier(0);
    issue(wa, ra, g_first, 0);
    __builtin_amdgcn_sched_barrier(0);
    float M = -INFINITY;
#pragma unroll
    for (int sp = 0; sp < SM; ++sp) M = fmaxf(M, sp < a.pS ? mv[sp] : -INFINITY);
    float L = 0.f;
    f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sp = 0; sp < SM; ++sp) {
      const float w = (sp < a.pS && mv[sp] != -INFINITY) ? exp2_fast(mv[sp] - M) : 0.f;
      L += w * lv[sp];
      o0 += w * ov[sp][0];
      o1 += w * ov[sp][1];
    }
    const float inv = 1.0f / L;
    // Unconditional: a thread past K stores its clamped chunk's merge again (the same bits
    // as the owner's). Under a bounds test the compiler would sink the partial loads into
    // it, behind the weight loads.
    *reinterpret_cast<f32x4*>(xs + xq_index(d0 / EPC, (d0 % EPC) / 4)) = o0 * inv;
    *reinterpret_cast<f32x4*>(xs + xq_index((d0 + 4) / EPC, ((d0 + 4) % EPC) / 4)) = o1 * inv;
    lds_barrier();
    if (ga >= gb1) return;
    if (gb < gb1) issue(wb, rb, gb, pb);
  } else if constexpr (PRO != PRO_DEPTH_ATTN) {
    // x (and alpha) -> registers, XR float4 per thread, clamped so every load is
    // unconditional; then the first item's weights; then x is staged in LDS (padded to
    // XR*NT*4 floats, so the stores are unconditional too). Straight-line code lets the
    // compiler wait for x alone, and lds_barrier() leaves the weight loads in flight.
    constexpr bool NORM = PRO == PRO_RMSNORM || PRO == PRO_LAYERNORM;
    f32x4 xv[XR], av[NORM ? XR : 1], bv[PRO == PRO_LAYERNORM ? XR : 1];
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      const int k = (i * NT + tid) * 4;
      const int kc = k < K ? k : K - 4;
      xv[i] = *reinterpret_cast<const f32x4*>(a.x + kc);
      if (NORM) av[i] = *reinterpret_cast<const f32x4*>(a.alpha + kc);
      if (PRO == PRO_LAYERNORM) bv[i] = *reinterpret_cast<const f32x4*>(a.beta + kc);
    }
    float rope_v = 0.f;
    if constexpr (EPI == EPI_QKV) {
      rope_v = a.rope[tid < a.dh ? tid : 0];
      if (a.pos < 0) pos = a.state[0];
    }
    issue(wa, ra, g_first, 0);  // unconditional: every block has >= 1 group
    float r = 1.f;
    if (PRO == PRO_RMSNORM) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < XR; ++i) {
        const float q = xv[i].x * xv[i].x + xv[i].y * xv[i].y + xv[i].z * xv[i].z + xv[i].w * xv[i].w;
        ss += (i * NT + tid) * 4 < K ? q : 0.f;
      }
      ss = wave_sum(ss);
      if (lane == 0) red[wid] = ss;
      lds_barrier();
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) tot += red[w];
      r = 1.0f / sqrtf(tot / (float)K + a.eps);
    }
    float mean = 0.f;
    if (PRO == PRO_LAYERNORM) {
      float sm = 0.f;
#pragma unroll
      for (int i = 0; i < XR; ++i) {
        const float q = (xv[i].x + xv[i].y) + (xv[i].z + xv[i].w);
        sm += (i * NT + tid) * 4 < K ? q : 0.f;
      }
      sm = wave_sum(sm);
      if (lane == 0) red[wid] = sm;
      lds_barrier();
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) tot += red[w];
      mean = tot / (float)K;
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < XR; ++i) {
        const f32x4 d = xv[i] - mean;
        const float q = d.x * d.x + d.y * d.y + d.z * d.z + d.w * d.w;
        ss += (i * NT + tid) * 4 < K ? q : 0.f;
      }
      ss = wave_sum(ss);
      if (lane == 0) red2[wid] = ss;
      lds_barrier();
      float var = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) var += red2[w];
      r = 1.0f / sqrtf(var / (float)K + a.eps);
    }
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      f32x4 v = xv[i];
      if (PRO == PRO_RMSNORM) v = (v * r) * av[i];
      if (PRO == PRO_LAYERNORM) v = ((v - mean) * r) * av[i] + bv[PRO == PRO_LAYERNORM ? i : 0];
      const int k = (i * NT + tid) * 4;  // float index; chunk k / EPC, quarter (k % EPC) / 4
      *reinterpret_cast<f32x4*>(xs + xq_index(k / EPC, (k % EPC) / 4)) = v;
    }
    if (EPI == EPI_QKV && tid < a.dh) ropes[tid] = rope_v;
    lds_barrier();
    if (ga >= gb1) return;
    if (gb < gb1) issue(wb, rb, gb, pb);
  } else {
    // Usual shape: the attention's rows are requested first and the first two items'
    // weights behind them, so the weights stream while the attention is computed.
    // Otherwise the weights go first and the general loop follows.
    const auto xpos = [&](int i) { return xq_index(i / EPC, (i % EPC) / 4) + (i % 4); };
    const bool fast = depth_attn_fast(a, NW);
    DepthRows dr;
    if (fast) depth_attn_request(a, dr);
    if (ga < gb1) issue(wa, ra, ga, pa);
    if (gb < gb1) issue(wb, rb, gb, pb);
    if (fast) depth_attn_finish(a, dr, xs, xpos);
    else depth_attention(a, xs, xpos);
    __syncthreads();
    if (ga >= gb1) return;
  }
  if constexpr (ONEPASS) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = u * kWave + lane;
#pragma unroll
      for (int e = 0; e < EPC; e += 4) {
        const f32x4 t = (FULL || c < nch) ? *reinterpret_cast<const f32x4*>(xs + xq_index(c, e / 4)) : f32x4{0.f, 0.f, 0.f, 0.f};
        xr[u][e] = t.x; xr[u][e + 1] = t.y; xr[u][e + 2] = t.z; xr[u][e + 3] = t.w;
      }
    }
  }

  float acc[RB], rg[RB];  // rg: residual rows of the group being accumulated
#pragma unroll
  for (int r = 0; r < RB; ++r) acc[r] = rg[r] = 0.f;

  auto consume = [&](const u32x4 (&buf)[RB][U], const float (&res)[RB], int gg, int pp) {
    // the residual was fetched with the group's first pass; the epilogue runs after its
    // last pass, which may sit in the other buffer
    if (EPI == EPI_RESID && pp == 0) {
#pragma unroll
      for (int r = 0; r < RB; ++r) rg[r] = res[r];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = pp * kWave * U + u * kWave + lane;
      float xw[EPC];
      if (ONEPASS) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) xw[e] = xr[u][e];
      } else if (FULL || c < nch) {
#pragma unroll
        for (int e = 0; e < EPC; e += 4) {
          const f32x4 t = *reinterpret_cast<const f32x4*>(xs + xq_index(c, e / 4));
          xw[e] = t.x; xw[e + 1] = t.y; xw[e + 2] = t.z; xw[e + 3] = t.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < EPC; ++e) xw[e] = 0.f;
      }
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        float wf[EPC];
        Elem<WT>::widen(buf[r][u], wf);
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[r] += wf[e] * xw[e];
      }
    }
    if (pp + 1 == np) {
#pragma unroll
      for (int r = 0; r < RB; ++r) acc[r] = wave_sum(acc[r]);
      if (lane == 0) epilogue<WT, RB, EPI>(a, gg, acc, rg, pos, ropes);
#pragma unroll
      for (int r = 0; r < RB; ++r) acc[r] = 0.f;
    }
  };

  // ---- 4. two buffers in flight: consume one, refill it two items ahead
  while (true) {
    consume(wa, ra, ga, pa);
    const int gc = next_g(gb, pb), pc = next_p(pb);
    if (gb >= gb1) break;
    if (gc < gb1) issue(wa, ra, gc, pc);
    consume(wb, rb, gb, pb);
    const int gd = next_g(gc, pc), pd = next_p(pc);
    if (gc >= gb1) break;
    if (gd < gb1) issue(wb, rb, gd, pd);
    ga = gc; pa = pc;
    gb = gd; pb = pd;
  }
}

template <typename WT, int RB, int U, bool ONEPASS, int PRO, int EPI, bool MM, bool FULL, int XR>
__global__ __launch_bounds__(kGemvWaves * 64) void k_gemv(GemvArgs a) {
  extern __shared__ float xs[];
  gemv_body<WT, RB, U, ONEPASS, PRO, EPI, MM, FULL, XR>(a, xs, blockIdx.x, gridDim.x);
}

template <typename WT, int RB, int U, bool OP, int PRO, int EPI, int XR>
static void launch_x(const GemvArgs& a, dim3 grid, dim3 block, size_t lds, hipStream_t s) {
  constexpr int EPC = Elem<WT>::kPerChunk;
  const bool full = (a.K / EPC) % (kWave * U) == 0;
  if constexpr (PRO == PRO_COPY && EPI == EPI_STORE) {
    if (a.rows_per_mat > 0) {
      if (full) hipLaunchKernelGGL((k_gemv<WT, RB, U, OP, PRO, EPI, true, true, XR>), grid, block, lds, s, a);
      else hipLaunchKernelGGL((k_gemv<WT, RB, U, OP, PRO, EPI, true, false, XR>), grid, block, lds, s, a);
      return;
    }
  }
  if (full) hipLaunchKernelGGL((k_gemv<WT, RB, U, OP, PRO, EPI, false, true, XR>), grid, block, lds, s, a);
  else hipLaunchKernelGGL((k_gemv<WT, RB, U, OP, PRO, EPI, false, false, XR>), grid, block, lds, s, a);
}

// XR: float4 of x per thread in the prologue; the LDS copy of x is padded to XR*NT*4 floats.
constexpr int kXPer = kGemvWaves * 64 * 4;
static int x_regs(int K) { return K <= kXPer ? 1 : (K <= 2 * kXPer ? 2 : 6); }

template <typename WT, int RB, int U, bool OP, int PRO, int EPI>
static void launch_u(const GemvArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  const int xr = x_regs(a.K);
  const size_t lds = (size_t)xr * kXPer * sizeof(float);
  if (xr == 1) launch_x<WT, RB, U, OP, PRO, EPI, 1>(a, grid, block, lds, s);
  else if (xr == 2) launch_x<WT, RB, U, OP, PRO, EPI, 2>(a, grid, block, lds, s);
  else launch_x<WT, RB, U, OP, PRO, EPI, 6>(a, grid, block, lds, s);
}

template <typename WT, int RB, int PRO, int EPI>
static hipError_t dispatch_u(const GemvArgs& a, int blocks, hipStream_t s) {
  constexpr int EPC = Elem<WT>::kPerChunk;
  const int nch = a.K / EPC;
  const dim3 grid(blocks), block(kGemvWaves * 64);
  if (a.K % EPC != 0 || a.K > 6 * kXPer) return hipErrorInvalidValue;
  if (PRO == PRO_DEPTH_ATTN && a.K > kXPer) return hipErrorInvalidValue;
  if (PRO == PRO_ATTN_MERGE && (a.K > kGemvWaves * 64 * 8 || a.pS < 1 || a.pS > 8 || a.adh % 8)) return hipErrorInvalidValue;
  if (a.rows_per_mat > 0 && (PRO != PRO_COPY || EPI != EPI_STORE)) return hipErrorInvalidValue;
  if (nch <= kWave * 1) launch_u<WT, RB, 1, true, PRO, EPI>(a, grid, block, s);
  else if (nch <= kWave * 2) launch_u<WT, RB, 2, true, PRO, EPI>(a, grid, block, s);
  else if (nch <= kWave * 4) launch_u<WT, RB, 4, true, PRO, EPI>(a, grid, block, s);
  else if (nch <= kWave * 6) launch_u<WT, RB, 6, true, PRO, EPI>(a, grid, block, s);
  else if (nch <= kWave * 8) launch_u<WT, RB, 8, true, PRO, EPI>(a, grid, block, s);
  else if (RB == 1 && nch % (kWave * 11) == 0) launch_u<WT, RB, (RB == 1 ? 11 : 8), false, PRO, EPI>(a, grid, block, s);
  else if (PRO == PRO_COPY && EPI == EPI_RESID && RB == 2 && nch % (kWave * 11) == 0)
    launch_u<WT, RB, (PRO == PRO_COPY && EPI == EPI_RESID ? 11 : 8), false, PRO, EPI>(a, grid, block, s);
  else launch_u<WT, RB, 8, false, PRO, EPI>(a, grid, block, s);
  return hipGetLastError();
}

template <typename WT, int PRO, int EPI>
static hipError_t dispatch_rb(int rb, const GemvArgs& a, int blocks, hipStream_t s) {
  if (rb == 2) return dispatch_u<WT, 2, PRO, EPI>(a, blocks, s);
  if constexpr (EPI != EPI_SWIGLU && EPI != EPI_QKV) {
    if (rb == 1) return dispatch_u<WT, 1, PRO, EPI>(a, blocks, s);
  }
  return hipErrorInvalidValue;
}

// One prologue/epilogue kind for both weight types; defined in gemv_<kind>.hip.
template <int PRO, int EPI>
hipError_t launch_gemv_kind(int rb, bool bf16, const GemvArgs& a, int blocks, hipStream_t s) {
  return bf16 ? dispatch_rb<bf16_t, PRO, EPI>(rb, a, blocks, s) : dispatch_rb<float, PRO, EPI>(rb, a, blocks, s);
}

}  // namespace pp
