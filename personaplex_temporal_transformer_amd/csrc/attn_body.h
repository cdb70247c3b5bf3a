// Decode attention body (split-K over keys).
//
// "PersonaPlex native LM audit", section 3: ordinary multi-head attention (query, key and
// value heads of d_head), scale 1/sqrt(d_head), softmax, no dropout; the declared mask
// admits keys with 0 <= query_pos - key_pos < context. Keys in the ring were rotated at
// their own positions when written. With the frame at position p written into slot
// p mod C first, the visible keys are exactly the slots 0 .. min(p+1, C)-1.
#pragma once

#include "device.h"
#include "frag_layout.h"
#include "internal.h"

namespace pp {

// Block (s, h): one pass over its keys with an online softmax. A group of LPK lanes reads
// one key row at a time (16 bytes per lane); the KPP groups of the block own contiguous,
// equal runs of the block's keys. A round loads NB keys' K and V rows per thread with
// buffer loads (slots past the group's run point out of range and read zeros without
// memory traffic); the next round is always issued before the current one is consumed.
// Each group keeps a running max m, sum l and output o (its lanes' EPC dimensions); the
// groups are merged through LDS at the end, all threads taking part (PARTS partial
// merges per output dimension, then their sum). With one split and a float16 output
// (a batched step whose sessions fill the grid) the block's merge is the head's output for
// session sess, written in the skinny products' fragment order; otherwise the block
// writes its partial.
template <typename KT, int DH, int NB, int NT>
__device__ __forceinline__ void attn_body(const AttnDecodeArgs& a, int s, int h, int sess) {
  constexpr int EPC = Elem<KT>::kPerChunk;  // elements per 16-byte chunk
  constexpr int LPK = DH / EPC;             // lanes per key row
  constexpr int KPP = NT / LPK;             // key groups per block
  constexpr int ROW = DH * (int)sizeof(KT); // bytes per key row
  constexpr int PARTS = NT / DH;            // partial merges per output dimension
  constexpr int GPP = KPP / PARTS;          // groups per partial merge
  static_assert(PARTS * DH == NT && GPP * PARTS == KPP, "merge layout");
  __shared__ float gm[KPP], gl[KPP];
  __shared__ float go[KPP][DH + 1];
  __shared__ float po[PARTS][DH], pl[PARTS];

  const int tid = threadIdx.x;
  const int sub = tid % LPK, kg = tid / LPK;
  const long long pos = a.pos >= 0 ? a.pos : a.state[0];
  const int n = pos + 1 < (long long)a.C ? (int)(pos + 1) : a.C;
  const int j0 = (int)((long long)s * n / a.S), j1 = (int)((long long)(s + 1) * n / a.S);
  const int cnt = j1 - j0;
  const int per_g = (cnt + KPP - 1) / KPP;
  const int gbeg = kg * per_g;
  const int gend = gbeg + per_g < cnt ? gbeg + per_g : cnt;
  const int rounds = (per_g + NB - 1) / NB;   // the same for every group

  float qv[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) qv[e] = a.q[h * DH + sub * EPC + e] * (a.scale * kLog2e);
  const size_t base = ((size_t)h * a.C + j0) * DH;
  const auto rk = make_rsrc(static_cast<const KT*>(a.k) + base, (uint32_t)cnt * ROW);
  const auto rv = make_rsrc(static_cast<const KT*>(a.v) + base, (uint32_t)cnt * ROW);

  float m = -INFINITY, l = 0.f, acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.f;

  auto issue = [&](u32x4 (&ck)[NB], u32x4 (&cv)[NB], int r) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int j = gbeg + r * NB + b;
      const int off = (r < rounds && j < gend) ? j * ROW + sub * 16 : kBufOutOfRange;
      ck[b] = buffer_load16_stream(rk, off);
      cv[b] = buffer_load16_stream(rv, off);
    }
  };
  auto consume = [&](const u32x4 (&ck)[NB], const u32x4 (&cv)[NB], int r) {
    float sc[NB];
    float mb = -INFINITY;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float kf[EPC];
      Elem<KT>::widen(ck[b], kf);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) d += qv[e] * kf[e];
      d = group_sum<LPK>(d);
      const int j = gbeg + r * NB + b;
      sc[b] = j < gend ? d : -INFINITY;
      mb = fmaxf(mb, sc[b]);
    }
    const float mn = fmaxf(m, mb);
    const float mref = mn == -INFINITY ? 0.f : mn;   // nothing visible yet: keep exponents finite
    const float scale = exp2_fast(m - mref);         // m = -inf -> 0
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] *= scale;
    l *= scale;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float p = exp2_fast(sc[b] - mref);       // masked keys: exp2(-inf) = 0
      l += p;
      float vf[EPC];
      Elem<KT>::widen(cv[b], vf);
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[e] += p * vf[e];
    }
    m = mn;
  };

  u32x4 ka[NB], va[NB], kb[NB], vb[NB];
  issue(ka, va, 0);
  issue(kb, vb, 1);
  for (int r = 0; r < rounds; r += 2) {
    consume(ka, va, r);
    if (r + 1 >= rounds) break;
    issue(ka, va, r + 2);
    consume(kb, vb, r + 1);
    if (r + 2 >= rounds) break;
    issue(kb, vb, r + 3);
  }
  // ---- merge the KPP groups of this block
  if (sub == 0) {
    gm[kg] = m;
    gl[kg] = l;
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) go[kg][sub * EPC + e] = acc[e];
  __syncthreads();
  float M = -INFINITY;
  for (int g = 0; g < KPP; ++g) M = fmaxf(M, gm[g]);
  const int d = tid % DH, part = tid / DH;
  float L = 0.f, o = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int i = 0; i < GPP; ++i) {
      const int g = part * GPP + i;
      const float w = exp2_fast(gm[g] - M);  // empty group: gm = -inf -> 0 (its o and l are 0)
      L += w * gl[g];
      o += w * go[g][d];
    }
  }
  po[part][d] = o;
  if (d == 0) pl[part] = L;
  __syncthreads();
  const bool direct = a.S == 1 && a.out16;
  if (tid < DH) {
    o = 0.f;
    L = 0.f;
#pragma unroll
    for (int i = 0; i < PARTS; ++i) {
      o += po[i][tid];
      L += pl[i];
    }
    if (direct) {   // L > 0: the key at the query's own position is visible
      a.out16[frag_act_index(sess, h * DH + tid, a.H * DH)] = f32_to_f16_sat(o / L * ldexpf(1.0f, -a.o16_exp));
    } else {
      a.part_o[((size_t)h * a.S + s) * DH + tid] = o;
      if (tid == 0) {
        a.part_ml[((size_t)h * a.S + s) * 2] = M;
        a.part_ml[((size_t)h * a.S + s) * 2 + 1] = L;
      }
    }
  }
}

}  // namespace pp
