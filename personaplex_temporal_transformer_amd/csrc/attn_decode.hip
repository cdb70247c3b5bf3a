// Decode attention over the temporal ring: one query per head against every visible key.
//
// "PersonaPlex native LM audit", section 3: ordinary multi-head attention (32 query, key
// and value heads of 128), scale 1/sqrt(d_head), softmax, no dropout; the declared mask
// admits keys with 0 <= query_pos - key_pos < context. Keys in the ring were rotated at
// their own positions when written, so nothing is rotated here. With the frame at
// position p written into slot p mod C first, the visible keys are exactly the slots
// 0 .. min(p+1, C)-1 (softmax does not depend on the order of keys).
//
// Split-K over keys: block (s, h) handles an equal share of head h's keys, so H x S
// blocks stream the K and V bytes once, 16 bytes per lane, and each forms a float32
// partial (o, max, sum). Scores are carried in base-2 units (q is pre-scaled by
// log2(e) / sqrt(d_head)), so every exponential is one exp2 and the partial max is in
// those units: softmax weights 2^(s - m) equal e^(s' - m') for the natural-unit scores. The S partials of a head are merged in split order -- a fixed order, so
// results are bit-reproducible -- by a small combine kernel. (Merging inside the split
// kernel by the last block to finish needs device-scope release/acquire fences, which on
// this multi-XCD part write back and invalidate L2 and measured slower.)
#include <stdlib.h>

#include "device.h"
#include "internal.h"

namespace pp {

constexpr int kMaxSplits = 64;

// Block (s, h): one pass over its keys with an online softmax. A group of LPK lanes reads
// one key row at a time (16 bytes per lane); the KPP groups of the block own contiguous,
// equal runs of the block's keys. A round loads NB keys' K and V rows per thread with
// buffer loads (slots past the group's run point out of range and read zeros without
// memory traffic); the next round is always issued before the current one is consumed.
// Each group keeps a running max m, sum l and output o (its lanes' EPC dimensions); the
// groups are merged through LDS at the end, all threads taking part (PARTS partial
// merges per output dimension, then their sum).
template <typename KT, int DH, int NB, int NT>
__global__ __launch_bounds__(NT) void k_attn_decode(AttnDecodeArgs a) {
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

  const int s = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
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
      sc[b] = (gbeg + r * NB + b) < gend ? d : -INFINITY;
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
  for (int r = 0; r < rounds; r += 2) {
    issue(kb, vb, r + 1);
    consume(ka, va, r);
    if (r + 1 >= rounds) break;
    issue(ka, va, r + 2);
    consume(kb, vb, r + 1);
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
  if (tid < DH) {
    o = 0.f;
    L = 0.f;
#pragma unroll
    for (int i = 0; i < PARTS; ++i) {
      o += po[i][tid];
      L += pl[i];
    }
    a.part_o[((size_t)h * a.S + s) * DH + tid] = o;
    if (tid == 0) {
      a.part_ml[((size_t)h * a.S + s) * 2] = M;
      a.part_ml[((size_t)h * a.S + s) * 2 + 1] = L;
    }
  }
}

// Merge the S partials (o_s, m_s, l_s) of head h in split order:
// o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s with M = max_s m_s (base-2 units).
// All partials of the head are first loaded into LDS in one parallel round.
template <int DH>
__global__ __launch_bounds__(kBlock) void k_attn_combine(AttnDecodeArgs a) {
  __shared__ float po[kMaxSplits * DH], pml[kMaxSplits * 2];
  const int h = blockIdx.x, t = threadIdx.x;
  for (int i = t; i < a.S * DH; i += kBlock) po[i] = a.part_o[(size_t)h * a.S * DH + i];
  for (int i = t; i < a.S * 2; i += kBlock) pml[i] = a.part_ml[(size_t)h * a.S * 2 + i];
  __syncthreads();
  if (t >= DH) return;
  float M = -INFINITY;
  for (int i = 0; i < a.S; ++i) M = fmaxf(M, pml[2 * i]);
  float L = 0.f, o = 0.f;
  for (int i = 0; i < a.S; ++i) {
    const float mi = pml[2 * i];
    if (mi == -INFINITY) continue;  // empty split
    const float w = exp2_fast(mi - M);
    L += w * pml[2 * i + 1];
    o += w * po[i * DH + t];
  }
  a.out[h * DH + t] = o / L;
}

hipError_t launch_attn_decode(const AttnDecodeArgs& a, bool bf16, int dh, hipStream_t s) {
  const dim3 grid(a.S, a.H);
  static const int nb_env = [] {
    const char* v = getenv("PP_ATTN_NB");
    return v ? atoi(v) : 6;
  }();
  static const int nt_env = [] {
    const char* v = getenv("PP_ATTN_THREADS");
    return v ? atoi(v) : 512;
  }();
  if (bf16 && dh == 128) {
    if (nt_env == 1024 && nb_env == 3) hipLaunchKernelGGL((k_attn_decode<bf16_t, 128, 3, 1024>), grid, dim3(1024), 0, s, a);
    else if (nt_env == 1024) hipLaunchKernelGGL((k_attn_decode<bf16_t, 128, 4, 1024>), grid, dim3(1024), 0, s, a);
    else if (nb_env == 4) hipLaunchKernelGGL((k_attn_decode<bf16_t, 128, 4, 512>), grid, dim3(512), 0, s, a);
    else hipLaunchKernelGGL((k_attn_decode<bf16_t, 128, 6, 512>), grid, dim3(512), 0, s, a);
  } else if (bf16 && dh == 64) hipLaunchKernelGGL((k_attn_decode<bf16_t, 64, 6, 512>), grid, dim3(512), 0, s, a);
  else if (!bf16 && dh == 128) hipLaunchKernelGGL((k_attn_decode<float, 128, 6, 512>), grid, dim3(512), 0, s, a);
  else if (!bf16 && dh == 64) hipLaunchKernelGGL((k_attn_decode<float, 64, 6, 512>), grid, dim3(512), 0, s, a);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.combine) return e;
  if (dh == 128) hipLaunchKernelGGL((k_attn_combine<128>), dim3(a.H), dim3(kBlock), 0, s, a);
  else hipLaunchKernelGGL((k_attn_combine<64>), dim3(a.H), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace pp
