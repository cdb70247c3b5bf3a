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
// partial (o, max, sum). The S partials of a head are merged in split order -- a fixed order, so
// results are bit-reproducible -- by a small combine kernel. (Merging inside the split
// kernel by the last block to finish needs device-scope release/acquire fences, which on
// this multi-XCD part write back and invalidate L2 and measured slower.)
#include "device.h"
#include "internal.h"

namespace pp {

constexpr int kMaxSplits = 64;

constexpr int kAttnThreads = 512;

// Block (s, h): one pass over its keys with an online softmax. A group of LPK lanes owns
// one key row per pass (16 bytes per lane); KPP groups cover KPP keys per pass and NB
// passes form a round. The K and V rows of the next round are loaded while the current
// round is scored and accumulated. Each group keeps a running max m, sum l and output
// o (its lanes' EPC dimensions); the groups are merged through LDS at the end.
template <typename KT, int DH>
__global__ __launch_bounds__(kAttnThreads) void k_attn_decode(AttnDecodeArgs a) {
  constexpr int EPC = Elem<KT>::kPerChunk;  // elements per 16-byte chunk
  constexpr int LPK = DH / EPC;             // lanes per key row
  constexpr int KPP = kAttnThreads / LPK;   // keys per pass
  constexpr int NB = 8;                     // passes per round
  constexpr int RK = KPP * NB;              // keys per round
  __shared__ float gm[KPP], gl[KPP];
  __shared__ float go[KPP][DH + 1];

  const int s = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int sub = tid % LPK, kg = tid / LPK;
  const long long pos = a.state[0];
  const int n = pos + 1 < (long long)a.C ? (int)(pos + 1) : a.C;
  const int j0 = (int)((long long)s * n / a.S), j1 = (int)((long long)(s + 1) * n / a.S);
  const int cnt = j1 - j0;

  float qv[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) qv[e] = a.q[h * DH + sub * EPC + e] * a.scale;
  const KT* kb = static_cast<const KT*>(a.k) + ((size_t)h * a.C + j0) * DH + sub * EPC;
  const KT* vb = static_cast<const KT*>(a.v) + ((size_t)h * a.C + j0) * DH + sub * EPC;

  float m = -INFINITY, l = 0.f, acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.f;

  auto issue = [&](u32x4 (&ck)[NB], u32x4 (&cv)[NB], int jb) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int j = jb + b * KPP + kg;
      ck[b] = j < cnt ? load_stream(kb + (size_t)j * DH) : u32x4{0u, 0u, 0u, 0u};
      cv[b] = j < cnt ? load_stream(vb + (size_t)j * DH) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto consume = [&](const u32x4 (&ck)[NB], const u32x4 (&cv)[NB], int jb) {
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
      sc[b] = (jb + b * KPP + kg) < cnt ? d : -INFINITY;
      mb = fmaxf(mb, sc[b]);
    }
    if (mb == -INFINITY) return;  // no key of this group in this round
    const float mn = fmaxf(m, mb);
    const float scale = expf(m - mn);  // m = -inf -> 0
    l *= scale;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] *= scale;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float p = expf(sc[b] - mn);  // -inf -> 0
      l += p;
      float vf[EPC];
      Elem<KT>::widen(cv[b], vf);
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[e] += p * vf[e];
    }
    m = mn;
  };

  u32x4 ka[NB], va[NB], kb2[NB], vb2[NB];
  if (cnt > 0) {
    issue(ka, va, 0);
    for (int jb = 0;; jb += 2 * RK) {
      if (jb + RK < cnt) issue(kb2, vb2, jb + RK);
      consume(ka, va, jb);
      if (jb + RK >= cnt) break;
      if (jb + 2 * RK < cnt) issue(ka, va, jb + 2 * RK);
      consume(kb2, vb2, jb + RK);
      if (jb + 2 * RK >= cnt) break;
    }
  }

  // ---- merge the KPP groups of this block
  if (sub == 0) {
    gm[kg] = m;
    gl[kg] = l;
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) go[kg][sub * EPC + e] = acc[e];
  __syncthreads();
  float* part = a.part + ((size_t)h * a.S + s) * (DH + 2);
  if (tid < DH) {
    float M = -INFINITY;
    for (int g = 0; g < KPP; ++g) M = fmaxf(M, gm[g]);
    float L = 0.f, o = 0.f;
    if (M != -INFINITY) {
      for (int g = 0; g < KPP; ++g) {
        if (gm[g] == -INFINITY) continue;
        const float w = expf(gm[g] - M);
        L += w * gl[g];
        o += w * go[g][tid];
      }
    }
    part[tid] = o;
    if (tid == 0) {
      part[DH] = M;
      part[DH + 1] = L;
    }
  }
}

// Merge the S partials (o_s, m_s, l_s) of head h in split order:
// o = sum_s exp(m_s - M) o_s / sum_s exp(m_s - M) l_s with M = max_s m_s.
// All partials of the head are first loaded into LDS in one parallel round.
template <int DH>
__global__ __launch_bounds__(kBlock) void k_attn_combine(AttnDecodeArgs a) {
  __shared__ float pp[kMaxSplits * (DH + 2)];
  const int h = blockIdx.x, t = threadIdx.x;
  const float* ph = a.part + (size_t)h * a.S * (DH + 2);
  for (int i = t; i < a.S * (DH + 2); i += kBlock) pp[i] = ph[i];
  __syncthreads();
  if (t >= DH) return;
  float M = -INFINITY;
  for (int i = 0; i < a.S; ++i) M = fmaxf(M, pp[i * (DH + 2) + DH]);
  float L = 0.f, o = 0.f;
  for (int i = 0; i < a.S; ++i) {
    const float mi = pp[i * (DH + 2) + DH];
    if (mi == -INFINITY) continue;  // empty split
    const float w = expf(mi - M);
    L += w * pp[i * (DH + 2) + DH + 1];
    o += w * pp[i * (DH + 2) + t];
  }
  a.out[h * DH + t] = o / L;
}

hipError_t launch_attn_decode(const AttnDecodeArgs& a, bool bf16, int dh, hipStream_t s) {
  const dim3 grid(a.S, a.H), block(kAttnThreads);
  if (bf16 && dh == 128) hipLaunchKernelGGL((k_attn_decode<bf16_t, 128>), grid, block, 0, s, a);
  else if (bf16 && dh == 64) hipLaunchKernelGGL((k_attn_decode<bf16_t, 64>), grid, block, 0, s, a);
  else if (!bf16 && dh == 128) hipLaunchKernelGGL((k_attn_decode<float, 128>), grid, block, 0, s, a);
  else if (!bf16 && dh == 64) hipLaunchKernelGGL((k_attn_decode<float, 64>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dh == 128) hipLaunchKernelGGL((k_attn_combine<128>), dim3(a.H), dim3(kBlock), 0, s, a);
  else hipLaunchKernelGGL((k_attn_combine<64>), dim3(a.H), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace pp
