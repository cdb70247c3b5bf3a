// Decode attention over the temporal ring: one query per head against every visible key.
//
// "PersonaPlex native LM audit", section 3: ordinary multi-head attention (32 query, key
// and value heads of 128), scale 1/sqrt(d_head), softmax, no dropout; the declared mask
// admits keys with 0 <= query_pos - key_pos < context. Keys in the ring were rotated at
// their own positions when written, so nothing is rotated here. With the frame at
// position p written into slot p mod C first, the visible keys are exactly the slots
// 0 .. min(p+1, C)-1 (softmax does not depend on the order of keys).
//
// Split-K over keys: block (s, h) handles an equal share of head h's keys, so
// H x S blocks stream the K and V bytes once, 16 bytes per lane, with a chunk of keys per
// load batch in flight. Each block keeps its scores in LDS and forms a float32 partial
// (o, max, sum). The S partials of a head are merged in split order -- a fixed order, so
// results are bit-reproducible -- by a small combine kernel. (Merging inside the split
// kernel by the last block to finish needs device-scope release/acquire fences, which on
// this multi-XCD part write back and invalidate L2 and measured slower.)
#include "device.h"
#include "internal.h"

namespace pp {

constexpr int kMaxChunk = 2048;   // keys per block (host keeps ceil(C / S) <= this)
constexpr int kMaxSplits = 64;

template <typename KT, int DH>
__global__ __launch_bounds__(kBlock) void k_attn_decode(AttnDecodeArgs a) {
  constexpr int EPC = Elem<KT>::kPerChunk;  // elements per 16-byte chunk
  constexpr int LPK = DH / EPC;             // lanes per key row
  constexpr int KPP = kBlock / LPK;         // keys per block pass
  constexpr int NB = 8;                     // passes batched per load round
  __shared__ float sc[kMaxChunk];
  __shared__ float red[4];
  __shared__ float osum[KPP][DH + 1];

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

  // ---- scores
  for (int jb = 0; jb < cnt; jb += KPP * NB) {
    u32x4 c[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int j = jb + b * KPP + kg;
      c[b] = j < cnt ? load_stream(kb + (size_t)j * DH) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int j = jb + b * KPP + kg;
      float kf[EPC];
      Elem<KT>::widen(c[b], kf);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) d += qv[e] * kf[e];
      d = group_sum<LPK>(d);
      if (sub == 0 && j < cnt) sc[j] = d;
    }
  }
  __syncthreads();

  // ---- softmax statistics of this chunk
  float mx = -INFINITY;
  for (int j = tid; j < cnt; j += kBlock) mx = fmaxf(mx, sc[j]);
  mx = wave_max(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float ls = 0.f;
  for (int j = tid; j < cnt; j += kBlock) {
    const float p = expf(sc[j] - m);
    sc[j] = p;
    ls += p;
  }
  const float l = cnt > 0 ? block_sum_256(ls, red) : 0.f;   // barrier inside: sc is ready

  // ---- P V
  float acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
  for (int jb = 0; jb < cnt; jb += KPP * NB) {
    u32x4 c[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int j = jb + b * KPP + kg;
      c[b] = j < cnt ? load_stream(vb + (size_t)j * DH) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int j = jb + b * KPP + kg;
      if (j < cnt) {
        float vf[EPC];
        Elem<KT>::widen(c[b], vf);
        const float p = sc[j];
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[e] += p * vf[e];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) osum[kg][sub * EPC + e] = acc[e];
  __syncthreads();

  float* part = a.part + ((size_t)h * a.S + s) * (DH + 2);
  if (tid < DH) {
    float o = 0.f;
    for (int g = 0; g < KPP; ++g) o += osum[g][tid];
    part[tid] = o;
  }
  if (tid == 0) {
    part[DH] = cnt > 0 ? m : -INFINITY;
    part[DH + 1] = l;
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
  const dim3 grid(a.S, a.H), block(kBlock);
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
