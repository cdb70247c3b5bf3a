// Matrix-vector kernels for batch-1 decode: y = W x with W [rows][K] row-major.
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

template <typename WT, int RB, int EPI>
__device__ __forceinline__ void epilogue(const GemvArgs& a, int g, const float (&acc)[RB]) {
  if (EPI == EPI_STORE) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int row = g * RB + r;
      a.out[row] = acc[r] + (a.add ? a.add[row] : 0.f);
    }
  } else if (EPI == EPI_RESID) {
#pragma unroll
    for (int r = 0; r < RB; ++r) a.out[g * RB + r] += acc[r];
  } else if (EPI == EPI_SWIGLU) {
    constexpr int P = RB / 2;
#pragma unroll
    for (int p = 0; p < P; ++p) a.out[g * P + p] = silu(acc[p]) * acc[P + p];
  } else if (EPI == EPI_QKV) {
    const long long pos = a.state[0];
    const int slot = (int)(pos % a.C);
#pragma unroll
    for (int p = 0; p < RB / 2; ++p) {
      const int row = g * RB + 2 * p;
      const int sec = row / a.D;             // 0 = Q, 1 = K, 2 = V
      const int w = row - sec * a.D;
      const int head = w / a.dh, d = w - head * a.dh;
      float y0 = acc[2 * p], y1 = acc[2 * p + 1];
      if (sec < 2) {
        const float c = a.rope[d], s = a.rope[d + 1];
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

// Depth attention for every head into x[0 .. aH*adh): scores q.k * scale over the keys
// of positions [aq_pos - awin + 1, aq_pos] (clipped at 0), softmax with max subtraction,
// then the weighted sum of values. `sc` holds aH x 32 floats of scratch LDS.
__device__ void depth_attention(const GemvArgs& a, float* x, float* sc) {
  const int tid = threadIdx.x;
  const int k0 = a.aq_pos - a.awin + 1 > 0 ? a.aq_pos - a.awin + 1 : 0;
  const int nk = a.aq_pos - k0 + 1;
  const int nt = blockDim.x;
  for (int i = tid; i < a.aH * nk; i += nt) {
    const int h = i / nk, j = i - h * nk;
    const float* qh = a.aq + h * a.adh;
    const float* kh = a.ak + ((size_t)h * a.acap + k0 + j) * a.adh;
    float d = 0.f;
    for (int e = 0; e < a.adh; ++e) d += qh[e] * kh[e];
    sc[h * 32 + j] = d * a.ascale;
  }
  __syncthreads();
  for (int h = tid; h < a.aH; h += nt) {
    float m = -INFINITY;
    for (int j = 0; j < nk; ++j) m = fmaxf(m, sc[h * 32 + j]);
    float l = 0.f;
    for (int j = 0; j < nk; ++j) {
      const float p = expf(sc[h * 32 + j] - m);
      sc[h * 32 + j] = p;
      l += p;
    }
    const float inv = 1.0f / l;
    for (int j = 0; j < nk; ++j) sc[h * 32 + j] *= inv;
  }
  __syncthreads();
  for (int i = tid; i < a.aH * a.adh; i += nt) {
    const int h = i / a.adh, d = i - h * a.adh;
    const float* vh = a.av + ((size_t)h * a.acap + k0) * a.adh + d;
    float o = 0.f;
    for (int j = 0; j < nk; ++j) o += sc[h * 32 + j] * vh[(size_t)j * a.adh];
    x[i] = o;
  }
}

constexpr int kGemvWaves = 8;                 // waves per GEMV workgroup
constexpr int kGemvThreads = kGemvWaves * kWave;

// Rows are processed in groups of RB rows; a lane streams 16-byte chunks c = p*64*U +
// u*64 + lane (u < U) of each row in pass p, so a wave reads 1 KB contiguous per load.
// Block b owns the contiguous groups [b*G/nb, (b+1)*G/nb) -- equal shares, so the grid
// (one block per CU) is balanced -- and its waves pull groups from an LDS counter.
// Loads are double-buffered: the next (group, pass) is in flight while the current one
// is multiplied and reduced. ONEPASS (a row fits in one pass): each lane keeps its slice
// of x in registers; otherwise x is read from LDS per pass.
template <typename WT, int RB, int U, bool ONEPASS, int PRO, int EPI>
__global__ __launch_bounds__(kGemvThreads) void k_gemv(GemvArgs a) {
  extern __shared__ float xs[];
  __shared__ float red[kGemvWaves];
  __shared__ int qnext;
  constexpr int EPC = Elem<WT>::kPerChunk;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int K = a.K;
  const int nch = K / EPC;
  const int np = ONEPASS ? 1 : (nch + kWave * U - 1) / (kWave * U);
  const int gb0 = (int)((long long)blockIdx.x * a.n_groups / gridDim.x);
  const int gb1 = (int)((long long)(blockIdx.x + 1) * a.n_groups / gridDim.x);
  if (tid == 0) qnext = gb0 + kGemvWaves;

  // ---- prologue: x (float32) -> LDS, optionally RMS-normalised
  if (PRO == PRO_DEPTH_ATTN) {
    depth_attention(a, xs, xs + K);
  } else {
    float ss = 0.f;
    for (int i = tid * 4; i < K; i += kGemvThreads * 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(a.x + i);
      *reinterpret_cast<f32x4*>(xs + i) = v;
      if (PRO == PRO_RMSNORM) ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    if (PRO == PRO_RMSNORM) {
      ss = wave_sum(ss);
      __syncthreads();
      if (lane == 0) red[wid] = ss;
      __syncthreads();
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < kGemvWaves; ++w) tot += red[w];
      const float r = 1.0f / sqrtf(tot / (float)K + a.eps);
      for (int i = tid * 4; i < K; i += kGemvThreads * 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(xs + i);
        const f32x4 al = *reinterpret_cast<const f32x4*>(a.alpha + i);
        *reinterpret_cast<f32x4*>(xs + i) = (v * r) * al;
      }
    }
  }
  __syncthreads();

  int g = gb0 + wid;
  if (g >= gb1) return;

  float xr[ONEPASS ? U : 1][EPC];
  if (ONEPASS) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = u * kWave + lane;
#pragma unroll
      for (int e = 0; e < EPC; ++e) xr[u][e] = c < nch ? xs[c * EPC + e] : 0.f;
    }
  }

  auto fetch = [&]() -> int {
    int v = 0;
    if (lane == 0) v = atomicAdd(&qnext, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };
  auto issue = [&](u32x4 (&buf)[RB][U], int gg, int pp) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int row = row_of<RB, EPI>(a, gg, r);
      const char* rp = a.rows_per_mat
                           ? static_cast<const char*>(a.mats[row / a.rows_per_mat]) +
                                 (size_t)(row % a.rows_per_mat) * K * sizeof(WT)
                           : static_cast<const char*>(a.W) + (size_t)row * K * sizeof(WT);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = pp * kWave * U + u * kWave + lane;
        buf[r][u] = c < nch ? load_stream(rp + (size_t)c * 16) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto accumulate = [&](const u32x4 (&buf)[RB][U], int pp, float (&acc)[RB]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = pp * kWave * U + u * kWave + lane;
      float xv[EPC];
      if (ONEPASS) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) xv[e] = xr[u][e];
      } else {
#pragma unroll
        for (int e = 0; e < EPC; ++e) xv[e] = c < nch ? xs[c * EPC + e] : 0.f;
      }
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        float wf[EPC];
        Elem<WT>::widen(buf[r][u], wf);
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[r] += wf[e] * xv[e];
      }
    }
  };

  u32x4 wa[RB][U], wb[RB][U];
  float acc[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) acc[r] = 0.f;
  int p = 0;
  issue(wa, g, 0);
  int gn = fetch();

#define PP_GEMV_STEP(CUR, NXT)                                   \
  {                                                              \
    const bool last_pass = p + 1 == np;                          \
    const int ng = last_pass ? gn : g;                           \
    const int npp = last_pass ? 0 : p + 1;                       \
    const bool more = ng < gb1;                                  \
    if (more) issue(NXT, ng, npp);                               \
    accumulate(CUR, p, acc);                                     \
    if (last_pass) {                                             \
      _Pragma("unroll") for (int r = 0; r < RB; ++r) acc[r] = wave_sum(acc[r]); \
      if (lane == 0) epilogue<WT, RB, EPI>(a, g, acc);           \
      _Pragma("unroll") for (int r = 0; r < RB; ++r) acc[r] = 0.f; \
    }                                                            \
    if (!more) break;                                            \
    if (last_pass) gn = fetch();                                 \
    g = ng;                                                      \
    p = npp;                                                     \
  }
  while (true) {
    PP_GEMV_STEP(wa, wb)
    PP_GEMV_STEP(wb, wa)
  }
#undef PP_GEMV_STEP
}

template <typename WT, int RB, int PRO, int EPI>
static hipError_t dispatch_u(const GemvArgs& a, int blocks, hipStream_t s) {
  constexpr int EPC = Elem<WT>::kPerChunk;
  const int nch = a.K / EPC;
  const size_t lds = (size_t)a.K * sizeof(float) + (PRO == PRO_DEPTH_ATTN ? 32 * 32 * sizeof(float) : 0);
  const dim3 grid(blocks), block(kGemvThreads);
  if (nch <= kWave * 1)
    hipLaunchKernelGGL((k_gemv<WT, RB, 1, true, PRO, EPI>), grid, block, lds, s, a);
  else if (nch <= kWave * 2)
    hipLaunchKernelGGL((k_gemv<WT, RB, 2, true, PRO, EPI>), grid, block, lds, s, a);
  else if (nch <= kWave * 4)
    hipLaunchKernelGGL((k_gemv<WT, RB, 4, true, PRO, EPI>), grid, block, lds, s, a);
  else if (nch <= kWave * 6)
    hipLaunchKernelGGL((k_gemv<WT, RB, 6, true, PRO, EPI>), grid, block, lds, s, a);
  else if (nch <= kWave * 8)
    hipLaunchKernelGGL((k_gemv<WT, RB, 8, true, PRO, EPI>), grid, block, lds, s, a);
  else if (nch % (kWave * 11) == 0)
    hipLaunchKernelGGL((k_gemv<WT, RB, 11, false, PRO, EPI>), grid, block, lds, s, a);
  else
    hipLaunchKernelGGL((k_gemv<WT, RB, 8, false, PRO, EPI>), grid, block, lds, s, a);
  return hipGetLastError();
}

template <typename WT, int PRO, int EPI>
static hipError_t dispatch_rb(int rb, const GemvArgs& a, int blocks, hipStream_t s) {
  if (rb == 2) return dispatch_u<WT, 2, PRO, EPI>(a, blocks, s);
  if (rb == 4) return dispatch_u<WT, 4, PRO, EPI>(a, blocks, s);
  return hipErrorInvalidValue;
}

template <typename WT>
static hipError_t dispatch_kind(int pro, int epi, int rb, const GemvArgs& a, int blocks,
                                hipStream_t s) {
  if (pro == PRO_RMSNORM && epi == EPI_QKV) return dispatch_rb<WT, PRO_RMSNORM, EPI_QKV>(rb, a, blocks, s);
  if (pro == PRO_COPY && epi == EPI_RESID) return dispatch_rb<WT, PRO_COPY, EPI_RESID>(rb, a, blocks, s);
  if (pro == PRO_RMSNORM && epi == EPI_SWIGLU) return dispatch_rb<WT, PRO_RMSNORM, EPI_SWIGLU>(rb, a, blocks, s);
  if (pro == PRO_RMSNORM && epi == EPI_STORE) return dispatch_rb<WT, PRO_RMSNORM, EPI_STORE>(rb, a, blocks, s);
  if (pro == PRO_COPY && epi == EPI_STORE) return dispatch_rb<WT, PRO_COPY, EPI_STORE>(rb, a, blocks, s);
  if (pro == PRO_RMSNORM && epi == EPI_DEPTH_QKV) return dispatch_rb<WT, PRO_RMSNORM, EPI_DEPTH_QKV>(rb, a, blocks, s);
  if (pro == PRO_DEPTH_ATTN && epi == EPI_RESID) return dispatch_rb<WT, PRO_DEPTH_ATTN, EPI_RESID>(rb, a, blocks, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gemv(int pro, int epi, bool bf16, int rows_per_group, const GemvArgs& a,
                       int blocks, hipStream_t s) {
  if (a.n_groups <= 0) return hipSuccess;
  if (blocks <= 0 || blocks > a.n_groups) blocks = a.n_groups;
  return bf16 ? dispatch_kind<bf16_t>(pro, epi, rows_per_group, a, blocks, s)
              : dispatch_kind<float>(pro, epi, rows_per_group, a, blocks, s);
}

}  // namespace pp
