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
//   EPI_QKV      rows Q|K|V of in_proj; RoPE on adjacent pairs (2j, 2j+1) of Q and K at
//                the frame's absolute position with omega_j = theta^(-2j/d_head), the
//                angle formed in float64; Q -> float32 buffer, K (rotated) and V (raw) ->
//                ring slot pos mod C (section 6, temporal attention cache)
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
        const double ang = (double)pos * exp(-a.log_theta * (double)d / (double)a.dh);
        double sn, cs;
        sincos(ang, &sn, &cs);
        const float c = (float)cs, s = (float)sn;
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

// RB rows per group, U 16-byte chunks per lane per pass over K. ONEPASS: the whole row
// fits in one pass (K/chunk <= 64*U), so each lane keeps its slice of x in registers.
template <typename WT, int RB, int U, bool ONEPASS, int PRO, int EPI>
__global__ __launch_bounds__(kBlock) void k_gemv(GemvArgs a) {
  extern __shared__ float xs[];
  __shared__ float red[4];
  constexpr int EPC = Elem<WT>::kPerChunk;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int K = a.K;
  const int nch = K / EPC;

  // ---- prologue: x (float32) -> LDS, optionally RMS-normalised
  float ss = 0.f;
  for (int i = tid * 4; i < K; i += kBlock * 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(a.x + i);
    *reinterpret_cast<f32x4*>(xs + i) = v;
    if (PRO == PRO_RMSNORM) ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  if (PRO == PRO_RMSNORM) {
    const float r = 1.0f / sqrtf(block_sum_256(ss, red) / (float)K + a.eps);
    for (int i = tid * 4; i < K; i += kBlock * 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(xs + i);
      const f32x4 al = *reinterpret_cast<const f32x4*>(a.alpha + i);
      *reinterpret_cast<f32x4*>(xs + i) = (v * r) * al;
    }
  }
  __syncthreads();

  // ---- rows: wave gw owns the contiguous groups [g0, g1)
  const int gw = blockIdx.x * (kBlock / kWave) + wid;
  const int TW = gridDim.x * (kBlock / kWave);
  const int g0 = (int)((long long)gw * a.n_groups / TW);
  const int g1 = (int)((long long)(gw + 1) * a.n_groups / TW);

  float xr[ONEPASS ? U : 1][EPC];
  if (ONEPASS) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = u * kWave + lane;
#pragma unroll
      for (int e = 0; e < EPC; ++e) xr[u][e] = c < nch ? xs[c * EPC + e] : 0.f;
    }
  }

  for (int g = g0; g < g1; ++g) {
    const char* rp[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r)
      rp[r] = static_cast<const char*>(a.W) + (size_t)row_of<RB, EPI>(a, g, r) * K * sizeof(WT);
    float acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[r] = 0.f;

    for (int c0 = 0; c0 < nch; c0 += kWave * U) {
      u32x4 w[RB][U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * kWave + lane;
#pragma unroll
        for (int r = 0; r < RB; ++r)
          w[r][u] = c < nch ? load_stream(rp[r] + (size_t)c * 16) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * kWave + lane;
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
          Elem<WT>::widen(w[r][u], wf);
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[r] += wf[e] * xv[e];
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[r] = wave_sum(acc[r]);
    if (lane == 0) epilogue<WT, RB, EPI>(a, g, acc);
  }
}

template <typename WT, int RB, int PRO, int EPI>
static hipError_t dispatch_u(const GemvArgs& a, int blocks, hipStream_t s) {
  constexpr int EPC = Elem<WT>::kPerChunk;
  const int nch = a.K / EPC;
  const size_t lds = (size_t)a.K * sizeof(float);
  const dim3 grid(blocks), block(kBlock);
  if (nch <= kWave * 1)
    hipLaunchKernelGGL((k_gemv<WT, RB, 1, true, PRO, EPI>), grid, block, lds, s, a);
  else if (nch <= kWave * 2)
    hipLaunchKernelGGL((k_gemv<WT, RB, 2, true, PRO, EPI>), grid, block, lds, s, a);
  else if (nch <= kWave * 4)
    hipLaunchKernelGGL((k_gemv<WT, RB, 4, true, PRO, EPI>), grid, block, lds, s, a);
  else if (nch <= kWave * 8)
    hipLaunchKernelGGL((k_gemv<WT, RB, 8, true, PRO, EPI>), grid, block, lds, s, a);
  else
    hipLaunchKernelGGL((k_gemv<WT, RB, 4, false, PRO, EPI>), grid, block, lds, s, a);
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
  return hipErrorInvalidValue;
}

hipError_t launch_gemv(int pro, int epi, bool bf16, int rows_per_group, const GemvArgs& a,
                       int waves, hipStream_t s) {
  if (a.n_groups <= 0) return hipSuccess;
  int w = waves > 0 ? waves : a.n_groups;
  if (w > a.n_groups) w = a.n_groups;
  const int blocks = (w + (kBlock / kWave) - 1) / (kBlock / kWave);
  return bf16 ? dispatch_kind<bf16_t>(pro, epi, rows_per_group, a, blocks, s)
              : dispatch_kind<float>(pro, epi, rows_per_group, a, blocks, s);
}

}  // namespace pp
