// Power-of-two scales that keep the float16 operands of the matrix-core paths (prefill,
// batched decode) inside float16's range for any weights.
//
// Those paths multiply float16 activations by a float16 copy of the bf16 weights. bfloat16
// reaches far beyond float16's range (65504) and far below its normal range (2^-14), so:
//   * every block matrix is copied as w * 2^-e_w with e_w chosen per matrix so that its
//     largest |w| lands in [2^14, 2^15): no overflow, and small weights keep their bits;
//   * every float16 activation is written as a * 2^-e_a, with e_a >= 0 per layer the
//     smallest exponent for which a bound on |a| that holds for every input stays below
//     2^15 -- so typical models (bounds below 2^15) are not scaled at all;
//   * the consumer multiplies its float32 accumulators by 2^(e_a + e_w). Powers of two are
//     exact, so nothing changes beyond the float16 roundings themselves.
// Bounds (Cauchy-Schwarz; "PersonaPlex native LM audit", section 3, for the operations):
//   u = alpha (.) x / sqrt(mean(x^2) + eps) has ||u||_2 <= max|alpha| sqrt(D), so every
//   |u_i| <= max|alpha| sqrt(D); a projection row w gives |w.u| <= ||w||_2 max|alpha| sqrt(D);
//   RoPE mixes the pair (2j, 2j+1): each rotated value is at most sqrt(2) times the larger;
//   attention averages values, so |o| <= max |v|; |SiLU(g) z| <= |g| |z|.
#include <hip/hip_runtime.h>

#include <cmath>
#include <string>
#include <vector>

#include "device.h"
#include "model.h"
#include "pp.h"

using namespace pp;

namespace pp {

// Per row of a bf16 matrix [rows][K]: the sum of squares and the largest |w| (float32; a
// non-finite weight gives a non-finite result). One wave per row.
__global__ __launch_bounds__(kBlock) void k_row_stats(const uint16_t* __restrict__ W, int rows, int K,
                                                      float* __restrict__ ss, float* __restrict__ amax) {
  const int row = blockIdx.x * (kBlock / 64) + (int)(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const uint16_t* r = W + (size_t)row * K;
  float s = 0.f, m = 0.f;
  for (int c = lane * 8; c < K; c += 64 * 8) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(r + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = bf16_lo(v[e]), b = bf16_hi(v[e]);
      s += a * a + b * b;
      m = fmaxf(m, fmaxf(fabsf(a), fabsf(b)));
      if (!(fabsf(a) <= 3.4e38f) || !(fabsf(b) <= 3.4e38f)) m = INFINITY;   // inf / NaN
    }
  }
  s = wave_sum(s);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (lane == 0) {
    ss[row] = s;
    amax[row] = m;
  }
}

hipError_t launch_row_stats(const void* W, int rows, int K, float* ss, float* amax, hipStream_t s) {
  if (K % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_row_stats, dim3((unsigned)((rows + 3) / 4)), dim3(kBlock), 0, s,
                     static_cast<const uint16_t*>(W), rows, K, ss, amax);
  return hipGetLastError();
}

}  // namespace pp

namespace {

// Smallest e >= 0 with bound * 2^-e <= 2^15.
int down_exp(double bound) {
  if (!(bound > 32768.0)) return 0;
  return (int)std::ceil(std::log2(bound / 32768.0));
}

// e with amax * 2^-e in [2^14, 2^15) (0 for an all-zero matrix).
int weight_exp(double amax) {
  if (!(amax > 0.0)) return 0;
  int e = 0;
  (void)std::frexp(amax, &e);   // amax in [2^(e-1), 2^e)
  return e - 15;
}

struct Stats {
  std::vector<float> ss, amax;
  double max_norm(int r0, int r1) const {
    double m = 0;
    for (int r = r0; r < r1; ++r) m = std::max(m, std::sqrt((double)ss[r]));
    return m;
  }
  double max_abs(int r0, int r1) const {
    double m = 0;
    for (int r = r0; r < r1; ++r) m = std::max(m, (double)amax[r]);
    return m;
  }
};

}  // namespace

pp_status pp_model::compute_f16_scales() {
  const pp_temporal_config& c = cfg;
  const int D = c.d_model, F = c.d_ff, L = c.n_layers, V = c.text_vocab - 1;
  const int max_rows = std::max(std::max(3 * D, 2 * F), text_head ? V : 0);
  float* dev = nullptr;
  if (hipMalloc(&dev, sizeof(float) * 2 * (size_t)max_rows) != hipSuccess)
    return pp_fail(PP_E_HIP, "hipMalloc of the weight-statistics buffer failed");
  Stats st;
  auto stats = [&](const void* W, int rows, int K) -> hipError_t {
    hipError_t e = launch_row_stats(W, rows, K, dev, dev + max_rows, nullptr);
    st.ss.assign(rows, 0.f);
    st.amax.assign(rows, 0.f);
    if (e == hipSuccess) e = hipMemcpy(st.ss.data(), dev, sizeof(float) * rows, hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(st.amax.data(), dev + max_rows, sizeof(float) * rows, hipMemcpyDeviceToHost);
    return e;
  };
  auto max_abs_dev = [&](const float* p, int n, double* out) -> hipError_t {
    std::vector<float> h(n);
    hipError_t e = hipMemcpy(h.data(), p, sizeof(float) * n, hipMemcpyDeviceToHost);
    double m = 0;
    for (float v : h) m = std::max(m, (double)std::fabs(v));
    *out = m;
    return e;
  };
  const double sqD = std::sqrt((double)D);
  hipError_t e = hipSuccess;
  std::string bad;
  f16e.assign(L, F16Exps{});
  for (int l = 0; l < L && e == hipSuccess && bad.empty(); ++l) {
    F16Exps& x = f16e[l];
    double a1 = 0, a2 = 0;
    if ((e = max_abs_dev(norm1[l], D, &a1)) != hipSuccess || (e = max_abs_dev(norm2[l], D, &a2)) != hipSuccess) break;
    if (!std::isfinite(a1) || !std::isfinite(a2)) bad = "a norm scale of layer " + std::to_string(l) + " is not finite";
    if ((e = stats(w_qkv[l], 3 * D, D)) != hipSuccess) break;
    const double nq = st.max_norm(0, D), nk = st.max_norm(D, 2 * D), nv = st.max_norm(2 * D, 3 * D);
    double aw = st.max_abs(0, 3 * D);
    if (!std::isfinite(aw)) bad = "W_QKV of layer " + std::to_string(l) + " has a non-finite weight";
    x.w_qkv = weight_exp(aw);
    if ((e = stats(w_o[l], D, D)) != hipSuccess) break;
    aw = st.max_abs(0, D);
    if (!std::isfinite(aw)) bad = "W_O of layer " + std::to_string(l) + " has a non-finite weight";
    x.w_o = weight_exp(aw);
    if ((e = stats(w_in[l], 2 * F, D)) != hipSuccess) break;
    const double ng = st.max_norm(0, F), nz = st.max_norm(F, 2 * F);
    aw = st.max_abs(0, 2 * F);
    if (!std::isfinite(aw)) bad = "W_in of layer " + std::to_string(l) + " has a non-finite weight";
    x.w_in = weight_exp(aw);
    if ((e = stats(w_out[l], D, F)) != hipSuccess) break;
    aw = st.max_abs(0, D);
    if (!std::isfinite(aw)) bad = "W_out of layer " + std::to_string(l) + " has a non-finite weight";
    x.w_out = weight_exp(aw);
    const double u1 = a1 * sqD, u2 = a2 * sqD;
    x.u1 = down_exp(u1);
    x.u2 = down_exp(u2);
    x.q = down_exp(std::sqrt(2.0) * nq * u1);
    x.k = down_exp(std::sqrt(2.0) * nk * u1);
    x.v = down_exp(nv * u1);
    x.s = down_exp((ng * u2) * (nz * u2));
  }
  if (e == hipSuccess && bad.empty() && text_head) {
    double ao = 0;
    e = max_abs_dev(out_norm, D, &ao);
    if (e == hipSuccess) e = stats(text_head, V, D);
    if (e == hipSuccess) {
      const double aw = st.max_abs(0, V);
      if (!std::isfinite(aw) || !std::isfinite(ao)) bad = "the text head or the output norm has a non-finite value";
      f16e_uout = down_exp(ao * sqD);
      f16e_whead = weight_exp(aw);
    }
  }
  (void)hipFree(dev);
  if (e != hipSuccess) return pp_fail(PP_E_HIP, std::string("weight statistics: ") + hipGetErrorString(e));
  if (!bad.empty()) return pp_fail(PP_E_ARG, bad);
  return PP_OK;
}
