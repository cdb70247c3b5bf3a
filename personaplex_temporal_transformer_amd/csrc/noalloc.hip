// Batch-1 decode step that allocates nothing: pp_temporal_decode_step_noalloc (pp.h).
//
// The same frame as pp_temporal_decode_step ("PersonaPlex native LM audit", section 3),
// with every kernel launched directly (no graph is captured or instantiated) and the
// step's intermediates -- residual stream, query, attention output, SiLU product,
// attention split partials, position word and RoPE table -- in `scratch`, a file-scope
// device array of kScratchBytes, instead of the model's workspace. Each GPU holds its own
// copy of the array for the life of the process; its address on a device is looked up
// once (hipGetSymbolAddress, the first call with that device current) and only that
// address is handed to kernels. Every call on one GPU shares the array: calls that
// overlap on one GPU race. Nothing needs clearing between calls: each step writes every
// value it later reads.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "model.h"
#include "pp.h"

using namespace pp;

namespace {
constexpr size_t kScratchBytes = size_t(1) << 20;   // per device
constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
char* g_scratch[kMaxDevices];   // device address of `scratch` on each device, once looked up
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Address of this device's copy of `scratch` (the current device must be `dev`).
static pp_status scratch_address(int dev, char** out) {
  if (dev < 0 || dev >= kMaxDevices) return pp_fail(PP_E_DEVICE, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return pp_fail(PP_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch[dev] = static_cast<char*>(p);
  }
  *out = g_scratch[dev];
  return PP_OK;
}

// Carve the step's buffers out of `base` (nullptr: only count); returns the bytes used.
static size_t carve(const pp_temporal_config& c, int S, char* base, DecodeBufs* b) {
  size_t off = 0;
  auto take = [&](size_t n) {
    char* p = base ? base + off : nullptr;
    off += (n + 255) / 256 * 256;
    return p;
  };
  const size_t D = c.d_model, F = c.d_ff, H = c.n_heads, dh = c.d_head;
  DecodeBufs t{};
  t.x = reinterpret_cast<float*>(take(4 * D));
  t.q = reinterpret_cast<float*>(take(4 * D));
  t.o = reinterpret_cast<float*>(take(4 * D));
  t.s = reinterpret_cast<float*>(take(4 * F));
  t.part_o = reinterpret_cast<float*>(take(4 * H * S * dh));
  t.part_ml = reinterpret_cast<float*>(take(4 * H * S * 2));
  t.state = reinterpret_cast<long long*>(take(4 * sizeof(long long)));
  t.rope = reinterpret_cast<float*>(take(4 * dh));
  if (b) *b = t;
  return off;
}

extern "C" pp_status pp_temporal_decode_step_noalloc(pp_model* m, pp_kv* kv, const int32_t* ids_host,
                                                     float* h_out_dev, float* text_logits_dev, void* stream) {
  if (!m || !kv || !ids_host || !h_out_dev) return pp_fail(PP_E_ARG, "NULL argument");
  if (kv->m != m) return pp_fail(PP_E_ARG, "kv ring belongs to another model");
  if (kv->B != 1) return pp_fail(PP_E_ARG, "the allocation-free step takes batch-1 rings only");
  if (m->readers.visible > 0) return pp_fail(PP_E_ARG, "the allocation-free step runs without visible memory readers");
  if (text_logits_dev && !m->text_head) return pp_fail(PP_E_ARG, "text logits requested but the model has no text head");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return pp_fail(PP_E_DEVICE, "no current HIP device");
  if (dev != m->device) return pp_fail(PP_E_DEVICE, "the model's device is not the current device");
  const size_t need = carve(m->cfg, m->S, nullptr, nullptr);
  if (need > kScratchBytes)
    return pp_fail(PP_E_CAPACITY, "the step needs " + std::to_string(need) + " bytes of scratch; the library holds " +
                                      std::to_string(kScratchBytes) + " per device");
  pp_status st = m->check_ids(ids_host, 1);
  if (st) return st;
  char* base = nullptr;
  if ((st = scratch_address(dev, &base))) return st;
  DecodeBufs b{};
  carve(m->cfg, m->S, base, &b);
  return m->decode_one(kv, ids_host, nullptr, h_out_dev, text_logits_dev, static_cast<hipStream_t>(stream), b, false);
}
