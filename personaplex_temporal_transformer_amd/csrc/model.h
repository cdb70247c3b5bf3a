// Handle types behind the opaque pointers of pp.h (host side only).
#pragma once

#include <hip/hip_runtime.h>

#include <string>
#include <vector>

#include "internal.h"
#include "pp.h"

pp_status pp_fail(pp_status st, const std::string& msg);
pp_status pp_device_check(int* n_cu);

struct pp_kv;

// Power-of-two exponents of the float16 operands of one layer (csrc/f16_scales.hip): the
// float16 copy of a matrix holds w * 2^-w_*, a float16 activation a * 2^-(its exponent).
struct F16Exps {
  int u1, u2;        // normalised rows entering QKV / W_in
  int q, k, v;       // prefill: Q and the K copy of the attention, the transposed V copy
                     // (so the attention output too); batched decode: its attention output
  int s;             // SiLU(g) * z entering W_out
  int w_qkv, w_o, w_in, w_out;
};

// The per-step intermediates of a batch-1 decode frame (device memory).
struct DecodeBufs {
  float* x;          // residual stream [D] float32
  float* q;          // rotated query [D]
  float* o;          // attention output [D]
  float* s;          // SiLU(g) * z [F]
  float* part_o;     // attention partial outputs [H][S][dh]
  float* part_ml;    // attention partial (max, sum) [H][S][2]
  long long* state;  // [0] = position of the frame being decoded (read by graph replays)
  float* rope;       // [dh] cos/sin table of that position
};

struct pp_model {
  pp_temporal_config cfg{};
  bool bf16 = true;
  int device = 0, n_cu = 0;
  int max_batch = 1, max_T = 0;

  // weights (caller-owned device memory)
  const void* text_emb = nullptr;
  std::vector<const void*> audio_emb;
  std::vector<const float*> norm1, norm2;
  std::vector<const void*> w_qkv, w_o, w_in, w_out;
  const float* out_norm = nullptr;
  const void* text_head = nullptr;

  // decode workspace (one hipMalloc)
  void* ws = nullptr;
  float* x = nullptr;        // residual stream [D] float32
  float* q = nullptr;        // rotated query [D]
  float* o = nullptr;        // attention output [D]
  float* s = nullptr;        // SiLU(g) * z [F]
  float* part_o = nullptr;   // attention partial outputs [H][S][dh]
  float* part_ml = nullptr;  // attention partial (max, sum) [H][S][2]
  long long* state = nullptr;  // [0] = position of the frame being decoded
  float* rope = nullptr;       // [dh] cos/sin table of that position
  DecodeBufs db{};             // the above, as one set
  // batched decode (max_batch > 1): residuals [B][D], queries [B][D] float32; float16
  // normalised rows [B][D], attention outputs [B][D], SiLU products [B][F]; partials
  float* bx = nullptr;
  float* bq = nullptr;
  uint16_t* bu16 = nullptr;
  uint16_t* bo16 = nullptr;
  uint16_t* bs16 = nullptr;
  float* bpart_o = nullptr;
  float* bpart_ml = nullptr;
  // batched decode: the matrices in the skinny products' fragment order (one allocation)
  void* pk_ws = nullptr;
  std::vector<const void*> pk_qkv, pk_o, pk_in, pk_out;
  const void* pk_head = nullptr;
  int S = 16;                // attention splits per head (batch-1 decode)
  int S_auto = 16;           // the automatic split count (batched decode always uses it)
  int gemv_blocks = 256;     // workgroups per GEMV launch (one per CU)
  int wout_rb = 1;           // rows per group of the W_out GEMV

  // prefill workspace (one hipMalloc, sized by max_T)
  void* pws = nullptr;
  int32_t* ids_dev = nullptr;  // [ids_frames][n_streams]
  size_t ids_frames = 0;       // frames of IDs the device region holds
  float* px = nullptr;         // residual stream [T][D] float32
  void* pu = nullptr;          // normalised rows [T][D]: float16 (bf16-weight path) or float32
  void* pq = nullptr;          // rotated Q [H][T][dh]: float16 (bf16-weight path) or float32
  void* pa = nullptr;          // attention output [T][D], same element type
  void* pg = nullptr;          // SiLU(g)*z [T][F], same element type
  float* psplit = nullptr;     // bf16-weight path: split-K partial sums of the small-M products
  size_t psplit_bytes = 0;
  float* prope = nullptr;      // RoPE table [T][dh] (cos, sin pairs)
  void* pvt = nullptr;         // bf16-weight path: V transposed, float16 [H][dh][vt_pitch] of a chunk's key space
  void* pkx = nullptr;         // a chunk's key space: K [H][x_pitch][dh] (float16 on the bf16-weight path, else float32)
  void* pvx = nullptr;         // float32 path: V [H][x_pitch][dh]
  int vt_pitch = 0, x_pitch = 0;
  void* pf16_ws = nullptr;     // bf16-weight path: float16 copies of the block matrices (one allocation)
  std::vector<const void*> f16_qkv, f16_o, f16_in, f16_out;   // keys of the key space: max_T + context + 16, rounded up to 64

  // float16 operand exponents (bf16 weights with prefill or batched decode): per layer, and
  // the final norm's rows / the text head of the batched step
  std::vector<F16Exps> f16e;
  int f16e_uout = 0, f16e_whead = 0;

  int32_t* ids_pinned = nullptr;
  size_t ids_cap = 0;
  hipEvent_t ids_event = nullptr;

  // memory readers (csrc/reader.cpp)
  struct Reader {
    int block = 0;
    pp_reader_weights w{};
    void* K = nullptr;   // [H][max_slots][dh], weight type
    void* V = nullptr;
  };
  struct ReaderSet {
    int n = 0, mem_dim = 0, max_slots = 0, visible = 0;
    double eps = 1e-5;
    std::vector<Reader> r;
    void* ws = nullptr;
    ~ReaderSet();
  } readers;
  hipError_t enqueue_reader(int l, hipStream_t s, const DecodeBufs& b);

  // launch mode and timing
  bool use_graph = true;
  int graph_gen = 0;
  int trace_layer = -1;
  int trace_repeat = 1;
  std::vector<hipEvent_t> trace_ev;
  size_t trace_used = 0;

  ~pp_model();
  pp_status alloc_decode(int D, int F, int H, int dh);
  pp_status compute_f16_scales();
  pp_status alloc_prefill();
  void free_prefill();
  pp_status check_ids(const int32_t* ids, size_t frames) const;
  void embed_tables(pp::EmbedArgs& a) const;
  pp_status stage_ids(const int32_t* ids_host, size_t n, hipStream_t s);
  hipError_t enqueue_layers(pp_kv* kv, hipStream_t s, bool traced, long long pos_arg, const DecodeBufs& b);
  pp_status run_layers(pp_kv* kv, hipStream_t s);
  pp_status decode(pp_kv* kv, const int32_t* ids_host, const int32_t* ids_dev, float* h_out_dev,
                   float* text_logits_dev, hipStream_t s);
  pp_status decode_one(pp_kv* kv, const int32_t* ids_host, const int32_t* ids_dev, float* h_out_dev,
                       float* text_logits_dev, hipStream_t s, const DecodeBufs& b, bool graph);
  hipError_t enqueue_layers_batched(pp_kv* kv, hipStream_t s, long long pos_arg);
  pp_status pack_batched();
  pp_status decode_batched(pp_kv* kv, const int32_t* ids_host, float* h_out_dev, float* text_logits_dev,
                           hipStream_t s);
};

struct pp_kv {
  pp_model* m = nullptr;
  void* ring = nullptr;   // [L][2][B][H][C][dh]
  size_t bytes = 0;
  int B = 1;
  int64_t pos = 0;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int exec_model_gen = -1;
  ~pp_kv();
};

// Depth transformer handle (depformer.cpp); its workspace holds the per-frame state.
struct pp_depformer {
  pp_depth_config cfg{};
  bool bf16 = true;
  int n_cu = 0;
  std::vector<const void*> in_proj, audio_emb, w_qkv, w_o, w_in, w_out, head;
  std::vector<const float*> norm1, norm2;
  const void* text_emb = nullptr;

  void* ws = nullptr;
  float *h = nullptr, *c_all = nullptr, *z = nullptr, *q = nullptr, *s = nullptr, *kv = nullptr,
        *logits = nullptr;
  int32_t* codes = nullptr;
  pp::DepthCtrl* ctrl = nullptr;
  int gemv_blocks = 256;
  int qkv_blocks = 256, attn_blocks = 256, ffn_blocks = 256;   // per-launch workgroups of the depth GEMVs
  bool use_graph = true;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;

  ~pp_depformer() {
    if (exec) (void)hipGraphExecDestroy(exec);
    if (graph) (void)hipGraphDestroy(graph);
    if (ws) (void)hipFree(ws);
  }
  hipError_t enqueue(hipStream_t st);
  pp_status run(hipStream_t st);
};

