/*
 * pp.h -- C ABI of libpp: the per-frame forward of the PersonaPlex/Moshi temporal
 * transformer and its 16-position depth transformer on an AMD Instinct MI355X (gfx950).
 *
 * What is computed follows "PersonaPlex native LM audit" (Clockless Inkling,
 * personaplex-research page): section 3 "Native temporal computation" (embedding sum,
 * the pre-norm block, RoPE, causal context mask, final norm and text head), section 4
 * "Native depth computation" (per-position depth inputs, blocks and heads) and
 * section 6 "Three distinct caches" (the temporal ring KV cache and the per-frame depth
 * cache). The device-resident, fixed, in-place cache follows the lessons of "Learnings:
 * PersonaPlex/Moshi full-duplex S2S export + real-time ORT inference" (onnxruntime/mobius
 * issue #369), sections 3a-3c and the follow-up on in-place KV.
 *
 * Conventions for every call
 *  - Pointers named *_dev are device pointers (memory on the current HIP device,
 *    allocated by the caller); pointers named *_host are host pointers. Neither is
 *    retained after the call returns, except the weight pointers given at create time,
 *    which must stay valid and unchanged until the handle is destroyed.
 *  - Linear weights are row-major [out_features, in_features]: y = W x.
 *  - `stream` is a hipStream_t (NULL = the null stream). Every call that touches the
 *    device is asynchronous on that stream; outputs are valid once it is synchronised.
 *  - Every call returns a pp_status. Argument, ID, capacity and device errors are
 *    detected on the host and returned BEFORE anything is enqueued; PP_E_HIP reports a
 *    HIP runtime error. pp_last_error() gives a message for the calling thread.
 *  - There is no CPU fallback: creating a handle fails with PP_E_DEVICE unless the
 *    current device is a gfx950 GPU.
 *  - Handles are not thread-safe; calls on one handle must not overlap.
 */
#ifndef PP_H
#define PP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PP_OK = 0,
  PP_E_ARG = 1,       /* bad pointer, size, config or handle */
  PP_E_ID = 2,        /* a stream ID outside [-1, vocab) (includes -2) */
  PP_E_CAPACITY = 3,  /* prefill longer than the ring or the workspace */
  PP_E_DEVICE = 4,    /* no gfx950 device current */
  PP_E_HIP = 5,       /* HIP runtime error */
  PP_E_DTYPE = 6      /* unsupported weight dtype */
} pp_status;

typedef enum { PP_F32 = 0, PP_BF16 = 1 } pp_dtype;

/* ------------------------------------------------------------------ temporal model */

/* Shapes of the temporal transformer. Full size: 32 layers, d_model 4096, 32 heads of
 * 128, d_ff (gated hidden width) 11264, context 3000, text vocab 32001 (IDs 0..32000),
 * audio vocab 2049 (IDs 0..2048), 16 audio streams, rope_theta 1e4, eps 1e-8.
 * Requirements: d_model == n_heads * d_head; d_head is 64 or 128; d_model and d_ff are
 * multiples of 8 and at most 12288. wdtype (a pp_dtype) is the type of every weight matrix and
 * embedding table AND of the KV ring; norm scales are always float32. */
typedef struct {
  int32_t n_layers, d_model, n_heads, d_head, d_ff, context;
  int32_t text_vocab, audio_vocab, n_audio;
  int32_t wdtype;
  double rope_theta;
  double eps;
} pp_temporal_config;

/* Weights (device pointers; the pointer ARRAYS are host arrays, copied at create).
 * Names follow the constructor's parameters (audit section 5):
 *   text_emb    text_emb.weight                               [text_vocab, d_model]
 *   audio_emb   emb.{0..n_audio-1}.weight (agent cb0-7, user cb0-7) [audio_vocab, d_model]
 *   norm1/2     transformer.layers.{l}.norm{1,2}.alpha         [d_model] float32
 *   w_qkv       transformer.layers.{l}.self_attn.in_proj_weight [3*d_model, d_model]
 *               rows: Q | K | V, head h owns rows h*d_head .. h*d_head+d_head-1 of each
 *   w_o         transformer.layers.{l}.self_attn.out_proj.weight [d_model, d_model]
 *   w_in        transformer.layers.{l}.gating.linear_in.weight  [2*d_ff, d_model]
 *               rows 0..d_ff-1 are the SiLU-gated half g, the rest the linear half z
 *   w_out       transformer.layers.{l}.gating.linear_out.weight [d_model, d_ff]
 *   out_norm    out_norm.alpha                                 [d_model] float32
 *   text_head   text_linear.weight                              [text_vocab-1, d_model] or NULL */
typedef struct {
  const void* text_emb;
  const void* const* audio_emb;
  const float* const* norm1;
  const float* const* norm2;
  const void* const* w_qkv;
  const void* const* w_o;
  const void* const* w_in;
  const void* const* w_out;
  const float* out_norm;
  const void* text_head;
} pp_temporal_weights;

typedef struct pp_model pp_model;
typedef struct pp_kv pp_kv;

/* Create a temporal model on the current device. max_batch (1..64) bounds the sessions a
 * KV ring may hold for batched decode (B is the tensors' leading axis, audit section 3;
 * the pages' server runs B = 1); max_batch > 1 needs bf16 weights, d_model % 32 == 0,
 * d_ff % 32 == 0 and text-head rows % 16 == 0. max_prefill_T (0..context) sizes the
 * prefill workspace. The library allocates its workspace here (hipMalloc); weights are
 * not copied, except that max_batch > 1 keeps one copy of every matrix (and the text
 * head) rearranged for the batched products (13.4 GB at full size), and max_prefill_T > 0
 * with bf16 weights keeps a float16 copy of every block matrix for the prefill's
 * matrix-core products (13.15 GB), both made here, plus 64 MB for the split-K and key-split
 * partial sums of short prefill chunks. */
pp_status pp_temporal_create(const pp_temporal_config* cfg, const pp_temporal_weights* w,
                             int32_t max_batch, int32_t max_prefill_T, pp_model** out);
pp_status pp_temporal_destroy(pp_model* m);

/* The temporal KV ring of one session: n_layers x [2][batch][n_heads][context][d_head]
 * of wdtype, allocated once (hipMalloc) and never grown. Keys are stored after RoPE,
 * values raw. Absolute position p lives in slot p mod context; a query at position p
 * sees the keys with 0 <= p - key_position < context (audit section 3, declared mask).
 * bytes = n_layers*2*batch*n_heads*context*d_head*sizeof(wdtype): 1,572,864,000 at
 * full size, bf16, B = 1 (audit section 6). */
pp_status pp_kv_alloc(const pp_model* m, int32_t batch, pp_kv** out);
pp_status pp_kv_free(pp_kv* kv);
/* Position := 0. No byte is cleared: slots become visible again only once rewritten. */
pp_status pp_kv_reset(pp_kv* kv);
pp_status pp_kv_info(const pp_kv* kv, int64_t* position, uint64_t* bytes);
/* Restore: copy n_frames frames [n_layers][2][batch][n_heads][n_frames][d_head] (wdtype,
 * keys already rotated for positions 0..n_frames-1) from src_dev into slots
 * 0..n_frames-1 and set position := n_frames. 0 < n_frames <= context. */
pp_status pp_kv_load(pp_kv* kv, const void* src_dev, int32_t n_frames, void* stream);
/* Copy the whole ring [n_layers][2][batch][n_heads][context][d_head] to dst_dev. */
pp_status pp_kv_store(const pp_kv* kv, void* dst_dev, void* stream);
/* Snapshot restore (audit section 9, cached voice prompts restored before live audio):
 * copy a whole ring written by pp_kv_store (same model and batch) from src_dev and set
 * position := the position the ring had when it was stored (position >= 0). */
pp_status pp_kv_restore(pp_kv* kv, const void* src_dev, int64_t position, void* stream);

/* Embedding sum (audit section 3, 'Input embedding sum'): for each of batch*T frames,
 * x = sum over the n_audio+1 streams of that stream's table row, in stream order,
 * accumulated in float32; ID -1 adds nothing (an exact zero vector).
 * ids_host [batch][T][n_audio+1]: stream 0 = agent text, 1..8 agent audio, 9..16 user
 * audio. Any ID < -1 or >= that stream's vocab gives PP_E_ID. x_out_dev [batch][T][d_model].
 * 1 <= batch <= max_batch; one frame (batch * T == 1) is always accepted, more frames go
 * through the model's ID region of max_prefill_T x max_batch frames: beyond it,
 * PP_E_CAPACITY. */
pp_status pp_embed_sum(const pp_model* m, const int32_t* ids_host, int32_t batch, int32_t T,
                       float* x_out_dev, void* stream);

/* One decode frame at the ring's current position p (audit section 3): embedding sum,
 * n_layers pre-norm blocks (RMSNorm in float32 -> fused QKV -> RoPE on Q and K at p ->
 * write K, V to slot p mod context -> attention over the visible keys -> W_O + residual ->
 * RMSNorm -> W_in -> SiLU(g)*z -> W_out + residual), then the final RMSNorm.
 * ids_host [batch][n_audio+1]. h_out_dev [batch][d_model] float32 receives the final-norm
 * hidden state; text_logits_dev [batch][text_vocab-1] float32, if not NULL, the text-head
 * logits (needs a text_head weight). The position then advances by one; past `context`
 * frames the ring wraps and positions keep counting. A ring with batch B > 1 holds B
 * sessions at one shared position, each attending only to its own keys; their step
 * streams every weight once for all B sessions (float16 activations into the matrix
 * cores, float32 accumulation, residual stream and norms in float32). */
pp_status pp_temporal_decode_step(pp_model* m, pp_kv* kv, const int32_t* ids_host,
                                  float* h_out_dev, float* text_logits_dev, void* stream);

/* For callers that cannot allocate device memory during a step (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same batch-1 frame
 * as pp_temporal_decode_step, with the same results bit for bit, that calls no allocating
 * routine. Every kernel is launched directly (no graph is captured), and the step's
 * intermediates live in a 1 MiB device array that the library holds on each GPU until the
 * process ends, instead of the model's workspace. The step needs
 * 4*(3*d_model + d_ff + n_heads*splits*(d_head + 2) + d_head) + 32 bytes of it (each of its
 * eight regions rounded up to 256 bytes; 228 KB at full size with the automatic 8
 * splits); more gives PP_E_CAPACITY. All calls on one GPU share that array: calls that
 * overlap on one GPU (two streams, threads or models) race. The first call on a device
 * looks up the array's address there. Requirements: a batch-1 ring, no visible memory
 * readers (else PP_E_ARG), the model's device current (else PP_E_DEVICE). */
pp_status pp_temporal_decode_step_noalloc(pp_model* m, pp_kv* kv, const int32_t* ids_host,
                                          float* h_out_dev, float* text_logits_dev, void* stream);

/* Full-sequence forward of T frames at positions p..p+T-1, p = the ring's position
 * (audit section 3; section 9 for prompts replayed into a live ring): causal attention
 * among the frames and, when p > 0, over the keys of the ring still inside each frame's
 * context window (0 <= position - key_position < context); K/V of the frames written to
 * slots (p+t) mod context; position := p+T afterwards, so decode continues there.
 * 1 <= T <= min(context, max_prefill_T), batch 1. ids_host [batch][T][n_audio+1];
 * h_out_dev [batch][T][d_model] float32 final-norm hidden. */
pp_status pp_temporal_prefill(pp_model* m, pp_kv* kv, const int32_t* ids_host, int32_t T,
                              float* h_out_dev, void* stream);

/* The same forward with the first block's inputs given directly: x_dev [T][d_model] float32
 * holds each frame's summed embedding (audit section 9: a cached voice prompt replays the
 * native summed embeddings instead of token IDs). Everything else as pp_temporal_prefill
 * (batch 1, positions p..p+T-1, K/V into the ring, position := p+T). x_dev is read only
 * during the call's stream work and may be reused once the stream has passed it. */
pp_status pp_temporal_prefill_embedded(pp_model* m, pp_kv* kv, const float* x_dev, int32_t T,
                                       float* h_out_dev, void* stream);

/* ------------------------------------------------------------------ depth transformer */

/* Shapes of the depth transformer (audit section 4). Full size: 6 layers, d_model 1024,
 * 16 heads of 64, d_ff 2816, 16 steps (weights_per_step), window 8, text vocab 32001,
 * audio vocab 2049, 2048 logits per step, d_temporal 4096, eps 1e-8. Requirements:
 * d_model == n_heads * d_head <= 2048, d_head <= 128, window >= 1, n_steps <= 32,
 * d_ff and d_temporal multiples of 8 and at most 12288, n_out even. */
typedef struct {
  int32_t n_layers, d_model, n_heads, d_head, d_ff, n_steps, window;
  int32_t text_vocab, audio_vocab, n_out, d_temporal;
  int32_t wdtype;
  double eps;
} pp_depth_config;

/* Depth weights (device pointers; host pointer arrays copied at create):
 *   in_proj   depformer_in.{q}.weight, q < n_steps                  [d_model, d_temporal]
 *   text_emb  depformer_text_emb.weight                              [text_vocab, d_model]
 *   audio_emb depformer_emb.{q}.weight, q < n_steps-1 (input of q+1)  [audio_vocab, d_model]
 *   w_qkv     depformer.layers.{m}.self_attn.in_proj_weight  [n_steps*3*d_model, d_model]
 *             step q uses rows q*3*d_model .. (q+1)*3*d_model-1 (Q | K | V)
 *   w_o       depformer.layers.{m}.self_attn.out_proj.weight [n_steps*d_model, d_model]
 *             step q uses rows q*d_model .. (q+1)*d_model-1
 *   w_in      depformer.layers.{m}.gating.{q}.linear_in.weight, index m*n_steps+q [2*d_ff, d_model]
 *   w_out     depformer.layers.{m}.gating.{q}.linear_out.weight, index m*n_steps+q [d_model, d_ff]
 *   norm1/2   depformer.layers.{m}.norm{1,2}.alpha, shared by all steps  [d_model] float32
 *   head      linears.{q}.weight                                          [n_out, d_model] */
typedef struct {
  const void* const* in_proj;
  const void* text_emb;
  const void* const* audio_emb;
  const void* const* w_qkv;
  const void* const* w_o;
  const void* const* w_in;
  const void* const* w_out;
  const float* const* norm1;
  const float* const* norm2;
  const void* const* head;
} pp_depth_weights;

typedef struct pp_depformer pp_depformer;

pp_status pp_depformer_create(const pp_depth_config* cfg, const pp_depth_weights* w,
                              pp_depformer** out);
pp_status pp_depformer_destroy(pp_depformer* d);

/* One frame of the depth loop (audit section 4): for q = 0..n_steps-1,
 * z = in_proj[q] h + (q == 0 ? text_emb[text token] : audio_emb[q-1][code of q-1]);
 * n_layers blocks on the step-q weights (no RoPE; position q attends to the positions
 * q' of this frame with 0 <= q - q' < window; the depth cache starts empty each call);
 * logits_q = head[q] z. The code of position q is forced_host[q] when >= 0, else the
 * argmax of logits_q (lowest index on ties); it feeds position q+1 on the device.
 * h_dev [batch][d_temporal] float32 (the final-norm temporal hidden state);
 * text_token_host [batch]; forced_host [batch][n_steps] or NULL (all selected);
 * codes_dev [batch][n_steps] int32 out; logits_dev [batch][n_steps][n_out] float32 or NULL.
 * batch must be 1. A text token outside [0, text_vocab) or a forced code outside
 * [-1, n_out) gives PP_E_ID. */
pp_status pp_depformer_step(pp_depformer* d, const float* h_dev, const int32_t* text_token_host,
                            const int32_t* forced_host, int32_t batch, int32_t* codes_dev,
                            float* logits_dev, void* stream);

/* Depth-step launch mode: 0 = launch each kernel, 1 = replay a captured HIP graph (default). */
pp_status pp_depformer_set_graph(pp_depformer* d, int32_t enable);

/* ------------------------------------------------------------------ sampling and the generator frame */

/* Temperature / top-k sampling of `rows` independent logit rows ("PersonaPlex native LM
 * audit", section 7 "One exact generator step" and the sampling defaults after it; the
 * page names the parameters, the procedure below is the plain reading of them):
 * the candidates are the top_k largest logits of the row, ordered by value (larger
 * first; equal values by lower index); weights w_i = exp((l_i - l_0) / temperature) in
 * float64 with the float32 temperature widened; with the row's draw u, the result is
 * the first candidate whose running sum w_0 + .. + w_i (added in candidate order)
 * exceeds u * (w_0 + .. + w_{k-1}), or the last candidate if none does.
 * top_k <= 1 or temperature <= 0 selects the largest logit (lowest index on ties).
 * logits_dev [rows][n] float32, finite; uniforms_dev [rows] float64 in [0, 1), or NULL
 * for all zeros (the largest logit); out_dev [rows] int32. 1 <= n <= 32768,
 * top_k <= 1024 (values above n act as n), else PP_E_ARG. */
pp_status pp_sample_top_k(const float* logits_dev, int32_t rows, int32_t n, float temperature,
                          int32_t top_k, const double* uniforms_dev, int32_t* out_dev, void* stream);

/* Generator parameters (audit section 7 and "Generator delayed-code cache"). Stream k
 * of the ring is stream k of the temporal embedding sum: 0 = agent text, 1..8 = agent
 * codebooks 0..7, 9..16 = user codebooks 0..7; depth position q selects stream q + 1.
 * Defaults of the released path: delays {0, 0, 1 x 7, 0, 1 x 7}, initial tokens 32000
 * (text) and 2048 (audio), text temperature 0.7 / top-k 25, audio temperature 0.8 /
 * top-k 250. Requirements: n_streams == n_audio + 1 of the model == n_steps + 1 of the
 * depformer; 0 <= delay <= 5 (the ring has max delay + 3 slots); initial tokens are rows
 * of their tables; top-k <= 1024; sampled audio needs n_out <= 2048 and the text head
 * at most 32768 classes. */
typedef struct {
  int32_t n_streams;
  int32_t delays[32];
  int32_t text_initial, audio_initial;
  float text_temperature;
  int32_t text_top_k;
  float audio_temperature;
  int32_t audio_top_k;
} pp_generator_config;

typedef struct pp_generator pp_generator;

/* A generator session over a temporal model with its KV ring (batch 1) and a
 * depformer, none of which it owns; they must outlive it and must not be used by other
 * calls while it runs. The temporal position continues from the ring's current position
 * (0 after pp_kv_reset, or past a prefilled prompt). The code ring starts empty at
 * cursor 0. */
pp_status pp_generator_create(pp_model* m, pp_kv* kv, pp_depformer* d, const pp_generator_config* cfg,
                              pp_generator** out);
pp_status pp_generator_destroy(pp_generator* g);

/* One generator call at cursor s (audit section 7, steps 1-7), all on the device:
 * supplied codes go to ring slot (s + delay_k) mod C, marked provided; at s = 0 slot 0
 * receives the initial tokens where nothing was supplied and the call ends; otherwise
 * the temporal step reads slot (s - 1) mod C, the text is drawn from its logits with
 * uniforms[0] (a supplied text of slot s mod C replaces it), depth position q draws with
 * uniforms[1 + q] (a supplied code replaces it and feeds position q + 1), selections fill
 * the unsupplied entries of slot s mod C, the flags of slot (s - 1) mod C are cleared, and
 * when s > max delay the aligned output of stream k is slot (s - max_delay + delay_k) mod C.
 * provided_host [n_streams] int32 (-1 = not supplied; text in [0, text_vocab), audio in
 * [0, n_out)) or NULL; uniforms_host [n_streams] float64 in [0, 1) or NULL (all zero);
 * out_dev [n_streams] int32 written when *has_output_host is set to 1 (NULL: not written).
 * The cursor advances by one per call. */
pp_status pp_generator_step(pp_generator* g, const int32_t* provided_host, const double* uniforms_host,
                            int32_t* out_dev, int32_t* has_output_host, void* stream);

/* Snapshot of a generator session's delayed-code ring (audit section 9: after a cached
 * prompt, the short token ring is restored): pp_generator_info gives the cursor s (calls
 * made so far) and the size of the ring state; pp_generator_store copies that state to
 * dst_dev; pp_generator_restore copies a stored state back from src_dev and sets the
 * cursor (>= 0). Together with pp_kv_store / pp_kv_restore of the model's ring this resumes
 * a session exactly where it was stored. */
pp_status pp_generator_info(const pp_generator* g, int64_t* cursor, uint64_t* state_bytes);
pp_status pp_generator_store(const pp_generator* g, void* dst_dev, void* stream);
pp_status pp_generator_restore(pp_generator* g, const void* src_dev, int64_t cursor, void* stream);

/* Copies of the last model step's intermediate values (any pointer may be NULL):
 * inputs_dev [n_streams] the temporal input IDs; chosen_dev [n_streams] the selection per
 * stream (supplied or drawn); text_logits_dev [text_vocab - 1]; depth_logits_dev
 * [n_steps][n_out]. Valid after the last pp_generator_step that ran the model. */
pp_status pp_generator_inspect(const pp_generator* g, int32_t* inputs_dev, int32_t* chosen_dev,
                               float* text_logits_dev, float* depth_logits_dev, void* stream);

/* ------------------------------------------------------------------ memory readers */

/* Memory readers inserted after temporal blocks ("Current sequence memory: one writer,
 * four readers" on the PersonaPlex + Inkling page, sections 1 and 6; the released
 * configuration has 4 readers after zero-based blocks 7, 15, 23, 31, 32 heads of 128, a
 * 1024-wide memory). A reader after block l adds, to the residual stream z,
 *   r = W_O concat_h(softmax_v(Q_h . K_h,v / sqrt(d_head)) V_h,v) + b_O,
 *   Q = W_Q LayerNorm(z) + b_Q (affine, eps ln_eps),  K_v = W_K m_v + b_K,  V_v = W_V m_v + b_V
 * over the visible memory rows m_v; no visible row adds nothing. Heads as the model's.
 * Weights (device pointers, kept until the model is destroyed): ln_w, ln_b [d_model]
 * float32; w_q, w_o [d_model][d_model], w_k, w_v [d_model][mem_dim] in wdtype; biases
 * [d_model] float32. Requirements: 1..8 readers on distinct blocks, mem_dim % 16 == 0,
 * d_model % 64 == 0. Readers act in batch-1 decode (and the generator); a prefill or a
 * batched step with visible memory gives PP_E_ARG. */
typedef struct {
  int32_t n_readers;
  int32_t blocks[8];
  int32_t mem_dim;
  int32_t max_slots;   /* memory rows the library keeps keys/values for */
  double ln_eps;       /* 1e-5 */
} pp_reader_config;

typedef struct {
  const float* ln_w;
  const float* ln_b;
  const void* w_q;
  const float* b_q;
  const void* w_k;
  const float* b_k;
  const void* w_v;
  const float* b_v;
  const void* w_o;
  const float* b_o;
} pp_reader_weights;

/* Attach readers (w: n_readers entries); allocates 2 x n_readers x n_heads x max_slots x
 * d_head keys/values (wdtype). Once per model. */
pp_status pp_readers_attach(pp_model* m, const pp_reader_config* cfg, const pp_reader_weights* w);
/* Write memory rows slot0 .. slot0+n-1 from mem_dev [n][mem_dim] (wdtype): every reader's
 * keys and values of those rows are formed now. slot0 + n <= max_slots, else PP_E_CAPACITY. */
pp_status pp_readers_write(pp_model* m, const void* mem_dev, int32_t slot0, int32_t n, void* stream);
/* Rows 0 .. n_visible-1 are visible to every reader from the next decode step on
 * (0 = empty memory: readers add nothing). 0 <= n_visible <= max_slots. */
pp_status pp_readers_set_visible(pp_model* m, int32_t n_visible);

/* ------------------------------------------------------------------ diagnostics */

/* Message of the last error on the calling thread ("" if none). */
const char* pp_last_error(void);

/* Decode-step launch mode of a temporal model: 0 = launch each kernel, 1 = replay a
 * captured HIP graph of the layer stack (default). */
pp_status pp_temporal_set_graph(pp_model* m, int32_t enable);

/* Split-K factor of the batch-1 decode attention: each head's visible keys are shared by
 * `splits` workgroups whose partial softmax results are merged afterwards (inside the W_O
 * product for up to 8 splits, else by a separate merge kernel). 0 = automatic (about one
 * workgroup per compute unit over all heads: 8 for 32 heads on 256 CUs); 1..64 forces a
 * value. The result does not depend on it beyond float32 rounding. Batched decode always
 * chooses its own: about one workgroup per compute unit over the B x H heads
 * (ceil(CUs / (H B)), at most the automatic value, one from B = 8 on at 32 heads). */
pp_status pp_temporal_set_attn_splits(pp_model* m, int32_t splits);

/* Kernel timing for roofline reports: when layer >= 0, every decode step brackets the
 * W_in (RMSNorm + gate/linear projection + SiLU product) kernel of that layer with HIP
 * events on the caller's stream. With repeat > 1 that kernel is launched `repeat` times
 * back to back between the two events (it reads the residual and rewrites the same
 * SwiGLU output, so the step's result is unchanged; only the step's time grows), which
 * spreads the events' own cost over the launches. pp_temporal_trace_read synchronises the
 * events and returns the number of timed launches (brackets x repeat) and the mean time
 * per launch in microseconds, then clears them. layer = -1 turns timing off; repeat must
 * be in [1, 64]. At most 2048 brackets are kept. */
pp_status pp_temporal_trace(pp_model* m, int32_t layer, int32_t repeat);
pp_status pp_temporal_trace_read(pp_model* m, int64_t* count, double* mean_us);

#ifdef __cplusplus
}
#endif

#endif /* PP_H */
