/*
 * mk.h -- C ABI of the MI355X (gfx950) low-latency decode megakernel.
 *
 * One call, mk_decode_step, runs the whole batch-1 decode forward pass of a
 * Llama-style decoder (pre-norm, GQA attention with RoPE, SwiGLU FFN, RMSNorm,
 * tied or untied LM head, greedy argmax) as ONE persistent GPU kernel: every
 * workgroup stays resident on its compute unit, walks a host-planned task tape
 * and waits on flags in device memory instead of on kernel boundaries.
 *
 * Source of the operations: the pages "Revolution der KI-Beschleunigung: Wie
 * ein Low-Latency Megakernel den Llama-1B Turbo zuendet" (dasgeld.co) and the
 * glossary entry "Megakernel" (synthszr.com).  The article describes fusing all
 * steps of the Llama-1B bf16 forward pass into one kernel, an instruction
 * interpreter fed with sequences planned once on the host and reused for every
 * forward pass, dependency tracking through global counters in GPU memory, and
 * a paged shared memory that lets the next load start while another finishes.
 * The glossary section "Wie eine ganze Rechenkette in ein Programm passt" adds
 * that the kernel is started once and takes its tasks from a work list, and
 * that counters and signals in memory replace host control between launches.
 * The pages give no API and no model formulas; the calls below follow the
 * problem as the pages state it (per-token decode with a reusable host plan)
 * and the model is the textbook Llama-style decoder.
 *
 * Conventions for every call:
 *   - return 0 (MK_OK) on success, a negative MK_E_* code on failure;
 *   - pointers marked "device" must be device memory of the current HIP device;
 *   - bf16 tensors are passed as uint16_t bit patterns;
 *   - matrices are row-major [out][in];
 *   - the library never frees memory it did not allocate.
 */
#ifndef MK_H_
#define MK_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Error codes. */
#define MK_OK 0
#define MK_E_INVAL (-1)       /* null, misaligned or inconsistent argument        */
#define MK_E_RANGE (-2)       /* position outside [0, max_seq)                     */
#define MK_E_HIP (-3)         /* a HIP runtime call failed                         */
#define MK_E_STATE (-4)       /* a device error is latched; call mk_reset          */
#define MK_E_TIMEOUT (-5)     /* a dependency wait exceeded the watchdog budget    */
#define MK_E_TOKEN (-6)       /* an input token id was outside [0, vocab)          */
#define MK_E_NOMEM (-7)       /* device or host allocation failed                  */
#define MK_E_UNSUPPORTED (-8) /* configuration not supported by this build         */
#define MK_E_DEVICE (-9)      /* device does not fit the persistent launch         */
#define MK_E_TOOBIG (-10)     /* the step needs more than the fixed static scratch  */

/* Execution modes of mk_decode_step. */
#define MK_MODE_MEGA 0       /* one persistent kernel per decode step                        */
#define MK_MODE_MULTI 1      /* the megakernel's executors, one launch per stage             */
#define MK_MODE_GRAPH 2      /* the MULTI launches captured once into a hipGraph             */
#define MK_MODE_CONV 3       /* conventional path: one plain kernel per operation (see
                                mk_conv_decode_step), the bubble baseline                    */
#define MK_MODE_CONV_GRAPH 4 /* the MK_MODE_CONV launches captured once into a hipGraph      */

/* Model and run configuration.
 * Llama-style decoder: n_layers, hidden H, n_heads query heads and n_kv_heads
 * key/value heads of head_dim each (n_heads % n_kv_heads == 0, head_dim even),
 * SwiGLU width ffn, vocabulary vocab.  max_seq bounds the positions and is
 * the slot count of the caller's KV cache; batch is the number of independent
 * sequences decoded per step (1..8; 2..8 run the GEMVs as skinny MFMA GEMMs
 * and need head_dim 64).  rms_eps and rope_theta are
 * the RMSNorm epsilon and the RoPE base.  tie_embeddings != 0 uses the
 * embedding matrix as LM head.  exec_mode is one of MK_MODE_*.
 * attn_chunks: split of [0, pos] per KV head in attention (0 = automatic).
 * num_wgs: persistent workgroups (0 = one per compute unit).
 * watchdog_ms: budget of any single dependency wait (0 = 2000 ms; a negative
 * value is a budget of -watchdog_ms device clock ticks, which lets tests drive
 * the timeout path with every workgroup still leaving the kernel normally).
 * trace: non-zero records, for every (workgroup, stage) of the latest step,
 * the device wall-clock stamps of mk_trace_copy, in a kernel build of its own
 * (head_dim 64, without partial_input; otherwise mk_load returns
 * MK_E_UNSUPPORTED); off for timing runs.
 * partial_input: non-zero starts every wave of the down projection as soon as
 * its quarter of the gate/up output is ready instead of waiting for all of it
 * (the pages' operations that begin on partial input; batch 1, head_dim 64;
 * a separate kernel build, slower than the default on MI355X, see the
 * repository's design notes).
 * prefill: non-zero makes the batch the next `batch` tokens of ONE sequence
 * (2..8 tokens, the batched MFMA executors): mk_decode_step then takes the
 * tokens of positions pos .. pos + batch - 1 in d_token[batch], kv points at
 * that one sequence's cache ([1][n_layers][n_kv_heads][max_seq][head_dim]),
 * every token attends to the cache below pos plus the tokens of this call up
 * to itself (causal), their K/V go to slots pos .. pos + batch - 1, and
 * out_logits[batch][vocab] / out_token[batch] are each token's next-token
 * logits and greedy token: a prompt is run `batch` tokens per launch, each
 * launch reading the weights once (the prompt as MFMA GEMM tasks).  Not with
 * mk_decode_steps or the MK_MODE_CONV modes. */
typedef struct mk_config {
  int32_t n_layers;
  int32_t hidden;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t ffn;
  int32_t vocab;
  int32_t max_seq;
  int32_t batch;
  float rms_eps;
  double rope_theta;
  int32_t tie_embeddings;
  int32_t exec_mode;
  int32_t attn_chunks;
  int32_t num_wgs;
  int32_t watchdog_ms;
  int32_t trace;
  int32_t partial_input;
  int32_t prefill;
  int32_t reserved[4];
} mk_config;

/* Device pointers to one layer's bf16 weights (row-major [out][in]):
 * attn_norm[H], wq[n_heads*head_dim][H], wk[n_kv_heads*head_dim][H],
 * wv[n_kv_heads*head_dim][H], wo[H][n_heads*head_dim], ffn_norm[H],
 * w_gate[ffn][H], w_up[ffn][H], w_down[H][ffn]. */
typedef struct mk_layer_weights {
  const uint16_t* attn_norm;
  const uint16_t* wq;
  const uint16_t* wk;
  const uint16_t* wv;
  const uint16_t* wo;
  const uint16_t* ffn_norm;
  const uint16_t* w_gate;
  const uint16_t* w_up;
  const uint16_t* w_down;
} mk_layer_weights;

/* Model weights: device pointers embed[vocab][H], final_norm[H], lm_head
 * [vocab][H] (NULL iff tie_embeddings), and a HOST array of n_layers
 * mk_layer_weights.  mk_load copies every layer matrix into a library-owned
 * packed layout.  embed is read in place (the first layer gathers its rows),
 * and so is the LM head (embed when tied, else lm_head) when hidden is a
 * multiple of 512 and needs no row padding: those buffers must stay valid
 * until mk_free; all others may be released once mk_load returns. */
typedef struct mk_weights {
  const uint16_t* embed;
  const uint16_t* final_norm;
  const uint16_t* lm_head;
  const mk_layer_weights* layers;
} mk_weights;

/* Caller-owned bf16 KV cache, device memory, layout
 * [batch][n_layers][n_kv_heads][max_seq][head_dim] for K and for V.
 * Keys are stored after the rotary embedding.  Both may be NULL when
 * n_layers == 0. */
typedef struct mk_kv {
  uint16_t* k;
  uint16_t* v;
} mk_kv;

/* Latched device status.  code is MK_OK or the first device error;
 * task/stage/wg locate a watchdog timeout, detail holds the bad token id
 * or the value the wait last observed. */
typedef struct mk_status_t {
  int32_t code;
  int32_t stage;
  int32_t wg;
  uint32_t detail;
} mk_status_t;

/* Plan summary (host only; see mk_plan_describe). */
typedef struct mk_plan_info {
  int32_t num_wgs;        /* persistent workgroups                          */
  int32_t num_stages;     /* stages on the tape (5 per layer + LM head)     */
  int32_t num_tasks;      /* non-empty (stage, workgroup) entries           */
  int32_t attn_chunks;    /* KV split per head used by attention            */
  int64_t weight_bytes;   /* bytes of the packed weight arena               */
  int64_t workspace_bytes;/* bytes of activations, flags, tape, tables      */
  int32_t lds_bytes;      /* dynamic LDS per workgroup                      */
  int32_t ring_units;     /* 1 KiB weight units each wave keeps in flight   */
  int32_t reserved[4];
} mk_plan_info;

typedef struct mk_handle mk_handle;

/* mk_load -- validate cfg, pack the weights, build the task tape, allocate the
 * workspace, and return a handle in *out.
 * The tape splits every matrix op of every layer into row tiles, one tile per
 * workgroup and stage (the article's instruction sequences planned on the host
 * once and reused for every forward pass).  All device work runs on the null
 * stream and is complete on return.
 * Errors: MK_E_INVAL (bad cfg/pointers), MK_E_UNSUPPORTED (includes, for
 * now, head_dim 128, hidden > 2048 and packed weights of 4 GiB or more in the
 * megakernel modes: such plans build on the host but are not run),
 * MK_E_DEVICE, MK_E_NOMEM, MK_E_HIP.  On error *out is NULL and nothing
 * leaks. */
int mk_load(const mk_config* cfg, const mk_weights* w, mk_handle** out);

/* mk_decode_step -- one decode step at position pos for every sequence.
 * This is the forward pass the article runs as one kernel: per layer RMSNorm,
 * the Q/K/V projections with the rotary embedding and the KV append, the
 * attention over the cache, the output projection with its residual, the
 * gated FFN with its residual, then the final norm, the LM head and the
 * greedy token (article, the paragraphs on the Llama-1B forward pass as one
 * kernel; glossary "Megakernel", "Wie eine ganze Rechenkette in ein Programm
 * passt": the kernel runs the whole chain of operations of one token).
 * d_token[batch] (device int32) holds the input token ids; the previous
 * step's out_token may be passed directly.  kv is the caller's cache: slot
 * pos of every (sequence, layer, kv head) is written, slots [0, pos] are read,
 * slots above pos are never touched.  out_logits[batch][vocab] (device fp32)
 * and out_token[batch] (device int32, first index of the maximum logit) are
 * written.  Asynchronous on stream; allocates nothing and never synchronises.
 * Synchronous errors: MK_E_INVAL, MK_E_RANGE, MK_E_STATE (an earlier step
 * latched a device error: see mk_status), MK_E_HIP.  A device-side bad token
 * latches MK_E_TOKEN and writes out_token = -1; a wait that exceeds the
 * watchdog latches MK_E_TIMEOUT and ends the kernel early.
 * One handle must not be used from two streams or threads at once. */
int mk_decode_step(mk_handle* h, const int32_t* d_token, int32_t pos, const mk_kv* kv,
                   float* out_logits, int32_t* out_token, hipStream_t stream);

/* mk_decode_steps -- n_steps greedy decode steps at positions pos ..
 * pos + n_steps - 1 for every sequence, the argmax of each step feeding the
 * embedding gather of the next on the device.  In MK_MODE_MEGA this is ONE
 * persistent launch that walks the task tape n_steps times (the glossary
 * entry "Megakernel", section "Wie eine ganze Rechenkette in ein Programm
 * passt": the kernel is started once and then keeps running): the last
 * workgroup of each step's argmax publishes the next tokens as tagged words
 * that every workgroup polls before the next step's first stage.  In every
 * other mode the steps are issued one by one (in the graph modes a step whose
 * pointers differ from the captured ones recaptures the graph).
 * d_token[batch] (device int32): the first step's input tokens.
 * out_tokens[n_steps][batch] (device int32): the greedy token of every step.
 * out_logits: [n_steps][batch][vocab] device fp32, or NULL when the logits
 * are not wanted (they then go to a buffer of the handle).  kv as in
 * mk_decode_step: slots pos .. pos + n_steps - 1 are written.  Asynchronous
 * on stream; allocates nothing and never synchronises.
 * Errors: MK_E_INVAL (null pointers, n_steps < 1, misalignment), MK_E_RANGE
 * (pos < 0 or pos + n_steps > max_seq), MK_E_STATE, MK_E_HIP.  A device error
 * (bad token, watchdog) is latched as in mk_decode_step; later steps of the
 * same call then stop early. */
int mk_decode_steps(mk_handle* h, const int32_t* d_token, int32_t pos, int32_t n_steps, const mk_kv* kv,
                    float* out_logits, int32_t* out_tokens, hipStream_t stream);

/* mk_reset -- wait for the handle's last stream, clear every flag, counter and
 * latched error and restart the step count.  Weights and the caller's cache
 * are untouched; a new sequence simply starts at pos = 0.  The plan built by
 * mk_load is kept: the article's instruction sequences are planned once on
 * the host and reused for every forward pass, so a new sequence only resets
 * the dependency state the kernel keeps in device memory.
 * Errors: MK_E_INVAL (null handle), MK_E_HIP. */
int mk_reset(mk_handle* h);

/* mk_free -- wait for outstanding work and release everything the handle owns. */
void mk_free(mk_handle* h);

/* mk_status -- copy the latched device status (no synchronisation). */
int mk_status(mk_handle* h, mk_status_t* out);

/* mk_error_string -- static text for an MK_* code. */
const char* mk_error_string(int code);

/* mk_trace_copy -- wait for the device, then copy the trace of the latest
 * step into host memory out[capacity_words]: num_wgs * num_stages records of
 * 20 uint64 stamps read from the device-wide constant-rate clock
 * (s_memrealtime): {stage entered, inputs ready, compute done, stage left,
 * then the time each of the 8 waves finished its own part, then the time each
 * wave had its first weight unit of the task}; record (wg, stage) starts at
 * word 20 * (wg * num_stages + stage), and a stamp of 0
 * means the workgroup (or wave) had no work there.  *words_written gets the
 * word count and *clock_khz the clock rate.  Errors: MK_E_INVAL (null,
 * capacity too small, handle loaded without cfg.trace), MK_E_HIP. */
int mk_trace_copy(mk_handle* h, uint64_t* out, int64_t capacity_words, int64_t* words_written,
                  int32_t* clock_khz);

/* mk_plan_describe -- build and validate the task tape for cfg on num_wgs
 * workgroups (0 = assume 256) on the HOST ONLY, without touching a GPU, and
 * fill *out.  Returns MK_OK if the tape passes the validator: stages in
 * dependency order, every row pair of every matrix covered exactly once
 * (in batched plans a 16-row block of the O- or down projection may be split
 * over two workgroups by halves of its columns: then once per half, on
 * neighbouring workgroups), every (kv head, chunk) attention task present
 * once, LDS and scratch bounds respected. */
int mk_plan_describe(const mk_config* cfg, int32_t num_wgs, mk_plan_info* out);

/* ---------------------------------------------------------------------------
 * The conventional path: one plain kernel launch per operation.
 *
 * The article's paragraphs on the typical challenges of decode and on mid-size
 * models, and the glossary entry "Megakernel", section "Warum die Pausen
 * zwischen den Rechenschritten teuer sind", describe the usual execution that
 * the megakernel replaces: the forward pass as a long series of short kernels,
 * each started separately, with idle gaps between them that streams and
 * graphs shorten but do not remove.  These calls run that usual execution on
 * the same weights and cache layout, with kernels that share nothing with the
 * megakernel: per layer RMSNorm, the Q, K and V GEMVs, RoPE + KV append,
 * split-KV attention and its merge, O projection + residual, RMSNorm, the
 * gate and up GEMVs, SiLU product, down projection + residual; then the final
 * RMSNorm, the LM head and a two-kernel argmax (4 + 13 * n_layers launches).
 * Activations are fp32.  The handle modes MK_MODE_CONV and MK_MODE_CONV_GRAPH
 * run it through mk_load / mk_decode_step; a caller can also capture one call
 * into its own hipGraph: every launch is a kernel and the position is read
 * from device memory.
 * ------------------------------------------------------------------------- */

/* mk_conv_workspace_size -- bytes of the fp32 workspace one conventional step
 * needs for cfg (activations, attention partials, argmax partials).  Only the
 * model dimensions, max_seq and batch (1..8) of cfg are used.
 * Errors: MK_E_INVAL (null, or dimensions that are not positive, head_dim,
 * hidden or ffn not multiples of 8, n_heads not a multiple of n_kv_heads),
 * MK_E_UNSUPPORTED (head_dim above 128 or not 8 times a power of two, batch
 * above 8). */
int mk_conv_workspace_size(const mk_config* cfg, size_t* bytes);

/* mk_conv_decode_step -- one decode step of cfg.batch sequences with the
 * conventional path, asynchronous on stream.
 * w: the caller's weights (device pointers, read in place; every matrix and
 * the LM head 16-byte aligned; the host array w->layers is read during the
 * call only).  d_token[batch] (device int32): input tokens.  d_pos (device
 * int32): the position, in [0, max_seq) (a position outside it makes every
 * kernel return without writing the cache).  kv: the caller's bf16 cache as in
 * mk_decode_step (16-byte aligned); slot pos is written, [0, pos] read.
 * out_logits[batch][vocab] (device fp32) and out_token[batch] (device int32,
 * first index of the maximum; -1 for an input token outside [0, vocab)) are
 * written.  workspace: device memory of at least mk_conv_workspace_size
 * bytes, 256-byte aligned, owned by the caller and not used by any other
 * work until the step has run.  Allocates nothing, never synchronises.
 * Errors: those of mk_conv_workspace_size, MK_E_INVAL (null or misaligned
 * pointers, workspace too small), MK_E_HIP (a launch failed). */
int mk_conv_decode_step(const mk_config* cfg, const mk_weights* w, const int32_t* d_token, const int32_t* d_pos,
                        const mk_kv* kv, float* out_logits, int32_t* out_token, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* mk_conv_decode_step_static -- mk_conv_decode_step for callers that cannot
 * allocate device memory at all (code under hipGraph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the workspace is a fixed buffer of
 * 8 MiB in the library's static device memory, one per GPU, looked up on the
 * first call made on that GPU (enough for the Llama-1B shape at batch 8 over
 * 8192 positions; compare mk_conv_workspace_size).  The
 * caller still passes inputs and outputs; arguments and results are exactly
 * those of mk_conv_decode_step.  Calls on one GPU share that buffer: calls
 * that overlap in time on one GPU (other streams, other threads) race and must
 * be serialised by the caller.  Allocates nothing, never synchronises.
 * Errors: those of mk_conv_decode_step, MK_E_TOOBIG (the configuration needs a
 * workspace larger than the buffer; see mk_conv_workspace_size), MK_E_HIP. */
int mk_conv_decode_step_static(const mk_config* cfg, const mk_weights* w, const int32_t* d_token,
                               const int32_t* d_pos, const mk_kv* kv, float* out_logits, int32_t* out_token,
                               hipStream_t stream);

/* ---------------------------------------------------------------------------
 * W2A8 matrix-vector product: ternary weights (-1, 0, 1) stored in two bits,
 * int8 activations.  After the page "BitNet 1.58bit GPU Inference Kernel:
 * Revolutionaere Effizienz fuer KI-Modelle mit W2A8-Quantisierung"
 * (dasgeld.co, body: two-bit weights and eight-bit activations, sixteen
 * two-bit values packed per 32-bit word for parallel decoding, 4-wide int8
 * dot products).  The page prints no quantiser; the activations are coded as
 * in BitNet b1.58:
 *   s = 127 / max(max_k |x_k|, 1e-5),  q_k = clamp(round_half_even(x_k * s), -128, 127)
 *   y_r = (float(sum_k Q_rk q_k) * gamma_r) / s        (float32, in this order)
 * with Q the ternary codes and gamma_r the scale of row r (per-row absmean,
 * or one value repeated for a per-tensor scale).
 * ------------------------------------------------------------------------- */

/* mk_w2a8_pack -- host: ternary codes [rows][cols] (int8, each -1, 0 or 1,
 * row-major) into the packed matrix [rows][cols / 16] (uint32): word w of a
 * row holds columns 16 w .. 16 w + 15, column 16 w + 4 k + m as code + 1 at
 * bits 8 m + 2 k (k, m in 0..3).  Both buffers are host memory owned by the
 * caller.  Errors: MK_E_INVAL (cols not a multiple of 64, negative sizes, null
 * pointers, a code outside -1..1; packed is then partly written). */
int mk_w2a8_pack(const int8_t* codes, int rows, int cols, uint32_t* packed);

/* mk_w2a8_quantize -- device: the int8 codes d_xq[cols] and the scale
 * *d_scale of the float32 vector d_x[cols], as above, enqueued on stream (one
 * workgroup).  0 <= cols <= 16384, cols a multiple of 64.  Non-finite inputs
 * give unspecified codes.  Errors: MK_E_INVAL, MK_E_HIP. */
int mk_w2a8_quantize(const float* d_x, int cols, int8_t* d_xq, float* d_scale, hipStream_t stream);

/* mk_w2a8_gemv -- device: d_y[rows] (float32) from the packed matrix
 * d_packed (mk_w2a8_pack's layout, 16-byte aligned), the row scales
 * d_gamma[rows], the activation codes d_xq[cols] (16-byte aligned) and their
 * scale *d_scale, enqueued on stream.  The integer sums are exact, so the
 * result is bit-for-bit the formula above.  0 <= cols <= 16384, cols a
 * multiple of 64; rows == 0 is a no-op.  Errors: MK_E_INVAL, MK_E_HIP. */
int mk_w2a8_gemv(const uint32_t* d_packed, const float* d_gamma, int rows, int cols, const int8_t* d_xq,
                 const float* d_scale, float* d_y, hipStream_t stream);

/* mk_w2a8_linear -- device: the whole product from a float32 input in one
 * launch: every workgroup finds max |x| over d_x[cols] (16-byte aligned) and
 * codes the columns it needs itself, so the codes, the scale and d_y[rows]
 * are bit-for-bit those of mk_w2a8_quantize followed by mk_w2a8_gemv.  Same
 * sizes and errors as mk_w2a8_gemv. */
int mk_w2a8_linear(const uint32_t* d_packed, const float* d_gamma, int rows, int cols, const float* d_x, float* d_y,
                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MK_H_ */
