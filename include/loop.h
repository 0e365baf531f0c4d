/*
 * loop.h -- C ABI of the MI355X (gfx950) forward pass of the looped hybrid
 * decoder.
 *
 * What is computed (page citations: [P1] = hncyxsy.com/news/268323, the
 * technical article; [P2] = yuliuswiki.com/sensenova-loop-9b; [P4] =
 * yeyulingfeng.com/a/1332585.html):
 *   - [P1 section 2], [P2 section 2]: n_layers weight layers run as
 *     head [0, loop_start), the block [loop_start, loop_end) loop_passes times
 *     (B(B(h)) for two passes), tail [loop_end, n_layers), then the head:
 *     4 + 24*2 + 4 = 56 executions for the full model.
 *   - [P1 section 3]: every 4-layer group is 3 Gated-DeltaNet layers then one
 *     full-attention layer (GQA 16 Q / 4 KV heads x 256, QK-norm, sigmoid
 *     output gate, rotary on 64 of 256 dims in adjacent pairs).
 *   - [P1 section 5], [P4 section 02]: a dual-stream mHC residual inside the
 *     loop, the 2x2 stream mix Sinkhorn-normalised (20 iterations, fp32).
 *   - [P1 section 4]: every execution keeps its own KV cache / GDN state.
 *   - [P2 section 4]: greedy decoding with the cache, one token per step.
 * Every layer has a SwiGLU FFN (d -> F -> d).  Precision: bf16 weights and
 * GEMM operands with fp32 accumulation, fp32 residual / streams / mHC / GDN
 * state, bf16 KV cache, fp32 logits.
 *
 * Conventions for every entry point:
 *   - Return 0 on success or a negative LOOP_E* code; loop_last_error()
 *     then holds a message (thread-local).  No exception crosses the ABI.
 *   - "device" pointers are HIP device memory (gfx950) owned by the caller;
 *     "host" pointers are read before the call returns (never kept).
 *   - All device work is enqueued on `stream` (a hipStream_t; NULL = the
 *     null stream) and the call returns without waiting for it.
 *   - A model handle is not thread-safe; calls on one handle must not
 *     overlap (they share the workspace).
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid call enqueues nothing.
 */
#ifndef LOOP_H_
#define LOOP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  LOOP_OK = 0,
  LOOP_EINVAL = -1,    /* null pointer, bad flag, bad enum */
  LOOP_ESHAPE = -2,    /* unsupported dimensions or layer layout */
  LOOP_ECAPACITY = -3, /* arena / workspace / slot / position out of capacity */
  LOOP_EHIP = -4,      /* a HIP runtime call failed */
  LOOP_EDEVICE = -5    /* the current device is not gfx950 */
};

/* Model dimensions and capacities.  Names follow the pages: d_model = hidden
 * size, d_ff = FFN size, vocab = vocabulary (0 = no embedding / head: the
 * caller passes hidden states in and reads hidden states out).  Supported:
 * loop bounds and n_layers multiples of 4, 1 <= loop_passes,
 * n_streams == 2, head_dim in {64, 256}, rotary_dim even <= head_dim,
 * n_q_heads multiple of n_kv_heads, gdn_dk == gdn_dv in {64, 128},
 * gdn_chunk == 64, d_model multiple of 256, max_seq multiple of 64. */
typedef struct loop_config {
  int32_t n_layers, loop_start, loop_end, loop_passes;
  int32_t d_model, d_ff, vocab;
  int32_t n_q_heads, n_kv_heads, head_dim, rotary_dim;
  int32_t gdn_heads, gdn_dk, gdn_dv;
  int32_t n_streams, sinkhorn_iters;
  float rope_theta, eps;
  int32_t max_batch;  /* sequence slots held by the cache arena */
  int32_t max_seq;    /* positions per sequence slot */
  int32_t max_tokens; /* largest batch*seq_len of one call (workspace size) */
  int32_t gdn_chunk;  /* chunk length of the chunked GDN prefill (64) */
} loop_config;

/* Weights of one weight layer; all device pointers, row-major [out, in]
 * like a linear layer's weight.  bf16 unless marked fp32.
 *   attn_norm, ffn_norm [d_model]         RMSNorm gains
 *   full attention layers (layer % 4 == 3):
 *     w_in  [2*Hq*D + 2*Hkv*D, d_model]   rows [q; gate; k; v]
 *     w_o   [d_model, Hq*D]
 *     q_norm, k_norm [D]                  QK-norm gains (shared by heads)
 *   Gated-DeltaNet layers:
 *     w_in  [2*H*Dk + 2*H*Dv + 2*H, d_model]  rows [q; k; v; z; a; b]
 *     w_o   [d_model, H*Dv]
 *     o_norm [Dv]                         output RMSNorm gain
 *   w_gateup [2*d_ff, d_model]            rows [gate; up]
 *   w_down   [d_model, d_ff]
 *   loop layers only (loop_start <= layer < loop_end), fp32:
 *     mhc_read_w [2, 2*d_model], mhc_read_b [2],
 *     mhc_write_w [2, d_model], mhc_write_b [2], mhc_mix [2, 2] (logits)
 * Unused pointers may be NULL. */
typedef struct loop_layer_weights {
  const void *attn_norm, *ffn_norm;
  const void *w_in, *w_o;
  const void *q_norm, *k_norm, *o_norm;
  const void *w_gateup, *w_down;
  const float *mhc_read_w, *mhc_read_b, *mhc_write_w, *mhc_write_b, *mhc_mix;
} loop_layer_weights;

typedef struct loop_weights {
  const void* embed;      /* bf16 [vocab, d_model] (device), NULL if vocab == 0 */
  const void* final_norm; /* bf16 [d_model] (device) */
  const void* head;       /* bf16 [vocab, d_model] (device), untied */
  int32_t n_layers;
  const loop_layer_weights* layers; /* host array [n_layers], copied at create */
} loop_weights;

typedef struct loop_model loop_model;

/* ---------------------------------------------------------------- sizes
 * [P1 section 4]: full-attention KV = n_full_exec * 2 (K, V) * n_kv_heads *
 * head_dim * 2 bytes per token (57,344 B per token for the full model); GDN
 * state = n_gdn_exec * H * Dk * Dv * 4 bytes per sequence, independent of
 * the context length.  All return -1 on an invalid configuration. */
int64_t loop_kv_bytes(const loop_config* cfg, int32_t batch, int64_t seq_len);
int64_t loop_state_bytes(const loop_config* cfg, int32_t batch);
/* Arena for create: kv_bytes(max_batch, max_seq) + state_bytes(max_batch). */
int64_t loop_arena_bytes(const loop_config* cfg);
/* Workspace for create, for calls of up to max_tokens tokens. */
int64_t loop_workspace_bytes(const loop_config* cfg, int32_t max_tokens);

/* Cache layout inside the arena (byte offsets from the arena base):
 *   K of (kv slot s, sequence slot b): bf16 [n_kv_heads][max_seq][head_dim]
 *   V of (s, b):                       bf16 [n_kv_heads][max_seq/32][head_dim][32]
 *                                      (transposed in blocks of 32 positions:
 *                                      block j holds positions 32j .. 32j+31,
 *                                      dim d of them contiguous at d * 32)
 *   per kv slot s the K blocks of sequence slots 0..max_batch-1 follow each
 *   other, then the V blocks; the GDN states follow all KV slots.
 *   GDN state of (gdn slot g, b):      fp32 [gdn_heads][gdn_dv][gdn_dk]
 * which = 0 for K, 1 for V, 2 for the GDN state (s = gdn slot).  kv slot /
 * gdn slot = rank of the execution among executions of its kind.  Returns -1
 * when out of range. */
int64_t loop_cache_offset(const loop_config* cfg, int32_t which, int32_t slot, int32_t seq_slot);

/* Execution schedule, 0-based ([P1 section 2], [P4 section 03]): writes
 * n_exec rows of 6 int32 {weight layer, kind (0 GDN, 1 full), slot, loop,
 * fork, merge} into host `out` (capacity `cap` rows) and returns n_exec, or
 * a negative code. */
int32_t loop_schedule(const loop_config* cfg, int32_t* out, int32_t cap);

/* -------------------------------------------------------------- the model
 * Borrows the caller's device buffers: weights, the cache arena
 * (loop_arena_bytes) and the workspace (loop_workspace_bytes(cfg,
 * cfg->max_tokens)); they must stay alive and unmoved until destroy.  No
 * device memory is allocated.  Checks that the current device is gfx950.
 * The arena contents are not touched: a sequence slot is reset by a prefill
 * with start_pos 0. */
int loop_model_create(const loop_config* cfg, const loop_weights* w, void* d_arena,
                      size_t arena_bytes, void* d_workspace, size_t ws_bytes,
                      loop_model** out);
void loop_model_destroy(loop_model* m);

/* Prefill: seq_len new tokens for each of `batch` sequences, appended to the
 * caches of their slots at positions start_pos[b] .. start_pos[b]+seq_len-1
 * (start_pos 0 = fresh sequence: GDN state starts at zero; chunked prefill =
 * repeated calls).  Exactly one of d_tokens / d_hidden_in is given.
 *   slots      host [batch]   sequence slot of each sequence (distinct)
 *   start_pos  host [batch]
 *   d_tokens   device int32 [batch*seq_len] token ids (vocab > 0; ids
 *              outside [0, vocab) are clamped into it)
 *   d_hidden_in device fp32 [batch*seq_len, d_model]
 *   d_logits   device fp32 [batch, vocab] logits of the last position, or NULL
 *   d_hidden_out device fp32 [batch*seq_len, d_model]: h after the last
 *              execution (before the final norm), or NULL
 *   d_final_out device fp32 [batch*seq_len, d_model]: the final RMSNorm of
 *              h at every position (gain final_norm; the bf16 values the
 *              head multiplies, stored as fp32), or NULL
 *   n_taps / tap_exec (host) / d_taps device fp32 [n_taps, batch, d_model]:
 *              hidden state after the listed executions at the last position
 *              (mean of the streams inside the loop), or 0 / NULL.
 *   taps_all_positions  nonzero: the taps hold every position instead,
 *              d_taps fp32 [n_taps, batch*seq_len, d_model].
 *   loop_passes number of times the shared block runs in this call: 0 = the
 *              configuration's loop_passes, else 1 .. loop_passes.  A p-pass
 *              call runs the head layers, the block's first p passes (each
 *              execution on the cache slot it has in the full schedule) and
 *              the tail ([P1 section 2]: the pass count is a property of the
 *              forward pass, fixed per sequence); tap_exec then indexes the
 *              p-pass execution list.  A sequence keeps the count of the call
 *              that prefilled it from position 0: later calls on its slot
 *              with another count are rejected (LOOP_EINVAL).
 * Requires batch*seq_len <= max_tokens, start_pos+seq_len <= max_seq,
 * slot < max_batch.  Zero-initialise the struct: fields may be appended. */
typedef struct loop_prefill_args {
  int32_t batch, seq_len;
  const int32_t* slots;
  const int32_t* start_pos;
  const int32_t* d_tokens;
  const float* d_hidden_in;
  float* d_logits;
  float* d_hidden_out;
  int32_t n_taps;
  const int32_t* tap_exec;
  float* d_taps;
  int32_t loop_passes;
  int32_t taps_all_positions;
  float* d_final_out;
} loop_prefill_args;
int loop_prefill(loop_model* m, const loop_prefill_args* a, void* stream);

/* Decode step: one new token per sequence at position pos[b] (its current
 * length), greedy next token = argmax of the logits, lowest index on ties.
 *   slots, pos  host [batch]
 *   d_tokens    device int32 [batch]
 *   d_logits    device fp32 [batch, vocab] or NULL
 *   d_next      device int32 [batch] or NULL
 *   d_hidden_out device fp32 [batch, d_model] (h before the final norm) or NULL
 *   loop_passes 0 = the configuration's, else 1 .. loop_passes; must equal
 *               the count each sequence was prefilled with (LOOP_EINVAL). */
typedef struct loop_decode_args {
  int32_t batch;
  const int32_t* slots;
  const int32_t* pos;
  const int32_t* d_tokens;
  float* d_logits;
  int32_t* d_next;
  float* d_hidden_out;
  int32_t loop_passes;
} loop_decode_args;
int loop_decode_step(loop_model* m, const loop_decode_args* a, void* stream);

/* Decode graph: the decode step of a fixed batch captured once into a HIP
 * graph and replayed, one step per launch, so a token costs one graph launch
 * on the host instead of ~600 kernel launches ([P1 section 2]: all 56
 * executions run per generated token; [P2 section 4]: greedy decoding one
 * token per step).  Each launch computes exactly what loop_decode_step does
 * at the graph's current positions (same kernels, same launch shapes: the
 * results are bit-identical), then advances every position by one.
 *   create: `a` as for loop_decode_step; slots, loop_passes and the device
 *           buffers d_tokens / d_logits / d_next / d_hidden_out are fixed for
 *           the graph's life (their contents are read / written at each
 *           launch: d_tokens may be d_next, so that each step feeds its greedy
 *           token to the next); a->pos (host) are the first launch's
 *           positions; max_steps >= 1 launches are allowed, and every
 *           pos[b] + max_steps must be <= max_seq (LOOP_ECAPACITY).  The
 *           capture runs on an internal stream and enqueues no work; the
 *           graph keeps its own positions in device memory (allocated here).
 *   launch: one step on `stream`; LOOP_ECAPACITY after max_steps launches.
 *           Calls on the model (prefill, decode, other graphs) may come
 *           between launches on the same stream; launches must not overlap
 *           other calls on the model (they share the workspace).
 *   positions: the next launch's positions (host [batch]).
 *   destroy: frees the graph; the model must outlive it.
 * Model changes after create (loop_model_set_int8 / _int4) do not reach the
 * captured graph. */
typedef struct loop_decode_graph loop_decode_graph;
int loop_decode_graph_create(loop_model* m, const loop_decode_args* a, int32_t max_steps, loop_decode_graph** out);
int loop_decode_graph_launch(loop_decode_graph* g, void* stream);
int loop_decode_graph_positions(const loop_decode_graph* g, int32_t* pos_out);
void loop_decode_graph_destroy(loop_decode_graph* g);

/* Verify step: k tokens per sequence (k <= LOOP_VERIFY_MAX) appended at
 * positions pos[b] .. pos[b]+k-1 -- a prefill of k tokens -- with the logits
 * (and greedy next tokens, and taps) of every position, as speculative
 * decoding checks k drafted tokens in one pass ([P4 section 03]: a small
 * draft model proposes several tokens that the full model then checks).  The
 * caches advance through all k tokens: after accepting j < k of them, a
 * caller continues at position pos+j (KV entries past it are overwritten by
 * later calls) but must first restore the GDN states it saved (they are the
 * arena's state blocks, loop_cache_offset(cfg, 2, slot, b)) and feed the j
 * accepted tokens again, or re-verify from the restored state.  The taps
 * are what a drafter reads ([P4 section 03]: the draft model looks at the
 * hidden states after executions 3, 27, 51, 53 and 54).
 *   slots, pos  host [batch]
 *   d_tokens    device int32 [batch*k], sequence-major
 *   d_logits    device fp32 [batch*k, vocab] or NULL
 *   d_next      device int32 [batch*k] greedy argmax of every position (needs
 *               d_logits) or NULL
 *   d_hidden_out device fp32 [batch*k, d_model] or NULL
 *   n_taps / tap_exec (host) / d_taps device fp32 [n_taps, batch*k, d_model]:
 *               hidden state after the listed executions at every position
 *   loop_passes as for decode.
 * Requires batch*k <= max_tokens. */
#define LOOP_VERIFY_MAX 16
typedef struct loop_verify_args {
  int32_t batch, k;
  const int32_t* slots;
  const int32_t* pos;
  const int32_t* d_tokens;
  float* d_logits;
  int32_t* d_next;
  float* d_hidden_out;
  int32_t n_taps;
  const int32_t* tap_exec;
  float* d_taps;
  int32_t loop_passes;
} loop_verify_args;
int loop_verify_step(loop_model* m, const loop_verify_args* a, void* stream);

/* One execution's sequence mixer on its own, on a given input projection:
 * the part of an execution between its two projections, run with the
 * execution's cache slot exactly as loop_prefill (decode = 0) or
 * loop_decode_step (decode = 1) run it inside the stack, so that the mixer
 * can be checked on identical inputs.
 *   full attention ([P1 section 3]): QK-norm over each head's dims, rotary
 *     on the first rotary_dim dims in adjacent pairs, K / V appended to the
 *     slot's cache at positions start_pos .. start_pos+seq_len-1 ([P1
 *     section 4]), causal GQA attention over the cache, output times
 *     sigmoid(gate);
 *   Gated-DeltaNet ([P1 section 3]): L2-norm of q, k, gates, the gated
 *     delta rule from the slot's state (zero at start_pos 0) with the final
 *     state stored back, RMSNorm of the output times SiLU(z).
 *   exec       execution index of the configuration's full schedule (its
 *              weight layer, kind and cache slot)
 *   batch, seq_len, slots (host [batch]), start_pos (host [batch]) as for
 *              loop_prefill; decode = 1 requires seq_len = 1
 *   d_proj     device bf16 [batch*seq_len][ld_proj]: the in-projection
 *              output, columns [q; g; k; v] (full) or [q; k; v; z; a; b] (GDN)
 *   d_out      device bf16 [batch*seq_len][ld_out]: the mixer output, the
 *              input of W_o (n_q_heads*head_dim or gdn_heads*gdn_dv columns)
 * Uses the model's workspace (calls on one model must not overlap). */
typedef struct loop_mixer_args {
  int32_t exec;
  int32_t batch, seq_len;
  const int32_t* slots;
  const int32_t* start_pos;
  int32_t decode;
  const void* d_proj;
  int64_t ld_proj;
  void* d_out;
  int64_t ld_out;
} loop_mixer_args;
int loop_exec_mixer(loop_model* m, const loop_mixer_args* a, void* stream);

/* Sinkhorn-normalised stream-mix matrices of every loop layer as the device
 * computes them ([P1 section 5]): fp32 [loop_end-loop_start, 2, 2] into
 * device d_out. */
int loop_debug_mhc(loop_model* m, float* d_out, void* stream);

/* ------------------------------------------------------------ int8 decode
 * Weight-only INT8 for the decode projections ([P1 section 7] estimates the
 * bf16 weights at about 18 GB, about 9 GB in INT8).  Per output row n of a
 * [N][K] matrix: scale s_n = max_k |w_nk| / 127 (fp32) and codes q_nk = the
 * nearest integer to w_nk / s_n (ties to even; fp32, correctly rounded
 * division), in [-127, 127]; a zero row has s_n = 0 and q = 0.  The decode
 * projections compute with s_n * q_nk.
 * loop_quantize_int8: codes and scales of one bf16 matrix, on the device.
 *   d_w bf16 [N][ldw] (device), d_q int8 [N][K] (device, row stride K),
 *   d_scale fp32 [N] (device).  LOOP_EINVAL for N < 1, K < 1, ldw < K or
 *   NULL buffers.
 * loop_model_set_int8: from now on decode steps (loop_decode_step) use the
 * codes of every layer's in / O / gate-up / down projection instead of its
 * bf16 matrix; prefill, verify and the head keep bf16.  layers: host
 * [n_layers] (copied); each matrix's codes (int8, the bf16 matrix's shape,
 * row stride = its K) and scales (fp32 [rows]) are device buffers borrowed
 * until the model is destroyed or int8 is turned off.  NULL turns it off
 * (and so does registering int4 codes).
 * Requires every K (d_model, the mixer widths, d_ff) to be a multiple of 128;
 * decode calls then take at most 64 sequences. */
typedef struct loop_q8_layer {
  const int8_t* w_in;
  const float* s_in;
  const int8_t* w_o;
  const float* s_o;
  const int8_t* w_gateup;
  const float* s_gateup;
  const int8_t* w_down;
  const float* s_down;
} loop_q8_layer;
int loop_quantize_int8(const void* d_w, int64_t N, int64_t K, int64_t ldw, int8_t* d_q, float* d_scale,
                       void* stream);
int loop_model_set_int8(loop_model* m, const loop_q8_layer* layers);

/* ------------------------------------------------------------ int4 decode
 * Weight-only INT4 for the decode projections ([P1 section 7] estimates
 * about 4.5 GB in INT4; the pages give no format).  Group-wise symmetric:
 * per output row n and group g of 128 consecutive k, scale
 * s_ng = max |w| over the group / 7 (fp32) and codes q = the nearest integer
 * to w / s_ng (ties to even; fp32, correctly rounded division) in [-7, 7];
 * a zero group has s = 0 and q = 0.  The decode projections compute with
 * the bf16 value nearest to the fp32 product q * s_ng.  Storage: codes + 8
 * in nibbles, each run of 8 consecutive k in 4 bytes, byte i holding k = i
 * in its low nibble and k = i + 4 in its high nibble (K / 2 bytes per row);
 * scales fp32 [N][K / 128].
 * loop_quantize_int4: codes and scales of one bf16 matrix, on the device.
 *   d_w bf16 [N][ldw] (device), d_q uint8 [N][K / 2] (device, row stride
 *   K / 2), d_scale fp32 [N][K / 128] (device).  LOOP_EINVAL for N < 1,
 *   K < 1 or not a multiple of 128, ldw < K or NULL buffers.
 * loop_model_set_int4: as loop_model_set_int8, with int4 codes (row stride
 * K / 2 bytes, 16-byte aligned) and group scales (fp32 [rows][K / 128]).
 * Registering int4 codes turns int8 off and the reverse; NULL turns int4
 * off. */
typedef struct loop_q4_layer {
  const uint8_t* w_in;
  const float* s_in;
  const uint8_t* w_o;
  const float* s_o;
  const uint8_t* w_gateup;
  const float* s_gateup;
  const uint8_t* w_down;
  const float* s_down;
} loop_q4_layer;
int loop_quantize_int4(const void* d_w, int64_t N, int64_t K, int64_t ldw, uint8_t* d_q, float* d_scale,
                       void* stream);
int loop_model_set_int4(loop_model* m, const loop_q4_layer* layers);

/* Weight-only quantized GEMM: one decode projection on its own, with the
 * kernels loop_decode_step runs when int8 / int4 codes are registered.
 * C[M,N] = A[M,K] . W[N,K]^T with W the dequantized codes of
 * loop_quantize_int8 (bits 8: W[n][k] = s_n q_nk) or loop_quantize_int4
 * (bits 4: W[n][k] = the bf16 value nearest to s_ng q_nk); the epilogues of
 * loop_op_gemm (SwiGLU: the codes and scales hold the gate rows then the up
 * rows, 2N rows).  A bf16 [M][lda] (device, 16-byte aligned); Bq the codes
 * (device, ldq bytes per row, 16-byte aligned rows); scale as the quantizer
 * writes it (device).  Requires 1 <= M <= 64, K % 128 == 0, lda % 8 == 0,
 * lda >= K, ldq % 16 == 0 and ldq >= the code bytes of a row; LOOP_ESHAPE /
 * LOOP_EINVAL otherwise (nothing enqueued).  d_ws / ws_bytes as for
 * loop_op_gemm (split-K partials, summed in split order). */
int loop_op_gemm_quant(int32_t bits, const void* A, int64_t lda, const void* Bq, int64_t ldq, const float* scale,
                       void* C, int64_t ldc, const float* R, int32_t M, int32_t N, int32_t K, int32_t epi,
                       float* d_ws, size_t ws_bytes, void* stream);

const char* loop_last_error(void);

/* Kernel timing of one kernel class inside the model calls: with class c
 * selected (c >= 0), every launch of that class made by loop_prefill /
 * loop_decode_step is bracketed by two HIP events on the call's stream;
 * loop_profile_read waits for them and returns the summed duration (ms) and
 * the number of launches since the last read, then clears them.  c = -1
 * turns it off.  Classes: */
enum {
  LOOP_K_GEMM_GATEUP = 0, LOOP_K_GEMM_DOWN = 1, LOOP_K_GEMM_IN = 2, LOOP_K_GEMM_O = 3,
  LOOP_K_ATTN_PREP = 4, LOOP_K_FLASH = 5, LOOP_K_GDN = 6, LOOP_K_DECODE_ATTN = 7,
  LOOP_K_ROWS = 8, LOOP_K_HEAD = 9, LOOP_K_NCLASS = 10
};
int loop_profile(loop_model* m, int32_t kernel_class);
int loop_profile_read(loop_model* m, double* total_ms, int64_t* launches);

/* ------------------------------------------------------ single operations
 * The kernels of the path, callable one at a time (same kernels the model
 * launches).  Device pointers; row-major; return codes as above.
 *
 * GEMM C[M,N] = A[M,K] . B[N,K]^T (bf16 operands, fp32 accumulation), with
 * the epilogue `epi`:
 *   LOOP_EPI_BF16     C bf16 [M, ldc]
 *   LOOP_EPI_F32      C fp32
 *   LOOP_EPI_F32_RES  C fp32 = R + A.B^T (R fp32 [M, ldc], may alias C)
 *   LOOP_EPI_SWIGLU   B holds [gate; up] (2*N rows); C bf16 [M, N] =
 *                     silu(A.gate^T) * (A.up^T)
 * Requires K % 64 == 0, lda and ldb multiples of 8, A and B 16-byte aligned.
 * d_ws / ws_bytes (device, optional): fp32 scratch for split-K partials,
 * used when M is small (< 512), or for the ragged edges of a large-M call
 * (rows past the last multiple of 256, columns past the last whole 256-wide
 * tile), and the buffer is large enough; the partials are summed in split
 * order (deterministic).  NULL = no split. */
enum { LOOP_EPI_BF16 = 0, LOOP_EPI_F32 = 1, LOOP_EPI_F32_RES = 2, LOOP_EPI_SWIGLU = 3 };
int loop_op_gemm(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                 const float* R, int32_t M, int32_t N, int32_t K, int32_t epi, float* d_ws,
                 size_t ws_bytes, void* stream);

/* GEMM that allocates nothing: loop_op_gemm for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same operands,
 * epilogues, kernels and results as loop_op_gemm given a large enough d_ws;
 * the split-K partials of small-M calls live in a static device array of the
 * library instead (LOOP_GEMM_STATIC_SCRATCH_BYTES, one copy per GPU, held
 * until the process ends).  Takes at most LOOP_GEMM_STATIC_MAX_ROWS rows
 * (decode-sized products); a call whose partials would not fit the array is
 * rejected with LOOP_ECAPACITY (nothing enqueued).  No hipMalloc / hipFree:
 * the device address of the array is looked up once per device on the
 * first call there.  Every call on one GPU shares that GPU's array, so calls
 * that overlap on one GPU (other streams, other threads) race; calls ordered
 * on one stream do not.  Every partial a call reads is written by that call
 * first, so the array needs no clearing. */
#define LOOP_GEMM_STATIC_SCRATCH_BYTES (32u << 20)
#define LOOP_GEMM_STATIC_MAX_ROWS 64
int loop_op_gemm_static(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                        const float* R, int32_t M, int32_t N, int32_t K, int32_t epi, void* stream);

/* -------------------------------------------------- synthetic inputs
 * Device implementation of the seeded input generator (Philox4x32-10,
 * Salmon et al. SC'11, + Box-Muller in float64): element i of stream
 * (seed, key) takes word i%4 of the Philox block i/4 (counter (i/4 lo,
 * i/4 hi, 0, 0), key (seed, key)); normals from word pairs (0,1), (2,3),
 * u = (x + 0.5) 2^-32, value = fp32(z*std + mean), optionally rounded to bf16
 * (nearest even).  dtype 0 = fp32, 1 = bf16.  Writes n elements to device
 * `dst`, element i of the call being stream element start+i. */
int loop_synth_normal(void* dst, int64_t n, int32_t dtype, uint32_t seed, uint32_t key,
                      int64_t start, double std, double mean, void* stream);
/* Uniform ids (x * vocab) >> 32, int32, stream elements 0 .. n-1. */
int loop_synth_token_ids(int32_t* dst, int64_t n, uint32_t vocab, uint32_t seed, uint32_t key,
                         void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LOOP_H_ */
