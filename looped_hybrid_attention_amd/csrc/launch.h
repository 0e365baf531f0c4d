// Host-side launchers of the kernels (one per kernel family).  Each enqueues
// on stream `s` and returns the launch status; argument checks are done by
// the callers in host.cpp.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "../../include/loop.h"

// ws / ws_bytes: optional fp32 buffer for split-K partials (small M); NULL
// or too small = no split.
hipError_t launch_gemm(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                       const float* R, int M, int N, int K, int epi, hipStream_t s, float* ws = nullptr,
                       size_t ws_bytes = 0);

// Split-K partial bytes that launch_gemm uses for a call of M < 512 rows when
// its buffer is large enough (0: the call does not split; M >= 512: 0).
size_t gemm_small_m_partial_bytes(int M, int N, int K, int epi, int64_t lda, int64_t ldb);

// C = A . B^T (+ R) as launch_gemm (fp32 output), then
// hn[m] = bf16(RMSNorm(C[m] + X2[m]; gain)) (X2 may be NULL; rows of C and
// X2 share the stride ldc; hn rows are N apart).
// Weight-only projections for decode rows (M <= 64), bits = 8: B is int8
// [rows][ldb] with a per-row fp32 scale; bits = 4: B is packed int4 codes
// (ldb bytes per row) with fp32 scales [rows][K / 128].  K a multiple of 128,
// ldb of 16, lda of 8.
hipError_t launch_gemm_wq(int bits, const void* A, int64_t lda, const void* Bq, int64_t ldb, const float* scale,
                          void* C, int64_t ldc, const float* R, int M, int N, int K, int epi, hipStream_t s, float* ws,
                          size_t ws_bytes);
hipError_t launch_gemm_norm_wq(int bits, const void* A, int64_t lda, const void* Bq, int64_t ldb, const float* scale,
                               float* C, int64_t ldc, const float* R, const float* X2, const void* gain, void* hn,
                               float eps, int M, int N, int K, hipStream_t s, float* ws, size_t ws_bytes);
hipError_t launch_quantize_int4(const void* w, int64_t ldw, int64_t N, int K, uint8_t* q, int64_t ldq, float* scale,
                                hipStream_t s);
hipError_t launch_quantize_int8(const void* w, int64_t ldw, int64_t N, int K, int8_t* q, int64_t ldq, float* scale,
                                hipStream_t s);
hipError_t launch_gemm_norm(const void* A, int64_t lda, const void* B, int64_t ldb, float* C, int64_t ldc,
                            const float* R, const float* X2, const void* gain, void* hn, float eps, int M, int N,
                            int K, hipStream_t s, float* ws, size_t ws_bytes);

hipError_t launch_synth_normal(void* dst, int64_t n, int dtype, uint32_t seed, uint32_t key,
                               int64_t start, double std, double mean, hipStream_t s);
hipError_t launch_synth_token_ids(int32_t* dst, int64_t n, uint32_t vocab, uint32_t seed,
                                  uint32_t key, hipStream_t s);

// ---- row kernels
hipError_t launch_embed(const int32_t* ids, const void* E, float* h, int M, int d, int vocab, hipStream_t s);
// y[i] = bf16(RMSNorm(x[row_i] (+ x2[row_i])) * g); rows = NULL: row i = i.
hipError_t launch_rmsnorm(const float* x, const float* x2, const int32_t* rows, int64_t x_stride,
                          const void* g, void* y, int M, int d, float eps, hipStream_t s);
// y fp32 [M][d]: the bf16 values of the RMSNorm above, stored as fp32
hipError_t launch_rmsnorm_f32(const float* x, const void* g, float* y, int M, int d, float eps, hipStream_t s);

enum { TR_IN_H = 0, TR_IN_WRITE = 1 };
enum { TR_OUT_NORM = 0, TR_OUT_READ = 1, TR_OUT_NONE = 2 };
struct TransitionArgs {
  int in_mode, out_mode, M, d, iters, rows_per_block;
  float eps;
  const float* h;    // in = H: current state
  const float* out;  // in = WRITE: layer branch a + f
  const float* s0;   // in = WRITE: streams before the write
  const float* s1;
  const float* write_w; const float* write_b;  // this exec's write params
  const float* P;          // this exec's 2x2 mix matrix (row-major), precomputed
  const float* read_w; const float* read_b;                      // next exec's read params
  const uint16_t* norm_g;  // next exec's attn_norm gain (bf16)
  float* s0_out; float* s1_out; float* x_out;  // out = READ
  float* h_out;            // in = WRITE, out != READ: merged h
  uint16_t* xn;            // normed input of the next exec (bf16)
};
hipError_t launch_transition(TransitionArgs t, hipStream_t s);
hipError_t launch_tap(const float* h, const float* s0, const float* s1, float* dst, int B, int T, int d,
                      hipStream_t s);
hipError_t launch_sinkhorn(const float* mix, int iters, float* out, hipStream_t s);
// mix matrices of up to 64 layers in one launch: out[4 l ..] = Sinkhorn(mix[l])
struct SinkhornBatch {
  const float* mix[64];
  int n, iters;
  float* out;
};
hipError_t launch_sinkhorn_layers(const SinkhornBatch& sb, hipStream_t s);
int argmax_chunks(int64_t n);
hipError_t launch_argmax(const float* x, int rows, int64_t n, float* pv, int* pi, int32_t* out, hipStream_t s);
// pos[b] += 1 for b < B (the positions of a replayed decode graph)
hipError_t launch_advance_pos(int32_t* pos, int B, hipStream_t s);

// ---- attention
struct AttnPrepArgs {
  const uint16_t* proj; int64_t proj_stride;  // [M][..]: q | gate | k | v
  int T, Hq, Hkv, D, R, max_seq;
  float theta, eps;
  const int32_t* pos;       // device [B] first position of the call
  const int32_t* seq_slot;  // device [B]
  const uint16_t* k_norm;
  uint16_t* k_cache;        // K block of the exec slot: [max_batch][Hkv][max_seq][D]
  uint16_t* v_cache;        // V block: [max_batch][Hkv][D][max_seq]
  float* rope;              // out: [M][R/2] (cos, sin) of each token's position
};
hipError_t launch_attn_prep(const AttnPrepArgs& a, int M, hipStream_t s);

// The attention kernels take the queries straight from the projection (row
// stride q_stride, head h at h * D) and apply QK-norm (gain q_norm, eps) and
// the partial rotary (first R dims; cos / sin of each token's position from
// the table the prep kernel wrote, rope [M][R/2]) themselves.
struct FlashArgs {
  const uint16_t* q; int64_t q_stride; const uint16_t* q_norm; int R; float eps; const float* rope;
  int T, Hq, Hkv, D, max_seq;
  const int32_t* pos; const int32_t* seq_slot;
  const uint16_t* k_cache; const uint16_t* v_cache;
  float scale_log2;
  const uint16_t* gate; int64_t gate_stride;
  uint16_t* out; int64_t out_stride;
};
hipError_t launch_flash_prefill(const FlashArgs& a, int B, hipStream_t s);

// Decode attention splits the keys of a sequence into DEC_SPLIT_KEYS-key
// pieces (one workgroup each); contexts of up to DEC_SPLIT_KEYS *
// DEC_MAX_SPLITS positions.
constexpr int DEC_SPLIT_KEYS = 1024;
constexpr int DEC_MAX_SPLITS = 1024;
struct DecodeAttnArgs {
  const uint16_t* q; int64_t q_stride; const uint16_t* q_norm; int R; float eps; const float* rope;
  int Hq, Hkv, D, max_seq;
  const int32_t* pos;  // device [B]: position of the new token (keys 0..pos)
  const int32_t* seq_slot;
  const uint16_t* k_cache; const uint16_t* v_cache;
  float scale_log2;
  int split_len, n_split;
  float* partial;      // [B][Hq][n_split][D + 2]
  const uint16_t* gate; int64_t gate_stride;
  uint16_t* out; int64_t out_stride;
};
hipError_t launch_decode_attn(const DecodeAttnArgs& a, int B, hipStream_t s);

// ---- Gated-DeltaNet
struct GdnArgs {
  const uint16_t* proj; int64_t proj_stride;
  int off_q, off_k, off_v, off_z, off_a, off_b;
  int H, Dk, T, n_chunks;
  float eps, q_scale;
  const int32_t* pos; const int32_t* seq_slot;
  float* state;  // state block of the exec slot: [max_batch][H][Dv][Dk]
  // chunk workspace, per (seq, head, chunk) at (seq H + head) n_chunks + chunk:
  float* W;      // W: fp32 [64][Dk]
  float* Ut;     // U~^T: fp32 [Dv][64] (prep); the scan overwrites it with U^T
  float* Mq;     // Mqk: fp32 [64][64]
  uint16_t* Kt;  // raw k of the chunk transposed: bf16 [Dk][64] (16-byte groups swizzled)
  float* sc;     // row scales: sq [64], dk [64], gC (gdn_chunk_scales() floats)
  float* Oq;     // Q S^T with the state entering the chunk (raw q): fp32 [64][Dv]
  const uint16_t* o_norm;
  uint16_t* out; int64_t out_stride;
};
int gdn_chunks(int T);
int gdn_chunk_scales();
hipError_t launch_gdn_prefill(const GdnArgs& a, int B, hipStream_t s);
hipError_t launch_gdn_recurrent(const GdnArgs& a, int B, hipStream_t s);
