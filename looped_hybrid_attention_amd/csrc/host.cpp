// Host side of the C ABI: argument validation, sizes, the execution
// schedule, error reporting, single-operation entry points and synthetic
// input generation.  The model entry points live in model.cpp.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "host.h"

static thread_local char g_err[512] = "";

int loop_fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int loop_hip_fail(hipError_t e, const char* what) {
  return loop_fail(LOOP_EHIP, "%s: %s", what, hipGetErrorString(e));
}

extern "C" const char* loop_last_error(void) { return g_err; }

// ------------------------------------------------------------ schedule
// [P1 section 2]: head [0, loop_start), block [loop_start, loop_end) run
// loop_passes times, tail [loop_end, n_layers).  [P1 section 3]: layer l is
// full attention iff l % 4 == 3 (three GDN layers then one full layer per
// group).  [P1 section 4]: one cache slot per execution (rank among its kind).
int build_schedule(const loop_config& c, std::vector<ExecDesc>& out) {
  out.clear();
  std::vector<int> layers;
  for (int l = 0; l < c.loop_start; ++l) layers.push_back(l);
  for (int p = 0; p < c.loop_passes; ++p)
    for (int l = c.loop_start; l < c.loop_end; ++l) layers.push_back(l);
  for (int l = c.loop_end; l < c.n_layers; ++l) layers.push_back(l);
  const int n_loop = (c.loop_end - c.loop_start) * c.loop_passes;
  const int first = c.loop_start, last = c.loop_start + n_loop - 1;
  int nf = 0, ng = 0;
  for (int e = 0; e < (int)layers.size(); ++e) {
    ExecDesc d;
    d.layer = layers[e];
    d.full = (d.layer % 4) == 3;
    d.slot = d.full ? nf++ : ng++;
    d.loop = n_loop > 0 && e >= first && e <= last;
    d.fork = d.loop && e == first;
    d.merge = d.loop && e == last;
    out.push_back(d);
  }
  return (int)out.size();
}

int validate_config(const loop_config* c) {
  if (!c) return loop_fail(LOOP_EINVAL, "config is NULL");
  if (c->n_layers <= 0 || c->n_layers % 4 || c->loop_start % 4 || c->loop_end % 4 ||
      c->loop_start < 0 || c->loop_end < c->loop_start || c->loop_end > c->n_layers)
    return loop_fail(LOOP_ESHAPE, "layer count and loop bounds must be multiples of 4 with 0 <= start <= end <= n_layers");
  if (c->loop_passes < 1) return loop_fail(LOOP_ESHAPE, "loop_passes must be >= 1");
  if (c->n_streams != 2) return loop_fail(LOOP_ESHAPE, "only 2 residual streams are supported");
  if (c->sinkhorn_iters < 0 || c->sinkhorn_iters > 1000) return loop_fail(LOOP_ESHAPE, "sinkhorn_iters out of range");
  if (c->head_dim != 64 && c->head_dim != 256) return loop_fail(LOOP_ESHAPE, "head_dim must be 64 or 256");
  if (c->rotary_dim < 0 || c->rotary_dim % 2 || c->rotary_dim > c->head_dim)
    return loop_fail(LOOP_ESHAPE, "rotary_dim must be even and <= head_dim");
  if (c->n_kv_heads <= 0 || c->n_q_heads <= 0 || c->n_q_heads % c->n_kv_heads)
    return loop_fail(LOOP_ESHAPE, "n_q_heads must be a positive multiple of n_kv_heads");
  if (c->gdn_dk != c->gdn_dv || (c->gdn_dk != 64 && c->gdn_dk != 128) || c->gdn_heads <= 0)
    return loop_fail(LOOP_ESHAPE, "gdn_dk == gdn_dv in {64, 128} required");
  if (c->gdn_chunk != 64) return loop_fail(LOOP_ESHAPE, "gdn_chunk must be 64");
  if (c->d_model <= 0 || c->d_model % 256) return loop_fail(LOOP_ESHAPE, "d_model must be a multiple of 256");
  if (c->loop_end - c->loop_start > 64) return loop_fail(LOOP_ESHAPE, "at most 64 layers in the loop block");
  if (c->d_ff <= 0 || c->d_ff % 64) return loop_fail(LOOP_ESHAPE, "d_ff must be a multiple of 64");
  if ((c->n_q_heads * c->head_dim) % 64 || (c->gdn_heads * c->gdn_dv) % 64)
    return loop_fail(LOOP_ESHAPE, "attention / GDN widths must be multiples of 64");
  if (c->vocab < 0) return loop_fail(LOOP_ESHAPE, "vocab must be >= 0");
  if (c->max_batch <= 0 || c->max_seq <= 0 || c->max_tokens <= 0)
    return loop_fail(LOOP_ECAPACITY, "max_batch, max_seq and max_tokens must be positive");
  if (c->max_seq % 64) return loop_fail(LOOP_ESHAPE, "max_seq must be a multiple of 64");
  if (c->max_seq > (int64_t)DEC_SPLIT_KEYS * DEC_MAX_SPLITS)
    return loop_fail(LOOP_ECAPACITY, "max_seq %d above %d", c->max_seq, DEC_SPLIT_KEYS * DEC_MAX_SPLITS);
  if (!(c->eps > 0.f)) return loop_fail(LOOP_ESHAPE, "eps must be positive");
  return 0;
}

static void exec_counts(const loop_config& c, int* n_full, int* n_gdn) {
  std::vector<ExecDesc> s;
  build_schedule(c, s);
  *n_full = *n_gdn = 0;
  for (auto& d : s) (d.full ? *n_full : *n_gdn) += 1;
}

// [P1 section 4]: bf16 K and V per KV head and head dim, per full execution.
extern "C" int64_t loop_kv_bytes(const loop_config* c, int32_t batch, int64_t seq_len) {
  if (validate_config(c) || batch < 0 || seq_len < 0) return -1;
  int nf, ng;
  exec_counts(*c, &nf, &ng);
  return (int64_t)nf * 2 * c->n_kv_heads * c->head_dim * 2 * (int64_t)batch * seq_len;
}

extern "C" int64_t loop_state_bytes(const loop_config* c, int32_t batch) {
  if (validate_config(c) || batch < 0) return -1;
  int nf, ng;
  exec_counts(*c, &nf, &ng);
  return (int64_t)ng * c->gdn_heads * c->gdn_dk * c->gdn_dv * 4 * (int64_t)batch;
}

extern "C" int64_t loop_arena_bytes(const loop_config* c) {
  if (validate_config(c)) return -1;
  return loop_kv_bytes(c, c->max_batch, c->max_seq) + loop_state_bytes(c, c->max_batch);
}

extern "C" int64_t loop_cache_offset(const loop_config* c, int32_t which, int32_t slot, int32_t b) {
  if (validate_config(c)) return -1;
  int nf, ng;
  exec_counts(*c, &nf, &ng);
  if (b < 0 || b >= c->max_batch) return -1;
  // exec slot s: K of all sequence slots, then V of all sequence slots
  const int64_t kv_one = (int64_t)c->n_kv_heads * c->max_seq * c->head_dim * 2;  // bytes of K (or V)
  if (which == 0 || which == 1) {
    if (slot < 0 || slot >= nf) return -1;
    return ((int64_t)slot * 2 + which) * c->max_batch * kv_one + (int64_t)b * kv_one;
  }
  if (which == 2) {
    if (slot < 0 || slot >= ng) return -1;
    const int64_t st_one = (int64_t)c->gdn_heads * c->gdn_dv * c->gdn_dk * 4;
    return loop_kv_bytes(c, c->max_batch, c->max_seq) + ((int64_t)slot * c->max_batch + b) * st_one;
  }
  return -1;
}

extern "C" int32_t loop_schedule(const loop_config* c, int32_t* out, int32_t cap) {
  if (int e = validate_config(c)) return e;
  std::vector<ExecDesc> s;
  int n = build_schedule(*c, s);
  if (out) {
    if (cap < n) return loop_fail(LOOP_ECAPACITY, "schedule needs %d rows", n);
    for (int i = 0; i < n; ++i) {
      int32_t* r = out + 6 * i;
      r[0] = s[i].layer; r[1] = s[i].full; r[2] = s[i].slot;
      r[3] = s[i].loop; r[4] = s[i].fork; r[5] = s[i].merge;
    }
  }
  return n;
}

// ------------------------------------------------------ single operations

extern "C" int loop_op_gemm(const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                            int64_t ldc, const float* R, int32_t M, int32_t N, int32_t K,
                            int32_t epi, float* d_ws, size_t ws_bytes, void* stream) {
  if (!A || !B || !C) return loop_fail(LOOP_EINVAL, "gemm: null operand");
  if (epi < 0 || epi > 3) return loop_fail(LOOP_EINVAL, "gemm: bad epilogue %d", epi);
  if (epi == LOOP_EPI_F32_RES && !R) return loop_fail(LOOP_EINVAL, "gemm: residual epilogue needs R");
  if (M < 0 || N <= 0 || K <= 0 || K % 64) return loop_fail(LOOP_ESHAPE, "gemm: need N > 0, K > 0, K %% 64 == 0");
  if (lda % 8 || ldb % 8 || lda < K || ldb < K || ldc < N)
    return loop_fail(LOOP_ESHAPE, "gemm: lda, ldb must be multiples of 8 and cover K; ldc >= N");
  if (((uintptr_t)A | (uintptr_t)B) % 16) return loop_fail(LOOP_EINVAL, "gemm: A and B must be 16-byte aligned");
  if (M == 0) return 0;
  hipError_t e = launch_gemm(A, lda, B, ldb, C, ldc, R, M, N, K, epi, (hipStream_t)stream, d_ws,
                             d_ws ? ws_bytes : 0);
  return e == hipSuccess ? 0 : loop_hip_fail(e, "gemm launch");
}

extern "C" int loop_op_gemm_quant(int32_t bits, const void* A, int64_t lda, const void* Bq, int64_t ldq,
                                  const float* scale, void* C, int64_t ldc, const float* R, int32_t M, int32_t N,
                                  int32_t K, int32_t epi, float* d_ws, size_t ws_bytes, void* stream) {
  if (bits != 8 && bits != 4) return loop_fail(LOOP_EINVAL, "gemm_quant: bits must be 8 or 4");
  if (!A || !Bq || !scale || !C) return loop_fail(LOOP_EINVAL, "gemm_quant: null operand");
  if (epi < 0 || epi > 3) return loop_fail(LOOP_EINVAL, "gemm_quant: bad epilogue %d", epi);
  if (epi == LOOP_EPI_F32_RES && !R) return loop_fail(LOOP_EINVAL, "gemm_quant: residual epilogue needs R");
  if (M < 1 || M > 64 || N <= 0 || K <= 0 || K % 128)
    return loop_fail(LOOP_ESHAPE, "gemm_quant: need 1 <= M <= 64, N > 0, K > 0, K %% 128 == 0");
  const int64_t row_bytes = bits == 8 ? K : K / 2;
  if (lda % 8 || lda < K || ldq % 16 || ldq < row_bytes || ldc < N)
    return loop_fail(LOOP_ESHAPE, "gemm_quant: lda %% 8, lda >= K, ldq %% 16, ldq >= %lld, ldc >= N",
                     (long long)row_bytes);
  if (((uintptr_t)A | (uintptr_t)Bq) % 16) return loop_fail(LOOP_EINVAL, "gemm_quant: A and Bq must be 16-byte aligned");
  hipError_t e = launch_gemm_wq(bits, A, lda, Bq, ldq, scale, C, ldc, R, M, N, K, epi, (hipStream_t)stream, d_ws,
                                d_ws ? ws_bytes : 0);
  return e == hipSuccess ? 0 : loop_hip_fail(e, "gemm_quant launch");
}

// ------------------------------------------------------- synthetic inputs

extern "C" int loop_synth_normal(void* dst, int64_t n, int32_t dtype, uint32_t seed, uint32_t key,
                                 int64_t start, double std, double mean, void* stream) {
  if (!dst && n > 0) return loop_fail(LOOP_EINVAL, "synth: null destination");
  if (dtype != 0 && dtype != 1) return loop_fail(LOOP_EINVAL, "synth: dtype must be 0 (fp32) or 1 (bf16)");
  if (n < 0 || start < 0) return loop_fail(LOOP_EINVAL, "synth: negative size");
  hipError_t e = launch_synth_normal(dst, n, dtype, seed, key, start, std, mean, (hipStream_t)stream);
  return e == hipSuccess ? 0 : loop_hip_fail(e, "synth launch");
}

extern "C" int loop_quantize_int8(const void* d_w, int64_t N, int64_t K, int64_t ldw, int8_t* d_q, float* d_scale,
                                  void* stream) {
  if (!d_w || !d_q || !d_scale) return loop_fail(LOOP_EINVAL, "quantize: NULL buffer");
  if (N < 1 || K < 1 || ldw < K || K > (1 << 30) || N > (1ll << 31))
    return loop_fail(LOOP_EINVAL, "quantize: bad shape N %lld K %lld ldw %lld", (long long)N, (long long)K, (long long)ldw);
  hipError_t e = launch_quantize_int8(d_w, ldw, N, (int)K, d_q, K, d_scale, (hipStream_t)stream);
  return e == hipSuccess ? 0 : loop_hip_fail(e, "quantize_int8");
}

extern "C" int loop_quantize_int4(const void* d_w, int64_t N, int64_t K, int64_t ldw, uint8_t* d_q, float* d_scale,
                                  void* stream) {
  if (!d_w || !d_q || !d_scale) return loop_fail(LOOP_EINVAL, "quantize: NULL buffer");
  if (N < 1 || K < 1 || K % 128 || ldw < K || K > (1 << 30) || N > (1ll << 31))
    return loop_fail(LOOP_EINVAL, "quantize_int4: bad shape N %lld K %lld ldw %lld (K a multiple of 128)",
                     (long long)N, (long long)K, (long long)ldw);
  hipError_t e = launch_quantize_int4(d_w, ldw, N, (int)K, d_q, K / 2, d_scale, (hipStream_t)stream);
  return e == hipSuccess ? 0 : loop_hip_fail(e, "quantize_int4");
}

extern "C" int loop_synth_token_ids(int32_t* dst, int64_t n, uint32_t vocab, uint32_t seed,
                                    uint32_t key, void* stream) {
  if (!dst && n > 0) return loop_fail(LOOP_EINVAL, "synth: null destination");
  if (n < 0 || vocab == 0) return loop_fail(LOOP_EINVAL, "synth: need n >= 0 and vocab > 0");
  hipError_t e = launch_synth_token_ids(dst, n, vocab, seed, key, (hipStream_t)stream);
  return e == hipSuccess ? 0 : loop_hip_fail(e, "synth launch");
}
